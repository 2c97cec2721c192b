"""Helpers for the GPU parity tests: move seeded inputs to the device, call
the library through its binding, and compare with the oracle."""
import numpy as np
import torch

import workloads as W

DEV = "cuda:0"


def dev(x, dtype=None):
    """numpy array or workloads.Stored -> device tensor (bf16 from its bits)."""
    if isinstance(x, W.Stored):
        if x.dtype == W.BF16:
            return torch.from_numpy(np.ascontiguousarray(x.bits).view(np.int16)).view(
                torch.bfloat16).to(DEV)
        return torch.from_numpy(np.ascontiguousarray(x.bits)).to(DEV)
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def kvcache(c):
    from speculative_decoding_attention_amd import KVCache
    return KVCache(dev(c.k), dev(c.v), dev(c.kv_len.astype(np.int32)),
                   page_table=dev(c.page_table.astype(np.int32)) if c.page_size else None,
                   page_size=c.page_size, max_len=c.max_len)


def oracle_kv(c):
    return dict(page_table=c.page_table, page_size=c.page_size)


def assert_attention_close(out, lse, ref_o, ref_l, q_len, dtype, tag=""):
    """Contract tolerance (1e-5 fp32, 2e-2 bf16) plus scale-aware guards:
    per (sequence, head) max error <= 1e-2 * max|O_ref| for bf16 inputs, and
    |LSE - LSE_ref| <= 1e-3 (both only on real rows; padded rows must be
    exactly O = 0 and LSE = -inf)."""
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    B, n_max, Hq, d = o.shape
    tol = 1e-5 if dtype == W.F32 else 2e-2
    for b in range(B):
        nb = int(q_len[b])
        err = np.abs(o[b, :nb] - ref_o[b, :nb])
        assert err.max(initial=0) <= tol, f"{tag} b={b} max err {err.max()}"
        if dtype == W.BF16 and nb:
            for h in range(Hq):
                scale = np.abs(ref_o[b, :nb, h]).max()
                e = err[:, h].max()
                assert e <= 1e-2 * scale + 1e-7, f"{tag} b={b} h={h} err {e} vs scale {scale}"
        lr = ref_l[b, :nb]
        fin = np.isfinite(lr)
        assert np.array_equal(fin, np.isfinite(l[b, :nb])), f"{tag} b={b} lse finiteness"
        if fin.any():
            le = np.abs(l[b, :nb][fin] - lr[fin]).max()
            assert le <= 1e-3, f"{tag} b={b} lse err {le}"
        assert np.all(o[b, nb:] == 0), f"{tag} padded rows must be zero"
        assert np.all(np.isneginf(l[b, nb:])), f"{tag} padded LSE must be -inf"

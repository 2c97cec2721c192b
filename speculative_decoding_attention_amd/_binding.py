"""ctypes binding of libspecattn (the C ABI declared in include/specattn.h).

Argument marshalling only: every step of the hot path runs in the HIP
library.  PyTorch provides device memory and the current stream.  Loading
fails loudly when the library has not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspecattn.so")

SPEC_F32 = 0
SPEC_BF16 = 1
SPEC_ABI_VERSION = 4
SPEC_WS_SYNC_BYTES = 1 << 20
SPEC_NOALLOC_SCRATCH_BYTES = 32 << 20

STATUS = {
    0: "SPEC_OK", 1: "SPEC_ERR_NULL", 2: "SPEC_ERR_SHAPE", 3: "SPEC_ERR_DTYPE",
    4: "SPEC_ERR_WORKSPACE", 5: "SPEC_ERR_UNSUPPORTED", 6: "SPEC_ERR_HIP",
}

# Every function the header declares, with its ctypes signature.
_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float
_S = ctypes.c_size_t


class SpecKV(ctypes.Structure):
    """Mirror of ``spec_kv_t``."""

    _fields_ = [("k", _P), ("v", _P), ("dtype", _I), ("num_kv_heads", _I), ("head_dim", _I),
                ("max_len", _I), ("kv_len", _P), ("page_size", _I), ("max_pages", _I),
                ("page_table", _P)]


_KVP = ctypes.POINTER(SpecKV)

SIGNATURES = {
    "spec_verify_attn_workspace": (_S, [_KVP, _I, _I, _I]),
    "spec_verify_attn": (_I, [_KVP, _I, _P, _I, _I, _P, _I, _F, _P, _I, _P, _P, _S, _P]),
    "spec_verify_attn_noalloc": (_I, [_KVP, _I, _P, _I, _I, _P, _I, _F, _P, _I, _P, _P]),
    "spec_vata_attn_workspace": (_S, [_KVP, _I, _I, _I, _I]),
    "spec_vata_attn": (_I, [_KVP, _I, _P, _I, _I, _P, _I, _P, _P, _I, _F, _P, _I, _P, _P, _S, _P]),
    "spec_topk_attn_workspace": (_S, [_KVP, _I, _I, _I]),
    "spec_topk_attn": (_I, [_KVP, _I, _P, _I, _I, _I, _F, _P, _P, _I, _P, _P, _S, _P]),
    "spec_hsr_fuse_workspace": (_S, [_I, _I]),
    "spec_hsr_fuse": (_I, [_P, _P, _P, _I, _I, _I, _P, _I, _P, _S, _P]),
    "spec_accept_workspace": (_S, [_I, _I, _I]),
    "spec_accept": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _S, _P]),
    "spec_status_str": (ctypes.c_char_p, [_I]),
    "spec_std_select_workspace": (_S, [_KVP, _I, _I, _I, _I]),
    "spec_std_select": (_I, [_KVP, _I, _P, _I, _I, _P, _P, _I, _I, _F, _P, _P, _P, _P, _P, _S,
                             _P]),
    "spec_sparse_attn_workspace": (_S, [_KVP, _I, _I, _I, _I, _I]),
    "spec_sparse_attn": (_I, [_KVP, _I, _P, _I, _I, _P, _I, _P, _P, _I, _P, _I, _F, _P, _I, _P,
                              _P, _S, _P]),
    "spec_commit": (_I, [_I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _I, _P]),
    "spec_abi_version": (_I, []),
    "spec_set_debug": (_I, [_I]),
    "spec_mark_main_kernel": (_I, [_P, _P]),
    "spec_read_probe": (_I, [_P, ctypes.c_size_t, _P, _P]),
}


class SpecError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {STATUS.get(status, status)}")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"libspecattn is not built ({path} missing); run "
                          "`python -m speculative_decoding_attention_amd.build` first")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.spec_abi_version() != SPEC_ABI_VERSION:
        raise ImportError("libspecattn ABI version mismatch")
    return lib


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = load_library()
    return _lib


# ---------------------------------------------------------------- helpers --

def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return SPEC_F32
    if t == torch.bfloat16:
        return SPEC_BF16
    raise TypeError(f"unsupported dtype {t}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype=None) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(fn: str, st: int):
    if st != 0:
        raise SpecError(fn, st)


class Workspace:
    """A device scratch buffer, grown on demand.

    A new buffer is zero-filled once: its first SPEC_WS_SYNC_BYTES bytes hold
    the library's synchronisation words, which every call leaves at zero, so
    one workspace serves consecutive calls of any entry point on one stream
    (never two overlapping calls).
    """

    def __init__(self, device=None):
        self.device = torch.device(device) if device is not None else None
        self.buf: Optional[torch.Tensor] = None

    def get(self, nbytes: int, device: torch.device):
        if nbytes == 0:
            return None, 0
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
            self.buf = torch.zeros(max(nbytes, SPEC_WS_SYNC_BYTES), dtype=torch.uint8, device=device)
        return ctypes.c_void_p(self.buf.data_ptr()), self.buf.numel()


_default_ws = {}


def _workspace(ws: Optional[Workspace], device: torch.device) -> Workspace:
    if ws is not None:
        return ws
    key = (device.type, device.index)
    if key not in _default_ws:
        _default_ws[key] = Workspace(device)
    return _default_ws[key]


class KVCache:
    """Descriptor of a KV cache held in torch device tensors.

    Contiguous: k, v ``[B, Hkv, max_len, d]``.  Paged: k, v
    ``[num_pages, Hkv, page_size, d]`` with ``page_table [B, max_pages]``
    int32 and a host-side bound ``max_len`` on the lengths.
    """

    def __init__(self, k: torch.Tensor, v: torch.Tensor, kv_len: torch.Tensor,
                 page_table: Optional[torch.Tensor] = None, page_size: int = 0,
                 max_len: Optional[int] = None):
        _dev(k, "k")
        _dev(v, "v", k.dtype)
        _dev(kv_len, "kv_len", torch.int32)
        if k.shape != v.shape or k.dim() != 4:
            raise ValueError("k and v must have the same 4-d shape")
        self.k, self.v, self.kv_len = k, v, kv_len
        self.page_size = int(page_size)
        self.page_table = page_table
        if self.page_size:
            _dev(page_table, "page_table", torch.int32)
            if k.shape[2] != self.page_size:
                raise ValueError("paged k/v must be [num_pages, Hkv, page_size, d]")
            if max_len is None:
                raise ValueError("paged caches need a host-side max_len bound")
            self.max_len = int(max_len)
        else:
            self.max_len = int(k.shape[2]) if max_len is None else int(max_len)
            if self.max_len != k.shape[2]:
                raise ValueError("contiguous max_len must equal k.shape[2]")
        self.struct = SpecKV(
            k.data_ptr(), v.data_ptr(), _dtype_code(k.dtype), int(k.shape[1]), int(k.shape[3]),
            self.max_len, kv_len.data_ptr(), self.page_size,
            int(page_table.shape[1]) if self.page_size else 0,
            page_table.data_ptr() if self.page_size else None)

    @property
    def num_kv_heads(self) -> int:
        return int(self.k.shape[1])

    @property
    def head_dim(self) -> int:
        return int(self.k.shape[3])

    @property
    def device(self) -> torch.device:
        return self.k.device


# -------------------------------------------------------- entry points ----

def spec_verify_attn(kv: KVCache, q: torch.Tensor, q_len: Optional[torch.Tensor] = None,
                     scale: Optional[float] = None, out_dtype: Optional[torch.dtype] = None,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     want_lse: bool = True, workspace: Optional[Workspace] = None):
    """Dense verification attention; returns (out, lse)."""
    L = lib()
    _dev(q, "q", kv.k.dtype)
    B, n_max, Hq, d = q.shape
    if q_len is not None:
        _dev(q_len, "q_len", torch.int32)
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty((B, n_max, Hq, d), dtype=out_dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, n_max, Hq), dtype=torch.float32, device=q.device)
    scale = float(d ** -0.5) if scale is None else float(scale)
    need = L.spec_verify_attn_workspace(ctypes.byref(kv.struct), B, n_max, Hq)
    wsp, wsn = _workspace(workspace, q.device).get(need, q.device)
    st = L.spec_verify_attn(ctypes.byref(kv.struct), B, _ptr(q), _dtype_code(q.dtype), n_max,
                            _ptr(q_len), Hq, scale, _ptr(out), _dtype_code(out.dtype), _ptr(lse),
                            wsp, wsn, _stream(q.device))
    _check("spec_verify_attn", st)
    return out, lse


def spec_verify_attn_noalloc(kv: KVCache, q: torch.Tensor, out: torch.Tensor,
                             lse: Optional[torch.Tensor] = None,
                             q_len: Optional[torch.Tensor] = None,
                             scale: Optional[float] = None):
    """Dense verification attention into caller-provided `out` (and `lse`)
    with no device allocation: the library's own scratch holds the split
    partials.  Returns (out, lse)."""
    L = lib()
    _dev(q, "q", kv.k.dtype)
    _dev(out, "out")
    B, n_max, Hq, d = q.shape
    if tuple(out.shape) != (B, n_max, Hq, d):
        raise ValueError("out must have the shape of q")
    if lse is not None:
        _dev(lse, "lse", torch.float32)
        if tuple(lse.shape) != (B, n_max, Hq):
            raise ValueError("lse must be [B, n_max, Hq]")
    if q_len is not None:
        _dev(q_len, "q_len", torch.int32)
    scale = float(d ** -0.5) if scale is None else float(scale)
    st = L.spec_verify_attn_noalloc(ctypes.byref(kv.struct), B, _ptr(q), _dtype_code(q.dtype),
                                    n_max, _ptr(q_len), Hq, scale, _ptr(out),
                                    _dtype_code(out.dtype), _ptr(lse), _stream(q.device))
    _check("spec_verify_attn_noalloc", st)
    return out, lse


def spec_vata_attn(kv: KVCache, q: torch.Tensor, text_idx: torch.Tensor, text_len: torch.Tensor,
                   q_len: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                   out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                   workspace: Optional[Workspace] = None):
    """Text-anchored draft attention over text_idx; returns (out, lse)."""
    L = lib()
    _dev(q, "q", kv.k.dtype)
    _dev(text_idx, "text_idx", torch.int32)
    _dev(text_len, "text_len", torch.int32)
    B, n_max, Hq, d = q.shape
    t_max = int(text_idx.shape[1])
    if q_len is not None:
        _dev(q_len, "q_len", torch.int32)
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty((B, n_max, Hq, d), dtype=out_dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, n_max, Hq), dtype=torch.float32, device=q.device)
    scale = float(d ** -0.5) if scale is None else float(scale)
    need = L.spec_vata_attn_workspace(ctypes.byref(kv.struct), B, n_max, Hq, t_max)
    wsp, wsn = _workspace(workspace, q.device).get(need, q.device)
    st = L.spec_vata_attn(ctypes.byref(kv.struct), B, _ptr(q), _dtype_code(q.dtype), n_max,
                          _ptr(q_len), Hq, _ptr(text_idx), _ptr(text_len), t_max, scale,
                          _ptr(out), _dtype_code(out.dtype), _ptr(lse), wsp, wsn,
                          _stream(q.device))
    _check("spec_vata_attn", st)
    return out, lse


def spec_topk_attn(kv: KVCache, q: torch.Tensor, top_k: int, scale: Optional[float] = None,
                   out_dtype: Optional[torch.dtype] = None, sel_idx: Optional[torch.Tensor] = None,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   want_lse: bool = True, workspace: Optional[Workspace] = None):
    """Top-K sparse draft attention for one query row; returns (sel_idx, out, lse)."""
    L = lib()
    _dev(q, "q", kv.k.dtype)
    B, one, Hq, d = q.shape
    if one != 1:
        raise ValueError("q must be [B, 1, Hq, d]")
    out_dtype = out_dtype or q.dtype
    if sel_idx is None:
        sel_idx = torch.empty((B, kv.num_kv_heads, top_k), dtype=torch.int32, device=q.device)
    if out is None:
        out = torch.empty((B, 1, Hq, d), dtype=out_dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, 1, Hq), dtype=torch.float32, device=q.device)
    scale = float(d ** -0.5) if scale is None else float(scale)
    need = L.spec_topk_attn_workspace(ctypes.byref(kv.struct), B, Hq, top_k)
    wsp, wsn = _workspace(workspace, q.device).get(need, q.device)
    st = L.spec_topk_attn(ctypes.byref(kv.struct), B, _ptr(q), _dtype_code(q.dtype), Hq, int(top_k),
                          scale, _ptr(sel_idx), _ptr(out), _dtype_code(out.dtype), _ptr(lse),
                          wsp, wsn, _stream(q.device))
    _check("spec_topk_attn", st)
    return sel_idx, out, lse


def spec_std_select(kv: KVCache, q_text: torch.Tensor, text_idx: torch.Tensor,
                    text_len: torch.Tensor, top_k: int, scale: Optional[float] = None,
                    want_keep: bool = True, want_score: bool = False,
                    sel_idx: Optional[torch.Tensor] = None,
                    keep_idx: Optional[torch.Tensor] = None,
                    keep_len: Optional[torch.Tensor] = None,
                    score: Optional[torch.Tensor] = None,
                    workspace: Optional[Workspace] = None):
    """Sparse-to-Dense prefill selection for one layer; returns
    (sel_idx, keep_idx, keep_len, score), the last three None unless asked."""
    L = lib()
    _dev(q_text, "q_text", kv.k.dtype)
    _dev(text_idx, "text_idx", torch.int32)
    _dev(text_len, "text_len", torch.int32)
    B, t_max, Hq, d = q_text.shape
    Hkv = kv.num_kv_heads
    dev = q_text.device
    if sel_idx is None:
        sel_idx = torch.empty((B, Hkv, top_k), dtype=torch.int32, device=dev)
    if want_keep and keep_idx is None:
        keep_idx = torch.empty((B, Hkv, top_k + t_max), dtype=torch.int32, device=dev)
    if keep_idx is not None and keep_len is None:
        keep_len = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    if want_score and score is None:
        score = torch.empty((B, Hkv, kv.max_len), dtype=torch.float32, device=dev)
    scale = float(d ** -0.5) if scale is None else float(scale)
    need = L.spec_std_select_workspace(ctypes.byref(kv.struct), B, Hq, t_max, int(top_k))
    wsp, wsn = _workspace(workspace, dev).get(need, dev)
    st = L.spec_std_select(ctypes.byref(kv.struct), B, _ptr(q_text), _dtype_code(q_text.dtype), Hq,
                           _ptr(text_idx), _ptr(text_len), t_max, int(top_k), scale,
                           _ptr(sel_idx), _ptr(keep_idx), _ptr(keep_len), _ptr(score), wsp, wsn,
                           _stream(dev))
    _check("spec_std_select", st)
    return sel_idx, keep_idx, keep_len, score


def spec_sparse_attn(kv: KVCache, q: torch.Tensor, list_idx: torch.Tensor,
                     list_len: torch.Tensor, tail_start: Optional[torch.Tensor] = None,
                     tail_max: int = 0, q_len: Optional[torch.Tensor] = None,
                     scale: Optional[float] = None, out_dtype: Optional[torch.dtype] = None,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     want_lse: bool = True, workspace: Optional[Workspace] = None):
    """Draft attention over per-head lists plus a dense tail (from
    tail_start, or the last tail_max positions without it); returns
    (out, lse)."""
    L = lib()
    _dev(q, "q", kv.k.dtype)
    _dev(list_idx, "list_idx", torch.int32)
    _dev(list_len, "list_len", torch.int32)
    if tail_start is not None:
        _dev(tail_start, "tail_start", torch.int32)
    if q_len is not None:
        _dev(q_len, "q_len", torch.int32)
    B, n_max, Hq, d = q.shape
    list_max = int(list_idx.shape[2])
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty((B, n_max, Hq, d), dtype=out_dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, n_max, Hq), dtype=torch.float32, device=q.device)
    scale = float(d ** -0.5) if scale is None else float(scale)
    tail_max = int(tail_max)
    need = L.spec_sparse_attn_workspace(ctypes.byref(kv.struct), B, n_max, Hq, list_max, tail_max)
    wsp, wsn = _workspace(workspace, q.device).get(need, q.device)
    st = L.spec_sparse_attn(ctypes.byref(kv.struct), B, _ptr(q), _dtype_code(q.dtype), n_max,
                            _ptr(q_len), Hq, _ptr(list_idx), _ptr(list_len), list_max,
                            _ptr(tail_start), tail_max, scale, _ptr(out), _dtype_code(out.dtype),
                            _ptr(lse), wsp, wsn, _stream(q.device))
    _check("spec_sparse_attn", st)
    return out, lse


def spec_hsr_fuse(e: torch.Tensor, h: torch.Tensor, w: torch.Tensor,
                  out_dtype: torch.dtype = torch.bfloat16, y: Optional[torch.Tensor] = None,
                  workspace: Optional[Workspace] = None):
    """HSR fusion FC: Y = concat(E, H) @ W^T; returns y."""
    L = lib()
    _dev(e, "e", torch.bfloat16)
    _dev(h, "h", torch.bfloat16)
    _dev(w, "w", torch.bfloat16)
    m, d = e.shape
    if h.shape != e.shape or tuple(w.shape) != (d, 2 * d):
        raise ValueError("expected e, h [m, d] and w [d, 2d]")
    if y is None:
        y = torch.empty((m, d), dtype=out_dtype, device=e.device)
    need = L.spec_hsr_fuse_workspace(m, d)
    wsp, wsn = _workspace(workspace, e.device).get(need, e.device)
    st = L.spec_hsr_fuse(_ptr(e), _ptr(h), _ptr(w), SPEC_BF16, m, d, _ptr(y), _dtype_code(y.dtype),
                         wsp, wsn, _stream(e.device))
    _check("spec_hsr_fuse", st)
    return y


def spec_accept(logits: torch.Tensor, draft: torch.Tensor, gamma: Optional[torch.Tensor] = None,
                target_tok: Optional[torch.Tensor] = None,
                accept_len: Optional[torch.Tensor] = None,
                next_tok: Optional[torch.Tensor] = None,
                workspace: Optional[Workspace] = None):
    """Greedy acceptance; returns (target_tok, accept_len, next_tok)."""
    L = lib()
    _dev(logits, "logits")
    B, n_max, V = logits.shape
    _dev(draft, "draft", torch.int32)
    if gamma is not None:
        _dev(gamma, "gamma", torch.int32)
    dev = logits.device
    if target_tok is None:
        target_tok = torch.empty((B, n_max), dtype=torch.int32, device=dev)
    if accept_len is None:
        accept_len = torch.empty((B,), dtype=torch.int32, device=dev)
    if next_tok is None:
        next_tok = torch.empty((B,), dtype=torch.int32, device=dev)
    need = L.spec_accept_workspace(B, n_max, V)
    wsp, wsn = _workspace(workspace, dev).get(need, dev)
    st = L.spec_accept(_ptr(logits), _dtype_code(logits.dtype), B, n_max, V, _ptr(draft),
                       _ptr(gamma), _ptr(target_tok), _ptr(accept_len), _ptr(next_tok), wsp, wsn,
                       _stream(dev))
    _check("spec_accept", st)
    return target_tok, accept_len, next_tok


def spec_commit(draft: torch.Tensor, accept_len: torch.Tensor, next_tok: torch.Tensor,
                kv_len: torch.Tensor, gamma: Optional[torch.Tensor] = None,
                last_tok: Optional[torch.Tensor] = None, tokens: Optional[torch.Tensor] = None,
                tok_len: Optional[torch.Tensor] = None, text_idx: Optional[torch.Tensor] = None,
                text_len: Optional[torch.Tensor] = None) -> None:
    """Post-acceptance bookkeeping on the device; updates kv_len (and the
    optional last_tok, tokens/tok_len, text_idx/text_len) in place."""
    L = lib()
    _dev(draft, "draft", torch.int32)
    for t, name in ((accept_len, "accept_len"), (next_tok, "next_tok"), (kv_len, "kv_len")):
        _dev(t, name, torch.int32)
    for t, name in ((gamma, "gamma"), (last_tok, "last_tok"), (tokens, "tokens"),
                    (tok_len, "tok_len"), (text_idx, "text_idx"), (text_len, "text_len")):
        if t is not None:
            _dev(t, name, torch.int32)
    B, g = draft.shape
    st = L.spec_commit(B, g + 1, _ptr(draft), _ptr(gamma), _ptr(accept_len), _ptr(next_tok),
                       _ptr(kv_len), _ptr(last_tok), _ptr(tokens), _ptr(tok_len),
                       int(tokens.shape[1]) if tokens is not None else 0, _ptr(text_idx),
                       _ptr(text_len), int(text_idx.shape[1]) if text_idx is not None else 0,
                       _stream(kv_len.device))
    _check("spec_commit", st)


def spec_status_str(status: int) -> str:
    return lib().spec_status_str(status).decode()


def spec_abi_version() -> int:
    return int(lib().spec_abi_version())


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence:
    recording it makes no system-scope cache write-back and invalidation, so
    a pair of them around one kernel measures little beyond the kernel.
    elapsed_ms() is valid once the stream has passed both records (after a
    device synchronisation); the event itself orders no memory."""

    _FLAGS = 0x20000000          # hipEventDisableSystemFence
    _hip: Optional[ctypes.CDLL] = None

    @classmethod
    def _rt(cls) -> ctypes.CDLL:
        if cls._hip is None:
            torch.cuda.init()
            # the runtime the process already has (torch's, and the library's)
            h = ctypes.CDLL("libamdhip64.so.7")
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                              ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            for f in (h.hipEventCreateWithFlags, h.hipEventElapsedTime, h.hipEventDestroy):
                f.restype = ctypes.c_int
            cls._hip = h
        return cls._hip

    def __init__(self):
        ev = ctypes.c_void_p()
        rc = self._rt().hipEventCreateWithFlags(ctypes.byref(ev), self._FLAGS)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.handle = ev.value

    def elapsed_ms(self, end: "TimingEvent") -> float:
        ms = ctypes.c_float()
        rc = self._rt().hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def __del__(self):
        if getattr(self, "handle", None) and TimingEvent._hip is not None:
            TimingEvent._hip.hipEventDestroy(self.handle)
            self.handle = None


def _event_handle(e) -> int:
    if isinstance(e, TimingEvent):
        return e.handle
    if not e.cuda_event:
        e.record()
    return e.cuda_event


def mark_main_kernel(before, after) -> None:
    """Measurement hook: the calling thread's next library call records
    `before` right before its main kernel and `after` right after it, on the
    call's stream (see spec_mark_main_kernel), for calls made outside
    stream capture.  Both are timing events of the call's device: TimingEvent
    or torch.cuda.Event (one that has no handle yet is recorded once first to
    make one)."""
    hb, ha = _event_handle(before), _event_handle(after)
    _check("spec_mark_main_kernel",
           lib().spec_mark_main_kernel(ctypes.c_void_p(hb), ctypes.c_void_p(ha)))


SPEC_READ_PROBE_SINK_WORDS = 1024


def read_probe(x: torch.Tensor, sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Measurement aid: one plain streaming read of x's bytes (contiguous,
    16-byte aligned, a multiple of 16 bytes); returns the sink of
    SPEC_READ_PROBE_SINK_WORDS int32 words whose XOR is the XOR of x's
    32-bit words."""
    if not (x.is_cuda and x.is_contiguous()):
        raise ValueError("x must be a contiguous device tensor")
    if sink is None:
        sink = torch.empty(SPEC_READ_PROBE_SINK_WORDS, dtype=torch.int32, device=x.device)
    _dev(sink, "sink", torch.int32)
    if sink.numel() < SPEC_READ_PROBE_SINK_WORDS:
        raise ValueError("sink too small")
    _check("spec_read_probe", lib().spec_read_probe(x.data_ptr(), x.numel() * x.element_size(),
                                                    sink.data_ptr(), _stream(x.device)))
    return sink


def spec_set_debug(on: bool) -> bool:
    """Debug mode on or off for this process: each call then checks its
    device index arrays first (synchronously) and raises SpecError with
    SPEC_ERR_SHAPE if one is out of range.  Returns the previous setting."""
    return bool(lib().spec_set_debug(1 if on else 0))

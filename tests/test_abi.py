"""The C-ABI library builds, loads, exports every function include/specattn.h
declares, and rejects every host-detectable argument error before anything is
enqueued (these calls never reach a launch, so they run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specattn.h")


@pytest.fixture(scope="module")
def L():
    from speculative_decoding_attention_amd import _binding, build
    other = os.environ.get("SPECATTN_TEST_LIB")   # e.g. the host-sanitizer build
    if other:
        return _binding.load_library(other)
    if not os.path.exists(_binding.LIB_PATH):
        build.build_library()
    return _binding.load_library()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:size_t|spec_status_t|const char\*|int32_t)\s+(spec_\w+)\s*\(",
                                 src, flags=re.M)))


def test_header_declares_the_five_entry_points():
    names = _declared_functions()
    for n in ["spec_verify_attn", "spec_vata_attn", "spec_topk_attn", "spec_hsr_fuse",
              "spec_accept"]:
        assert n in names and n + "_workspace" in names


def test_every_declared_symbol_is_exported(L):
    from speculative_decoding_attention_amd import _binding
    for name in _declared_functions():
        assert hasattr(L, name), name
        assert name in _binding.SIGNATURES, name


def test_version_and_status_strings(L):
    assert L.spec_abi_version() == 4
    for code in range(7):
        s = L.spec_status_str(code).decode()
        assert s.startswith("SPEC_")
    assert L.spec_status_str(99).decode() == "unknown spec_status_t"


FAKE = 0x10000   # never dereferenced: every call below fails validation first


def _kv(**over):
    from speculative_decoding_attention_amd._binding import SpecKV
    f = dict(k=FAKE, v=FAKE, dtype=1, num_kv_heads=4, head_dim=128, max_len=1024,
             kv_len=FAKE, page_size=0, max_pages=0, page_table=None)
    f.update(over)
    return SpecKV(**f)


def _verify(L, kv, B=1, q=FAKE, q_dtype=1, n_max=6, Hq=28, scale=0.088, out=FAKE, out_dtype=1,
            ws=None, ws_bytes=0):
    return L.spec_verify_attn(ctypes.byref(kv), B, q, q_dtype, n_max, None, Hq, scale, out,
                              out_dtype, None, ws, ws_bytes, None)


@pytest.mark.parametrize("over,code", [
    (dict(k=None), 1), (dict(kv_len=None), 1), (dict(dtype=7), 3), (dict(head_dim=96), 5),
    (dict(num_kv_heads=0), 2), (dict(max_len=0), 2), (dict(page_size=12), 2),
    (dict(page_size=16, page_table=None, max_pages=4), 1),
    (dict(page_size=16, page_table=FAKE, max_pages=4), 2),     # 4*16 < max_len
])
def test_verify_rejects_bad_kv(L, over, code):
    assert _verify(L, _kv(**over)) == code


def test_verify_rejects_bad_args(L):
    kv = _kv()
    assert _verify(L, kv, q=None) == 1
    assert _verify(L, kv, out=None) == 1
    assert _verify(L, kv, Hq=30) == 2                 # 30 % 4 != 0
    assert _verify(L, kv, B=0) == 2
    assert _verify(L, kv, n_max=0) == 2
    assert _verify(L, kv, q_dtype=0) == 3             # q dtype != kv dtype
    assert _verify(L, kv, out_dtype=5) == 3
    assert _verify(L, kv, n_max=10) == 5              # 10 * 7 rows > 64
    assert _verify(L, kv, scale=float("nan")) == 2
    assert _verify(L, kv, scale=float("inf")) == 2
    assert _verify(L, kv, scale=0.0) == 2             # the kernels need scale > 0
    assert _verify(L, kv, scale=-1.0) == 2
    need = L.spec_verify_attn_workspace(ctypes.byref(kv), 1, 6, 28)
    assert need > 0
    assert _verify(L, kv, ws=None, ws_bytes=0) == 1
    assert _verify(L, kv, ws=FAKE, ws_bytes=need - 1) == 4
    assert _verify(L, kv, ws=FAKE + 128, ws_bytes=need) == 4   # not 256-byte aligned


def test_verify_noalloc_rejects_before_touching_the_device(L):
    """The allocation-free verification checks its arguments as spec_verify_attn
    does, and refuses shapes whose split partials exceed its fixed scratch
    (SPEC_ERR_WORKSPACE), all before any device call."""
    from speculative_decoding_attention_amd import _binding
    kv = _kv()
    call = lambda kv_, B=1, n_max=6, Hq=28, scale=0.088, q=FAKE: L.spec_verify_attn_noalloc(
        ctypes.byref(kv_), B, q, 1, n_max, None, Hq, scale, FAKE, 1, None, None)
    assert call(kv, q=None) == 1
    assert call(kv, Hq=30) == 2
    assert call(kv, scale=0.0) == 2
    assert call(_kv(head_dim=96)) == 5
    # 16 sequences x 32,768 positions with 64 rows per KV head need 33.75 MiB
    big = _kv(max_len=32768)
    need = L.spec_verify_attn_workspace(ctypes.byref(big), 16, 16, 16)
    assert need > _binding.SPEC_NOALLOC_SCRATCH_BYTES
    assert call(big, B=16, n_max=16, Hq=16) == 4
    # the 25k-visual-token step fits
    assert L.spec_verify_attn_workspace(ctypes.byref(_kv(max_len=25512)), 1, 6, 28) < \
        _binding.SPEC_NOALLOC_SCRATCH_BYTES


def test_vata_topk_rejections(L):
    kv = _kv()
    assert L.spec_vata_attn(ctypes.byref(kv), 1, FAKE, 1, 1, None, 28, None, FAKE, 512, 0.1, FAKE,
                            1, None, None, 0, None) == 1
    assert L.spec_vata_attn(ctypes.byref(kv), 1, FAKE, 1, 1, None, 28, FAKE, FAKE, 0, 0.1, FAKE,
                            1, None, None, 0, None) == 2
    assert L.spec_topk_attn(ctypes.byref(kv), 1, FAKE, 1, 28, 0, 0.1, FAKE, FAKE, 1, None, None,
                            0, None) == 2
    assert L.spec_topk_attn(ctypes.byref(kv), 1, FAKE, 1, 28, 16, 0.1, None, FAKE, 1, None, None,
                            0, None) == 1
    need = L.spec_topk_attn_workspace(ctypes.byref(kv), 1, 28, 16)
    assert need >= 8 * 4 * 1024                        # fp64 scores for every key
    assert L.spec_topk_attn(ctypes.byref(kv), 1, FAKE, 1, 28, 16, 0.1, FAKE, FAKE, 1, None,
                            FAKE, need - 1, None) == 4


def test_hsr_and_accept_rejections(L):
    assert L.spec_hsr_fuse(None, FAKE, FAKE, 1, 4, 64, FAKE, 1, None, 0, None) == 1
    assert L.spec_hsr_fuse(FAKE, FAKE, FAKE, 0, 4, 64, FAKE, 1, None, 0, None) == 3
    assert L.spec_hsr_fuse(FAKE, FAKE, FAKE, 1, 4, 96, FAKE, 1, None, 0, None) == 2
    assert L.spec_hsr_fuse(FAKE, FAKE, FAKE, 1, 0, 64, FAKE, 1, None, 0, None) == 2
    assert L.spec_accept(None, 1, 1, 6, 100, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == 1
    assert L.spec_accept(FAKE, 1, 1, 6, 100, None, None, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == 1
    assert L.spec_accept(FAKE, 2, 1, 6, 100, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == 3
    assert L.spec_accept(FAKE, 1, 1, 0, 100, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == 2
    need = L.spec_accept_workspace(64, 6, 152064)
    assert need >= 64 * 6 * 8
    assert L.spec_accept(FAKE, 1, 64, 6, 152064, FAKE, None, FAKE, FAKE, FAKE, FAKE, need - 1,
                         None) == 4


def test_set_debug_returns_the_previous_setting(L):
    first = L.spec_set_debug(1)
    try:
        assert L.spec_set_debug(0) == 1
        assert L.spec_set_debug(0) == 0
        assert L.spec_set_debug(7) == 0
        assert L.spec_set_debug(1) == 1
    finally:
        L.spec_set_debug(first)


def test_debug_mode_leaves_host_checks_first(L):
    """Host-side rejections come before any device check, so they need no GPU
    in debug mode either."""
    prev = L.spec_set_debug(1)
    try:
        assert L.spec_hsr_fuse(None, FAKE, FAKE, 1, 4, 64, FAKE, 1, None, 0, None) == 1
        assert L.spec_accept(FAKE, 2, 1, 6, 100, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 20,
                             None) == 3
    finally:
        L.spec_set_debug(prev)


def test_std_and_sparse_rejections(L):
    kv = _kv()
    # spec_std_select(kv, B, q_text, q_dtype, Hq, text_idx, text_len, t_max, top_k, scale,
    #                 sel, keep, keep_len, score, ws, ws_bytes, stream)
    assert L.spec_std_select(ctypes.byref(kv), 1, None, 1, 28, FAKE, FAKE, 8, 4, 0.1, FAKE,
                             None, None, None, None, 0, None) == 1
    assert L.spec_std_select(ctypes.byref(kv), 1, FAKE, 1, 28, FAKE, FAKE, 8, 4, 0.1, FAKE,
                             FAKE, None, None, None, 0, None) == 1      # keep without keep_len
    assert L.spec_std_select(ctypes.byref(kv), 1, FAKE, 0, 28, FAKE, FAKE, 8, 4, 0.1, FAKE,
                             None, None, None, None, 0, None) == 3      # q dtype != kv dtype
    assert L.spec_std_select(ctypes.byref(kv), 1, FAKE, 1, 28, FAKE, FAKE, 0, 4, 0.1, FAKE,
                             None, None, None, None, 0, None) == 2
    for bad in (0.0, -1.0):                             # scale must be > 0
        assert L.spec_std_select(ctypes.byref(kv), 1, FAKE, 1, 28, FAKE, FAKE, 8, 4, bad, FAKE,
                                 None, None, None, None, 0, None) == 2
        assert L.spec_vata_attn(ctypes.byref(kv), 1, FAKE, 1, 1, None, 28, FAKE, FAKE, 512, bad,
                                FAKE, 1, None, None, 0, None) == 2
        assert L.spec_topk_attn(ctypes.byref(kv), 1, FAKE, 1, 28, 16, bad, FAKE, FAKE, 1, None,
                                None, 0, None) == 2
        assert L.spec_sparse_attn(ctypes.byref(kv), 1, FAKE, 1, 1, None, 28, FAKE, FAKE, 16,
                                  None, 0, bad, FAKE, 1, None, None, 0, None) == 2
    assert L.spec_std_select(ctypes.byref(kv), 1, FAKE, 1, 28, FAKE, FAKE, 8, 0, 0.1, FAKE,
                             None, None, None, None, 0, None) == 2
    assert L.spec_std_select(ctypes.byref(kv), 1, FAKE, 1, 27, FAKE, FAKE, 8, 4, 0.1, FAKE,
                             None, None, None, None, 0, None) == 2
    need = L.spec_std_select_workspace(ctypes.byref(kv), 1, 28, 8, 4)
    assert need > 0
    assert L.spec_std_select(ctypes.byref(kv), 1, FAKE, 1, 28, FAKE, FAKE, 8, 4, 0.1, FAKE,
                             None, None, None, FAKE, need - 1, None) == 4
    # spec_sparse_attn(kv, B, q, q_dtype, n_max, q_len, Hq, list, list_len, list_max,
    #                  tail_start, tail_max, scale, out, out_dtype, lse, ws, ws_bytes, stream)
    assert L.spec_sparse_attn(ctypes.byref(kv), 1, FAKE, 1, 1, None, 28, None, FAKE, 16, None,
                              0, 0.1, FAKE, 1, None, None, 0, None) == 1
    assert L.spec_sparse_attn(ctypes.byref(kv), 1, FAKE, 1, 1, None, 28, FAKE, FAKE, 0, None,
                              0, 0.1, FAKE, 1, None, None, 0, None) == 2
    assert L.spec_sparse_attn(ctypes.byref(kv), 1, FAKE, 1, 1, None, 28, FAKE, FAKE, 16, FAKE,
                              -1, 0.1, FAKE, 1, None, None, 0, None) == 2
    assert L.spec_sparse_attn(ctypes.byref(kv), 1, FAKE, 1, 10, None, 28, FAKE, FAKE, 16, None,
                              0, 0.1, FAKE, 1, None, None, 0, None) == 5    # 70 rows > 64
    assert L.spec_sparse_attn_workspace(ctypes.byref(kv), 1, 1, 28, 16, 8) >= 0


def test_commit_rejections(L):
    # spec_commit(B, n_max, draft, gamma, accept_len, next_tok, kv_len, last_tok, tokens,
    #             tok_len, tok_cap, text_idx, text_len, t_max, stream)
    assert L.spec_commit(1, 6, FAKE, None, None, FAKE, FAKE, None, None, None, 0, None, None, 0,
                         None) == 1
    assert L.spec_commit(1, 6, None, None, FAKE, FAKE, FAKE, None, None, None, 0, None, None, 0,
                         None) == 1                      # drafts needed when n_max > 1
    assert L.spec_commit(1, 6, FAKE, None, FAKE, FAKE, FAKE, None, FAKE, None, 4, None, None, 0,
                         None) == 1                      # tokens without tok_len
    assert L.spec_commit(0, 6, FAKE, None, FAKE, FAKE, FAKE, None, None, None, 0, None, None, 0,
                         None) == 2
    assert L.spec_commit(1, 6, FAKE, None, FAKE, FAKE, FAKE, None, FAKE, FAKE, 0, None, None, 0,
                         None) == 2                      # tokens with no capacity


def test_mark_main_kernel_takes_both_events_or_neither(L):
    assert L.spec_mark_main_kernel(None, None) == 0
    assert L.spec_mark_main_kernel(FAKE, None) == 1      # SPEC_ERR_NULL, nothing kept
    assert L.spec_mark_main_kernel(None, FAKE) == 1
    assert L.spec_mark_main_kernel(None, None) == 0


def test_read_probe_rejects_bad_arguments(L):
    assert L.spec_read_probe(None, 16, FAKE, None) == 1          # SPEC_ERR_NULL
    assert L.spec_read_probe(FAKE, 16, None, None) == 1
    for p, n in ((FAKE, 0), (FAKE, 15), (FAKE, 24), (FAKE + 8, 16)):
        assert L.spec_read_probe(p, n, FAKE, None) == 2          # SPEC_ERR_SHAPE

"""MI355X-native speculative-decoding attention hot path.

Python entry points with the names of the C ABI (include/specattn.h); each
marshals torch device tensors into one call of libspecattn.so.
"""
from ._binding import (SPEC_BF16, SPEC_F32, SPEC_READ_PROBE_SINK_WORDS, SPEC_WS_SYNC_BYTES, KVCache,
                       SpecError, TimingEvent, Workspace, lib, load_library,
                       mark_main_kernel, read_probe, spec_abi_version, spec_accept, spec_commit, spec_hsr_fuse,
                       spec_set_debug, spec_sparse_attn, spec_status_str, spec_std_select, spec_topk_attn,
                       spec_vata_attn, spec_verify_attn, spec_verify_attn_noalloc)

__all__ = ["SPEC_BF16", "SPEC_F32", "SPEC_READ_PROBE_SINK_WORDS", "SPEC_WS_SYNC_BYTES", "KVCache",
           "SpecError", "TimingEvent", "Workspace", "lib", "load_library", "mark_main_kernel",
           "read_probe", "spec_abi_version", "spec_accept", "spec_commit", "spec_hsr_fuse",
           "spec_set_debug", "spec_sparse_attn", "spec_status_str", "spec_std_select", "spec_topk_attn",
           "spec_vata_attn", "spec_verify_attn", "spec_verify_attn_noalloc"]

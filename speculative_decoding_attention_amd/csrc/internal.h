// Host-side interfaces between the C-ABI layer (api.hip) and the kernel
// translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/specattn.h"

namespace spec {

// Arguments of the split-K attention kernel.  One "unit" is a (sequence b,
// KV head g) pair; its key slots t in [0, T_b) map to positions through
// `mode`:
//   0  dense:        position = t,                         T_b = kv_len[b]
//   1  text list:    position = slots[b*stride + t],       T_b = slot_len[b]
//   2  top-K list:   position = slots[(b*Hkv+g)*stride+t], T_b = min(stride, kv_len[b])
//   3  per-head list + tail: slots[(b*Hkv+g)*stride + t] for t < slot_len[b*Hkv+g]
//                    (entries inside the tail skipped), then the tail positions
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* kv_len;
  const int32_t* q_len;       // may be null (= n_max)
  const int32_t* page_table;  // paged layout when page_shift >= 0
  int32_t max_pages;
  int32_t page_shift;
  // Key slots of a unit: mode 0 every position below kv_len; mode 1 a list
  // per sequence (slots[b, :slot_len[b]]); mode 2 a list per unit of
  // min(slot_stride, kv_len) entries; mode 3 a list per unit
  // (slots[u, :slot_len[u]]) followed by the tail t0..kv_len-1, where t0 =
  // tail_start[b], or kv_len - min(tail_window, kv_len) without tail_start;
  // list entries at or past t0 are skipped (the tail holds them).
  const int32_t* slots;
  const int32_t* slot_len;
  const int32_t* tail_start;
  int32_t tail_window;
  int32_t slot_stride;
  int32_t mode;
  int32_t B, Hq, Hkv, G, n_max, R, max_len;
  int32_t S, chunk;           // splits per unit and slots per split
  int32_t SP;                 // partials per unit: S, or S * phases when each wave writes its own
  float scale_log2;           // softmax scale * log2(e)
  float* part_acc;            // [U*S, R, D] unnormalised partial outputs
  float* part_ml;             // [U*S, 3, R] partial (max, sum, rounded-weight sum), log2 domain
  // Balanced splits from the device lengths (bf16, d = 128, dense
  // verification of 2..64 sequences): the slots actually present are spread over
  // dyn_groups workgroups; partials are numbered split by split, unit by
  // unit (see dyn_split in attention.hip).
  int32_t dyn;
  int32_t dyn_groups;
  void* out;
  int32_t out_bf16;
  float* lse;
};

// Every workspace starts with a reserved region of synchronisation words
// (arrival counters, packed row maxima, selection histograms).  It must be
// zero when the workspace is first used; every call leaves the words it used
// at zero again, and no call keeps scratch data in it.  Scratch follows it.
constexpr size_t kSyncBytes = SPEC_WS_SYNC_BYTES;

struct AttnPlan {
  int S = 1;
  int sp_max = 1;             // partials per unit the workspace holds (S + 1, or S * 4)
  int chunk = 0;
  int grid = 0;
  bool gather = false;        // slots resolved through a list or a page table
  size_t off_acc = 0;         // byte offsets of the partials in the workspace
  size_t off_ml = 0;
  size_t ws_bytes = 0;
};

int device_cu_count();

// Split plan for U units of at most t_max slots and R rows of width d.
// `gather`: slot positions come from a list, or rows from a page table.
// `dense_page_shift` >= 0: every position of a paged cache with pages of
// 2^shift rows (splits then stage pages, not slots).
// The partials start at byte `scratch_off` (at least kSyncBytes); ws_bytes is
// the end of the whole layout, or 0 when a single split needs no workspace.
AttnPlan plan_attention(int units, int t_max, int rows, int d, bool gather,
                        size_t scratch_off = kSyncBytes, int dense_page_shift = -1);

spec_status_t launch_attention(AttnArgs a, int d, int dtype, const AttnPlan& plan, void* ws,
                               hipStream_t stream);

// Top-K: scores + selection into sel_idx, then attention via launch_attention.
struct TopkPlan {
  size_t off_scores = 0;    // fp64 [U, max_len]
  size_t off_key16 = 0;     // uint16 [U, max_len]
  size_t off_hist = 0;      // uint32 [U, 4096]
  bool hist_in_sync = false;  // histogram inside the sync region (no clearing launch)
  AttnPlan attn;            // offsets relative to the same workspace
  size_t ws_bytes = 0;
};
TopkPlan plan_topk(int units, int max_len, int top_k, int rows, int d);
spec_status_t launch_topk_select(const AttnArgs& a, int d, int dtype, int top_k,
                                 int32_t* sel_idx, const TopkPlan& plan, void* ws,
                                 hipStream_t stream);

// Sparse-to-Dense prefill selection (std.hip: the two score passes;
// topk.hip: the mean, the ranking and the kept lists).
struct StdArgs {
  const void* q;               // [B, t_max, Hq, D] text-token queries
  const void* k;
  const int32_t* kv_len;
  const int32_t* page_table;   // paged layout when page_shift >= 0
  int32_t max_pages, page_shift;
  const int32_t* text_idx;     // [B, t_max] ascending positions
  const int32_t* text_len;     // [B]
  int32_t B, Hq, Hkv, G, t_max, max_len;
  int32_t RB, RBP;             // 128-row blocks per unit, and RB * 128
  int32_t S, chunk;            // key splits and keys per split
  float scale_log2;
  float2* ml;                  // [U, S, RBP] per-split (reference max, sum of exp2)
  float* colsum;               // [U, RB, max_len] per-row-block sums of attention
};
struct StdRankPlan {
  size_t off_scores = 0;       // fp64 [U, max_len] ranking scores
  size_t off_key16 = 0;        // uint16 [U, max_len]
  size_t off_hist = 0;         // uint32 [U, 4096]
  bool hist_in_sync = false;
  size_t ws_bytes = 0;
};
struct StdPlan {
  int RB = 0, RBP = 0, S = 1, chunk = 0, grid = 0;
  size_t off_ml = 0, off_col = 0;
  StdRankPlan rank;
  size_t ws_bytes = 0;
};
StdPlan plan_std(int units, int max_len, int t_max, int G, int top_k);
StdRankPlan plan_std_rank(int units, int max_len, size_t scratch_off);
spec_status_t launch_std_select(StdArgs a, int d, int dtype, int top_k, int32_t* sel_idx,
                                int32_t* keep_idx, int32_t* keep_len, float* score,
                                const StdPlan& plan, void* ws, hipStream_t stream);
spec_status_t launch_std_rank(const StdArgs& a, int top_k, int32_t* sel_idx, int32_t* keep_idx,
                              int32_t* keep_len, float* score, const StdRankPlan& plan, void* ws,
                              hipStream_t stream);

// HSR fusion GEMM.
size_t hsr_workspace(int m, int d_model);
spec_status_t launch_hsr(const void* e, const void* h, const void* w, int m, int d_model,
                         void* y, int out_bf16, void* ws, hipStream_t stream);

// Greedy acceptance.
size_t accept_workspace(int batch, int n_max, int vocab);
spec_status_t launch_accept(const void* logits, int dtype, int batch, int n_max, int vocab,
                            const int32_t* draft, const int32_t* gamma, int32_t* target_tok,
                            int32_t* accept_len, int32_t* next_tok, void* ws,
                            hipStream_t stream);

// Bookkeeping after acceptance (spec_commit).
struct CommitArgs {
  int32_t B, n_max;
  const int32_t* draft;        // [B, n_max-1]
  const int32_t* gamma;        // [B] or null (n_max-1)
  const int32_t* accept_len;
  const int32_t* next_tok;
  int32_t* kv_len;             // in: verification length; out: committed length
  int32_t* last_tok;           // may be null
  int32_t* tokens;             // [B, tok_cap] or null
  int32_t* tok_len;
  int32_t tok_cap;
  int32_t* text_idx;           // [B, t_max] or null
  int32_t* text_len;
  int32_t t_max;
};
spec_status_t launch_commit(const CommitArgs& a, hipStream_t stream);

// Debug-mode checks of device index arrays (see validate.hip).  Null
// pointers and zero counts skip the corresponding check.
struct ValidateArgs {
  int32_t B = 0;
  const int32_t* kv_len = nullptr;
  int32_t max_len = 0;
  const int32_t* q_len = nullptr;
  int32_t rows = 0;                 // query rows per sequence (0: no check)
  const int32_t* page_table = nullptr;
  int32_t page_size = 0, max_pages = 0;
  const int32_t* text_idx = nullptr;
  const int32_t* text_len = nullptr;
  int32_t t_max = 0;
  bool text_sorted = false;         // text list strictly ascending
  const int32_t* gamma = nullptr;
  int32_t gamma_n = 0;              // gamma[b] must be in [0, gamma_n - 1]
  // spec_commit: 0 <= accept_len[b] <= gamma_b, gamma_b + 1 <= kv_len[b]
  // (kv_len without max_len), 0 <= tok_len <= tok_cap, 0 <= text_len <= t_max
  const int32_t* accept_len = nullptr;
  const int32_t* tok_len = nullptr;
  int32_t tok_cap = 0;
  // per-unit lists (spec_sparse_attn): list_idx[b, g, :list_len[b, g]] in
  // [0, kv_len[b]); tail_start[b] in [kv_len[b] - tail_max, kv_len[b]]
  int32_t Hkv = 0;
  const int32_t* list_idx = nullptr;
  const int32_t* list_len = nullptr;
  int32_t list_max = 0;
  const int32_t* tail_start = nullptr;
  int32_t tail_max = 0;
};
bool debug_enabled();
int set_debug(int on);

// Measurement hook (spec_mark_main_kernel): the events the calling thread
// set are recorded on the stream right before and right after the main
// kernel of its next call, then forgotten.  No effect on any result.
void mark_before_main(hipStream_t s);
void mark_after_main(hipStream_t s);

// stream.hip: the plain streaming read behind spec_read_probe
spec_status_t launch_read_probe(const void* p, size_t bytes, uint32_t* sink, hipStream_t stream);
// Runs the checks on `stream` and waits for them: SPEC_ERR_SHAPE when a
// value is out of range.
spec_status_t validate(const ValidateArgs& v, hipStream_t stream);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Clears `bytes` (a multiple of 4) at `p` with a fill kernel, so it is safe
// inside captured graphs.
spec_status_t launch_zero(void* p, size_t bytes, hipStream_t stream);

}  // namespace spec

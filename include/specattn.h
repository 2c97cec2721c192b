/*
 * specattn.h -- C ABI of the speculative-decoding attention hot path for
 * AMD Instinct MI355X (gfx950).
 *
 * One speculative iteration of a video LLM has four data-parallel steps:
 *   draft:   u = FC([e_t ; h_{t-1}])                    spec_hsr_fuse
 *            text-anchored attention over text rows     spec_vata_attn
 *            (or top-K sparse attention over all rows)  spec_topk_attn
 *            (or lists kept since prefill:              spec_std_select
 *             selection once, then attention)           spec_sparse_attn
 *   verify:  gamma+1 rows against the full KV cache     spec_verify_attn
 *   accept:  argmax + longest matching prefix           spec_accept
 *   commit:  keep the accepted rows, append tokens      spec_commit
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are DEVICE pointers unless marked (host).  The caller owns every
 *   buffer; the library never allocates, frees or retains caller memory.
 * - Every call is asynchronous on `stream`.  SPEC_OK means the work was
 *   enqueued; faults surface at the caller's next synchronisation.  Every
 *   argument error the host can detect returns a non-zero status before
 *   anything is enqueued, so nothing is partially written.
 * - Workspace: scratch memory comes from the caller (`ws`, `ws_bytes`), sized
 *   by the matching spec_*_workspace() query (which depends only on shapes;
 *   a size of 0 means the call needs none and `ws` may be NULL; otherwise
 *   `ws` is 256-byte aligned, as every hipMalloc allocation is).  Its first
 *   SPEC_WS_SYNC_BYTES bytes are a synchronisation region (arrival counters,
 *   packed row maxima, selection histograms): the caller zero-fills a new
 *   workspace once, before its first use, and every call returns the words
 *   it used to zero before it completes, so a workspace can be reused by any
 *   entry point and any shape without clearing it again (and inside captured
 *   graphs).  The rest is scratch that needs no initialisation.  Calls that
 *   share a workspace must not run concurrently (same stream, or ordered by
 *   events); calls with distinct workspaces may run concurrently on
 *   different streams.  A call cut short by a device fault can leave the
 *   region dirty; zero it again after such an error.
 * - Query heads: q and out are [B, n_max, Hq, d] row-major; query head h
 *   reads KV head h / (Hq / Hkv) (consecutive query heads share a KV head).
 * - Positions: sequence b holds kv_len[b] KV positions, which include the
 *   query rows' own K/V (the caller writes them before the call).  Query row
 *   i < q_len[b] sits at absolute position P = kv_len[b] - q_len[b] + i and
 *   sees key position j iff j <= P (bottom-right causal mask).  Rows
 *   i >= q_len[b] are padding and are written as O = 0, LSE = -inf.
 * - LSE is the natural-log log-sum-exp of the scaled scores, fp32
 *   [B, n_max, Hq]; pass NULL to skip it.
 * - Scores use the caller's `scale` (normally 1/sqrt(d)), which must be
 *   finite and > 0 (else SPEC_ERR_SHAPE); Q and K are post-rotary.
 *   Accumulation is fp32 for every input dtype.
 * - Contents of device index arrays (kv_len, q_len, text_idx, text_len,
 *   page_table, gamma) are preconditions: values outside the stated ranges
 *   are undefined behaviour, unless debug mode is on (spec_set_debug, or
 *   SPEC_DEBUG=1 in the environment at first use).  Then each call first
 *   checks them on its stream, waits, and returns SPEC_ERR_SHAPE without
 *   launching anything if one is out of range: 1 <= kv_len <= max_len;
 *   1 <= q_len <= min(n_max, kv_len) (n_max <= kv_len without q_len);
 *   0 <= text_len <= t_max; 0 <= text_idx < kv_len for listed entries; the
 *   pages a sequence needs fit max_pages and their table entries are >= 0
 *   (the pool size is not known to the library); 0 <= gamma <= n_max - 1;
 *   for spec_std_select the text list is strictly ascending; for
 *   spec_sparse_attn 0 <= list_len <= list_max, list entries lie in
 *   [0, kv_len) and kv_len - tail_max <= tail_start <= kv_len; for
 *   spec_commit 0 <= accept_len <= gamma <= kv_len - 1, 0 <= tok_len <=
 *   tok_cap and 0 <= text_len <= t_max.
 *   Debug calls are synchronous, must not be captured into graphs, and must
 *   not run concurrently on one device (their finding word is per device).
 *
 * Sources (the pages this library implements; titles as published):
 * - "Sparrow: Text-Anchored Window Attention with Visual-Semantic Glimpsing
 *   for Speculative Decoding in Video LLMs" (arXiv 2602.15318), as explained
 *   on gist.science (zh and pt, technical summary section 3 / 3.A) and
 *   summarised on shd-paper.top (method details).
 * - "Sparse-to-Dense: A Free Lunch for Lossless Acceleration of Video
 *   Understanding in LLMs", as explained on gist.science (pt), technical
 *   summary "Metodologia" (decoding procedure, KV-cache selection).
 */
#ifndef SPECATTN_H
#define SPECATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_ABI_VERSION 4

/* Bytes at the start of every non-empty workspace that must be zero before
 * its first use (see Workspace above). */
#define SPEC_WS_SYNC_BYTES (1u << 20)

typedef enum { SPEC_F32 = 0, SPEC_BF16 = 1 } spec_dtype_t;

typedef enum {
  SPEC_OK = 0,
  SPEC_ERR_NULL = 1,        /* a required pointer is NULL                     */
  SPEC_ERR_SHAPE = 2,       /* a size is out of range or inconsistent         */
  SPEC_ERR_DTYPE = 3,       /* unsupported dtype or dtype combination         */
  SPEC_ERR_WORKSPACE = 4,   /* ws_bytes below the spec_*_workspace() size,
                               or ws not 256-byte aligned                  */
  SPEC_ERR_UNSUPPORTED = 5, /* valid request outside what the library supports */
  SPEC_ERR_HIP = 6          /* the HIP runtime refused a launch or query      */
} spec_status_t;

/*
 * KV-cache descriptor.  Two layouts:
 *  contiguous (page_size == 0): k, v are [B, num_kv_heads, max_len, head_dim];
 *      position p of sequence b, head g is row (b*Hkv + g)*max_len + p.
 *  paged (page_size a power of two, 1..256): k, v are a pool
 *      [num_pages, num_kv_heads, page_size, head_dim]; position p of sequence
 *      b lives in physical page page_table[b*max_pages + p/page_size] at slot
 *      p % page_size.  max_len is then a host-side upper bound on kv_len[b]
 *      (used only to size the launch).
 * dtype is SPEC_F32 or SPEC_BF16 (both K and V); head_dim is 64 or 128.
 * kv_len (device, [B]) gives 1 <= kv_len[b] <= max_len.
 */
typedef struct spec_kv {
  const void* k;
  const void* v;
  int32_t dtype;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t max_len;
  const int32_t* kv_len;
  int32_t page_size;
  int32_t max_pages;
  const int32_t* page_table;
} spec_kv_t;

/*
 * spec_verify_attn -- dense verification attention (Sparse-to-Dense,
 * "Metodologia", decoding procedure: the dense model checks all gamma
 * speculative tokens in parallel with one I/O pass over the full KV cache,
 * using standard attention).
 *
 * q:      [B, n_max, Hq, head_dim] in q_dtype (must equal kv->dtype).
 * q_len:  device [B], 1 <= q_len[b] <= min(n_max, kv_len[b]); NULL = n_max.
 * out:    [B, n_max, Hq, head_dim] in out_dtype (SPEC_F32 or SPEC_BF16,
 *         rounded to nearest even).
 * lse:    fp32 [B, n_max, Hq] or NULL.
 * Limits: n_max * (Hq / Hkv) <= 64; Hq % Hkv == 0.
 * For every valid row: O = softmax(scale * q K^T + causal mask) V over key
 * positions 0..P.
 */
size_t spec_verify_attn_workspace(const spec_kv_t* kv, int32_t batch, int32_t n_max,
                                  int32_t num_q_heads);
spec_status_t spec_verify_attn(const spec_kv_t* kv, int32_t batch, const void* q,
                               int32_t q_dtype, int32_t n_max, const int32_t* q_len,
                               int32_t num_q_heads, float scale, void* out, int32_t out_dtype,
                               float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * spec_verify_attn_noalloc -- spec_verify_attn for callers that cannot
 * allocate device memory (code under HIP graph capture that may not call
 * hipMalloc, tight serving loops, harnesses that forbid allocation).
 *
 * Same arguments, limits, results and errors as spec_verify_attn, without
 * the workspace: the split partials live in the library's own scratch
 * array, SPEC_NOALLOC_SCRATCH_BYTES per device, held from the library's
 * load until the process ends.  The call allocates nothing (no hipMalloc,
 * no allocating library routine); its first call on a device looks the
 * array up once.  Returns SPEC_ERR_WORKSPACE, with nothing enqueued, when
 * the shapes need more scratch than that (spec_verify_attn_workspace()
 * reports the need; the 25k-visual-token step needs about 6.5 MB, 16
 * sequences of 32,768 positions about 23 MB).
 * Every call on one device shares that device's array: calls that may
 * overlap on one device (different streams, or host threads without
 * ordering) race and must be serialised by the caller.
 */
#define SPEC_NOALLOC_SCRATCH_BYTES (32u << 20)
spec_status_t spec_verify_attn_noalloc(const spec_kv_t* kv, int32_t batch, const void* q,
                                       int32_t q_dtype, int32_t n_max, const int32_t* q_len,
                                       int32_t num_q_heads, float scale, void* out,
                                       int32_t out_dtype, float* lse, hipStream_t stream);

/*
 * spec_vata_attn -- text-anchored draft attention (Sparrow, technical summary
 * 3.1 / 3.A: the draft drops the visual KV cache and attends only to
 * text-anchored positions, so its cost scales with the text length).
 *
 * text_idx: device [B, t_max] int32 logical positions, 0 <= idx < kv_len[b];
 * text_len: device [B], 0 <= text_len[b] <= t_max.  Only the K/V rows named
 * by text_idx[b, 0..text_len[b]) are read.  Row i sees list entry t iff
 * text_idx[b, t] <= P (its own absolute position); a repeated position counts
 * twice; a row that sees no entry gets O = 0, LSE = -inf.
 * Other arguments as spec_verify_attn.
 */
size_t spec_vata_attn_workspace(const spec_kv_t* kv, int32_t batch, int32_t n_max,
                                int32_t num_q_heads, int32_t t_max);
spec_status_t spec_vata_attn(const spec_kv_t* kv, int32_t batch, const void* q,
                             int32_t q_dtype, int32_t n_max, const int32_t* q_len,
                             int32_t num_q_heads, const int32_t* text_idx,
                             const int32_t* text_len, int32_t t_max, float scale, void* out,
                             int32_t out_dtype, float* lse, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/*
 * spec_topk_attn -- top-K sparse draft attention (Sparse-to-Dense,
 * "Metodologia": the sparse draft attends only to the most relevant KV
 * entries; "Selecao de Cache KV": relevance is the group-mean attention
 * score).  One query row per sequence at position kv_len[b]-1.
 *
 * Per (b, KV head g): qbar = sum of the group's query vectors (fp64, heads in
 * increasing order); score_j = sum_c qbar[c]*K[b,g,j,c] (fp64, c increasing,
 * every product and sum rounded, no fused multiply-add) for j < kv_len[b].
 * Keys are ranked by (score descending, index ascending) and the first
 * min(top_k, kv_len[b]) are kept.
 * sel_idx: device [B, Hkv, top_k] int32, the kept positions in ascending
 *          order, then -1 in unused slots.
 * q:       [B, 1, Hq, head_dim]; out [B, 1, Hq, head_dim]; lse [B, 1, Hq].
 * Every head of group g attends with plain softmax over the kept keys only.
 */
size_t spec_topk_attn_workspace(const spec_kv_t* kv, int32_t batch, int32_t num_q_heads,
                                int32_t top_k);
spec_status_t spec_topk_attn(const spec_kv_t* kv, int32_t batch, const void* q,
                             int32_t q_dtype, int32_t num_q_heads, int32_t top_k, float scale,
                             int32_t* sel_idx, void* out, int32_t out_dtype, float* lse,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * spec_std_select -- Sparse-to-Dense prefill KV selection ("Selecao de Cache
 * KV": the top-K visual KV entries are chosen once, during prefill, by the
 * mean attention that the text tokens pay to the visual tokens, separately
 * per layer and attention head; the text KV is kept).  One call covers one
 * layer; the selection is per (sequence b, KV head g).
 *
 * q_text:   [B, t_max, Hq, head_dim] in kv->dtype (q_dtype must match): row
 *           t is the prefill query of the text token at text_idx[b, t].
 * text_idx: device [B, t_max] int32, strictly ascending in [0, kv_len[b]) for
 *           t < text_len[b]; text_len: device [B], 0 <= text_len <= t_max.
 * Text row t sees positions j <= text_idx[b, t] (causal prefill); with
 * A[h, t, j] its softmax weight (scale applied to the dot products),
 *   mean[b, g, j] = 1/(G*T) * sum over the group's heads h and t < T of
 *                   A[h, t, j]  (0 when T = 0), for j < kv_len[b].
 * Visual positions (j < kv_len[b], not in the text list) are ranked by
 * (mean descending, index ascending).
 * sel_idx:  device [B, Hkv, top_k] out: the first min(top_k, #visual) in
 *           ascending order, then -1.
 * keep_idx: device [B, Hkv, top_k + t_max] out, or NULL: the ascending union
 *           of the selection and the text positions, then -1;
 *           keep_len: device [B, Hkv] out (required with keep_idx): its
 *           length.  keep_idx/keep_len feed spec_sparse_attn.
 * score:    device [B, Hkv, max_len] float out, or NULL: mean[b, g, j] for
 *           j < kv_len[b] (text positions included); later entries are not
 *           written.
 * Precision: bf16 inputs use exact products with fp32 sums on the matrix
 * cores, fp32 exponentials, and fp64 for the final sum over row blocks; the
 * ranking is taken on those values, so positions whose means differ by less
 * than about 1e-5 relative may rank in either order.  fp32 inputs use fp32
 * FMAs.  Limits: t_max * (Hq / Hkv) <= 2^20 rows; top_k >= 1.
 */
size_t spec_std_select_workspace(const spec_kv_t* kv, int32_t batch, int32_t num_q_heads,
                                 int32_t t_max, int32_t top_k);
spec_status_t spec_std_select(const spec_kv_t* kv, int32_t batch, const void* q_text,
                              int32_t q_dtype, int32_t num_q_heads, const int32_t* text_idx,
                              const int32_t* text_len, int32_t t_max, int32_t top_k,
                              float scale, int32_t* sel_idx, int32_t* keep_idx,
                              int32_t* keep_len, float* score, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/*
 * spec_sparse_attn -- Sparse-to-Dense draft attention over the kept lists
 * ("Metodologia": the sparse mode of the same model attends only to the
 * selected KV entries; decoding continues with the entries written since).
 *
 * The tail of sequence b starts at t0 = tail_start[b]; without tail_start it
 * is a sliding window over the last tail_max positions, t0 = kv_len[b] -
 * min(tail_max, kv_len[b]) (tail_max = 0: no tail).  For (b, KV head g) the
 * attended positions are the union of
 *   list_idx[b, g, 0 .. list_len[b, g]-1] below t0  (used as given), and
 *   t0 .. kv_len[b]-1;
 * list entries at or past t0 are skipped (the tail already holds them).
 * Query row i < q_len[b] sits at P = kv_len[b] - q_len[b] + i and sees the
 * members at positions <= P; rows past q_len are padding (O = 0,
 * LSE = -inf), as for spec_verify_attn.  Per-head anchor lists with a
 * window give the text-anchored window variants (Sparrow's explainers name
 * the window's size and placement as key design choices, without values);
 * the kept lists of
 * spec_std_select with tail_start = the prefill length give the
 * Sparse-to-Dense decode.
 * list_idx: device [B, Hkv, list_max] int32, entries in [0, kv_len[b]);
 *           list_len: device [B, Hkv], 0 <= list_len <= list_max.
 * tail_start: device [B] or NULL; with it kv_len[b] - tail_max <=
 *           tail_start[b] <= kv_len[b].  tail_max: host bound on the tail
 *           length (sizes the launch), or the window without tail_start.
 * q, out, lse, scale, dtypes: as spec_verify_attn.
 */
size_t spec_sparse_attn_workspace(const spec_kv_t* kv, int32_t batch, int32_t n_max,
                                  int32_t num_q_heads, int32_t list_max, int32_t tail_max);
spec_status_t spec_sparse_attn(const spec_kv_t* kv, int32_t batch, const void* q,
                               int32_t q_dtype, int32_t n_max, const int32_t* q_len,
                               int32_t num_q_heads, const int32_t* list_idx,
                               const int32_t* list_len, int32_t list_max,
                               const int32_t* tail_start, int32_t tail_max, float scale,
                               void* out, int32_t out_dtype, float* lse, void* ws,
                               size_t ws_bytes, hipStream_t stream);

/*
 * spec_hsr_fuse -- hidden-state-reuse fusion FC (Sparrow, technical summary
 * 3.1 HSR: the current text embedding is concatenated with the target's
 * reused text hidden state and projected by one fully connected layer).
 *
 * Y[r, o] = sum_{k < 2D} X[r, k] * W[o, k],  X[r] = concat(E[r], H[r]).
 * e, h:  [m, d_model] bf16 row-major.   w: [d_model, 2*d_model] bf16
 *        (output-major, the PyTorch Linear layout).  No bias.
 * y:     [m, d_model] in out_dtype (SPEC_F32 or SPEC_BF16).
 * fp32 accumulation on the matrix cores.  Limits: d_model % 64 == 0,
 * 1 <= m <= 65536.
 */
size_t spec_hsr_fuse_workspace(int32_t m, int32_t d_model);
spec_status_t spec_hsr_fuse(const void* e, const void* h, const void* w, int32_t dtype,
                            int32_t m, int32_t d_model, void* y, int32_t out_dtype, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/*
 * spec_accept -- greedy acceptance (Sparse-to-Dense, "Metodologia", decoding
 * procedure: keep the longest prefix of draft tokens that match the dense
 * model's predictions, plus one bonus token from the dense model).
 *
 * logits:     [B, n_max, vocab] in dtype (SPEC_F32 or SPEC_BF16), finite.
 * draft:      device [B, n_max-1] int32 draft tokens.
 * gamma:      device [B] with 0 <= gamma[b] <= n_max-1; NULL = n_max-1.
 * target_tok: device [B, n_max]: t[b,i] = lowest index of the maximum of row
 *             i for i <= gamma[b] (IEEE compare, so -0 == +0), else -1.
 * accept_len: device [B]: n_b = the largest n <= gamma[b] with
 *             draft[b,j] == t[b,j] for all j < n.
 * next_tok:   device [B]: t[b, n_b], the bonus token.
 * The sequence grows by draft[b, 0..n_b) followed by next_tok[b].
 */
size_t spec_accept_workspace(int32_t batch, int32_t n_max, int32_t vocab);
spec_status_t spec_accept(const void* logits, int32_t dtype, int32_t batch, int32_t n_max,
                          int32_t vocab, const int32_t* draft, const int32_t* gamma,
                          int32_t* target_tok, int32_t* accept_len, int32_t* next_tok,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* Human-readable name of a status code (static string, never NULL).  Takes
 * any int: a value that is no spec_status_t gives "unknown spec_status_t". */
const char* spec_status_str(int32_t status);

/*
 * spec_commit -- the bookkeeping that follows acceptance, on the device, so a
 * whole speculative round needs no host synchronisation (Sparse-to-Dense,
 * "Metodologia": the accepted tokens and the bonus token join the context).
 *
 * Convention: during verification sequence b's cache held kv_len[b]
 * positions, the last gamma_b + 1 of them the verified rows (the last
 * committed token at C = kv_len[b] - gamma_b - 1, then the drafts); n =
 * accept_len[b] and next_tok[b] come from spec_accept.  Rows C..C+n stay
 * valid and the rest is rolled back (their contents are simply overwritten
 * later):
 *   kv_len[b]   <- C + n + 1                       (in/out)
 *   last_tok[b] <- next_tok[b]   (its K/V is written by the next round)
 *   tokens[b, tok_len[b] + i] <- draft[b, i] for i < n, then next_tok[b];
 *                  tok_len[b] += n + 1            (stops at tok_cap)
 *   text_idx[b, text_len[b] + i] <- C + i for i <= n;
 *                  text_len[b] += n + 1           (stops at t_max)
 * draft: [B, n_max-1]; gamma: [B] or NULL (n_max-1), as for spec_accept.
 * last_tok, tokens (with tok_len) and text_idx (with text_len) may be NULL.
 * Preconditions: gamma_b + 1 <= kv_len[b]; 0 <= accept_len[b] <= gamma_b.
 * Paged caches: pages past the new length stay with the caller's allocator.
 */
spec_status_t spec_commit(int32_t batch, int32_t n_max, const int32_t* draft,
                          const int32_t* gamma, const int32_t* accept_len,
                          const int32_t* next_tok, int32_t* kv_len, int32_t* last_tok,
                          int32_t* tokens, int32_t* tok_len, int32_t tok_cap,
                          int32_t* text_idx, int32_t* text_len, int32_t t_max,
                          hipStream_t stream);

/* SPEC_ABI_VERSION of the loaded library. */
int32_t spec_abi_version(void);

/* Debug mode on (non-zero) or off for this process; returns the previous
 * setting.  The initial setting comes from SPEC_DEBUG in the environment. */
int32_t spec_set_debug(int32_t on);

/* Measurement hook, for timing one kernel without a profiler.  The calling
 * thread's next call of an entry point records `before` on that call's
 * stream right before its main kernel is launched and `after` right after
 * it, then forgets both (they are not recorded again).  Main kernel: the
 * split attention pass of verify, text-anchored, sparse and the no-allocation
 * verify; the score pass of spec_topk_attn; the GEMM (or the one-row stream
 * pass) of spec_hsr_fuse; the vocabulary scan of spec_accept; the first
 * score pass of spec_std_select.  A call that fails before its launches
 * leaves both set.  Both NULL clears them; exactly one NULL is
 * SPEC_ERR_NULL.  Meant for calls made outside stream capture (the records
 * are plain ones).  The events belong to the caller and must outlive the
 * call; nothing the call computes depends on them. */
spec_status_t spec_mark_main_kernel(hipEvent_t before, hipEvent_t after);

/* Measurement aid: a plain streaming read of `bytes` bytes at device
 * address `p` (16-byte aligned, `bytes` a non-zero multiple of 16), the
 * reference rate for the library's HBM-bound kernels at a given size.
 * SPEC_READ_PROBE_SINK_WORDS workgroups each write one 32-bit word to
 * `sink` (device, that many words): the XOR of the 32-bit words they read,
 * so the XOR of all sink words is the XOR of the buffer's words.  Errors:
 * SPEC_ERR_NULL, SPEC_ERR_SHAPE (alignment or size), SPEC_ERR_HIP. */
#define SPEC_READ_PROBE_SINK_WORDS 1024
spec_status_t spec_read_probe(const void* p, size_t bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECATTN_H */

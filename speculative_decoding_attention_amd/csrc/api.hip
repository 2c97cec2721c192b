// C ABI of libspecattn: argument validation, workspace sizing and launch.
// Every argument error the host can detect is reported before anything is
// enqueued on the caller's stream.
#include <math.h>
#include <string.h>

#include <mutex>

#include "internal.h"

using namespace spec;

// Scratch of spec_verify_attn_noalloc: the split partials of callers that
// cannot allocate device memory.  One copy per device, held from module load
// until the process ends; every call on a device reuses it.  No word of it
// needs to start at zero (each partial is written before it is read), so
// nothing is cleared.  In host code the name stands for a host-side shadow,
// never a device address: host code reaches the memory only through the
// per-device pointer that noalloc_scratch() obtains.
static __device__ __align__(256) unsigned char scratch[SPEC_NOALLOC_SCRATCH_BYTES];

namespace {

// This device's copy of `scratch`, looked up once per device (with that
// device current) under a lock; nullptr if the runtime cannot resolve it.
void* noalloc_scratch() {
  static std::mutex mu;
  static void* ptr[64] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    ptr[dev] = p;
  }
  return ptr[dev];
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int log2_int(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

spec_status_t check_kv(const spec_kv_t* kv) {
  if (!kv || !kv->k || !kv->v || !kv->kv_len) return SPEC_ERR_NULL;
  if (kv->dtype != SPEC_F32 && kv->dtype != SPEC_BF16) return SPEC_ERR_DTYPE;
  if (kv->head_dim != 64 && kv->head_dim != 128) return SPEC_ERR_UNSUPPORTED;
  if (kv->num_kv_heads < 1 || kv->max_len < 1) return SPEC_ERR_SHAPE;
  if (kv->page_size != 0) {
    if (!is_pow2(kv->page_size) || kv->page_size > 256) return SPEC_ERR_SHAPE;
    if (!kv->page_table) return SPEC_ERR_NULL;
    if (kv->max_pages < 1) return SPEC_ERR_SHAPE;
    if ((long long)kv->max_pages * kv->page_size < kv->max_len) return SPEC_ERR_SHAPE;
  }
  return SPEC_OK;
}

spec_status_t check_common(const spec_kv_t* kv, int32_t batch, const void* q, int32_t q_dtype,
                           int32_t n_max, int32_t num_q_heads, float scale, const void* out,
                           int32_t out_dtype) {
  const spec_status_t st = check_kv(kv);
  if (st != SPEC_OK) return st;
  if (!q || !out) return SPEC_ERR_NULL;
  if (batch < 1 || n_max < 1 || num_q_heads < 1) return SPEC_ERR_SHAPE;
  if (num_q_heads % kv->num_kv_heads != 0) return SPEC_ERR_SHAPE;
  if (q_dtype != kv->dtype) return SPEC_ERR_DTYPE;
  if (out_dtype != SPEC_F32 && out_dtype != SPEC_BF16) return SPEC_ERR_DTYPE;
  // the kernels take the masked keys' -inf and the running maxima as the
  // small and large ends of the scaled scores, which holds for scale > 0 only
  if (!(scale > 0.f) || !isfinite(scale)) return SPEC_ERR_SHAPE;
  if ((long long)n_max * (num_q_heads / kv->num_kv_heads) > 64) return SPEC_ERR_UNSUPPORTED;
  if ((long long)batch * kv->num_kv_heads > (1 << 24)) return SPEC_ERR_SHAPE;
  // contiguous caches address rows with 32-bit indices
  if (kv->page_size == 0 && (long long)batch * kv->num_kv_heads * kv->max_len >= (1LL << 32))
    return SPEC_ERR_SHAPE;
  return SPEC_OK;
}

AttnArgs make_args(const spec_kv_t* kv, int32_t batch, const void* q, int32_t n_max,
                   const int32_t* q_len, int32_t num_q_heads, float scale, void* out,
                   int32_t out_dtype, float* lse) {
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = kv->k;
  a.v = kv->v;
  a.kv_len = kv->kv_len;
  a.q_len = q_len;
  a.page_table = kv->page_size ? kv->page_table : nullptr;
  a.max_pages = kv->max_pages;
  a.page_shift = kv->page_size ? log2_int(kv->page_size) : -1;
  a.B = batch;
  a.Hq = num_q_heads;
  a.Hkv = kv->num_kv_heads;
  a.G = num_q_heads / kv->num_kv_heads;
  a.n_max = n_max;
  a.R = n_max * a.G;
  a.max_len = kv->max_len;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = out;
  a.out_bf16 = (out_dtype == SPEC_BF16);
  a.lse = lse;
  return a;
}

// Debug mode: the device index arrays of an attention call.
ValidateArgs kv_checks(const spec_kv_t* kv, int32_t batch, const int32_t* q_len, int32_t rows) {
  ValidateArgs v;
  v.B = batch;
  v.kv_len = kv->kv_len;
  v.max_len = kv->max_len;
  v.q_len = q_len;
  v.rows = rows;
  if (kv->page_size) {
    v.page_table = kv->page_table;
    v.page_size = kv->page_size;
    v.max_pages = kv->max_pages;
  }
  return v;
}

spec_status_t check_ws(size_t need, const void* ws, size_t ws_bytes) {
  if (need == 0) return SPEC_OK;
  if (!ws) return SPEC_ERR_NULL;
  if (ws_bytes < need) return SPEC_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return SPEC_ERR_WORKSPACE;   // 256-byte aligned
  return SPEC_OK;
}

}  // namespace

namespace spec {
namespace {
// events of the measurement hook, per calling thread (one-shot)
thread_local hipEvent_t g_mark_before = nullptr;
thread_local hipEvent_t g_mark_after = nullptr;
void set_main_marks(hipEvent_t before, hipEvent_t after) {
  g_mark_before = before;
  g_mark_after = after;
}
}  // namespace

void mark_before_main(hipStream_t s) {
  if (g_mark_before) hipEventRecord(g_mark_before, s);
  g_mark_before = nullptr;
}

void mark_after_main(hipStream_t s) {
  if (g_mark_after) hipEventRecord(g_mark_after, s);
  g_mark_after = nullptr;
}
}  // namespace spec

extern "C" {

int32_t spec_abi_version(void) { return SPEC_ABI_VERSION; }

int32_t spec_set_debug(int32_t on) { return set_debug(on); }

spec_status_t spec_read_probe(const void* p, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!p || !sink) return SPEC_ERR_NULL;
  if (bytes == 0 || bytes % 16 || reinterpret_cast<uintptr_t>(p) % 16) return SPEC_ERR_SHAPE;
  return launch_read_probe(p, bytes, sink, stream);
}

spec_status_t spec_mark_main_kernel(hipEvent_t before, hipEvent_t after) {
  if ((before == nullptr) != (after == nullptr)) return SPEC_ERR_NULL;
  set_main_marks(before, after);
  return SPEC_OK;
}

const char* spec_status_str(int32_t status) {
  switch (status) {
    case SPEC_OK: return "SPEC_OK";
    case SPEC_ERR_NULL: return "SPEC_ERR_NULL: a required pointer is NULL";
    case SPEC_ERR_SHAPE: return "SPEC_ERR_SHAPE: a size is out of range or inconsistent";
    case SPEC_ERR_DTYPE: return "SPEC_ERR_DTYPE: unsupported dtype or dtype combination";
    case SPEC_ERR_WORKSPACE: return "SPEC_ERR_WORKSPACE: workspace smaller than required";
    case SPEC_ERR_UNSUPPORTED: return "SPEC_ERR_UNSUPPORTED: outside what the library supports";
    case SPEC_ERR_HIP: return "SPEC_ERR_HIP: the HIP runtime refused a launch or query";
  }
  return "unknown spec_status_t";
}

// ------------------------------------------------------------- verify ----

size_t spec_verify_attn_workspace(const spec_kv_t* kv, int32_t batch, int32_t n_max,
                                  int32_t num_q_heads) {
  if (check_kv(kv) != SPEC_OK || batch < 1 || n_max < 1 || num_q_heads < 1 ||
      num_q_heads % kv->num_kv_heads)
    return 0;
  const int R = n_max * (num_q_heads / kv->num_kv_heads);
  return plan_attention(batch * kv->num_kv_heads, kv->max_len, R, kv->head_dim,
                        kv->page_size != 0, kSyncBytes,
                        kv->page_size ? log2_int(kv->page_size) : -1).ws_bytes;
}

spec_status_t spec_verify_attn(const spec_kv_t* kv, int32_t batch, const void* q,
                               int32_t q_dtype, int32_t n_max, const int32_t* q_len,
                               int32_t num_q_heads, float scale, void* out, int32_t out_dtype,
                               float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  spec_status_t st =
      check_common(kv, batch, q, q_dtype, n_max, num_q_heads, scale, out, out_dtype);
  if (st != SPEC_OK) return st;
  AttnArgs a = make_args(kv, batch, q, n_max, q_len, num_q_heads, scale, out, out_dtype, lse);
  a.mode = 0;
  const AttnPlan plan = plan_attention(batch * kv->num_kv_heads, kv->max_len, a.R, kv->head_dim,
                                       kv->page_size != 0, kSyncBytes, a.page_shift);
  st = check_ws(plan.ws_bytes, ws, ws_bytes);
  if (st != SPEC_OK) return st;
  if (debug_enabled() && (st = validate(kv_checks(kv, batch, q_len, n_max), stream)) != SPEC_OK)
    return st;
  return launch_attention(a, kv->head_dim, kv->dtype, plan, ws, stream);
}

spec_status_t spec_verify_attn_noalloc(const spec_kv_t* kv, int32_t batch, const void* q,
                                       int32_t q_dtype, int32_t n_max, const int32_t* q_len,
                                       int32_t num_q_heads, float scale, void* out,
                                       int32_t out_dtype, float* lse, hipStream_t stream) {
  spec_status_t st =
      check_common(kv, batch, q, q_dtype, n_max, num_q_heads, scale, out, out_dtype);
  if (st != SPEC_OK) return st;
  AttnArgs a = make_args(kv, batch, q, n_max, q_len, num_q_heads, scale, out, out_dtype, lse);
  a.mode = 0;
  const AttnPlan plan = plan_attention(batch * kv->num_kv_heads, kv->max_len, a.R, kv->head_dim,
                                       kv->page_size != 0, kSyncBytes, a.page_shift);
  if (plan.ws_bytes > SPEC_NOALLOC_SCRATCH_BYTES) return SPEC_ERR_WORKSPACE;
  void* ws = nullptr;
  if (plan.ws_bytes > 0 && !(ws = noalloc_scratch())) return SPEC_ERR_HIP;
  if (debug_enabled() && (st = validate(kv_checks(kv, batch, q_len, n_max), stream)) != SPEC_OK)
    return st;
  return launch_attention(a, kv->head_dim, kv->dtype, plan, ws, stream);
}

// --------------------------------------------------------------- VATA ----

size_t spec_vata_attn_workspace(const spec_kv_t* kv, int32_t batch, int32_t n_max,
                                int32_t num_q_heads, int32_t t_max) {
  if (check_kv(kv) != SPEC_OK || batch < 1 || n_max < 1 || num_q_heads < 1 || t_max < 1 ||
      num_q_heads % kv->num_kv_heads)
    return 0;
  const int R = n_max * (num_q_heads / kv->num_kv_heads);
  return plan_attention(batch * kv->num_kv_heads, t_max, R, kv->head_dim, true).ws_bytes;
}

spec_status_t spec_vata_attn(const spec_kv_t* kv, int32_t batch, const void* q,
                             int32_t q_dtype, int32_t n_max, const int32_t* q_len,
                             int32_t num_q_heads, const int32_t* text_idx,
                             const int32_t* text_len, int32_t t_max, float scale, void* out,
                             int32_t out_dtype, float* lse, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  spec_status_t st =
      check_common(kv, batch, q, q_dtype, n_max, num_q_heads, scale, out, out_dtype);
  if (st != SPEC_OK) return st;
  if (!text_idx || !text_len) return SPEC_ERR_NULL;
  if (t_max < 1) return SPEC_ERR_SHAPE;
  AttnArgs a = make_args(kv, batch, q, n_max, q_len, num_q_heads, scale, out, out_dtype, lse);
  a.mode = 1;
  a.slots = text_idx;
  a.slot_len = text_len;
  a.slot_stride = t_max;
  const AttnPlan plan = plan_attention(batch * kv->num_kv_heads, t_max, a.R, kv->head_dim, true);
  st = check_ws(plan.ws_bytes, ws, ws_bytes);
  if (st != SPEC_OK) return st;
  if (debug_enabled()) {
    ValidateArgs v = kv_checks(kv, batch, q_len, n_max);
    v.text_idx = text_idx;
    v.text_len = text_len;
    v.t_max = t_max;
    if ((st = validate(v, stream)) != SPEC_OK) return st;
  }
  return launch_attention(a, kv->head_dim, kv->dtype, plan, ws, stream);
}

// -------------------------------------------------------------- top-K ----

size_t spec_topk_attn_workspace(const spec_kv_t* kv, int32_t batch, int32_t num_q_heads,
                                int32_t top_k) {
  if (check_kv(kv) != SPEC_OK || batch < 1 || num_q_heads < 1 || top_k < 1 ||
      num_q_heads % kv->num_kv_heads)
    return 0;
  const int G = num_q_heads / kv->num_kv_heads;
  return plan_topk(batch * kv->num_kv_heads, kv->max_len, top_k, G, kv->head_dim).ws_bytes;
}

spec_status_t spec_topk_attn(const spec_kv_t* kv, int32_t batch, const void* q,
                             int32_t q_dtype, int32_t num_q_heads, int32_t top_k, float scale,
                             int32_t* sel_idx, void* out, int32_t out_dtype, float* lse,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  spec_status_t st = check_common(kv, batch, q, q_dtype, 1, num_q_heads, scale, out, out_dtype);
  if (st != SPEC_OK) return st;
  if (!sel_idx) return SPEC_ERR_NULL;
  if (top_k < 1) return SPEC_ERR_SHAPE;
  if ((long long)batch * kv->num_kv_heads * kv->max_len > (1LL << 31)) return SPEC_ERR_SHAPE;
  AttnArgs a = make_args(kv, batch, q, 1, nullptr, num_q_heads, scale, out, out_dtype, lse);
  const TopkPlan plan = plan_topk(batch * kv->num_kv_heads, kv->max_len, top_k, a.R, kv->head_dim);
  st = check_ws(plan.ws_bytes, ws, ws_bytes);
  if (st != SPEC_OK) return st;
  if (debug_enabled() && (st = validate(kv_checks(kv, batch, nullptr, 1), stream)) != SPEC_OK)
    return st;
  st = launch_topk_select(a, kv->head_dim, kv->dtype, top_k, sel_idx, plan, ws, stream);
  if (st != SPEC_OK) return st;
  a.mode = 2;
  a.slots = sel_idx;
  a.slot_stride = top_k;
  return launch_attention(a, kv->head_dim, kv->dtype, plan.attn, ws, stream);
}

// ---------------------------------------------- Sparse-to-Dense prefill ----

size_t spec_std_select_workspace(const spec_kv_t* kv, int32_t batch, int32_t num_q_heads,
                                 int32_t t_max, int32_t top_k) {
  if (check_kv(kv) != SPEC_OK || batch < 1 || num_q_heads < 1 || t_max < 1 || top_k < 1 ||
      num_q_heads % kv->num_kv_heads)
    return 0;
  const int G = num_q_heads / kv->num_kv_heads;
  if ((long long)t_max * G > (1 << 20)) return 0;
  return plan_std(batch * kv->num_kv_heads, kv->max_len, t_max, G, top_k).ws_bytes;
}

spec_status_t spec_std_select(const spec_kv_t* kv, int32_t batch, const void* q_text,
                              int32_t q_dtype, int32_t num_q_heads, const int32_t* text_idx,
                              const int32_t* text_len, int32_t t_max, int32_t top_k,
                              float scale, int32_t* sel_idx, int32_t* keep_idx,
                              int32_t* keep_len, float* score, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  spec_status_t st = check_kv(kv);
  if (st != SPEC_OK) return st;
  if (!q_text || !text_idx || !text_len || !sel_idx) return SPEC_ERR_NULL;
  if (keep_idx && !keep_len) return SPEC_ERR_NULL;
  if (batch < 1 || num_q_heads < 1 || num_q_heads % kv->num_kv_heads) return SPEC_ERR_SHAPE;
  if (q_dtype != kv->dtype) return SPEC_ERR_DTYPE;
  if (!(scale > 0.f) || !isfinite(scale) || t_max < 1 || top_k < 1) return SPEC_ERR_SHAPE;
  const int G = num_q_heads / kv->num_kv_heads;
  if ((long long)t_max * G > (1 << 20)) return SPEC_ERR_UNSUPPORTED;
  if ((long long)batch * kv->num_kv_heads * kv->max_len > (1LL << 31)) return SPEC_ERR_SHAPE;
  if ((long long)batch * kv->num_kv_heads * ((long long)top_k + t_max) > (1LL << 31))
    return SPEC_ERR_SHAPE;
  const int units = batch * kv->num_kv_heads;
  const StdPlan plan = plan_std(units, kv->max_len, t_max, G, top_k);
  st = check_ws(plan.ws_bytes, ws, ws_bytes);
  if (st != SPEC_OK) return st;
  if (debug_enabled()) {
    ValidateArgs v = kv_checks(kv, batch, nullptr, 0);
    v.text_idx = text_idx;
    v.text_len = text_len;
    v.t_max = t_max;
    v.text_sorted = true;
    if ((st = validate(v, stream)) != SPEC_OK) return st;
  }
  StdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q_text;
  a.k = kv->k;
  a.kv_len = kv->kv_len;
  a.page_table = kv->page_size ? kv->page_table : nullptr;
  a.max_pages = kv->max_pages;
  a.page_shift = kv->page_size ? log2_int(kv->page_size) : -1;
  a.text_idx = text_idx;
  a.text_len = text_len;
  a.B = batch;
  a.Hq = num_q_heads;
  a.Hkv = kv->num_kv_heads;
  a.G = G;
  a.t_max = t_max;
  a.max_len = kv->max_len;
  a.scale_log2 = scale * 1.4426950408889634f;
  return launch_std_select(a, kv->head_dim, kv->dtype, top_k, sel_idx, keep_idx, keep_len, score,
                           plan, ws, stream);
}

// ------------------------------------------------ sparse (kept lists) ----

size_t spec_sparse_attn_workspace(const spec_kv_t* kv, int32_t batch, int32_t n_max,
                                  int32_t num_q_heads, int32_t list_max, int32_t tail_max) {
  if (check_kv(kv) != SPEC_OK || batch < 1 || n_max < 1 || num_q_heads < 1 || list_max < 1 ||
      tail_max < 0 || num_q_heads % kv->num_kv_heads)
    return 0;
  const int R = n_max * (num_q_heads / kv->num_kv_heads);
  return plan_attention(batch * kv->num_kv_heads, list_max + tail_max, R, kv->head_dim, true)
      .ws_bytes;
}

spec_status_t spec_sparse_attn(const spec_kv_t* kv, int32_t batch, const void* q,
                               int32_t q_dtype, int32_t n_max, const int32_t* q_len,
                               int32_t num_q_heads, const int32_t* list_idx,
                               const int32_t* list_len, int32_t list_max,
                               const int32_t* tail_start, int32_t tail_max, float scale,
                               void* out, int32_t out_dtype, float* lse, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  spec_status_t st =
      check_common(kv, batch, q, q_dtype, n_max, num_q_heads, scale, out, out_dtype);
  if (st != SPEC_OK) return st;
  if (!list_idx || !list_len) return SPEC_ERR_NULL;
  if (list_max < 1 || tail_max < 0) return SPEC_ERR_SHAPE;
  if ((long long)list_max + tail_max > (1 << 30)) return SPEC_ERR_SHAPE;
  AttnArgs a = make_args(kv, batch, q, n_max, q_len, num_q_heads, scale, out, out_dtype, lse);
  a.mode = 3;
  a.slots = list_idx;
  a.slot_len = list_len;
  a.slot_stride = list_max;
  a.tail_start = tail_start;
  a.tail_window = tail_start ? 0 : tail_max;
  const AttnPlan plan =
      plan_attention(batch * kv->num_kv_heads, list_max + tail_max, a.R, kv->head_dim, true);
  st = check_ws(plan.ws_bytes, ws, ws_bytes);
  if (st != SPEC_OK) return st;
  if (debug_enabled()) {
    ValidateArgs v = kv_checks(kv, batch, q_len, n_max);
    v.Hkv = kv->num_kv_heads;
    v.list_idx = list_idx;
    v.list_len = list_len;
    v.list_max = list_max;
    v.tail_start = tail_start;
    v.tail_max = tail_max;
    if ((st = validate(v, stream)) != SPEC_OK) return st;
  }
  return launch_attention(a, kv->head_dim, kv->dtype, plan, ws, stream);
}

// ------------------------------------------------------------- commit ----

spec_status_t spec_commit(int32_t batch, int32_t n_max, const int32_t* draft,
                          const int32_t* gamma, const int32_t* accept_len,
                          const int32_t* next_tok, int32_t* kv_len, int32_t* last_tok,
                          int32_t* tokens, int32_t* tok_len, int32_t tok_cap,
                          int32_t* text_idx, int32_t* text_len, int32_t t_max,
                          hipStream_t stream) {
  if (!accept_len || !next_tok || !kv_len) return SPEC_ERR_NULL;
  if (n_max > 1 && !draft) return SPEC_ERR_NULL;
  if ((tokens && !tok_len) || (text_idx && !text_len)) return SPEC_ERR_NULL;
  if (batch < 1 || n_max < 1 || batch > (1 << 24)) return SPEC_ERR_SHAPE;
  if ((tokens && tok_cap < 1) || (text_idx && t_max < 1)) return SPEC_ERR_SHAPE;
  if (debug_enabled()) {
    ValidateArgs v;
    v.B = batch;
    v.kv_len = kv_len;
    v.gamma = gamma;
    v.gamma_n = n_max;
    v.accept_len = accept_len;
    v.tok_len = tokens ? tok_len : nullptr;
    v.tok_cap = tok_cap;
    v.text_len = text_idx ? text_len : nullptr;
    v.t_max = t_max;
    const spec_status_t st = validate(v, stream);
    if (st != SPEC_OK) return st;
  }
  CommitArgs a;
  a.B = batch;
  a.n_max = n_max;
  a.draft = draft;
  a.gamma = gamma;
  a.accept_len = accept_len;
  a.next_tok = next_tok;
  a.kv_len = kv_len;
  a.last_tok = last_tok;
  a.tokens = tokens;
  a.tok_len = tok_len;
  a.tok_cap = tok_cap;
  a.text_idx = text_idx;
  a.text_len = text_len;
  a.t_max = t_max;
  return launch_commit(a, stream);
}

// ---------------------------------------------------------------- HSR ----

size_t spec_hsr_fuse_workspace(int32_t m, int32_t d_model) {
  if (m < 1 || m > 65536 || d_model < 64 || d_model % 64) return 0;
  return hsr_workspace(m, d_model);
}

spec_status_t spec_hsr_fuse(const void* e, const void* h, const void* w, int32_t dtype,
                            int32_t m, int32_t d_model, void* y, int32_t out_dtype, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  if (!e || !h || !w || !y) return SPEC_ERR_NULL;
  if (dtype != SPEC_BF16) return SPEC_ERR_DTYPE;
  if (out_dtype != SPEC_F32 && out_dtype != SPEC_BF16) return SPEC_ERR_DTYPE;
  if (m < 1 || m > 65536 || d_model < 64 || d_model % 64 || d_model > (1 << 16))
    return SPEC_ERR_SHAPE;
  const spec_status_t st = check_ws(hsr_workspace(m, d_model), ws, ws_bytes);
  if (st != SPEC_OK) return st;
  return launch_hsr(e, h, w, m, d_model, y, out_dtype == SPEC_BF16, ws, stream);
}

// ------------------------------------------------------------- accept ----

size_t spec_accept_workspace(int32_t batch, int32_t n_max, int32_t vocab) {
  if (batch < 1 || n_max < 1 || vocab < 1) return 0;
  return accept_workspace(batch, n_max, vocab);
}

spec_status_t spec_accept(const void* logits, int32_t dtype, int32_t batch, int32_t n_max,
                          int32_t vocab, const int32_t* draft, const int32_t* gamma,
                          int32_t* target_tok, int32_t* accept_len, int32_t* next_tok,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!logits || !target_tok || !accept_len || !next_tok) return SPEC_ERR_NULL;
  if (n_max > 1 && !draft) return SPEC_ERR_NULL;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_DTYPE;
  if (batch < 1 || n_max < 1 || vocab < 1 || vocab >= 0x7fffffff) return SPEC_ERR_SHAPE;
  if ((long long)batch * n_max > (1 << 24)) return SPEC_ERR_SHAPE;
  spec_status_t st = check_ws(accept_workspace(batch, n_max, vocab), ws, ws_bytes);
  if (st != SPEC_OK) return st;
  if (debug_enabled() && gamma) {
    ValidateArgs v;
    v.B = batch;
    v.gamma = gamma;
    v.gamma_n = n_max;
    if ((st = validate(v, stream)) != SPEC_OK) return st;
  }
  return launch_accept(logits, dtype, batch, n_max, vocab, draft, gamma, target_tok, accept_len,
                       next_tok, ws, stream);
}

}  // extern "C"

// Debug-mode validation of the device index arrays that every entry point
// takes as preconditions (lengths, position lists, page tables, gamma).
// When enabled (environment SPEC_DEBUG=1 at first use, or spec_set_debug),
// an entry point runs one check kernel on its stream, waits for it, and
// returns SPEC_ERR_SHAPE instead of launching anything if a value is out of
// range.  The wait makes such calls synchronous, so debug mode is for
// testing, not for captured graphs.  The finding word is one per device,
// so debug calls on one device must not run concurrently from several host
// threads.
#include <stdlib.h>

#include <atomic>

#include "internal.h"

namespace spec {

namespace {

// One word per device: the checks OR their findings into it.
__device__ uint32_t g_violation;

__device__ __forceinline__ void flag(bool bad) {
  if (bad) atomicOr(&g_violation, 1u);
}

// Per sequence b: 1 <= kv_len <= max_len; 1 <= q_len <= min(rows, kv_len)
// (rows <= kv_len without q_len); 0 <= text_len <= t_max and every listed
// position in [0, kv_len) (strictly ascending when asked); pages needed
// within max_pages and every used page-table entry >= 0; 0 <= gamma <=
// gamma_n - 1; per-unit list lengths in [0, list_max], entries in
// [0, kv_len), and the tail start in [kv_len - tail_max, kv_len].
__global__ __launch_bounds__(256) void check_kernel(ValidateArgs v) {
  const int b = blockIdx.x;
  const int L = v.kv_len ? v.kv_len[b] : 0;
  // (max_len 0: no upper bound on kv_len, as for spec_commit)
  const bool len_ok = !v.kv_len || (L >= 1 && (v.max_len == 0 || L <= v.max_len));
  if (threadIdx.x == 0) {
    flag(!len_ok);
    if (v.kv_len && v.rows > 0) {
      if (v.q_len) {
        const int n = v.q_len[b];
        flag(n < 1 || n > v.rows || n > L);
      } else {
        flag(v.rows > L);
      }
    }
    if (v.text_len) {
      const int t = v.text_len[b];
      flag(t < 0 || t > v.t_max);
    }
    if (v.gamma) {
      const int gm = v.gamma[b];
      flag(gm < 0 || gm > v.gamma_n - 1);
    }
    if (v.accept_len) {
      const int gm = v.gamma ? v.gamma[b] : v.gamma_n - 1;
      const int n = v.accept_len[b];
      flag(n < 0 || n > gm || (v.kv_len && L < gm + 1));
      if (v.tok_len) flag(v.tok_len[b] < 0 || v.tok_len[b] > v.tok_cap);
    }
  }
  if (v.page_table && v.kv_len && len_ok) {
    const int pages = (L + v.page_size - 1) / v.page_size;
    flag(threadIdx.x == 0 && pages > v.max_pages);
    for (int p = threadIdx.x; p < pages && p < v.max_pages; p += blockDim.x)
      flag(v.page_table[(size_t)b * v.max_pages + p] < 0);
  }
  if (v.text_idx && v.kv_len && len_ok) {
    const int t = min(max(v.text_len[b], 0), v.t_max);
    for (int i = threadIdx.x; i < t; i += blockDim.x) {
      const int pos = v.text_idx[(size_t)b * v.t_max + i];
      flag(pos < 0 || pos >= L);
      if (v.text_sorted && i > 0) flag(v.text_idx[(size_t)b * v.t_max + i - 1] >= pos);
    }
  }
  if (v.list_idx && v.kv_len && len_ok) {
    if (v.tail_start && threadIdx.x == 0) {
      const int t0 = v.tail_start[b];
      flag(t0 < L - v.tail_max || t0 > L);
    }
    for (int g = 0; g < v.Hkv; ++g) {
      const size_t u = (size_t)b * v.Hkv + g;
      const int n = v.list_len[u];
      if (threadIdx.x == 0) flag(n < 0 || n > v.list_max);
      const int nn = min(max(n, 0), v.list_max);
      for (int i = threadIdx.x; i < nn; i += blockDim.x) {
        const int pos = v.list_idx[u * v.list_max + i];
        flag(pos < 0 || pos >= L);
      }
    }
  }
}

std::atomic<int> debug_state{-1};   // -1: not yet read from the environment

}  // namespace

bool debug_enabled() {
  int s = debug_state.load(std::memory_order_relaxed);
  if (s < 0) {
    const char* e = getenv("SPEC_DEBUG");
    s = (e && e[0] && e[0] != '0') ? 1 : 0;
    int expected = -1;
    debug_state.compare_exchange_strong(expected, s, std::memory_order_relaxed);
    s = debug_state.load(std::memory_order_relaxed);
  }
  return s == 1;
}

int set_debug(int on) {
  const int prev = debug_enabled() ? 1 : 0;
  debug_state.store(on ? 1 : 0, std::memory_order_relaxed);
  return prev;
}

spec_status_t validate(const ValidateArgs& v, hipStream_t stream) {
  if (v.B < 1) return SPEC_OK;
  static const uint32_t zero = 0;
  if (hipMemcpyToSymbolAsync(HIP_SYMBOL(g_violation), &zero, sizeof(zero), 0,
                             hipMemcpyHostToDevice, stream) != hipSuccess)
    return SPEC_ERR_HIP;
  hipLaunchKernelGGL(check_kernel, dim3((unsigned)v.B), dim3(256), 0, stream, v);
  if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
  uint32_t found = 0;
  if (hipMemcpyFromSymbolAsync(&found, HIP_SYMBOL(g_violation), sizeof(found), 0,
                               hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return SPEC_ERR_HIP;
  return found ? SPEC_ERR_SHAPE : SPEC_OK;
}

}  // namespace spec

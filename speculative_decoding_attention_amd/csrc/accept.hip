// Greedy acceptance on gfx950: per-row argmax over the vocabulary, then the
// longest prefix of draft tokens that match, plus the bonus token.
//
// The vocabulary scan is split into chunks so every CU streams the logits.
// A workgroup reduces its chunk to one packed 64-bit key
//   (order-preserving bits of the value) << 32 | (0xFFFFFFFF - index)
// whose maximum is "largest value, then lowest index" in any reduction order,
// and merges it into its row with a 64-bit atomic max.  The last workgroup of
// each sequence (arrival counter) turns the row maxima into target tokens,
// counts the matching prefix and writes the outputs, and returns the maxima
// and its counter to zero for the next call.
#include "common.h"
#include "internal.h"

namespace spec {

namespace {

constexpr int kAcceptThreads = 256;
constexpr int kAccLoads = 4;      // 16-byte loads in flight per thread

struct AcceptArgs {
  const void* logits;
  const int32_t* draft;
  const int32_t* gamma;
  int32_t* target_tok;
  int32_t* accept_len;
  int32_t* next_tok;
  unsigned long long* best;   // [B, n_max] packed maxima (cleared per call)
  uint32_t* tick;             // [B] arrival counters (cleared per call)
  int32_t B, n_max, V, chunk, chunks, vec;
};

__device__ __forceinline__ unsigned long long pack_key(float x, uint32_t idx) {
  if (x == 0.f) x = 0.f;                       // IEEE: -0 == +0
  const uint32_t u = __float_as_uint(x);
  const uint32_t k = (u >> 31) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)k << 32) | (0xFFFFFFFFu - idx);
}

__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}

template <bool BF16>
__global__ __launch_bounds__(kAcceptThreads) void accept_kernel(AcceptArgs a) {
  constexpr int EPV = BF16 ? 8 : 4;                 // elements per 16-byte load
  constexpr int SCALAR = kAccLoads * EPV;           // scalar loads per thread (ragged vocab)
  __shared__ unsigned long long red[kAcceptThreads / 64];
  __shared__ uint32_t s_tick;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x / a.chunks;              // b * n_max + i
  const int ch = blockIdx.x - row * a.chunks;
  const int b = row / a.n_max;
  const int v0 = ch * a.chunk, v1 = min(a.V, v0 + a.chunk);
  // Every row is scanned (rows past gamma are ignored at the end), so the
  // loads do not wait for gamma; all of a thread's loads are in flight at once.
  unsigned long long best = 0;
  if (a.vec) {
    const unsigned char* p = reinterpret_cast<const unsigned char*>(a.logits) +
                             (size_t)row * a.V * (BF16 ? 2 : 4);
    u32x4_t w[kAccLoads];
#pragma unroll
    for (int k = 0; k < kAccLoads; ++k) {
      const int v = v0 + (k * kAcceptThreads + tid) * EPV;
      w[k] = (v < v1) ? ld16(p + (size_t)v * (BF16 ? 2 : 4)) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int k = 0; k < kAccLoads; ++k) {
      const int v = v0 + (k * kAcceptThreads + tid) * EPV;
      if (v < v1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (BF16) {
            best = umax64(best, pack_key(__uint_as_float(w[k][j] << 16), v + 2 * j));
            best = umax64(best, pack_key(__uint_as_float(w[k][j] & 0xFFFF0000u), v + 2 * j + 1));
          } else {
            best = umax64(best, pack_key(__uint_as_float(w[k][j]), v + j));
          }
        }
      }
    }
  } else {
    // unconditional loads from clamped indices (a guarded load becomes a
    // branch with its own wait); out-of-range lanes are masked below
    float x[SCALAR];
#pragma unroll
    for (int k = 0; k < SCALAR; ++k) {
      const size_t v = (size_t)row * a.V + min(v0 + k * kAcceptThreads + tid, v1 - 1);
      x[k] = BF16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(a.logits)[v])
                  : reinterpret_cast<const float*>(a.logits)[v];
    }
#pragma unroll
    for (int k = 0; k < SCALAR; ++k) {
      const int v = v0 + k * kAcceptThreads + tid;
      if (v < v1) best = umax64(best, pack_key(x[k], v));
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long other =
        ((unsigned long long)(uint32_t)__shfl_xor((int)(best >> 32), o) << 32) |
        (uint32_t)__shfl_xor((int)(uint32_t)best, o);
    best = umax64(best, other);
  }
  if (lane == 0) red[wave] = best;
  __syncthreads();
  // The maxima are device-scope atomics, read back with atomic exchanges, so
  // no cache write-back is needed: thread 0 only waits for its own atomicMax
  // to complete before it arrives.
  if (tid == 0) {
    unsigned long long m = red[0];
    for (int w = 1; w < kAcceptThreads / 64; ++w) m = umax64(m, red[w]);
    atomicMax(&a.best[row], m);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    s_tick = atomicAdd(&a.tick[b], 1u);
  }
  __syncthreads();
  if (s_tick != (uint32_t)(a.n_max * a.chunks - 1) || wave != 0) return;
  // Last arrival of sequence b: lane r takes row r (64 rows per round), so
  // the maxima, the draft tokens and the outputs move in one round trip.
  const int gam = a.gamma ? min(max(a.gamma[b], 0), a.n_max - 1) : a.n_max - 1;
  int n = -1, nxt = 0;
  for (int r0 = 0; r0 < a.n_max; r0 += 64) {
    const int r = r0 + lane;
    unsigned long long k = 0;
    int d = -1;
    if (r < a.n_max) {
      k = atomicExch(&a.best[(size_t)b * a.n_max + r], 0ull);
      if (r < gam) d = a.draft[(size_t)b * (a.n_max - 1) + r];
    }
    const int t = (r <= gam) ? (int)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull)) : -1;
    if (r < a.n_max) a.target_tok[(size_t)b * a.n_max + r] = t;
    const unsigned long long stop = __builtin_amdgcn_ballot_w64(r <= gam && (r == gam || d != t));
    if (n < 0 && stop) {
      const int first = __ffsll((long long)stop) - 1;
      n = r0 + first;
      nxt = __shfl(t, first);
    }
  }
  if (lane == 0) {
    a.accept_len[b] = n;
    a.next_tok[b] = nxt;
    a.tick[b] = 0u;
  }
}

struct AcceptPlan {
  int chunk, chunks, vec;
  bool in_sync;
  size_t off_best, off_tick, ws_bytes;
};

AcceptPlan plan_accept(int batch, int n_max, int vocab, bool bf16) {
  AcceptPlan p;
  const int vw = bf16 ? 8 : 4;
  p.chunk = kAcceptThreads * kAccLoads * vw;        // 64 B of logits per thread
  p.vec = (vocab % vw == 0) ? 1 : 0;
  if (p.chunk > vocab) p.chunk = ((vocab + vw - 1) / vw) * vw;
  p.chunks = (vocab + p.chunk - 1) / p.chunk;
  // The maxima and counters live in the sync region when they fit: the
  // finishing workgroup of each sequence returns them to zero, so no clearing
  // launch is needed.  Otherwise they sit in scratch and are cleared first.
  const size_t best_bytes = align_up((size_t)batch * n_max * sizeof(unsigned long long), 256);
  const size_t words = best_bytes + align_up((size_t)batch * sizeof(uint32_t), 256);
  p.in_sync = words <= kSyncBytes;
  p.off_best = p.in_sync ? 0 : kSyncBytes;
  p.off_tick = p.off_best + best_bytes;
  p.ws_bytes = p.in_sync ? kSyncBytes : kSyncBytes + words;
  return p;
}

}  // namespace

size_t accept_workspace(int batch, int n_max, int vocab) {
  const AcceptPlan a = plan_accept(batch, n_max, vocab, true);
  const AcceptPlan b = plan_accept(batch, n_max, vocab, false);
  return a.ws_bytes > b.ws_bytes ? a.ws_bytes : b.ws_bytes;
}

spec_status_t launch_accept(const void* logits, int dtype, int batch, int n_max, int vocab,
                            const int32_t* draft, const int32_t* gamma, int32_t* target_tok,
                            int32_t* accept_len, int32_t* next_tok, void* ws,
                            hipStream_t stream) {
  const bool bf16 = (dtype == SPEC_BF16);
  const AcceptPlan p = plan_accept(batch, n_max, vocab, bf16);
  AcceptArgs a;
  a.logits = logits;
  a.draft = draft;
  a.gamma = gamma;
  a.target_tok = target_tok;
  a.accept_len = accept_len;
  a.next_tok = next_tok;
  a.best = reinterpret_cast<unsigned long long*>(reinterpret_cast<char*>(ws) + p.off_best);
  a.tick = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(ws) + p.off_tick);
  a.B = batch;
  a.n_max = n_max;
  a.V = vocab;
  a.chunk = p.chunk;
  a.chunks = p.chunks;
  a.vec = p.vec;
  if (!p.in_sync) {
    const spec_status_t st =
        launch_zero(a.best, p.off_tick - p.off_best + (size_t)batch * sizeof(uint32_t), stream);
    if (st != SPEC_OK) return st;
  }
  const dim3 grid((unsigned)batch * n_max * p.chunks), block(kAcceptThreads);
  if (bf16)
    hipLaunchKernelGGL(accept_kernel<true>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(accept_kernel<false>, grid, block, 0, stream, a);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

}  // namespace spec

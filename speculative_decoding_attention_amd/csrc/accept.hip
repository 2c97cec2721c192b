// Greedy acceptance on gfx950: per-row argmax over the vocabulary, then the
// longest prefix of draft tokens that match, plus the bonus token.
//
// accept_scan_kernel: the vocabulary of every row is cut into chunks so that
// every CU streams logits; a workgroup reduces its chunk to one packed
// 64-bit key (see below) and stores it to its own slot (no atomics:
// device-scope atomics on shared words serialise and cost tens of
// microseconds at batch 64).
// accept_finish_kernel: one wave per sequence takes the maximum over each
// row's slots, turns it into the target token and counts the matching
// prefix.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace spec {

namespace {

constexpr int kAcceptThreads = 256;

struct AcceptArgs {
  const void* logits;
  const int32_t* draft;
  const int32_t* gamma;
  int32_t* target_tok;
  int32_t* accept_len;
  int32_t* next_tok;
  unsigned long long* best;   // [B, n_max, chunks] packed chunk maxima (every slot written)
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

__device__ __forceinline__ unsigned long long shfl_xor64(unsigned long long v, int o) {
  return ((unsigned long long)(uint32_t)__shfl_xor((int)(v >> 32), o) << 32) |
         (uint32_t)__shfl_xor((int)(uint32_t)v, o);
}

// Running maximum of one thread: elements arrive in increasing index order,
// and only a strictly larger value replaces the current one, so the kept
// index is the lowest of the maximum (IEEE compare: -0 does not replace +0,
// nor +0 -0).
__device__ __forceinline__ void take(float x, int v, bool ok, float& m, int& mi) {
  const bool gt = ok & (x > m);
  m = gt ? x : m;
  mi = gt ? v : mi;
}

// Chunk maximum of one row: every thread requests its NL 16-byte loads at
// once (rows past gamma are scanned too, so no load waits for gamma), keeps
// a (value, index) pair, and packs it into the 64-bit key
//   (order-preserving bits of the value) << 32 | (0xFFFFFFFF - index)
// only once, for the workgroup reduction: the key's maximum is "largest
// value, then lowest index" in any reduction order.
template <bool BF16, int NL>
__global__ __launch_bounds__(kAcceptThreads) void accept_scan_kernel(AcceptArgs a) {
  constexpr int EPV = BF16 ? 8 : 4;                 // elements per 16-byte load
  constexpr int SCALAR = NL * EPV;                  // scalar loads per thread (ragged vocab)
  __shared__ unsigned long long red[kAcceptThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x / a.chunks;              // b * n_max + i
  const int ch = blockIdx.x - row * a.chunks;
  const int v0 = ch * a.chunk, v1 = min(a.V, v0 + a.chunk);
  float m = -INFINITY;
  int mi = -1;
  if (a.vec) {
    const unsigned char* p = reinterpret_cast<const unsigned char*>(a.logits) +
                             (size_t)row * a.V * (BF16 ? 2 : 4);
    // clamped, unconditional loads (a guarded load waits for itself before
    // the next is issued); elements past the chunk are masked below
    u32x4_t w[NL];
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int v = min(v0 + (k * kAcceptThreads + tid) * EPV, v1 - EPV);
      w[k] = ld16(p + (size_t)v * (BF16 ? 2 : 4));
    }
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int v = v0 + (k * kAcceptThreads + tid) * EPV;
      const bool ok = v < v1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (BF16) {
          take(__uint_as_float(w[k][j] << 16), v + 2 * j, ok, m, mi);
          take(__uint_as_float(w[k][j] & 0xFFFF0000u), v + 2 * j + 1, ok, m, mi);
        } else {
          take(__uint_as_float(w[k][j]), v + j, ok, m, mi);
        }
      }
    }
  } else {
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
      take(x[k], v, v < v1, m, mi);
    }
  }
  unsigned long long best = (mi >= 0) ? pack_key(m, (uint32_t)mi) : 0ull;
  for (int o = 32; o > 0; o >>= 1) best = umax64(best, shfl_xor64(best, o));
  if (lane == 0) red[wave] = best;
  __syncthreads();
  if (tid == 0) {
    unsigned long long mm = red[0];
    for (int w = 1; w < kAcceptThreads / 64; ++w) mm = umax64(mm, red[w]);
    a.best[(size_t)row * a.chunks + ch] = mm;
  }
}

// One wave per sequence: row r's target token is the maximum over its chunk
// slots (every slot load in flight at once, reduced in LDS), and a lane per
// row finds the first mismatch with a ballot, 64 rows per round.  The draft
// tokens go out with the slot loads and gamma is a scalar load, so the
// sequence pays one round trip to memory before its stores.
__global__ __launch_bounds__(64) void accept_finish_kernel(AcceptArgs a) {
  constexpr int kRows = 64;                 // rows reduced per round (one per lane)
  __shared__ unsigned long long rmax[kRows];
  const int b = blockIdx.x, lane = threadIdx.x;
  const int gam = a.gamma ? min(max(ld_uniform(a.gamma, b), 0), a.n_max - 1) : a.n_max - 1;
  int n = -1, nxt = 0;
  for (int r0 = 0; r0 < a.n_max; r0 += kRows) {
    const int rows = min(kRows, a.n_max - r0);
    const int r = r0 + lane;
    // draft token of row r (index clamped; only rows below gamma use it)
    const int dr = (a.n_max > 1) ? a.draft[(size_t)b * (a.n_max - 1) + min(r, a.n_max - 2)] : -1;
    rmax[lane] = 0ull;
    __syncthreads();
    const int total = rows * a.chunks;
    const unsigned long long* src = a.best + ((size_t)b * a.n_max + r0) * a.chunks;
    for (int i0 = 0; i0 < total; i0 += kRows * 8) {
      unsigned long long v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = src[min(i0 + k * kRows + lane, total - 1)];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = i0 + k * kRows + lane;
        if (i < total) atomicMax(&rmax[i / a.chunks], v[k]);   // LDS atomic
      }
    }
    __syncthreads();
    const unsigned long long k = (lane < rows) ? rmax[lane] : 0ull;
    const int d = (r < gam) ? dr : -1;
    const int t = (r <= gam) ? (int)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull)) : -1;
    if (r < a.n_max) a.target_tok[(size_t)b * a.n_max + r] = t;
    const unsigned long long stop =
        __builtin_amdgcn_ballot_w64(r < a.n_max && r <= gam && (r == gam || d != t));
    if (n < 0 && stop) {
      const int first = __ffsll((long long)stop) - 1;
      n = r0 + first;
      nxt = __shfl(t, first);
    }
    __syncthreads();   // every lane has read rmax before the next round clears it
  }
  if (lane == 0) {
    a.accept_len[b] = n;
    a.next_tok[b] = nxt;
  }
}

// 16-byte loads per thread and chunk: two (32 bytes in flight per thread,
// 4,096 bf16 logits per 256-thread chunk).  More per thread measured slower
// at batch 64 (117 MB of logits): 8 loads gave 27.3 us per call (22.9 us
// scan), 6 loads 25.9 and 2 loads 26.0 (21.3-21.7 us scan); small,
// register-light workgroups keep more of them resident per CU.
constexpr int kAcceptLoads = 2;

struct AcceptPlan {
  int chunk, chunks, vec;
  size_t ws_bytes;
};

// Chunks of 256 threads x kAcceptLoads 16-byte loads.
AcceptPlan plan_accept(int batch, int n_max, int vocab, bool bf16) {
  AcceptPlan p;
  const int vw = bf16 ? 8 : 4;
  p.chunk = kAcceptThreads * kAcceptLoads * vw;
  p.vec = (vocab % vw == 0) ? 1 : 0;
  if (p.chunk > vocab) p.chunk = ((vocab + vw - 1) / vw) * vw;
  p.chunks = (vocab + p.chunk - 1) / p.chunk;
  // chunk maxima in scratch after the sync region; every slot is written
  p.ws_bytes = kSyncBytes +
               align_up((size_t)batch * n_max * p.chunks * sizeof(unsigned long long), 256);
  return p;
}

// One workgroup per sequence.  Thread 0 reads the round's lengths and
// hands them to the others through LDS before it overwrites them.  Values
// outside their ranges (a precondition) are clamped so that every access
// stays inside the arrays.
__global__ __launch_bounds__(64) void commit_kernel(CommitArgs a) {
  __shared__ int s_v[4];
  const int b = blockIdx.x;
  if (threadIdx.x == 0) {
    const int gam = min(max(a.gamma ? a.gamma[b] : a.n_max - 1, 0), a.n_max - 1);
    s_v[0] = a.kv_len[b] - gam - 1;                 // C: the last committed token's row
    s_v[1] = min(max(a.accept_len[b], 0), gam);
    s_v[2] = a.tokens ? max(a.tok_len[b], 0) : 0;
    s_v[3] = a.text_idx ? max(a.text_len[b], 0) : 0;
  }
  __syncthreads();
  const int C = s_v[0], n = s_v[1], t0 = s_v[2], x0 = s_v[3];
  const int nxt = a.next_tok[b];
  for (int i = threadIdx.x; i <= n; i += blockDim.x) {
    if (a.tokens && t0 + i < a.tok_cap)
      a.tokens[(size_t)b * a.tok_cap + t0 + i] =
          (i < n) ? a.draft[(size_t)b * (a.n_max - 1) + i] : nxt;
    if (a.text_idx && x0 + i < a.t_max) a.text_idx[(size_t)b * a.t_max + x0 + i] = C + i;
  }
  if (threadIdx.x == 0) {
    a.kv_len[b] = C + n + 1;
    if (a.last_tok) a.last_tok[b] = nxt;
    if (a.tokens) a.tok_len[b] = min(t0 + n + 1, a.tok_cap);
    if (a.text_idx) a.text_len[b] = min(x0 + n + 1, a.t_max);
  }
}

}  // namespace

spec_status_t launch_commit(const CommitArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(commit_kernel, dim3((unsigned)a.B), dim3(64), 0, stream, a);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

size_t accept_workspace(int batch, int n_max, int vocab) {
  // the larger of the two dtypes' plans
  size_t need = 0;
  for (int vw : {4, 8}) {
    const int chunk = std::min(kAcceptThreads * kAcceptLoads * vw, ((vocab + vw - 1) / vw) * vw);
    const size_t chunks = (size_t)((vocab + chunk - 1) / chunk);
    need = std::max(need, kSyncBytes + align_up((size_t)batch * n_max * chunks *
                                                    sizeof(unsigned long long), 256));
  }
  return need;
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
  a.best = reinterpret_cast<unsigned long long*>(reinterpret_cast<char*>(ws) + kSyncBytes);
  a.B = batch;
  a.n_max = n_max;
  a.V = vocab;
  a.chunk = p.chunk;
  a.chunks = p.chunks;
  a.vec = p.vec;
  const dim3 grid((unsigned)batch * n_max * p.chunks), block(kAcceptThreads);
  mark_before_main(stream);
  if (bf16)
    hipLaunchKernelGGL((accept_scan_kernel<true, kAcceptLoads>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((accept_scan_kernel<false, kAcceptLoads>), grid, block, 0, stream, a);
  mark_after_main(stream);
  if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
  hipLaunchKernelGGL(accept_finish_kernel, dim3((unsigned)batch), dim3(64), 0, stream, a);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

}  // namespace spec

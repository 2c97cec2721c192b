// Sparse-to-Dense prefill selection for gfx950: the mean attention that the
// text tokens of a prompt pay to every KV position, per (sequence b, KV
// head g) (Sparse-to-Dense pt explainer, "Seleção de Cache KV").
//
// The rows of a unit are the text tokens' prefill queries, row r = t*G + hh
// (text token t at position p_t = text_idx[b, t], query head g*G + hh).  Row r
// sees keys j <= p_t, and its attention is
//   A[r, j] = exp2(s2[r, j] - c_r),  s2 = scale*log2(e) * <q_r, k_j>,
//   c_r     = log2 sum_{j <= p_t} exp2(s2[r, j])     (exp2-domain LSE),
// so the per-key sum over rows needs c_r first.  Two passes over the same
// score tiles, both on v_mfma_f32_16x16x32_bf16 (exact bf16 products, fp32
// sums; the fp32 path uses plain FMAs):
//   pass A (rows):  per row, a lazily re-referenced (max, sum of exp2) over the
//                   keys of one split; partials go to the workspace;
//   pass B (keys):  merge the row partials into c_r, then per key the sum over
//                   the block's 128 rows of exp2(s2 - c_r); one partial per
//                   (unit, row block, key).
// The final mean, the ranking and the kept lists follow in topk.hip.
//
// Work decomposition: a workgroup owns 128 rows (8 groups of 16) of one unit
// and one split of the keys.  Its four waves hold all 128 query rows as MFMA
// operands in registers and stream disjoint 16-key blocks straight from
// global memory (no LDS, no barriers in the loop).  Pass A computes
// S^T = K Q^T, so each lane sees 4 keys of one row per group and keeps that
// row's statistics to itself; pass B computes S = Q K^T with the same
// registers, so each lane sees one key and 4 rows per group and the sum over
// rows stays in one register until a final 4-lane reduction.  Rows are
// ordered by position, so keys past a block's last text position are never
// computed.
#include <float.h>
#include <math.h>

#include "common.h"
#include "internal.h"

namespace spec {

namespace {

constexpr int kBR = 128;            // rows per workgroup
constexpr int kRG = kBR / 16;       // 16-row groups
constexpr int kKeysPerIter = 64;    // 4 waves x 16 keys
constexpr float kNoMax = -3.0e38f;  // finite "no key seen yet" reference

__device__ __forceinline__ size_t key_row(const StdArgs& a, int b, int g, int j) {
  if (a.page_shift >= 0) {
    const int page = a.page_table[(size_t)b * a.max_pages + (j >> a.page_shift)];
    return (((size_t)page * a.Hkv + g) << a.page_shift) + (j & ((1 << a.page_shift) - 1));
  }
  return ((size_t)b * a.Hkv + g) * (size_t)a.max_len + j;
}

struct Block {
  int u, b, g, s, rb;
  int rows;      // valid rows of the unit (text_len * G)
  int r0;        // first row of the block
  int L, k0, k1; // sequence length and this split's keys [k0, k1)
};

__device__ __forceinline__ bool decode_block(const StdArgs& a, Block& k) {
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  k.rb = wg % a.RB;
  const int us = wg / a.RB;
  k.s = us % a.S;
  k.u = us / a.S;
  k.b = k.u / a.Hkv;
  k.g = k.u - k.b * a.Hkv;
  k.rows = a.text_len[k.b] * a.G;
  k.r0 = k.rb * kBR;
  k.L = a.kv_len[k.b];
  k.k0 = k.s * a.chunk;
  k.k1 = min(k.L, k.k0 + a.chunk);
  return k.r0 < k.rows;
}

// Row positions of the block into LDS (-1 for rows past the unit's rows).
__device__ __forceinline__ void stage_positions(const StdArgs& a, const Block& k, int* s_pos) {
  if (threadIdx.x < kBR) {
    const int r = k.r0 + (int)threadIdx.x;
    s_pos[threadIdx.x] = (r < k.rows) ? a.text_idx[(size_t)k.b * a.t_max + r / a.G] : -1;
  }
}

// Pass B prologue: c_r from the S split partials of pass A, in split order
// (+inf for rows past the unit's rows, so their terms vanish).
__device__ __forceinline__ void stage_offsets(const StdArgs& a, const Block& k, float* s_c) {
  if (threadIdx.x < kBR) {
    const int r = k.r0 + (int)threadIdx.x;
    float c = INFINITY;
    if (r < k.rows) {
      const float2* ml = a.ml + (size_t)k.u * a.S * a.RBP + r;
      float M = kNoMax;
      for (int sp = 0; sp < a.S; ++sp) M = fmaxf(M, ml[(size_t)sp * a.RBP].x);
      float Ls = 0.f;
      for (int sp = 0; sp < a.S; ++sp) {
        const float2 v = ml[(size_t)sp * a.RBP];
        Ls += v.y * exp2f(v.x - M);
      }
      c = M + log2f(Ls);
    }
    s_c[threadIdx.x] = c;
  }
}

// ------------------------------------------------------------ MFMA path ----

template <int D>
__device__ __forceinline__ void load_q(const StdArgs& a, const Block& k, int r16, int q4,
                                       bf16x8_t (&qop)[kRG][D / 32]) {
  const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q);
#pragma unroll
  for (int rg = 0; rg < kRG; ++rg) {
    const int r = k.r0 + rg * 16 + r16;
    const bool ok = r < k.rows;
    const int rr = ok ? r : k.r0;                        // clamped, masked after
    const int t = rr / a.G, hh = rr - (rr / a.G) * a.G;
    const uint16_t* row = q + (((size_t)k.b * a.t_max + t) * a.Hq + k.g * a.G + hh) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const u32x4_t v = ld16(row + 32 * ks + 8 * q4);
      qop[rg][ks] = as_bf16x8(ok ? v : u32x4_t{0, 0, 0, 0});
    }
  }
}

template <int D>
__device__ __forceinline__ void load_k(const StdArgs& a, const Block& k, int key, int q4,
                                       u32x4_t (&kf)[D / 32]) {
  const uint16_t* kp = reinterpret_cast<const uint16_t*>(a.k) +
                       key_row(a, k.b, k.g, min(key, k.L - 1)) * D;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) kf[ks] = ld16(kp + 32 * ks + 8 * q4);
}

template <int D, int PASS>
__global__ __launch_bounds__(256, 2) void std_mfma_kernel(StdArgs a) {
  constexpr int KS = D / 32;
  __shared__ __align__(16) int s_pos[kBR];
  __shared__ float s_c[kBR];
  __shared__ float s_m[4][kBR], s_l[4][kBR];

  Block k;
  if (!decode_block(a, k)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, q4 = lane >> 4;
  stage_positions(a, k, s_pos);
  if (PASS == 1) stage_offsets(a, k, s_c);
  bf16x8_t qop[kRG][KS];
  load_q<D>(a, k, r16, q4, qop);
  __syncthreads();

  const int nrow = min(k.rows - k.r0, kBR);
  const int p_max = s_pos[nrow - 1];
  const int p_min = (nrow < kBR) ? -1 : s_pos[0];     // -1: padded rows need the mask
  const int kend = min(k.k1, p_max + 1);               // no row sees a key at or past this

  if (PASS == 0) {
    int pos[kRG];
    float m[kRG], l[kRG];
#pragma unroll
    for (int rg = 0; rg < kRG; ++rg) {
      pos[rg] = s_pos[rg * 16 + r16];
      m[rg] = kNoMax;
      l[rg] = 0.f;
    }
    int kb = k.k0 + 16 * wave;
    u32x4_t kc[KS];
    if (kb < kend) load_k<D>(a, k, kb + r16, q4, kc);
    for (; kb < kend; kb += kKeysPerIter) {
      u32x4_t kn[KS];
      const bool more = kb + kKeysPerIter < kend;
      if (more) load_k<D>(a, k, kb + kKeysPerIter + r16, q4, kn);
      const bool need_mask = kb + 15 > p_min;
#pragma unroll
      for (int rg = 0; rg < kRG; ++rg) {
        f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kc[ks]), qop[rg][ks], c, 0, 0, 0);
        float sv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sv[i] = c[i] * a.scale_log2;
          if (need_mask) sv[i] = (kb + 4 * q4 + i <= pos[rg]) ? sv[i] : -INFINITY;
        }
        const float tmax = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        // lazily raised reference: terms stay <= 2^8 and rescales are rare
        if (tmax > m[rg] + 8.f) {
          l[rg] *= exp2f(m[rg] - tmax);
          m[rg] = tmax;
        }
        l[rg] += (exp2f(sv[0] - m[rg]) + exp2f(sv[1] - m[rg])) +
                 (exp2f(sv[2] - m[rg]) + exp2f(sv[3] - m[rg]));
      }
      if (more) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kc[ks] = kn[ks];
      }
    }
    // the four lanes of a row, then the four waves, in a fixed order
#pragma unroll
    for (int rg = 0; rg < kRG; ++rg) {
#pragma unroll
      for (int x = 16; x <= 32; x <<= 1) {
        const float m2 = __shfl_xor(m[rg], x), l2 = __shfl_xor(l[rg], x);
        const float mn = fmaxf(m[rg], m2);
        l[rg] = l[rg] * exp2f(m[rg] - mn) + l2 * exp2f(m2 - mn);
        m[rg] = mn;
      }
      if (q4 == 0) {
        s_m[wave][rg * 16 + r16] = m[rg];
        s_l[wave][rg * 16 + r16] = l[rg];
      }
    }
    __syncthreads();
    if (threadIdx.x < kBR && (int)threadIdx.x < nrow) {
      const int r = threadIdx.x;
      float M = kNoMax;
      for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][r]);
      float Ls = 0.f;
      for (int w = 0; w < 4; ++w) Ls += s_l[w][r] * exp2f(s_m[w][r] - M);
      a.ml[((size_t)k.u * a.S + k.s) * a.RBP + k.r0 + r] = make_float2(M, Ls);
    }
  } else {
    float crow[kRG][4];
#pragma unroll
    for (int rg = 0; rg < kRG; ++rg)
#pragma unroll
      for (int i = 0; i < 4; ++i) crow[rg][i] = s_c[rg * 16 + 4 * q4 + i];
    float* out = a.colsum + ((size_t)k.u * a.RB + k.rb) * a.max_len;
    int kb = k.k0 + 16 * wave;
    u32x4_t kc[KS];
    if (kb < kend) load_k<D>(a, k, kb + r16, q4, kc);
    for (; kb < kend; kb += kKeysPerIter) {
      u32x4_t kn[KS];
      const bool more = kb + kKeysPerIter < kend;
      if (more) load_k<D>(a, k, kb + kKeysPerIter + r16, q4, kn);
      const bool need_mask = kb + 15 > p_min;
      const int key = kb + r16;
      float acc = 0.f;
#pragma unroll
      for (int rg = 0; rg < kRG; ++rg) {
        f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qop[rg][ks], as_bf16x8(kc[ks]), c, 0, 0, 0);
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = exp2f(c[i] * a.scale_log2 - crow[rg][i]);
        if (need_mask) {
          const int4 pr = *reinterpret_cast<const int4*>(&s_pos[rg * 16 + 4 * q4]);
          p[0] = (key <= pr.x) ? p[0] : 0.f;
          p[1] = (key <= pr.y) ? p[1] : 0.f;
          p[2] = (key <= pr.z) ? p[2] : 0.f;
          p[3] = (key <= pr.w) ? p[3] : 0.f;
        }
        acc += (p[0] + p[1]) + (p[2] + p[3]);
      }
      acc = sum_across_rows(acc);
      if (q4 == 0 && key < k.k1) out[key] = acc;
      if (more) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kc[ks] = kn[ks];
      }
    }
    // keys of the split that no row of the block sees
    const int kcov = k.k0 + ((max(kend - k.k0, 0) + 15) / 16) * 16;
    for (int j = kcov + (int)threadIdx.x; j < k.k1; j += blockDim.x) out[j] = 0.f;
  }
}

// ---------------------------------------------------------- scalar path ----
// fp32 (and any other case without the MFMA layout): one thread per row in
// pass A, one thread per key in pass B, products and sums in fp32 with d in
// order.

template <int D>
__device__ __forceinline__ float dot_row(const float* q, const float* kr) {
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < D; ++c) s = fmaf(q[c], kr[c], s);
  return s;
}

template <int D, int PASS>
__global__ __launch_bounds__(256) void std_scalar_kernel(StdArgs a) {
  __shared__ int s_pos[kBR];
  __shared__ float s_c[kBR];
  __shared__ float s_q[PASS == 1 ? kBR * D : 1];

  Block k;
  if (!decode_block(a, k)) return;
  stage_positions(a, k, s_pos);
  if (PASS == 1) stage_offsets(a, k, s_c);
  const float* q = reinterpret_cast<const float*>(a.q);
  const float* kb = reinterpret_cast<const float*>(a.k);
  const int nrow = min(k.rows - k.r0, kBR);
  if (PASS == 1) {
    for (int e = threadIdx.x; e < kBR * D; e += blockDim.x) {
      const int rl = e / D, c = e - (e / D) * D;
      float v = 0.f;
      if (rl < nrow) {
        const int r = k.r0 + rl, t = r / a.G, hh = r - (r / a.G) * a.G;
        v = q[(((size_t)k.b * a.t_max + t) * a.Hq + k.g * a.G + hh) * D + c];
      }
      s_q[e] = v;
    }
  }
  __syncthreads();
  const int p_max = s_pos[nrow - 1];

  if (PASS == 0) {
    const int rl = threadIdx.x;
    if (rl >= nrow) return;
    const int r = k.r0 + rl, t = r / a.G, hh = r - (r / a.G) * a.G;
    float qr[D];
    const float* qp = q + (((size_t)k.b * a.t_max + t) * a.Hq + k.g * a.G + hh) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) qr[c] = qp[c];
    const int end = min(k.k1, s_pos[rl] + 1);
    float m = kNoMax, l = 0.f;
    for (int j = k.k0; j < end; ++j) {
      const float s2 = dot_row<D>(qr, kb + key_row(a, k.b, k.g, j) * D) * a.scale_log2;
      if (s2 > m + 8.f) {
        l *= exp2f(m - s2);
        m = s2;
      }
      l += exp2f(s2 - m);
    }
    a.ml[((size_t)k.u * a.S + k.s) * a.RBP + r] = make_float2(m, l);
  } else {
    float* out = a.colsum + ((size_t)k.u * a.RB + k.rb) * a.max_len;
    for (int j = k.k0 + (int)threadIdx.x; j < k.k1; j += blockDim.x) {
      float acc = 0.f;
      if (j <= p_max) {
        const float* kr = kb + key_row(a, k.b, k.g, j) * D;
        for (int rl = 0; rl < nrow; ++rl) {
          if (j > s_pos[rl]) continue;
          const float s2 = dot_row<D>(s_q + rl * D, kr) * a.scale_log2;
          acc += exp2f(s2 - s_c[rl]);
        }
      }
      out[j] = acc;
    }
  }
}

template <int D>
hipError_t launch_passes(const StdArgs& a, int dtype, int grid, hipStream_t stream) {
  if (dtype == SPEC_BF16) {
    hipLaunchKernelGGL((std_mfma_kernel<D, 0>), dim3(grid), dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    hipLaunchKernelGGL((std_mfma_kernel<D, 1>), dim3(grid), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((std_scalar_kernel<D, 0>), dim3(grid), dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    hipLaunchKernelGGL((std_scalar_kernel<D, 1>), dim3(grid), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

StdPlan plan_std(int units, int max_len, int t_max, int G, int top_k) {
  StdPlan p;
  p.RB = (t_max * G + kBR - 1) / kBR;
  p.RBP = p.RB * kBR;
  // enough workgroups for several per CU (two fit at once), splits of at
  // least 256 keys, every split a whole number of 64-key iterations
  const long target = 8L * device_cu_count();
  const long blocks = (long)units * p.RB;
  long S = (target + blocks - 1) / blocks;
  const long smax = (max_len + 255) / 256;
  if (S > smax) S = smax;
  if (S < 1) S = 1;
  long chunk = (max_len + S - 1) / S;
  chunk = ((chunk + kKeysPerIter - 1) / kKeysPerIter) * kKeysPerIter;
  p.chunk = (int)chunk;
  p.S = (int)((max_len + chunk - 1) / chunk);
  p.grid = units * p.RB * p.S;
  p.off_ml = kSyncBytes;
  p.off_col = align_up(p.off_ml + (size_t)units * p.S * p.RBP * sizeof(float2), 256);
  const size_t rank_off = align_up(p.off_col + (size_t)units * p.RB * max_len * sizeof(float), 256);
  p.rank = plan_std_rank(units, max_len, rank_off);
  p.ws_bytes = p.rank.ws_bytes;
  (void)top_k;
  return p;
}

spec_status_t launch_std_select(StdArgs a, int d, int dtype, int top_k, int32_t* sel_idx,
                                int32_t* keep_idx, int32_t* keep_len, float* score,
                                const StdPlan& plan, void* ws, hipStream_t stream) {
  char* w = reinterpret_cast<char*>(ws);
  a.RB = plan.RB;
  a.RBP = plan.RBP;
  a.S = plan.S;
  a.chunk = plan.chunk;
  a.ml = reinterpret_cast<float2*>(w + plan.off_ml);
  a.colsum = reinterpret_cast<float*>(w + plan.off_col);
  const hipError_t e = (d == 64) ? launch_passes<64>(a, dtype, plan.grid, stream)
                                 : launch_passes<128>(a, dtype, plan.grid, stream);
  if (e != hipSuccess) return SPEC_ERR_HIP;
  return launch_std_rank(a, top_k, sel_idx, keep_idx, keep_len, score, plan.rank, ws, stream);
}

}  // namespace spec

// Split-K flash-decoding attention for gfx950: the shared engine behind
// verification attention (dense positions), text-anchored draft attention
// (positions from a text index list) and top-K sparse draft attention
// (positions from a per-head selection list).
//
// Work decomposition.  A unit is a (sequence b, KV head g) pair; its query
// block is the n_max * G rows (query position i, head-in-group hh), row
// r = i*G + hh, padded to NB*16 rows.  The unit's key slots are cut into S
// splits of `chunk` slots; one 256-thread workgroup (4 waves) owns one split
// and each wave streams 32-slot tiles of it independently with its own
// online-softmax state.  The waves merge in LDS; the workgroup writes either
// the final output (S == 1) or an unnormalised partial that a small merge
// kernel combines with the log-sum-exp rule.
//
// Per tile and wave (bf16, d = 128):
//   S^T = K Q^T   on v_mfma_f32_16x16x32_bf16: A = 16 keys x 32 d straight
//                 from global memory, B = the query block held in registers;
//                 the key order inside a tile is permuted so that each lane's
//                 8 scores are 8 consecutive keys of one query row.
//   online softmax in fp32 (exp2 domain), row maxima across the four 16-lane
//                 rows of the wave.
//   O^T += V^T P^T on the same MFMA: the probabilities are already laid out
//                 as the B operand; V is transposed through LDS as packed
//                 (key, key+1) bf16 pairs so each lane reads its A operand
//                 with one 16-byte LDS load.
// The fp32 variant uses v_mfma_f32_16x16x4_f32, where V needs no transpose.
#include <math.h>

#include "common.h"
#include "internal.h"

namespace spec {

namespace {

constexpr int kTK = 32;   // key slots per tile
constexpr int kNW = 4;    // waves per workgroup
constexpr int kPV = 20;   // dwords per LDS row of a transposed V tile (16 + 4 pad)

__device__ __forceinline__ int slot_position(const AttnArgs& a, int b, int g, int t) {
  if (a.mode == 0) return t;
  if (a.mode == 1) return a.slots[(size_t)b * a.slot_stride + t];
  return a.slots[((size_t)b * a.Hkv + g) * a.slot_stride + t];
}

// Row index (in units of head_dim elements) of position `pos` of (b, g).
__device__ __forceinline__ size_t kv_row(const AttnArgs& a, int b, int g, int pos) {
  if (a.page_shift >= 0) {
    const int page = a.page_table[(size_t)b * a.max_pages + (pos >> a.page_shift)];
    const int slot = pos & ((1 << a.page_shift) - 1);
    return (((size_t)page * a.Hkv + g) << a.page_shift) + slot;
  }
  return ((size_t)b * a.Hkv + g) * (size_t)a.max_len + pos;
}

// Shared epilogue: merge the 4 waves' (m, l, l_rnd, acc) in LDS in a fixed
// order, then write the final output (S == 1) or this split's partial.
template <int D, int NB>
__device__ __forceinline__ void finish_split(const AttnArgs& a, float* smem, int wave, int lane,
                                             int u, int s, int b, int g, int nq,
                                             const float (&m_run)[NB], const float (&l_run)[NB],
                                             const float (&l_rnd)[NB],
                                             f32x4_t (&acc)[D / 16][NB]) {
  constexpr int RP = NB * 16;
  constexpr int DP = D + 4;        // padded row pitch of the merge buffer
  constexpr int DB = D / 16;
  float* macc = smem;              // [RP][DP]
  float* mm = smem + RP * DP;      // [kNW][RP]
  float* ml = mm + kNW * RP;       // [kNW][RP]
  float* mr = ml + kNW * RP;       // [kNW][RP]
  float* mrow = mr + kNW * RP;     // [3][RP]: merged max, exact sum, rounded-weight sum
  const int r16 = lane & 15, q4 = lane >> 4;

  float l_tot[NB], r_tot[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    l_tot[nb] = sum_across_rows(l_run[nb]);
    r_tot[nb] = sum_across_rows(l_rnd[nb]);
  }

  __syncthreads();   // every wave is done with its V tile buffer
  if (q4 == 0) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      mm[wave * RP + nb * 16 + r16] = m_run[nb];
      ml[wave * RP + nb * 16 + r16] = l_tot[nb];
      mr[wave * RP + nb * 16 + r16] = r_tot[nb];
    }
  }
  __syncthreads();
  if (threadIdx.x < RP) {
    const int r = threadIdx.x;
    float M = -INFINITY;
    for (int w = 0; w < kNW; ++w) M = fmaxf(M, mm[w * RP + r]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float Ls = 0.f, Lr = 0.f;
    for (int w = 0; w < kNW; ++w) {
      const float f = exp2f(mm[w * RP + r] - Mu);
      Ls += ml[w * RP + r] * f;
      Lr += mr[w * RP + r] * f;
    }
    mrow[r] = M;
    mrow[RP + r] = Ls;
    mrow[2 * RP + r] = Lr;
  }
  __syncthreads();
  float f[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float M = mrow[nb * 16 + r16];
    const float Mu = (M == -INFINITY) ? 0.f : M;
    f[nb] = exp2f(m_run[nb] - Mu);   // m_run = -inf (no visible key) -> 0
  }
  for (int w = 0; w < kNW; ++w) {
    if (wave == w) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int idx = (nb * 16 + r16) * DP + db * 16 + q4 * 4 + i;
            const float val = acc[db][nb][i] * f[nb];
            macc[idx] = (w == 0) ? val : macc[idx] + val;
          }
    }
    __syncthreads();
  }

  const int R = a.R;
  if (a.S == 1) {
    // final output: O = acc / l_rnd, LSE = (M + log2 l) * ln 2
    const int Hq = a.Hq, G = a.G;
    for (int e = threadIdx.x; e < R * D; e += blockDim.x) {
      const int r = e / D, d = e - r * D;
      const int i = r / G, hh = r - i * G;
      const float Ls = mrow[RP + r], Lr = mrow[2 * RP + r];
      const bool live = (i < nq) && (Ls > 0.f);
      const float o = live ? macc[r * DP + d] / Lr : 0.f;
      const size_t oi = (((size_t)b * a.n_max + i) * Hq + g * G + hh) * D + d;
      if (a.out_bf16)
        reinterpret_cast<uint16_t*>(a.out)[oi] = (uint16_t)f32_to_bf16_bits(o);
      else
        reinterpret_cast<float*>(a.out)[oi] = o;
      if (a.lse && d == 0) {
        const float lse = live ? (mrow[r] + log2f(Ls)) * 0.69314718055994531f : -INFINITY;
        a.lse[((size_t)b * a.n_max + i) * Hq + g * G + hh] = lse;
      }
    }
  } else {
    const size_t base = (size_t)u * a.S + s;
    float* pa = a.part_acc + base * R * D;
    for (int e = threadIdx.x; e < R * D; e += blockDim.x) {
      const int r = e / D, d = e - r * D;
      pa[e] = macc[r * DP + d];
    }
    float* pm = a.part_ml + base * 3 * R;
    for (int r = threadIdx.x; r < R; r += blockDim.x) {
      pm[r] = mrow[r];
      pm[R + r] = mrow[RP + r];
      pm[2 * R + r] = mrow[2 * RP + r];
    }
  }
}

// Online-softmax update for one row block: scores sc (already scaled to the
// log2 domain and masked) -> probabilities; rescales the sums and acc.
// l_run sums the exact probabilities (it gives the LSE).  With ROUND_BF16 the
// probabilities fed to the P.V product are rounded to bf16 here and l_rnd
// sums exactly those weights, so O = acc / l_rnd stays an exact convex
// combination of V rows.
template <int DB, bool ROUND_BF16>
__device__ __forceinline__ void softmax_update(f32x4_t (&sc)[2], float& m_run, float& l_run,
                                               float& l_rnd, f32x4_t (&acc)[DB], float (&p)[8]) {
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[kb][i]);
  mx = max_across_rows(mx);
  const float m_new = fmaxf(m_run, mx);
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = exp2f(m_run - m_use);
  m_run = m_new;
  float ls = 0.f, lr = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = exp2f(sc[kb][i] - m_use);
      ls += e;
      const float er = ROUND_BF16 ? __uint_as_float(f32_to_bf16_bits(e) << 16) : e;
      lr += er;
      p[kb * 4 + i] = er;
    }
  l_run = l_run * alpha + ls;
  l_rnd = ROUND_BF16 ? l_rnd * alpha + lr : l_run;
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] *= alpha;
}

// ---------------------------------------------------------------- bf16 ----

template <int D>
struct Bf16Tile {
  static constexpr int KS = D / 32;
  u32x4_t k[2][KS];
  u32x4_t v[8];
  int kpos[2][4];
};

template <int D>
__device__ __forceinline__ void bf16_load_k(const AttnArgs& a, int b, int g, int t0, int t_end,
                                            int lane, Bf16Tile<D>& T) {
  constexpr int KS = D / 32;
  const int r16 = lane & 15, q4 = lane >> 4;
  const uint16_t* kb_ = reinterpret_cast<const uint16_t*>(a.k);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int slot = t0 + 8 * (r16 >> 2) + 4 * kb + (r16 & 3);
    if (slot < t_end) {
      const uint16_t* p = kb_ + kv_row(a, b, g, slot_position(a, b, g, slot)) * D + 8 * q4;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) T.k[kb][ks] = ld16(p + 32 * ks);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) T.k[kb][ks] = u32x4_t{0, 0, 0, 0};
    }
  }
}

template <int D>
__device__ __forceinline__ void bf16_load_v(const AttnArgs& a, int b, int g, int t0, int t_end,
                                            int lane, Bf16Tile<D>& T) {
  const int q4 = lane >> 4;
  const uint16_t* vb_ = reinterpret_cast<const uint16_t*>(a.v);
  const int o = lane & 3, c = lane >> 2;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const int slot = t0 + 8 * o + kk;
    if (c < D / 8 && slot < t_end)
      T.v[kk] = ld16(vb_ + kv_row(a, b, g, slot_position(a, b, g, slot)) * D + 8 * c);
    else
      T.v[kk] = u32x4_t{0, 0, 0, 0};
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int slot = t0 + 8 * q4 + 4 * kb + i;
      T.kpos[kb][i] = (slot < t_end) ? slot_position(a, b, g, slot) : 0x7fffffff;
    }
}

// One tile: S^T = K Q^T, online softmax, V^T -> LDS, O^T += V^T P^T.  The
// next tile's K loads are issued as soon as this tile's K registers are
// consumed, and its V loads as soon as this tile's V is in LDS, so one
// register set keeps a tile of loads in flight behind the softmax and PV.
template <int D, int NB>
__device__ __forceinline__ void bf16_tile(const AttnArgs& a, int b, int g, int t_next, int t_end,
                                          int lane, Bf16Tile<D>& T,
                                          const bf16x8_t (&qop)[NB][D / 32],
                                          const int (&rowP)[NB], uint32_t* vbuf,
                                          float (&m_run)[NB], float (&l_run)[NB],
                                          float (&l_rnd)[NB], f32x4_t (&acc)[D / 16][NB]) {
  constexpr int KS = D / 32, DB = D / 16;
  const int r16 = lane & 15, q4 = lane >> 4;
  const bool more = t_next < t_end;
  f32x4_t sc[NB][2];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x4_t c4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(T.k[kb][ks]), qop[nb][ks], c4, 0,
                                                     0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        c4[i] = (T.kpos[kb][i] <= rowP[nb]) ? c4[i] * a.scale_log2 : -INFINITY;
      sc[nb][kb] = c4;
    }
  if (more) bf16_load_k<D>(a, b, g, t_next, t_end, lane, T);

  // V tile -> LDS as (key 2p, key 2p+1) bf16 pairs, one LDS row per d.
  const int o = lane & 3, c = lane >> 2;
  if (c < D / 8) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      u32x4_t lo, hi;
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const uint32_t x = T.v[2 * pp][w], y = T.v[2 * pp + 1][w];
        lo[pp] = __builtin_amdgcn_perm(y, x, 0x05040100u);
        hi[pp] = __builtin_amdgcn_perm(y, x, 0x07060302u);
      }
      *reinterpret_cast<u32x4_t*>(vbuf + (8 * c + 2 * w) * kPV + 4 * o) = lo;
      *reinterpret_cast<u32x4_t*>(vbuf + (8 * c + 2 * w + 1) * kPV + 4 * o) = hi;
    }
  }
  if (more) bf16_load_v<D>(a, b, g, t_next, t_end, lane, T);

  bf16x8_t pop[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float p[8];
    f32x4_t accn[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) accn[db] = acc[db][nb];
    softmax_update<DB, true>(sc[nb], m_run[nb], l_run[nb], l_rnd[nb], accn, p);
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db][nb] = accn[db];
    u32x4_t pk;
    pk[0] = pack_bf16x2(p[0], p[1]);
    pk[1] = pack_bf16x2(p[2], p[3]);
    pk[2] = pack_bf16x2(p[4], p[5]);
    pk[3] = pack_bf16x2(p[6], p[7]);
    pop[nb] = as_bf16x8(pk);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const u32x4_t va = *reinterpret_cast<const u32x4_t*>(vbuf + (16 * db + r16) * kPV + 4 * q4);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      acc[db][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), pop[nb], acc[db][nb],
                                                            0, 0, 0);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D, int NB>
__global__ __launch_bounds__(256, 1) void attn_bf16_kernel(AttnArgs a) {
  constexpr int KS = D / 32, DB = D / 16, RP = NB * 16;
  constexpr int V_DW = kNW * D * kPV;
  constexpr int M_DW = RP * (D + 4) + 3 * kNW * RP + 3 * RP;
  __shared__ float smem[(V_DW > M_DW) ? V_DW : M_DW];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, q4 = lane >> 4;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int u = wg / a.S, s = wg - u * a.S;
  const int b = u / a.Hkv, g = u - b * a.Hkv;
  const int L = a.kv_len[b];
  const int nq = a.q_len ? a.q_len[b] : a.n_max;
  const int T = (a.mode == 0) ? L : (a.mode == 1 ? a.slot_len[b] : min(a.slot_stride, L));
  const int t_beg = s * a.chunk;
  const int t_end = min(T, t_beg + a.chunk);

  const int stride = kNW * kTK;
  int t0 = t_beg + wave * kTK;
  Bf16Tile<D> tile;
  if (t0 < t_end) {
    bf16_load_k<D>(a, b, g, t0, t_end, lane, tile);
    bf16_load_v<D>(a, b, g, t0, t_end, lane, tile);
  }

  bf16x8_t qop[NB][KS];
  int rowP[NB];
  const uint16_t* qb = reinterpret_cast<const uint16_t*>(a.q);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = nb * 16 + r16;
    const bool valid = n < nq * a.G;
    const int i = n / a.G, hh = n - (n / a.G) * a.G;
    rowP[nb] = valid ? L - nq + i : 0x7fffffff;
    const uint16_t* qp = qb + (((size_t)b * a.n_max + i) * a.Hq + g * a.G + hh) * D + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qop[nb][ks] = valid ? as_bf16x8(ld16(qp + 32 * ks)) : as_bf16x8(u32x4_t{0, 0, 0, 0});
  }

  float m_run[NB], l_run[NB], l_rnd[NB];
  f32x4_t acc[DB][NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m_run[nb] = -INFINITY;
    l_run[nb] = 0.f;
    l_rnd[nb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  uint32_t* vbuf = reinterpret_cast<uint32_t*>(smem) + wave * D * kPV;

  for (; t0 < t_end; t0 += stride)
    bf16_tile<D, NB>(a, b, g, t0 + stride, t_end, lane, tile, qop, rowP, vbuf, m_run, l_run,
                     l_rnd, acc);
  finish_split<D, NB>(a, smem, wave, lane, u, s, b, g, nq, m_run, l_run, l_rnd, acc);
}

// ---------------------------------------------------------------- fp32 ----
// v_mfma_f32_16x16x4_f32: A 16x4, B 4x16, lane l holds A[l%16][l/16] and
// B[l/16][l%16]; C as for the bf16 shape.  Keys in a tile are natural
// (key = 16*kb + m).  For S^T = K Q^T the contraction index d of k-step ks in
// lane row q4 is q4*(D/4) + ks, so each lane reads a contiguous quarter of a
// K row and of a Q row.  For O^T = V^T P^T, k-step s (0..7) takes key
// 16*(s/4) + 4*q4 + s%4 in lane row q4: exactly the probability that lane
// already holds, and V rows read straight from global memory.

template <int D, int NB>
__global__ __launch_bounds__(256, 1) void attn_f32_kernel(AttnArgs a) {
  constexpr int DB = D / 16, Q4 = D / 4, RP = NB * 16;
  constexpr int M_DW = RP * (D + 4) + 3 * kNW * RP + 3 * RP;
  __shared__ float smem[M_DW];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, q4 = lane >> 4;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int u = wg / a.S, s = wg - u * a.S;
  const int b = u / a.Hkv, g = u - b * a.Hkv;
  const int L = a.kv_len[b];
  const int nq = a.q_len ? a.q_len[b] : a.n_max;
  const int T = (a.mode == 0) ? L : (a.mode == 1 ? a.slot_len[b] : min(a.slot_stride, L));
  const int t_beg = s * a.chunk;
  const int t_end = min(T, t_beg + a.chunk);
  const float* qf = reinterpret_cast<const float*>(a.q);
  const float* kf = reinterpret_cast<const float*>(a.k);
  const float* vf = reinterpret_cast<const float*>(a.v);

  float qop[NB][Q4];
  int rowP[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = nb * 16 + r16;
    const bool valid = n < nq * a.G;
    const int i = n / a.G, hh = n - (n / a.G) * a.G;
    rowP[nb] = valid ? L - nq + i : 0x7fffffff;
    const float* qp = qf + (((size_t)b * a.n_max + i) * a.Hq + g * a.G + hh) * D + q4 * Q4;
#pragma unroll
    for (int j = 0; j < Q4; ++j) qop[nb][j] = valid ? qp[j] : 0.f;
  }
  float m_run[NB], l_run[NB], l_rnd[NB];
  f32x4_t acc[DB][NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m_run[nb] = -INFINITY;
    l_run[nb] = 0.f;
    l_rnd[nb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  for (int t0 = t_beg + wave * kTK; t0 < t_end; t0 += kNW * kTK) {
    // K rows: lane row m = r16 holds key 16*kb + r16, d in [q4*Q4, q4*Q4 + Q4)
    float kr[2][Q4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int slot = t0 + 16 * kb + r16;
      if (slot < t_end) {
        const float* p = kf + kv_row(a, b, g, slot_position(a, b, g, slot)) * D + q4 * Q4;
#pragma unroll
        for (int j = 0; j < Q4; ++j) kr[kb][j] = p[j];
      } else {
#pragma unroll
        for (int j = 0; j < Q4; ++j) kr[kb][j] = 0.f;
      }
    }
    // V: for k-step s the lane needs key 16*(s/4) + 4*q4 + s%4 at d = 16*db + r16
    float vr[8][DB];
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const int slot = t0 + 16 * (st >> 2) + 4 * q4 + (st & 3);
      if (slot < t_end) {
        const float* p = vf + kv_row(a, b, g, slot_position(a, b, g, slot)) * D + r16;
#pragma unroll
        for (int db = 0; db < DB; ++db) vr[st][db] = p[16 * db];
      } else {
#pragma unroll
        for (int db = 0; db < DB; ++db) vr[st][db] = 0.f;
      }
    }
    int kpos[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int slot = t0 + 16 * kb + 4 * q4 + i;
        kpos[kb][i] = (slot < t_end) ? slot_position(a, b, g, slot) : 0x7fffffff;
      }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      f32x4_t sc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x4_t c4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < Q4; ++j)
          c4 = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[kb][j], qop[nb][j], c4, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          c4[i] = (kpos[kb][i] <= rowP[nb]) ? c4[i] * a.scale_log2 : -INFINITY;
        sc[kb] = c4;
      }
      float p[8];
      f32x4_t accn[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) accn[db] = acc[db][nb];
      softmax_update<DB, false>(sc, m_run[nb], l_run[nb], l_rnd[nb], accn, p);
#pragma unroll
      for (int st = 0; st < 8; ++st)
#pragma unroll
        for (int db = 0; db < DB; ++db)
          accn[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(vr[st][db], p[st], accn[db], 0, 0, 0);
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db][nb] = accn[db];
    }
  }
  finish_split<D, NB>(a, smem, wave, lane, u, s, b, g, nq, m_run, l_run, l_rnd, acc);
}

// --------------------------------------------------------------- merge ----
// One workgroup per (unit, row): combine the S partials with the log-sum-exp
// rule in a fixed split order.
template <int D>
__global__ __launch_bounds__(D) void attn_merge_kernel(AttnArgs a) {
  const int R = a.R;
  const int u = blockIdx.x / R, r = blockIdx.x - (blockIdx.x / R) * R;
  const int b = u / a.Hkv, g = u - b * a.Hkv;
  const int nq = a.q_len ? a.q_len[b] : a.n_max;
  const int i = r / a.G, hh = r - i * a.G;
  const int d = threadIdx.x;
  const float* pm = a.part_ml + (size_t)u * a.S * 3 * R;
  float M = -INFINITY;
  for (int s = 0; s < a.S; ++s) M = fmaxf(M, pm[s * 3 * R + r]);
  const float Mu = (M == -INFINITY) ? 0.f : M;
  float Ls = 0.f, Lr = 0.f, o = 0.f;
  const float* pa = a.part_acc + (size_t)u * a.S * R * D + (size_t)r * D + d;
  for (int s = 0; s < a.S; ++s) {
    const float w = exp2f(pm[s * 3 * R + r] - Mu);
    Ls += pm[s * 3 * R + R + r] * w;
    Lr += pm[s * 3 * R + 2 * R + r] * w;
    o += pa[(size_t)s * R * D] * w;
  }
  const bool live = (i < nq) && (Ls > 0.f);
  o = live ? o / Lr : 0.f;
  const size_t oi = (((size_t)b * a.n_max + i) * a.Hq + g * a.G + hh) * D + d;
  if (a.out_bf16)
    reinterpret_cast<uint16_t*>(a.out)[oi] = (uint16_t)f32_to_bf16_bits(o);
  else
    reinterpret_cast<float*>(a.out)[oi] = o;
  if (a.lse && d == 0)
    a.lse[((size_t)b * a.n_max + i) * a.Hq + g * a.G + hh] =
        live ? (M + log2f(Ls)) * 0.69314718055994531f : -INFINITY;
}

template <int D, int NB>
hipError_t launch_d_nb(const AttnArgs& a, int dtype, int grid, hipStream_t st) {
  if (dtype == SPEC_BF16)
    hipLaunchKernelGGL((attn_bf16_kernel<D, NB>), dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((attn_f32_kernel<D, NB>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnArgs& a, int dtype, int grid, hipStream_t st) {
  const int nb = (a.R + 15) / 16;
  switch (nb) {
    case 1: return launch_d_nb<D, 1>(a, dtype, grid, st);
    case 2: return launch_d_nb<D, 2>(a, dtype, grid, st);
    case 3: return launch_d_nb<D, 3>(a, dtype, grid, st);
    default: return launch_d_nb<D, 4>(a, dtype, grid, st);
  }
}

__global__ __launch_bounds__(256) void zero_fill_kernel(uint32_t* p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

}  // namespace

spec_status_t launch_zero(void* p, size_t bytes, hipStream_t stream) {
  const size_t words = bytes / 4;
  if (words == 0) return SPEC_OK;
  size_t blocks = (words + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<uint32_t*>(p), words);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

AttnPlan plan_attention(int units, int t_max, int rows, int d) {
  AttnPlan p;
  const int target = device_cu_count();            // about one workgroup per CU
  const long total = (long)units * (long)(t_max > 0 ? t_max : 1);
  long chunk = (total + target - 1) / target;
  chunk = ((chunk + kTK - 1) / kTK) * kTK;
  if (chunk < kTK * kNW) chunk = kTK * kNW;        // every wave gets a tile
  int S = (int)(((long)(t_max > 0 ? t_max : 1) + chunk - 1) / chunk);
  if (S < 1) S = 1;
  p.S = S;
  p.chunk = (int)chunk;
  p.grid = units * S;
  if (S > 1) {
    const size_t acc_bytes = (size_t)units * S * rows * d * sizeof(float);
    p.off_ml = align_up(acc_bytes, 256);
    p.ws_bytes = p.off_ml + align_up((size_t)units * S * 3 * rows * sizeof(float), 256);
  }
  return p;
}

spec_status_t launch_attention(AttnArgs a, int d, int dtype, const AttnPlan& plan, void* ws,
                               hipStream_t stream) {
  a.S = plan.S;
  a.chunk = plan.chunk;
  if (plan.S > 1) {
    a.part_acc = reinterpret_cast<float*>(ws);
    a.part_ml = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + plan.off_ml);
  } else {
    a.part_acc = nullptr;
    a.part_ml = nullptr;
  }
  if (plan.grid == 0) return SPEC_OK;
  hipError_t e = (d == 64) ? launch_d<64>(a, dtype, plan.grid, stream)
                           : launch_d<128>(a, dtype, plan.grid, stream);
  if (e != hipSuccess) return SPEC_ERR_HIP;
  if (plan.S > 1) {
    const int blocks = a.B * a.Hkv * a.R;
    if (d == 64)
      hipLaunchKernelGGL(attn_merge_kernel<64>, dim3(blocks), dim3(64), 0, stream, a);
    else
      hipLaunchKernelGGL(attn_merge_kernel<128>, dim3(blocks), dim3(128), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
  }
  return SPEC_OK;
}

}  // namespace spec

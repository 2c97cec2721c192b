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
constexpr int kMaxChunk = 2048;     // keys per split (their rows and sums are staged in LDS)

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
  k.rows = ld_uniform(a.text_len, k.b) * a.G;
  k.r0 = k.rb * kBR;
  k.L = ld_uniform(a.kv_len, k.b);
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

// Key rows of this workgroup's split: computed for a contiguous cache, read
// from LDS (resolved once through the page table) for a paged one, so the key
// loop issues no dependent global loads.
template <bool PAGED>
struct KeyRows {
  size_t base;          // contiguous: first row of (b, g)
  const uint32_t* row;  // paged: LDS rows of keys k0..
  int k0;
  __device__ __forceinline__ size_t operator()(int key) const {
    return PAGED ? (size_t)row[key - k0] : base + (size_t)key;
  }
};

// 2^x on the transcendental unit (v_exp_f32) without the library's
// denormal-result fix-up: every term here is a probability-like weight, and
// results below 2^-126 are negligible against the sums they join.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Per-wave LDS ring of key blocks.  Each wave streams its own 16-key blocks
// through kNSW stages filled by global_load_lds_dwordx4 (no registers in
// flight, and the loads cannot be moved by the compiler); only the wave that
// fills a stage reads it, so a vmcnt wait is the only synchronisation.  A
// stage holds 16 rows of D bf16; the 16-byte chunk c of row r sits at slot
// c ^ swz(r), which makes the operand reads (16 rows, one chunk column)
// bank-conflict free.
constexpr int kNSW = 3;

template <int D>
struct Stage {
  static constexpr int ROWB = D * 2;             // bytes per key row
  static constexpr int CH = D / 8;               // 16-byte chunks per row
  static constexpr int BYTES = 16 * ROWB;
  static constexpr int NDMA = BYTES / 1024;      // 1 KB DMA instructions per stage
  static constexpr int RPD = 1024 / ROWB;        // rows per DMA instruction
  __device__ static __forceinline__ int swz(int r) {
    return CH == 16 ? (r & 15) : ((r >> 1) & 7);
  }
};

template <int D, bool PAGED>
__device__ __forceinline__ void issue_stage(const StdArgs& a, const KeyRows<PAGED>& kr, int kb,
                                            int kend, uint32_t lds, int lane) {
  using St = Stage<D>;
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(a.k);
#pragma unroll
  for (int j = 0; j < St::NDMA; ++j) {
    const int row = j * St::RPD + lane / St::CH;
    const int chunk = (lane % St::CH) ^ St::swz(row);
    const int key = min(kb + row, kend - 1);           // a row that exists
    dma16(kbase + kr(key) * St::ROWB + chunk * 16, lds + (uint32_t)(j * 1024));
  }
}

// This lane's operand for chunk c: row r16 of the stage.
template <int D>
__device__ __forceinline__ u32x4_t read_op(const unsigned char* stage, int r16, int c) {
  using St = Stage<D>;
  return *reinterpret_cast<const u32x4_t*>(stage + r16 * St::ROWB + 16 * (c ^ St::swz(r16)));
}

template <int D>
__device__ __forceinline__ void read_block(const unsigned char* stage, int r16, int q4,
                                           u32x4_t (&kc)[D / 32]) {
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) kc[ks] = read_op<D>(stage, r16, 4 * ks + q4);
}

// Waits until at most N of this wave's vector memory operations are pending.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Pass A on one 16-key block: S^T = K Q^T, lane (r16, q4) holds keys
// kb + 4*q4 + i of row 16*rg + r16; per-lane lazily re-referenced sums.  All
// eight MFMA chains are issued before any result is used, and the code is
// straight-line (MASK and the rare re-reference are wave-uniform branches),
// so the matrix and vector pipes overlap.
template <int D, bool MASK>
__device__ __forceinline__ void tile_rows(const StdArgs& a, const u32x4_t (&kc)[D / 32],
                                          const bf16x8_t (&qop)[kRG][D / 32], int kb, int q4,
                                          const int (&pos)[kRG], float (&m)[kRG],
                                          float (&l)[kRG]) {
  f32x4_t c[kRG];
#pragma unroll
  for (int rg = 0; rg < kRG; ++rg) {
    c[rg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      c[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kc[ks]), qop[rg][ks], c[rg], 0,
                                                      0, 0);
  }
  float tmax[kRG];
  bool raise = false;
#pragma unroll
  for (int rg = 0; rg < kRG; ++rg) {
    if (MASK) {
#pragma unroll
      for (int i = 0; i < 4; ++i) c[rg][i] = (kb + 4 * q4 + i <= pos[rg]) ? c[rg][i] : -INFINITY;
    }
    // the scale is positive, so the maximum can be taken before scaling; the
    // IEEE maximum (NaN-propagating) needs no canonicalisation of the
    // matrix-core results, unlike fmaxf
    tmax[rg] = __builtin_elementwise_maximum(__builtin_elementwise_maximum(c[rg][0], c[rg][1]),
                                             __builtin_elementwise_maximum(c[rg][2], c[rg][3])) *
               a.scale_log2;
    raise |= tmax[rg] > m[rg] + 8.f;
  }
  // lazily raised reference: terms stay <= 2^8 and raises are rare
  if (__builtin_amdgcn_ballot_w64(raise)) {
#pragma unroll
    for (int rg = 0; rg < kRG; ++rg) {
      const bool up = tmax[rg] > m[rg] + 8.f;
      l[rg] = up ? l[rg] * ex2(m[rg] - tmax[rg]) : l[rg];
      m[rg] = up ? tmax[rg] : m[rg];
    }
  }
#pragma unroll
  for (int rg = 0; rg < kRG; ++rg) {
    const float nm = -m[rg];
    l[rg] += (ex2(fmaf(c[rg][0], a.scale_log2, nm)) + ex2(fmaf(c[rg][1], a.scale_log2, nm))) +
             (ex2(fmaf(c[rg][2], a.scale_log2, nm)) + ex2(fmaf(c[rg][3], a.scale_log2, nm)));
  }
}

// Pass B on one 16-key block: S = Q K^T, lane (r16, q4) holds rows
// 16*rg + 4*q4 + i of key kb + r16; returns the key's sum over the 128 rows.
template <int D, bool MASK>
__device__ __forceinline__ float tile_keys(const StdArgs& a, const u32x4_t (&kc)[D / 32],
                                           const bf16x8_t (&qop)[kRG][D / 32], int key, int q4,
                                           const int* s_pos, const float (&crow)[kRG][4]) {
  f32x4_t c[kRG];
#pragma unroll
  for (int rg = 0; rg < kRG; ++rg) {
    c[rg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      c[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qop[rg][ks], as_bf16x8(kc[ks]), c[rg], 0,
                                                      0, 0);
  }
  float acc = 0.f;
#pragma unroll
  for (int rg = 0; rg < kRG; ++rg) {
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = ex2(fmaf(c[rg][i], a.scale_log2, -crow[rg][i]));
    if (MASK) {
      const int4 pr = *reinterpret_cast<const int4*>(&s_pos[rg * 16 + 4 * q4]);
      p[0] = (key <= pr.x) ? p[0] : 0.f;
      p[1] = (key <= pr.y) ? p[1] : 0.f;
      p[2] = (key <= pr.z) ? p[2] : 0.f;
      p[3] = (key <= pr.w) ? p[3] : 0.f;
    }
    acc += (p[0] + p[1]) + (p[2] + p[3]);
  }
  return sum_across_rows(acc);
}

template <int D, int PASS, bool PAGED>
__global__ __launch_bounds__(256, 2) void std_mfma_kernel(StdArgs a) {
  constexpr int KS = D / 32;
  using St = Stage<D>;
  __shared__ __align__(16) unsigned char ring[4 * kNSW * St::BYTES];
  __shared__ __align__(16) int s_pos[kBR];
  __shared__ float s_c[kBR];
  __shared__ float s_m[4][kBR], s_l[4][kBR];
  __shared__ uint32_t s_row[PAGED ? kMaxChunk : 1];
  __shared__ float s_out[PASS == 1 ? kMaxChunk : 1];

  Block k;
  if (!decode_block(a, k)) return;
  // wave-uniform values live in scalar registers, so the key loop is a plain
  // scalar loop
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, q4 = lane >> 4;
  stage_positions(a, k, s_pos);
  if (PASS == 1) stage_offsets(a, k, s_c);
  KeyRows<PAGED> kr;
  kr.base = ((size_t)k.b * a.Hkv + k.g) * (size_t)a.max_len;
  kr.row = s_row;
  kr.k0 = k.k0;
  if (PAGED) {
    for (int j = k.k0 + (int)threadIdx.x; j < k.k1; j += blockDim.x)
      s_row[j - k.k0] = (uint32_t)key_row(a, k.b, k.g, j);
  }
  bf16x8_t qop[kRG][KS];
  load_q<D>(a, k, r16, q4, qop);
  __syncthreads();
  wait_vm<0>();                 // the ring's wait counts below start from zero

  const int nrow = min(k.rows - k.r0, kBR);
  const int p_max = __builtin_amdgcn_readfirstlane(s_pos[nrow - 1]);
  const int p_min = (nrow < kBR) ? -1 : __builtin_amdgcn_readfirstlane(s_pos[0]);
  const int kend = min(k.k1, p_max + 1);               // no row sees a key at or past this
  // (p_min = -1: padded rows need the mask everywhere)

  // Key blocks of this wave: kb = k0 + 16*wave + 64*i < kend.  Stage i%kNSW
  // of the wave's ring holds block i; kNSW-1 blocks are in flight while one
  // is computed.  Every loaded row is clamped to key kend-1 (a row that
  // exists); keys past it are masked by position.
  const unsigned char* wring = ring + wave * kNSW * St::BYTES;
  const uint32_t wring_lds = (uint32_t)(size_t)(lds_u8_t*)wring;
  const int kb0 = k.k0 + 16 * wave;
  const int nblk = (kend > kb0) ? (kend - kb0 + kKeysPerIter - 1) / kKeysPerIter : 0;

  float m[kRG], l[kRG];
  int pos[kRG];
  float crow[kRG][4];
  if (PASS == 0) {
#pragma unroll
    for (int rg = 0; rg < kRG; ++rg) {
      pos[rg] = s_pos[rg * 16 + r16];
      m[rg] = kNoMax;
      l[rg] = 0.f;
    }
  } else {
#pragma unroll
    for (int rg = 0; rg < kRG; ++rg)
#pragma unroll
      for (int i = 0; i < 4; ++i) crow[rg][i] = s_c[rg * 16 + 4 * q4 + i];
  }

  if (nblk > 0) {
#pragma unroll
    for (int i = 0; i < kNSW - 1; ++i)
      issue_stage<D, PAGED>(a, kr, kb0 + i * kKeysPerIter, kend,
                            wring_lds + (uint32_t)(i * St::BYTES), lane);
    for (int i = 0; i < nblk; ++i) {
      const int nxt = i + kNSW - 1;                      // always issued, clamped
      issue_stage<D, PAGED>(a, kr, kb0 + nxt * kKeysPerIter, kend,
                            wring_lds + (uint32_t)((nxt % kNSW) * St::BYTES), lane);
      wait_vm<(kNSW - 1) * St::NDMA>();                  // block i has landed
      const int kb = kb0 + i * kKeysPerIter;
      u32x4_t kc[KS];
      read_block<D>(wring + (i % kNSW) * St::BYTES, r16, q4, kc);
      const bool mask = kb + 15 > p_min;   // wave-uniform
      if (PASS == 0) {
        if (mask) tile_rows<D, true>(a, kc, qop, kb, q4, pos, m, l);
        else tile_rows<D, false>(a, kc, qop, kb, q4, pos, m, l);
      } else {
        const float acc = mask ? tile_keys<D, true>(a, kc, qop, kb + r16, q4, s_pos, crow)
                               : tile_keys<D, false>(a, kc, qop, kb + r16, q4, s_pos, crow);
        if (q4 == 0) s_out[kb + r16 - k.k0] = acc;
      }
    }
    wait_vm<0>();                // no DMA into the ring outlives the loop
  }

  if (PASS == 0) {
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
    // the split's keys: computed blocks from LDS, keys no row sees as 0
    __syncthreads();
    float* out = a.colsum + ((size_t)k.u * a.RB + k.rb) * a.max_len;
    const int kcov = k.k0 + ((max(kend - k.k0, 0) + 15) / 16) * 16;
    for (int j = k.k0 + (int)threadIdx.x; j < k.k1; j += blockDim.x)
      out[j] = (j < kcov) ? s_out[j - k.k0] : 0.f;
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

// The first pass is the call's main kernel for the measurement hook.
template <int D>
hipError_t launch_passes(const StdArgs& a, int dtype, int grid, hipStream_t stream) {
  mark_before_main(stream);
  if (dtype == SPEC_BF16 && a.page_shift >= 0) {
    hipLaunchKernelGGL((std_mfma_kernel<D, 0, true>), dim3(grid), dim3(256), 0, stream, a);
    mark_after_main(stream);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    hipLaunchKernelGGL((std_mfma_kernel<D, 1, true>), dim3(grid), dim3(256), 0, stream, a);
  } else if (dtype == SPEC_BF16) {
    hipLaunchKernelGGL((std_mfma_kernel<D, 0, false>), dim3(grid), dim3(256), 0, stream, a);
    mark_after_main(stream);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    hipLaunchKernelGGL((std_mfma_kernel<D, 1, false>), dim3(grid), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((std_scalar_kernel<D, 0>), dim3(grid), dim3(256), 0, stream, a);
    mark_after_main(stream);
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
  // about four workgroups per CU (two fit at once), splits of at least 256
  // keys, every split a whole number of 64-key iterations.  Longer splits
  // amortise each workgroup's query-row set-up: at 25k keys x 512 text rows,
  // 10 splits per row block take 278 us against 295 us for 19 (eight per
  // CU); 7 splits (two or three per CU) take the same 278, 37 take 396
  const long target = 4L * device_cu_count();
  const long blocks = (long)units * p.RB;
  long S = (target + blocks - 1) / blocks;
  const long smax = (max_len + 255) / 256;
  if (S > smax) S = smax;
  if (S < 1) S = 1;
  if (S < (max_len + kMaxChunk - 1) / kMaxChunk) S = (max_len + kMaxChunk - 1) / kMaxChunk;
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

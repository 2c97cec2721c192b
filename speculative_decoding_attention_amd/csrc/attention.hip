// Split-K flash-decoding attention for gfx950: the shared engine behind
// verification attention (dense positions), text-anchored draft attention
// (positions from a text index list), top-K sparse draft attention
// (positions from a per-head selection list) and the Sparse-to-Dense draft
// attention (a per-head kept list plus a dense tail).
//
// Work decomposition.  A unit is a (sequence b, KV head g) pair; its query
// block is the n_max * G rows (query position i, head-in-group hh), row
// r = i*G + hh, padded to NB*16 rows.  The unit's key slots are cut into S
// splits of `chunk` slots, about one workgroup per CU in all.  A workgroup
// writes either the final output (S == 1) or unnormalised partials that
// attn_merge_kernel combines with the log-sum-exp rule.
//
// bf16, d = 128 (attn_bf16_pipe_kernel): K/V rows move HBM -> LDS by DMA
// (global_load_lds_dwordx4) into a 128 KiB ring of tiles, so data in flight
// costs no registers.  Each wave owns up to 16 query rows (NB row blocks) and
// one 32-key sub-tile phase of every tile; with NB >= 3 eight waves form two
// teams on alternate sub-tiles.  Per sub-tile:
//   S^T = K Q^T   on v_mfma_f32_16x16x32_bf16, K from the swizzled LDS tile,
//                 Q^T held in registers;
//   online softmax in fp32 (exp2 domain) against a lazily raised reference;
//   O^T += V^T P^T with V^T read transposed from LDS (ds_read_b64_tr_b16)
//                 and P already laid out as the B operand.
// At the end the phases are merged in LDS, or, when a unit has few splits,
// every wave writes its own partial.
//
// d = 64 bf16 and fp32 (attn_bf16_kernel, attn_f32_kernel): four waves per
// workgroup stream 32-slot tiles from global memory into registers, each
// with its own online-softmax state, and merge in LDS; the fp32 variant uses
// v_mfma_f32_16x16x4_f32, where V needs no transpose.
#include <math.h>

#include <atomic>

#include "common.h"
#include "internal.h"

namespace spec {

namespace {

constexpr int kTK = 32;   // key slots per tile
constexpr int kNW = 4;    // waves per workgroup
constexpr int kPV = 20;   // dwords per LDS row of a transposed V tile (16 + 4 pad)

// Slots per split whose (position, row) are staged in LDS; with the 128 KiB
// ring and the per-32-slot maxima this fills the 160 KiB of LDS.
constexpr int kMaxChunk = 4032;

// Where the key slots of one split live.  Dense contiguous splits compute
// position and row arithmetically; every other layout (a text index list, a
// top-K list, a paged pool) is resolved once per workgroup into LDS before
// the streaming loop, so the loop's only global loads are K and V rows.
template <bool GATHER>
struct SlotMap {
  int t_beg;
  uint32_t base_row;      // dense: first row of (b, g)
  const int* pos;         // gather: LDS positions of slots t_beg..
  const uint32_t* row;    // gather: LDS row indices of slots t_beg.. (or pages, below)
  // Dense slots in a paged cache (every position in order): row[] holds the
  // split's pages instead, from page pg0 on, so a split can span 4031 pages
  // rather than 4032 slots.  shift = log2(page size), or -1 for a list.
  int shift, pg0;
  uint32_t hkv, g;
  __device__ __forceinline__ int position(int slot) const {
    return !GATHER ? slot : (shift >= 0 ? slot : pos[slot - t_beg]);
  }
  __device__ __forceinline__ uint32_t rowof(int slot) const {
    if (!GATHER) return base_row + (uint32_t)slot;
    if (shift < 0) return row[slot - t_beg];
    return ((row[(slot >> shift) - pg0] * hkv + g) << shift) + (uint32_t)(slot & ((1 << shift) - 1));
  }
  __device__ __forceinline__ void set_pages(const AttnArgs& a, int g_) {
    shift = (a.mode == 0) ? a.page_shift : -1;
    pg0 = (shift >= 0) ? (t_beg >> shift) : 0;
    hkv = (uint32_t)a.Hkv;
    g = (uint32_t)g_;
  }
};

// Mode 3: first position of the tail (kv_len without a tail).
__device__ __forceinline__ int tail_begin(const AttnArgs& a, int b, int L) {
  return a.tail_start ? ld_uniform(a.tail_start, b) : L - min(a.tail_window, L);
}

// Number of key slots of unit (b, g) (see AttnArgs::mode).
__device__ __forceinline__ int unit_slots(const AttnArgs& a, int b, int g, int L) {
  if (a.mode == 0) return L;
  if (a.mode == 1) return ld_uniform(a.slot_len, b);
  if (a.mode == 2) return min(a.slot_stride, L);
  return ld_uniform(a.slot_len, b * a.Hkv + g) + max(0, L - tail_begin(a, b, L));
}

// Balanced split plan from the device lengths.  One lane per sequence (at
// most 64) loads its slot count T_b (modes 0-2: the same for each of its KV
// heads); every unit of sequence b gets S_b = max(1, ceil(T_b / ch)) splits
// of ch slots, where ch is the smallest multiple of 32 (at least 128) with
// at most `dyn_groups` splits in all -- found by bisection between the
// total over dyn_groups and the capacity plan's split length, which always
// fits.  So every split fits the capacity plan's LDS staging and the grid
// (one workgroup per CU), and the longest split is as short as the whole
// tiles allow.  Splits are numbered unit by unit (b, then g, then s); split
// w's partial is slot w.  Each wave computes the plan itself (one vector
// load, then shuffles).
struct DynSplit {
  int b, g, s;      // unit (b, g) and split index within it
  int ch;           // slots per split
  int S;            // splits of the unit
  int first;        // slot of the unit's first partial
  int w;            // split index (= partial slot)
  bool valid;       // false: this workgroup has no split
};

// by_unit: `key` is a unit index (the merge's query).  Otherwise `key` is
// the workgroup index: workgroups below the number of splits take one each,
// through the XCD-aware order over exactly that many (the hardware deals
// workgroup i to XCD i mod 8, so the splits spread evenly over the XCDs and
// neighbouring splits share one), the rest have nothing to do.
__device__ __forceinline__ DynSplit dyn_split(const AttnArgs& a, int key, bool by_unit) {
  const int lane = threadIdx.x & 63;
  const int bb = min(lane, a.B - 1);
  int t = (a.mode == 1) ? a.slot_len[bb] : a.kv_len[bb];
  if (a.mode == 2) t = min(t, a.slot_stride);
  const int T = (lane < a.B) ? max(t, 0) : 0;
  // 32-bit arithmetic in the search (lengths and split lengths stay below
  // 2^30; only the batch's total needs 64 bits, here from two 32-bit sums):
  // a 64-bit division is a long emulated sequence, and every split and merge
  // workgroup runs this search.  Its sums over the batch are DPP sums.
  const long tot = ((long)wave_sum((uint32_t)T >> 6) * 64 + (long)wave_sum((uint32_t)T & 63u)) *
                   a.Hkv;
  int lo = (int)((tot + a.dyn_groups - 1) / a.dyn_groups);
  lo = max(((lo + kTK - 1) / kTK) * kTK, kTK * kNW);
  int hi = max(a.chunk, lo);                         // the capacity plan's length fits
  while (lo < hi) {                                  // multiples of kTK: smallest that fits
    const int mid = ((lo + hi) / 2 / kTK) * kTK;
    const int c = max(mid, lo);
    const int n = (int)wave_sum(
        (lane < a.B) ? max(1u, ((unsigned)T + (unsigned)c - 1u) / (unsigned)c) : 0u);
    if (n * a.Hkv <= a.dyn_groups) hi = c;
    else lo = c + kTK;
  }
  const int ch = hi;
  const int Sb = (lane < a.B) ? max(1, (T + ch - 1) / ch) : 0;
  const int cnt = Sb * a.Hkv;
  const int incl = (int)wave_prefix_sum((uint32_t)cnt);
  DynSplit d;
  d.ch = ch;
  if (by_unit) {
    d.b = __builtin_amdgcn_readfirstlane(key / a.Hkv);   // a unit of the workgroup
    d.g = key - d.b * a.Hkv;
    d.s = 0;
    d.S = __builtin_amdgcn_readlane(Sb, d.b);
    d.first = __builtin_amdgcn_readlane(incl - cnt, d.b) + d.g * d.S;
    d.w = d.first;
    d.valid = true;
    return d;
  }
  const int total = __builtin_amdgcn_readlane(incl, 63);   // lanes past B add nothing
  d.valid = key < total;
  key = d.valid ? xcd_remap(key, total) : 0;
  d.w = key;
  const uint64_t m = __builtin_amdgcn_ballot_w64(lane < a.B && key < incl);
  d.b = d.valid ? __ffsll((long long)m) - 1 : 0;
  d.S = max(1, __builtin_amdgcn_readlane(Sb, d.b));
  const int off = key - __builtin_amdgcn_readlane(incl - cnt, d.b);
  d.g = off / d.S;
  d.s = off - d.g * d.S;
  d.first = key - d.s;
  return d;
}

// The list entry of this thread's first slot, t_beg + threadIdx.x, requested
// before the lengths that bound the split are known: the index is clamped to
// the list's extent, so the load is always in bounds, and stage_slots ignores
// it where the slot turns out to lie past the list.  This takes one global
// round trip off the path to the first K/V request.
__device__ __forceinline__ int prefetch_slot(const AttnArgs& a, int b, int g, int t_beg) {
  if (a.mode == 0 || a.slot_stride <= 0) return 0;
  const size_t base = (size_t)(a.mode == 1 ? b : b * a.Hkv + g) * a.slot_stride;
  return a.slots[base + min(t_beg + (int)threadIdx.x, a.slot_stride - 1)];
}

// Resolves slots [t_beg, t_end) of (b, g) into LDS: logical position from the
// slot list (or the slot itself), then the physical row through the page
// table when the cache is paged.  Rows fit 32 bits for any pool that fits in
// device memory.  `pre` is prefetch_slot's value for the first slot.  `bmax`
// (optional) receives the largest visible position of every 32 slots.
__device__ __forceinline__ void stage_slots(const AttnArgs& a, int b, int g, int L, int t_beg,
                                            int t_end, int* pos, uint32_t* row, int* bmax,
                                            int pre) {
  const size_t u = (size_t)b * a.Hkv + g;
  if (a.mode == 0) {              // every position of a paged cache: stage the pages
    if (t_end <= t_beg) return;
    const int pg0 = t_beg >> a.page_shift, pg1 = (t_end - 1) >> a.page_shift;
    for (int pg = pg0 + (int)threadIdx.x; pg <= pg1; pg += blockDim.x)
      row[pg - pg0] = (uint32_t)a.page_table[(size_t)b * a.max_pages + pg];
    return;
  }
  const int n_list = (a.mode == 3) ? ld_uniform(a.slot_len, (int)u) : 0;
  const int t0 = (a.mode == 3) ? tail_begin(a, b, L) : 0;
  const int first = t_beg + (int)threadIdx.x;
  // Every thread runs every round (t_beg and blockDim are multiples of 32),
  // so each 32-lane half of a wave can also reduce the largest position of
  // its 32 consecutive slots: a sub-tile whose largest position precedes
  // every query row needs no mask.  List reads past t_end are clamped.
  for (int r0 = t_beg; r0 < t_end; r0 += blockDim.x) {
    const int t = r0 + (int)threadIdx.x;
    const int tc = min(t, t_end - 1);
    int p;
    bool skip = false;          // a list entry inside the tail: the tail has it
    if (a.mode == 1) p = (t == first) ? pre : a.slots[(size_t)b * a.slot_stride + tc];
    else if (a.mode == 2) p = (t == first) ? pre : a.slots[u * a.slot_stride + tc];
    else if (tc < n_list) {
      p = (t == first) ? pre : a.slots[u * a.slot_stride + tc];
      skip = p >= t0;
    } else {
      p = t0 + (tc - n_list);
    }
    const int vis = skip ? 0x7fffffff : p;      // never visible; its row is still a real one
    if (t < t_end) {
      uint32_t r;
      if (a.page_shift >= 0) {
        const int page = a.page_table[(size_t)b * a.max_pages + (p >> a.page_shift)];
        r = (((uint32_t)page * (uint32_t)a.Hkv + (uint32_t)g) << a.page_shift) +
            (uint32_t)(p & ((1 << a.page_shift) - 1));
      } else {
        r = ((uint32_t)b * (uint32_t)a.Hkv + (uint32_t)g) * (uint32_t)a.max_len + (uint32_t)p;
      }
      pos[t - t_beg] = vis;
      row[t - t_beg] = r;
    }
    int mx = (t < t_end) ? vis : 0x7fffffff;
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) mx = max(mx, __shfl_xor(mx, o));
    if (bmax && (threadIdx.x & 31) == 0 && t < t_end) bmax[(t - t_beg) >> 5] = mx;
  }
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

template <int D, bool GATHER>
__device__ __forceinline__ void bf16_load_k(const AttnArgs& a, const SlotMap<GATHER>& sm, int t0,
                                            int t_end, int lane, Bf16Tile<D>& T) {
  constexpr int KS = D / 32;
  const int r16 = lane & 15, q4 = lane >> 4;
  const uint16_t* kb_ = reinterpret_cast<const uint16_t*>(a.k);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int slot = t0 + 8 * (r16 >> 2) + 4 * kb + (r16 & 3);
    if (slot < t_end) {
      const uint16_t* p = kb_ + (size_t)sm.rowof(slot) * D + 8 * q4;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) T.k[kb][ks] = ld16(p + 32 * ks);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) T.k[kb][ks] = u32x4_t{0, 0, 0, 0};
    }
  }
}

template <int D, bool GATHER>
__device__ __forceinline__ void bf16_load_v(const AttnArgs& a, const SlotMap<GATHER>& sm, int t0,
                                            int t_end, int lane, Bf16Tile<D>& T) {
  const int q4 = lane >> 4;
  const uint16_t* vb_ = reinterpret_cast<const uint16_t*>(a.v);
  const int o = lane & 3, c = lane >> 2;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const int slot = t0 + 8 * o + kk;
    if (c < D / 8 && slot < t_end)
      T.v[kk] = ld16(vb_ + (size_t)sm.rowof(slot) * D + 8 * c);
    else
      T.v[kk] = u32x4_t{0, 0, 0, 0};
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int slot = t0 + 8 * q4 + 4 * kb + i;
      const int pos = sm.position(min(slot, t_end - 1));   // unconditional read, no branch
      T.kpos[kb][i] = (slot < t_end) ? pos : 0x7fffffff;
    }
}

// One tile: S^T = K Q^T, online softmax, V^T -> LDS, O^T += V^T P^T.  The
// next tile's K loads are issued as soon as this tile's K registers are
// consumed, and its V loads as soon as this tile's V is in LDS, so one
// register set keeps a tile of loads in flight behind the softmax and PV.
template <int D, int NB, bool GATHER>
__device__ __forceinline__ void bf16_tile(const AttnArgs& a, const SlotMap<GATHER>& sm, int t_next,
                                          int t_end,
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
  if (more) bf16_load_k<D, GATHER>(a, sm, t_next, t_end, lane, T);

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
  if (more) bf16_load_v<D, GATHER>(a, sm, t_next, t_end, lane, T);

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

template <int D, int NB, bool GATHER>
__global__ __launch_bounds__(256, 1) void attn_bf16_kernel(AttnArgs a) {
  constexpr int KS = D / 32, DB = D / 16, RP = NB * 16;
  constexpr int V_DW = kNW * D * kPV;
  constexpr int M_DW = RP * (D + 4) + 3 * kNW * RP + 3 * RP;
  __shared__ float smem[(V_DW > M_DW) ? V_DW : M_DW];
  __shared__ int s_pos[GATHER ? kMaxChunk : 1];
  __shared__ uint32_t s_row[GATHER ? kMaxChunk : 1];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, q4 = lane >> 4;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int u = wg / a.S, s = wg - u * a.S;
  const int b = u / a.Hkv, g = u - b * a.Hkv;
  const int pre = GATHER ? prefetch_slot(a, b, g, s * a.chunk) : 0;
  const int L = ld_uniform(a.kv_len, b);
  const int nq = a.q_len ? ld_uniform(a.q_len, b) : a.n_max;
  const int T = unit_slots(a, b, g, L);
  const int t_beg = s * a.chunk;
  const int t_end = min(T, t_beg + a.chunk);

  SlotMap<GATHER> sm;
  sm.t_beg = t_beg;
  sm.base_row = ((uint32_t)b * (uint32_t)a.Hkv + (uint32_t)g) * (uint32_t)a.max_len;
  sm.pos = s_pos;
  sm.row = s_row;
  sm.set_pages(a, g);
  if (GATHER) {
    stage_slots(a, b, g, L, t_beg, t_end, s_pos, s_row, nullptr, pre);
    __syncthreads();
  }

  const int stride = kNW * kTK;
  int t0 = t_beg + wave * kTK;
  Bf16Tile<D> tile;
  if (t0 < t_end) {
    bf16_load_k<D, GATHER>(a, sm, t0, t_end, lane, tile);
    bf16_load_v<D, GATHER>(a, sm, t0, t_end, lane, tile);
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
    bf16_tile<D, NB, GATHER>(a, sm, t0 + stride, t_end, lane, tile, qop, rowP, vbuf, m_run,
                             l_run, l_rnd, acc);
  finish_split<D, NB>(a, smem, wave, lane, u, s, b, g, nq, m_run, l_run, l_rnd, acc);
}

// ------------------------------------------------- bf16 d=128 pipeline ----
// The streaming kernel every bf16 head_dim-128 call runs.  K and V rows go
// straight from HBM into an LDS ring by DMA (global_load_lds_dwordx4), so
// data in flight costs no registers and up to NS-1 tiles are outstanding
// per workgroup.  Each of the 4 waves owns one 16-row query block (NB >= 3)
// or one 32-key sub-tile of the tile (NB < 3, KP = 4/NB sub-tiles per tile).
//
// LDS layout of a 32-key sub-tile (K or V): key row r at r*256 bytes, its
// 16-byte chunk c at slot c ^ swz(r), swz(r) = 2*(r&7) ^ ((r>>3)&1).  With
// this swizzle the K operand reads (16 keys, one chunk) and the transposed V
// reads (ds_read_b64_tr_b16 over 4 keys x 32 bytes per 16-lane group) both
// hit 16 distinct 16-byte bank groups.
//
// Keys inside a sub-tile are in natural order: the S^T = K Q^T output gives
// lane (q4, i) keys 16*kb + 4*q4 + i, which is exactly the order in which two
// transposed reads (keys 4*q4.., 16 + 4*q4..) assemble the V^T operand.

__device__ __forceinline__ uint32_t swz(uint32_t r) { return ((r & 7u) << 1) ^ ((r >> 3) & 1u); }

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

template <int NB, bool GATHER = false>
struct PipeCfg {
  // NB >= 3: 8 waves in two teams; each team's waves own one 16-row block and
  // the teams take alternate 32-key sub-tiles, so every SIMD runs two waves.
  // NB <= 2: 4 waves, the spare waves take further sub-tiles.
  static constexpr int WAVES = (NB >= 3) ? 8 : 4;
  static constexpr int SLOTS = (NB >= 3) ? 4 : NB;        // row-block slots per team
  static constexpr int KP = WAVES / SLOTS;                 // 32-key sub-tiles per tile
  static constexpr int TILE_KEYS = 32 * KP;
  static constexpr int SUB_BYTES = 32 * 256;               // one sub-tile of K (or V)
  static constexpr int TILE_BYTES = KP * 2 * SUB_BYTES;
  // Splits of 64-key tiles keep a three-stage ring (two tiles in flight
  // while one is computed); a gathered split's slot tables take the LDS
  // beside it.  Deeper rings measured slower: dense at 25k keys over 248
  // splits, four stages about 1 us per call more, five about 2 us (also with
  // the first burst held at two tiles, so the cost is in the steady state,
  // not in the prologue); gathered, four stages against three, C5's
  // text-anchored batch 57.3 against 56.4 us and the ragged paged
  // verification 116.3 against 114.8 us.  128-key tiles (NB = 1) keep two.
  static constexpr int RING_BYTES = (NB >= 2 ? 96 : 128) * 1024;
  static constexpr int NS = RING_BYTES / TILE_BYTES;       // 2 to 4 stages
  static constexpr int INSTR = TILE_BYTES / 1024;          // 1 KB DMA instructions per tile
  static constexpr int PER_WAVE = INSTR / WAVES;
  static_assert(NS >= 2, "ring depth");
};

template <int NB, bool GATHER>
__device__ __forceinline__ void pipe_issue_tile(const AttnArgs& a, const SlotMap<GATHER>& sm,
                                                int tile_start, int t_end, uint32_t slot_lds,
                                                int wave, int lane) {
  using C = PipeCfg<NB, GATHER>;
  const unsigned char* kg = reinterpret_cast<const unsigned char*>(a.k);
  const unsigned char* vg = reinterpret_cast<const unsigned char*>(a.v);
  // All source addresses first: a gathered row comes from LDS, and each DMA
  // statement is a compiler memory barrier, so resolving rows between them
  // would cost one LDS round trip per instruction.
  const unsigned char* src[C::PER_WAVE];
#pragma unroll
  for (int jj = 0; jj < C::PER_WAVE; ++jj) {
    const int j = wave + C::WAVES * jj;          // DMA instruction index within the tile
    const int p = j >> 4, kind = (j >> 3) & 1, grp = j & 7;
    const int key = 4 * grp + (lane >> 4);       // key row inside the 32-key sub-tile
    int slot = tile_start + 32 * p + key;
    slot = slot < t_end ? slot : t_end - 1;      // past the end: any valid row (masked later)
    const uint32_t chunk = (uint32_t)(lane & 15) ^ swz((uint32_t)key);
    src[jj] = (kind ? vg : kg) + (size_t)sm.rowof(slot) * 256 + chunk * 16;
  }
#pragma unroll
  for (int jj = 0; jj < C::PER_WAVE; ++jj) {
    const int j = wave + C::WAVES * jj;
    const int p = j >> 4, kind = (j >> 3) & 1, grp = j & 7;
    dma16(src[jj], slot_lds + (uint32_t)((2 * p + kind) * C::SUB_BYTES + grp * 1024));
  }
}

// Epilogue of the pipelined kernel: wave (nb, p) holds rows nb*16.. of
// sub-tile phase p.  Phases are merged in LDS in a fixed order.
template <int NB>
__device__ __forceinline__ void pipe_finish(const AttnArgs& a, float* smem, int wave, int lane,
                                            bool active, int nb, int p, int u, int s, int b,
                                            int g, int nq, int S_unit, size_t pidx, float m_run,
                                            float l_run, float l_rnd, f32x4_t (&acc)[8]) {
  constexpr int D = 128, RP = NB * 16, DP = D + 4;
  constexpr int KP = PipeCfg<NB>::KP;
  constexpr int PARK = (KP > 1) ? KP - 1 : 1;
  const int R = a.R;
  if (a.SP != a.S) {
    // Few splits (a short list): every wave writes its own partial, split
    // s * KP + p, and the merge kernel combines them; no LDS merge and no
    // barrier here.  The wave's running maximum is the partial's reference.
    const float lt = sum_across_rows(l_run), rt = sum_across_rows(l_rnd);
    const int r16 = lane & 15, q4 = lane >> 4;
    const int n = nb * 16 + r16;
    if (active && n < R) {
      const size_t sp = (size_t)u * a.SP + (size_t)s * KP + p;
      float* pa = a.part_acc + sp * R * D + (size_t)n * D;
#pragma unroll
      for (int db = 0; db < 8; ++db)
        __builtin_nontemporal_store(acc[db], reinterpret_cast<f32x4_t*>(pa + db * 16 + 4 * q4));
      if (q4 == 0) {
        float* pm = a.part_ml + sp * 3 * R;
        pm[n] = m_run;
        pm[R + n] = lt;
        pm[2 * R + n] = rt;
      }
    }
    return;
  }
  float* macc = smem;                 // [PARK][RP][DP] parked accumulators of phases 1..KP-1
  float* mm = macc + PARK * RP * DP;  // [KP][RP]
  float* ml = mm + KP * RP;
  float* mr = ml + KP * RP;
  float* mrow = mr + KP * RP;         // [3][RP]
  const int r16 = lane & 15, q4 = lane >> 4;
  const float lt = sum_across_rows(l_run), rt = sum_across_rows(l_rnd);
  __syncthreads();                    // the ring is free from here on
  if (active && q4 == 0) {
    mm[p * RP + nb * 16 + r16] = m_run;
    ml[p * RP + nb * 16 + r16] = lt;
    mr[p * RP + nb * 16 + r16] = rt;
  }
  __syncthreads();
  if (threadIdx.x < RP) {
    const int r = threadIdx.x;
    float M = -INFINITY;
    for (int k = 0; k < KP; ++k) M = fmaxf(M, mm[k * RP + r]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float Ls = 0.f, Lr = 0.f;
    for (int k = 0; k < KP; ++k) {
      const float f = exp2f(mm[k * RP + r] - Mu);
      Ls += ml[k * RP + r] * f;
      Lr += mr[k * RP + r] * f;
    }
    mrow[r] = M;
    mrow[RP + r] = Ls;
    mrow[2 * RP + r] = Lr;
  }
  __syncthreads();
  float f = 0.f;
  if (active) {
    const float M = mrow[nb * 16 + r16];
    f = exp2f(m_run - ((M == -INFINITY) ? 0.f : M));
  }
  // Phases p >= 1 park their rescaled accumulators in LDS; phase 0 adds them
  // in phase order and writes straight from registers: lane (r16, q4) of
  // block db holds 4 consecutive d of row nb*16 + r16, one 16-byte store.
  const int n = nb * 16 + r16;
  if (active && p > 0) {
#pragma unroll
    for (int db = 0; db < 8; ++db)
      *reinterpret_cast<f32x4_t*>(macc + ((p - 1) * RP + n) * DP + db * 16 + 4 * q4) = acc[db] * f;
  }
  __syncthreads();
  if (active && p == 0 && n < R) {
    f32x4_t o[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      o[db] = acc[db] * f;
#pragma unroll
      for (int k = 1; k < KP; ++k)
        o[db] += *reinterpret_cast<const f32x4_t*>(macc + ((k - 1) * RP + n) * DP + db * 16 + 4 * q4);
    }
    if (S_unit == 1) {
      const int i = n / a.G, hh = n - i * a.G;
      const float Ls = mrow[RP + n], Lr = mrow[2 * RP + n];
      const bool live = (i < nq) && (Ls > 0.f);
      const size_t ob = (((size_t)b * a.n_max + i) * a.Hq + g * a.G + hh) * D;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        f32x4_t v = o[db];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = live ? v[e] / Lr : 0.f;
        const size_t oi = ob + db * 16 + 4 * q4;
        if (a.out_bf16) {
          const uint32_t lo = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
          const uint32_t hi = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + oi) = make_uint2(lo, hi);
        } else {
          *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(a.out) + oi) = v;
        }
      }
      if (a.lse && q4 == 0)
        a.lse[((size_t)b * a.n_max + i) * a.Hq + g * a.G + hh] =
            live ? (mrow[n] + log2f(Ls)) * 0.69314718055994531f : -INFINITY;
    } else {
      // Partials are read once, by the merge launch: non-temporal stores
      // (the ragged paged text-anchored call 18.1 -> 17.1 us; no change at
      // C2).  The HSR split-K partials measured slower that way (31 -> 34 us).
      float* pa = a.part_acc + pidx * R * D + (size_t)n * D;
#pragma unroll
      for (int db = 0; db < 8; ++db)
        __builtin_nontemporal_store(o[db], reinterpret_cast<f32x4_t*>(pa + db * 16 + 4 * q4));
    }
  }
  if (S_unit > 1) {
    float* pm = a.part_ml + pidx * 3 * R;
    for (int r = threadIdx.x; r < R; r += blockDim.x) {
      pm[r] = mrow[r];
      pm[R + r] = mrow[RP + r];
      pm[2 * R + r] = mrow[2 * RP + r];
    }
  }
}

// DMA of the unit's NB*16 query rows (256 bytes each, row-major) to LDS at
// q_lds: 1 KB instructions of 4 rows, spread over the waves.  Rows past the
// block (n >= n_max*G) fetch row 0 instead; every row that is not a live
// query is masked when read.
template <int NB>
__device__ __forceinline__ void pipe_issue_q(const AttnArgs& a, int b, int g, uint32_t q_lds,
                                             int wave, int lane) {
  using C = PipeCfg<NB>;
  for (int j = wave; j < NB * 4; j += C::WAVES) {
    int n = 4 * j + (lane >> 4);
    if (n >= a.R) n = 0;
    const int qi = n / a.G, hh = n - qi * a.G;
    const unsigned char* src = reinterpret_cast<const unsigned char*>(a.q) +
                               ((((size_t)b * a.n_max + qi) * a.Hq + g * a.G + hh) * 128) * 2 +
                               16 * (lane & 15);
    dma16(src, q_lds + (uint32_t)(j * 1024));
  }
}

template <int NB, bool GATHER>
__global__ __launch_bounds__(PipeCfg<NB>::WAVES * 64, 1) void attn_bf16_pipe_kernel(AttnArgs a) {
  using C = PipeCfg<NB, GATHER>;
  constexpr int D = 128;
  __shared__ __align__(16) unsigned char ring[C::RING_BYTES];
  // slot tables of gathered splits (a dense split has no LDS beside the ring)
  int* s_pos = nullptr;
  uint32_t* s_row = nullptr;
  int* s_bmax = nullptr;
  if constexpr (GATHER) {
    __shared__ int g_pos[kMaxChunk];
    __shared__ uint32_t g_row[kMaxChunk];
    __shared__ int g_bmax[kMaxChunk / 32];
    s_pos = g_pos;
    s_row = g_row;
    s_bmax = g_bmax;
  }
  static_assert(((C::KP > 1) ? C::KP - 1 : 1) * (NB * 16) * (D + 4) * 4 + 7 * C::KP * NB * 16 * 4 <=
                    C::RING_BYTES,
                "epilogue fits the ring");

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, q4 = lane >> 4;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  int u, s, b, g, chunk, S_unit;
  size_t pidx;
  if (a.dyn) {
    // the split comes from the device lengths; a workgroup past the last
    // split has nothing to do (it has touched neither LDS nor the ring)
    const DynSplit d = dyn_split(a, blockIdx.x, false);
    if (!d.valid) return;
    b = d.b;
    g = d.g;
    s = d.s;
    chunk = d.ch;
    S_unit = d.S;
    pidx = (size_t)d.w;
  } else {
    u = wg / a.S;
    s = wg - u * a.S;
    b = u / a.Hkv;
    g = u - b * a.Hkv;
    chunk = a.chunk;
    S_unit = a.S;
    pidx = (size_t)u * a.S + s;
  }
  u = b * a.Hkv + g;
  lds_u8_t* const ring_l = (lds_u8_t*)ring;        // the ring as an LDS-address-space pointer
  const uint32_t ring_lds = (uint32_t)(size_t)ring_l;
  constexpr uint32_t kQSlot = (uint32_t)((C::NS - 1) * C::TILE_BYTES);
  const int t_beg = s * chunk;
  SlotMap<GATHER> sm;
  sm.t_beg = t_beg;
  sm.base_row = ((uint32_t)b * (uint32_t)a.Hkv + (uint32_t)g) * (uint32_t)a.max_len;
  sm.pos = s_pos;
  sm.row = s_row;
  sm.set_pages(a, g);
  // The lengths are requested first (scalar loads, not queued behind the
  // DMA requests below); their values are waited for only where used.
  const int pre = GATHER ? prefetch_slot(a, b, g, t_beg) : 0;
  const int L = ld_uniform(a.kv_len, b);
  const int nq = a.q_len ? ld_uniform(a.q_len, b) : a.n_max;
  // Dense splits of the capacity plan: the first tile and the query block go
  // out before the sequence length is known, so their round trips overlap
  // the length's.  Their slots are clamped to the split's end as planned
  // over the cache capacity, so every row they name lies inside the cache.
  // Rows past the sequence's end may hold anything (a masked key still adds
  // 0 * V), so when the sequence ends inside that tile it is requested again
  // below.  (A balanced split already knows its lengths.)  One early tile
  // rather than NS - 1: the smaller first burst lands sooner, and a split
  // past a short sequence's end wastes half as much (measured 0.5-1 us per
  // call faster, on full and on short sequences).
  const bool spec = !GATHER && !a.dyn;
  const int spec_end = min(t_beg + chunk, a.max_len);
  const int spec_tiles = spec ? 1 : 0;               // a planned split starts below max_len
  if (spec) {
    pipe_issue_tile<NB, GATHER>(a, sm, t_beg, spec_end, ring_lds, wave, lane);
    pipe_issue_q<NB>(a, b, g, ring_lds + kQSlot, wave, lane);
  }
  const int T = GATHER ? unit_slots(a, b, g, L) : L;   // a dense split is mode 0
  const int t_end = min(T, t_beg + chunk);
  const int n_tiles = t_end > t_beg ? (t_end - t_beg + C::TILE_KEYS - 1) / C::TILE_KEYS : 0;
  if (GATHER) {
    stage_slots(a, b, g, L, t_beg, t_end, s_pos, s_row, s_bmax, pre);
    __syncthreads();
  }

  // this wave's rows and sub-tile phase
  const int nb = wave % C::SLOTS;
  const int p = wave / C::SLOTS;
  const bool active = nb < NB;
  const int n = nb * 16 + r16;
  const bool valid = active && n < nq * a.G;
  const int qi = n / a.G;
  const int rowP = valid ? L - nq + qi : 0x7fffffff;
  // Gathered and balanced splits resolve their slots first (plain loads the
  // compiler waits for), then send the query block ahead of the first tiles.
  if (!spec) pipe_issue_q<NB>(a, b, g, ring_lds + kQSlot, wave, lane);
  bf16x8_t qop[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qop[ks] = as_bf16x8(u32x4_t{0, 0, 0, 0});

  if (spec && n_tiles > 0 &&
      t_end < min(t_beg + min(spec_tiles, n_tiles) * C::TILE_KEYS, spec_end)) {
    // an early tile that is read named rows past the sequence: every wave's
    // requests land before any wave re-requests those slots (early tiles
    // past n_tiles are never read, and the loop's waits cover them)
    wait_dma_barrier<0>();
    for (int j = 0; j < spec_tiles && j < n_tiles; ++j)
      pipe_issue_tile<NB, GATHER>(a, sm, t_beg + j * C::TILE_KEYS, t_end,
                                  ring_lds + (uint32_t)(j * C::TILE_BYTES), wave, lane);
  }
  for (int j = spec_tiles; j < C::NS - 1 && j < n_tiles; ++j)
    pipe_issue_tile<NB, GATHER>(a, sm, t_beg + j * C::TILE_KEYS, t_end,
                                ring_lds + (uint32_t)(j * C::TILE_BYTES), wave, lane);

  float m_run = -INFINITY, l_run = 0.f, l_rnd = 0.f;
  f32x4_t acc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) acc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int t = 0; t < n_tiles; ++t) {
    if (t == 0) {
      wait_tiles_barrier<C::PER_WAVE, C::NS - 2>(n_tiles - 1);
      // the query block landed with (before) tile 0; every wave copies its
      // rows out before tile NS-1 reuses the slot
      if (valid) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          qop[ks] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(
              ring + kQSlot + n * 256 + 16 * q4 + 64 * ks));
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (C::NS - 1 < n_tiles)
        pipe_issue_tile<NB, GATHER>(a, sm, t_beg + (C::NS - 1) * C::TILE_KEYS, t_end,
                                    ring_lds + (uint32_t)((C::NS - 1) * C::TILE_BYTES), wave,
                                    lane);
    } else {
      // Every wave is done with tile t-1, so its slot is refilled at once,
      // before tile t is waited for: NS-1 tiles stay in flight while this
      // tile is computed, whenever its data arrives.
      asm volatile("s_barrier" ::: "memory");
      if (t + C::NS - 1 < n_tiles)
        pipe_issue_tile<NB, GATHER>(a, sm, t_beg + (t + C::NS - 1) * C::TILE_KEYS, t_end,
                                    ring_lds +
                                        (uint32_t)(((t + C::NS - 1) % C::NS) * C::TILE_BYTES),
                                    wave, lane);
      wait_tiles_barrier<C::PER_WAVE, C::NS - 1>(n_tiles - 1 - t);
    }
    if (!active) continue;
    const uint32_t kofs = (uint32_t)((t % C::NS) * C::TILE_BYTES + (2 * p) * C::SUB_BYTES);
    const uint32_t vofs = kofs + C::SUB_BYTES;
    const int sub0 = t_beg + t * C::TILE_KEYS + 32 * p;

    // Every LDS read of the sub-tile is requested at once, so their latency
    // is paid once per tile: the K fragments, then the transposed V
    // fragments (they do not depend on the scores).  The V^T operand of lane
    // (i, q4) for output block db is V[keys 4q4.. and 16+4q4..][d = 16*db+i].
    u32x4_t kfr[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint32_t row = 16 * kb + r16;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint32_t chunk = (uint32_t)(4 * ks + q4) ^ swz(row);
        kfr[kb][ks] = *reinterpret_cast<const u32x4_t*>(ring + kofs + row * 256 + chunk * 16);
      }
    }
    short4_t vlo[8], vhi[8];
    {
      const int sl = lane & 15;
      const uint32_t r0 = (uint32_t)(4 * q4 + (sl >> 2)), r1 = r0 + 16;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const uint32_t chunk = (uint32_t)(2 * db + ((sl & 3) >> 1));
        const uint32_t o0 = vofs + r0 * 256 + ((chunk ^ swz(r0)) * 16) + 8 * (sl & 1);
        const uint32_t o1 = vofs + r1 * 256 + ((chunk ^ swz(r1)) * 16) + 8 * (sl & 1);
        vlo[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(ring_l + o0));
        vhi[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(ring_l + o1));
      }
    }
    // S^T = K Q^T for keys 16*kb + m of the sub-tile (unscaled scores)
    f32x4_t sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x4_t c4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kfr[kb][ks]), qop[ks], c4, 0, 0, 0);
      sc[kb] = c4;
    }
    // causal / list / tail mask; a dense tile that lies entirely before the
    // first query row's position and before the split end needs none
    // (no short circuit: a guarded LDS read becomes a branch with its own wait)
    const int smax = GATHER ? ((sm.shift >= 0) ? sub0 + 31
                                               : s_bmax[min((sub0 - t_beg) >> 5, kMaxChunk / 32 - 1)])
                            : sub0 + 31;
    const bool full = (sub0 + 32 <= t_end) & (smax <= L - nq);
    if (!full) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int slot = sub0 + 16 * kb + 4 * q4 + i;
          // no short circuit: a guarded LDS read becomes a branch with its own wait
          const int pos = sm.position(min(slot, t_end - 1));
          const bool vis = (slot < t_end) & (pos <= rowP);
          sc[kb][i] = vis ? sc[kb][i] : -INFINITY;
        }
    }
    // Online softmax with a lazily moved reference max: the reference m_run
    // (log2 units) is only raised when some score exceeds it by more than
    // 2^8, so probabilities stay <= 256 and, in most tiles, no cross-lane
    // reduction and no rescale of acc are needed.  Exact: every term uses the
    // same reference as the running sums it joins.
    float lmax = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                       fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    lmax *= a.scale_log2;
    if (__builtin_amdgcn_ballot_w64(lmax > m_run + 8.0f)) {
      const float m_new = fmaxf(m_run, max_across_rows(lmax));
      const float alpha = exp2f(m_run - ((m_new == -INFINITY) ? 0.f : m_new));
      m_run = m_new;
      l_run *= alpha;
      l_rnd *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) acc[db] *= alpha;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float pr[8];
    float ls = 0.f, lr = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][i], a.scale_log2, -m_use));
        ls += e;
        pr[kb * 4 + i] = e;
      }
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    u32x4_t pk;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x2_t h2 = {(__bf16)pr[2 * j], (__bf16)pr[2 * j + 1]};
      const uint32_t w = __builtin_bit_cast(uint32_t, h2);
      pk[j] = w;
      lr += __uint_as_float(w << 16) + __uint_as_float(w & 0xFFFF0000u);
    }
    l_run += ls;
    l_rnd += lr;
    const bf16x8_t pop = as_bf16x8(pk);

    // O^T += V^T P^T with the V^T fragments requested above
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const short4_t lo = vlo[db], hi = vhi[db];
      u32x4_t va;
      va[0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
      va[1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
      va[2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
      va[3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), pop, acc[db], 0, 0, 0);
    }
  }
  if (n_tiles == 0) wait_dma_barrier<0>();   // the query DMA still targets the ring
  pipe_finish<NB>(a, reinterpret_cast<float*>(ring), wave, lane, active, nb, p, u, s, b, g, nq,
                  S_unit, pidx, m_run, l_run, l_rnd, acc);
}

// ---------------------------------------------------------------- fp32 ----
// v_mfma_f32_16x16x4_f32: A 16x4, B 4x16, lane l holds A[l%16][l/16] and
// B[l/16][l%16]; C as for the bf16 shape.  Keys in a tile are natural
// (key = 16*kb + m).  For S^T = K Q^T the contraction index d of k-step ks in
// lane row q4 is q4*(D/4) + ks, so each lane reads a contiguous quarter of a
// K row and of a Q row.  For O^T = V^T P^T, k-step s (0..7) takes key
// 16*(s/4) + 4*q4 + s%4 in lane row q4: exactly the probability that lane
// already holds, and V rows read straight from global memory.

template <int D, int NB, bool GATHER>
__global__ __launch_bounds__(256, 1) void attn_f32_kernel(AttnArgs a) {
  constexpr int DB = D / 16, Q4 = D / 4, RP = NB * 16;
  constexpr int M_DW = RP * (D + 4) + 3 * kNW * RP + 3 * RP;
  __shared__ float smem[M_DW];
  __shared__ int s_pos[GATHER ? kMaxChunk : 1];
  __shared__ uint32_t s_row[GATHER ? kMaxChunk : 1];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, q4 = lane >> 4;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int u = wg / a.S, s = wg - u * a.S;
  const int b = u / a.Hkv, g = u - b * a.Hkv;
  const int pre = GATHER ? prefetch_slot(a, b, g, s * a.chunk) : 0;
  const int L = ld_uniform(a.kv_len, b);
  const int nq = a.q_len ? ld_uniform(a.q_len, b) : a.n_max;
  const int T = unit_slots(a, b, g, L);
  const int t_beg = s * a.chunk;
  const int t_end = min(T, t_beg + a.chunk);
  const float* qf = reinterpret_cast<const float*>(a.q);
  const float* kf = reinterpret_cast<const float*>(a.k);
  const float* vf = reinterpret_cast<const float*>(a.v);
  SlotMap<GATHER> sm;
  sm.t_beg = t_beg;
  sm.base_row = ((uint32_t)b * (uint32_t)a.Hkv + (uint32_t)g) * (uint32_t)a.max_len;
  sm.pos = s_pos;
  sm.row = s_row;
  sm.set_pages(a, g);
  if (GATHER) {
    stage_slots(a, b, g, L, t_beg, t_end, s_pos, s_row, nullptr, pre);
    __syncthreads();
  }

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
        const float* p = kf + (size_t)sm.rowof(slot) * D + q4 * Q4;
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
        const float* p = vf + (size_t)sm.rowof(slot) * D + r16;
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
        const int pos = sm.position(min(slot, t_end - 1));   // unconditional read, no branch
        kpos[kb][i] = (slot < t_end) ? pos : 0x7fffffff;
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
// One workgroup per (unit, row, slice of 64 * CPT output columns): combine
// the S partials with the log-sum-exp rule.  Threads form kMergeThreads / 64
// groups over the splits (group k takes splits k, k + NG, ...), and each
// thread of a group takes CPT adjacent columns.  Each thread requests its
// partials and their splits' (m, l, l_rnd) in one round of loads, merges
// them against its group's own running maximum, and the groups are then
// combined in a fixed order against the overall maximum.  One load round
// trip and one barrier on the critical path; no thread waits for another's
// weights.  Two columns per thread (one workgroup per row at d = 128) when
// the rows are many: half the workgroups and 8-byte loads (C2's
// verification, 168 rows: 20.0 -> 19.7 us); one column per thread when they
// are few, so that more workgroups share the load round trip (7 rows: 9.8
// against 10.2 us for the text-anchored call).
constexpr int kMaxSplits = 4096;
// Up to this many partials per unit, the pipelined kernel's waves write one
// each (no LDS merge at the end of a split).
constexpr int kWavePartials = 64;
constexpr int kMergeThreads = 512;   // 8 groups of 64 threads over the splits
constexpr int kMergeWideRows = 128;   // rows (units x R) from which a thread takes two columns
constexpr int kMergeVecStats = 32;    // partials per unit from which statistics are vector loads
constexpr int kMergeLoads = 4096;     // partial values one workgroup requests per round

template <int D, int CPT, bool VSTAT>
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(AttnArgs a) {
  constexpr int DS = 64 * CPT;                      // output columns per workgroup
  constexpr int NG = kMergeThreads / 64;            // groups of 64 threads over the splits
  constexpr int PB = kMergeLoads / kMergeThreads;   // splits per thread per load round
  static_assert(D % DS == 0 && PB >= 1, "merge shape");
  typedef float vec_t __attribute__((ext_vector_type(CPT)));
  __shared__ vec_t part[NG][64];
  __shared__ float gstat[3][NG];
  const int R = a.R;
  const int row = blockIdx.x / (D / DS), slice = blockIdx.x - row * (D / DS);
  const int u = row / R, r = row - u * R;
  const int b = u / a.Hkv, g = u - b * a.Hkv;
  const int i = r / a.G, hh = r - i * a.G;
  const int tid = threadIdx.x, dl = tid % 64, d = slice * DS + CPT * dl;
  // requested first: only the epilogue needs it, and a load there would add
  // a round trip after the merge
  const int nq = a.q_len ? ld_uniform(a.q_len, b) : a.n_max;
  // the unit's partials: S per unit in the capacity plan, or the balanced
  // plan's (a unit with one split wrote its output itself)
  int S = a.SP;
  size_t first = (size_t)u * a.SP;
  if (a.dyn) {
    const DynSplit ds = dyn_split(a, u, true);
    if (ds.S == 1) return;
    S = ds.S;
    first = (size_t)ds.first;
  }
  // the group index is uniform over a wave, so the per-split statistics
  // below can be scalar loads (see VSTAT)
  const int grp = __builtin_amdgcn_readfirstlane(tid / 64);
  const float* pm = a.part_ml + first * 3 * R + r;
  const float* pa = a.part_acc + first * R * D + (size_t)r * D + d;

  float M = -INFINITY, ls = 0.f, lr = 0.f;
  vec_t o = {};
  for (int base = grp; base < S; base += NG * PB) {
    // clamped indices, loaded unconditionally and masked afterwards: a guarded
    // load would wait for itself before the next one is issued
    vec_t v[PB];
    float mv[PB], lv[PB], rv[PB];
#pragma unroll
    for (int j = 0; j < PB; ++j) {
      const int sp = min(base + NG * j, S - 1);
      v[j] = *reinterpret_cast<const vec_t*>(pa + (size_t)sp * R * D);
    }
    // VSTAT: the statistics are requested after the partials, and as vector
    // loads (the compiler otherwise issues them first, as scalar loads, with
    // waits at the scalar unit's limit of outstanding loads before any
    // partial is requested): one round trip for all, faster when most of
    // the PB splits per thread are real (C2 verification 19.7 -> 19.5 us,
    // top-K 32.1 -> 31.7), slower when most are clamped repeats (the 7-row
    // text-anchored call, 16 partials: 9.8 -> 10.0)
    if constexpr (VSTAT) asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < PB; ++j) {
      const int sp = min(base + NG * j, S - 1);
      mv[j] = pm[(size_t)sp * 3 * R];
      lv[j] = pm[(size_t)sp * 3 * R + R];
      rv[j] = pm[(size_t)sp * 3 * R + 2 * R];
    }
    float mr = M;
#pragma unroll
    for (int j = 0; j < PB; ++j) {
      if (base + NG * j >= S) mv[j] = -INFINITY;   // contributes a zero weight
      mr = fmaxf(mr, mv[j]);
    }
    const float Mu = (mr == -INFINITY) ? 0.f : mr;
    const float sc = __builtin_amdgcn_exp2f(M - Mu);   // M = -inf: nothing merged yet -> 0
#pragma unroll
    for (int c = 0; c < CPT; ++c) o[c] *= sc;
    ls *= sc;
    lr *= sc;
#pragma unroll
    for (int j = 0; j < PB; ++j) {
      const float w = __builtin_amdgcn_exp2f(mv[j] - Mu);
#pragma unroll
      for (int c = 0; c < CPT; ++c) o[c] = __builtin_fmaf(v[j][c], w, o[c]);
      ls = __builtin_fmaf(lv[j], w, ls);
      lr = __builtin_fmaf(rv[j], w, lr);
    }
    M = mr;
  }
  part[grp][dl] = o;
  if (dl == 0) {
    gstat[0][grp] = M;
    gstat[1][grp] = ls;
    gstat[2][grp] = lr;
  }
  __syncthreads();
  if (grp != 0) return;
  float Mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < NG; ++k) Mx = fmaxf(Mx, gstat[0][k]);
  const float Mu = (Mx == -INFINITY) ? 0.f : Mx;
  float Ls = 0.f, Lr = 0.f;
  o = vec_t{};
#pragma unroll
  for (int k = 0; k < NG; ++k) {
    const float f = __builtin_amdgcn_exp2f(gstat[0][k] - Mu);
    const vec_t pk = part[k][dl];
#pragma unroll
    for (int c = 0; c < CPT; ++c) o[c] = __builtin_fmaf(pk[c], f, o[c]);
    Ls = __builtin_fmaf(gstat[1][k], f, Ls);
    Lr = __builtin_fmaf(gstat[2][k], f, Lr);
  }
  const bool live = (i < nq) && (Ls > 0.f);
#pragma unroll
  for (int c = 0; c < CPT; ++c) o[c] = live ? o[c] / Lr : 0.f;
  const size_t oi = (((size_t)b * a.n_max + i) * a.Hq + g * a.G + hh) * D + d;
  if constexpr (CPT == 2) {                      // one 4- or 8-byte store
    if (a.out_bf16)
      reinterpret_cast<uint32_t*>(a.out)[oi / 2] = pack_bf16x2(o[0], o[1]);
    else
      *reinterpret_cast<vec_t*>(reinterpret_cast<float*>(a.out) + oi) = o;
  } else {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      if (a.out_bf16)
        reinterpret_cast<uint16_t*>(a.out)[oi + c] = (uint16_t)f32_to_bf16_bits(o[c]);
      else
        reinterpret_cast<float*>(a.out)[oi + c] = o[c];
    }
  }
  if (a.lse && d == 0)
    a.lse[((size_t)b * a.n_max + i) * a.Hq + g * a.G + hh] =
        live ? (Mx + log2f(Ls)) * 0.69314718055994531f : -INFINITY;
}

// Few partials per unit (a batch of short or ragged units): one wave per
// row, each thread D / 64 adjacent columns (one 8-byte load per partial at
// D = 128, against two 4-byte loads with one column per thread: the ragged
// paged batch's verification 118.3 -> 115.9 us, its text-anchored call
// 19.7 -> 18.0 us), 4 rows per workgroup.  The row's partials are requested
// kMergeSmall at a time (one round for the capacity plan's few partials; the
// balanced plan's units may have more, merged round by round against a
// running maximum).  The grouped kernel above would spend a 512-thread
// workgroup on each (row, 64 columns) with most groups idle.
constexpr int kMergeSmall = 8;
constexpr int kMergeSmallRows = 4;     // rows (waves) per workgroup

template <int D, bool VSTAT>
__global__ __launch_bounds__(64 * kMergeSmallRows) void attn_merge_small_kernel(AttnArgs a) {
  constexpr int CPT = D / 64;          // columns per thread
  typedef float vec_t __attribute__((ext_vector_type(CPT)));
  const int R = a.R;
  const int blocks_per_unit = (R + kMergeSmallRows - 1) / kMergeSmallRows;
  const int u = blockIdx.x / blocks_per_unit, rb = blockIdx.x - u * blocks_per_unit;
  int S = a.SP;
  size_t first = (size_t)u * a.SP;
  if (a.dyn) {
    const DynSplit ds = dyn_split(a, u, true);
    if (ds.S == 1) return;                 // the split wrote the output itself
    S = ds.S;
    first = (size_t)ds.first;
  }
  // the row is the wave's: scalar statistics
  const int r = __builtin_amdgcn_readfirstlane(rb * kMergeSmallRows + (int)threadIdx.x / 64);
  if (r >= R) return;
  const int d = CPT * ((int)threadIdx.x % 64);
  const int b = u / a.Hkv, g = u - b * a.Hkv;
  const int i = r / a.G, hh = r - i * a.G;
  const int nq = a.q_len ? ld_uniform(a.q_len, b) : a.n_max;   // requested first
  const float* pm = a.part_ml + first * 3 * R + r;
  const float* pa = a.part_acc + first * R * D + (size_t)r * D + d;
  float M = -INFINITY, Ls = 0.f, Lr = 0.f;
  vec_t o = {};
  for (int base = 0; base < S; base += kMergeSmall) {
    vec_t v[kMergeSmall];
    float mv[kMergeSmall], lv[kMergeSmall], rv[kMergeSmall];
#pragma unroll
    for (int j = 0; j < kMergeSmall; ++j) {          // clamped, masked after
      const int sp = min(base + j, S - 1);
      v[j] = *reinterpret_cast<const vec_t*>(pa + (size_t)sp * R * D);
    }
    // VSTAT (balanced plans, whose rounds hold mostly real splits): the
    // statistics as vector loads after the partials, as in the grouped merge
    // (4 x 32,768 verification 59.1 -> 58.5 us); with the capacity plan's
    // few partials per unit the scalar order stays faster
    if constexpr (VSTAT) asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < kMergeSmall; ++j) {
      const int sp = min(base + j, S - 1);
      mv[j] = pm[(size_t)sp * 3 * R];
      lv[j] = pm[(size_t)sp * 3 * R + R];
      rv[j] = pm[(size_t)sp * 3 * R + 2 * R];
    }
    float mr = M;
#pragma unroll
    for (int j = 0; j < kMergeSmall; ++j) {
      if (base + j >= S) mv[j] = -INFINITY;
      mr = fmaxf(mr, mv[j]);
    }
    const float Mu = (mr == -INFINITY) ? 0.f : mr;
    const float sc = __builtin_amdgcn_exp2f(M - Mu);   // M = -inf: nothing merged yet -> 0
#pragma unroll
    for (int c = 0; c < CPT; ++c) o[c] *= sc;
    Ls *= sc;
    Lr *= sc;
#pragma unroll
    for (int j = 0; j < kMergeSmall; ++j) {
      const float w = __builtin_amdgcn_exp2f(mv[j] - Mu);
#pragma unroll
      for (int c = 0; c < CPT; ++c) o[c] = __builtin_fmaf(v[j][c], w, o[c]);
      Ls = __builtin_fmaf(lv[j], w, Ls);
      Lr = __builtin_fmaf(rv[j], w, Lr);
    }
    M = mr;
  }
  const bool live = (i < nq) && (Ls > 0.f);
#pragma unroll
  for (int c = 0; c < CPT; ++c) o[c] = live ? o[c] / Lr : 0.f;
  const size_t oi = (((size_t)b * a.n_max + i) * a.Hq + g * a.G + hh) * D + d;
  if constexpr (CPT == 2) {                      // one 4- or 8-byte store
    if (a.out_bf16)
      reinterpret_cast<uint32_t*>(a.out)[oi / 2] = pack_bf16x2(o[0], o[1]);
    else
      *reinterpret_cast<vec_t*>(reinterpret_cast<float*>(a.out) + oi) = o;
  } else {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      if (a.out_bf16)
        reinterpret_cast<uint16_t*>(a.out)[oi + c] = (uint16_t)f32_to_bf16_bits(o[c]);
      else
        reinterpret_cast<float*>(a.out)[oi + c] = o[c];
    }
  }
  if (a.lse && d == 0)
    a.lse[((size_t)b * a.n_max + i) * a.Hq + g * a.G + hh] =
        live ? (M + log2f(Ls)) * 0.69314718055994531f : -INFINITY;
}

template <int D, int NB, bool GATHER>
hipError_t launch_d_nb(const AttnArgs& a, int dtype, int grid, hipStream_t st) {
  if (dtype == SPEC_BF16 && D == 128)
    hipLaunchKernelGGL((attn_bf16_pipe_kernel<NB, GATHER>), dim3(grid),
                       dim3(PipeCfg<NB>::WAVES * 64), 0, st, a);
  else if (dtype == SPEC_BF16)
    hipLaunchKernelGGL((attn_bf16_kernel<D, NB, GATHER>), dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((attn_f32_kernel<D, NB, GATHER>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D, bool GATHER>
hipError_t launch_d(const AttnArgs& a, int dtype, int grid, hipStream_t st) {
  const int nb = (a.R + 15) / 16;
  switch (nb) {
    case 1: return launch_d_nb<D, 1, GATHER>(a, dtype, grid, st);
    case 2: return launch_d_nb<D, 2, GATHER>(a, dtype, grid, st);
    case 3: return launch_d_nb<D, 3, GATHER>(a, dtype, grid, st);
    default: return launch_d_nb<D, 4, GATHER>(a, dtype, grid, st);
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

// Per-device CU count, queried once per device; calls from several host
// threads may race to fill an entry, with the same value.
int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

AttnPlan plan_attention(int units, int t_max, int rows, int d, bool gather, size_t scratch_off,
                        int dense_page_shift) {
  AttnPlan p;
  const int target = device_cu_count();            // about one workgroup per CU
  const long T = t_max > 0 ? t_max : 1;
  const long total = (long)units * T;
  long chunk = (total + target - 1) / target;
  if (chunk < (T + kMaxSplits - 1) / kMaxSplits) chunk = (T + kMaxSplits - 1) / kMaxSplits;
  chunk = ((chunk + kTK - 1) / kTK) * kTK;
  // Dense splits of whole tiles of the pipelined kernel (128 keys up to 16
  // rows, else 64): a split that ends inside a tile still spends a whole
  // tile's requests and compute on it, and fewer, fuller splits leave fewer
  // partials.  At 25,512 keys: 6 rows 19.1 -> 18.9 us, 9 rows 20.6 -> 19.8,
  // 1 row 18.5 -> 18.1.
  if (!gather) {
    const long tile = rows <= 16 ? 128 : 64;
    chunk = ((chunk + tile - 1) / tile) * tile;
  }
  if (chunk < kTK * kNW) chunk = kTK * kNW;        // every wave gets a tile
  if (gather) {
    // LDS holds kMaxChunk staged entries: slots, or pages when the split
    // covers every position of a paged cache
    const long cap = dense_page_shift >= 0
                         ? (((long)(kMaxChunk - 1) << dense_page_shift) / kTK) * kTK
                         : kMaxChunk;
    if (chunk > cap) chunk = cap;
  }
  int S = (int)((T + chunk - 1) / chunk);
  if (S < 1) S = 1;
  p.S = S;
  // partials per unit: one per wave of every split when few, and room for
  // the balanced plan's (at most grid + units splits)
  p.sp_max = (S > 1 && S * 4 <= kWavePartials) ? S * 4 : S + 1;
  p.chunk = (int)chunk;
  p.grid = units * S;
  p.gather = gather;
  if (S > 1) {
    const size_t sp = (size_t)units * p.sp_max;
    p.off_acc = align_up(scratch_off, 256);
    p.off_ml = p.off_acc + align_up(sp * rows * d * sizeof(float), 256);
    p.ws_bytes = p.off_ml + align_up(sp * 3 * rows * sizeof(float), 256);
  }
  return p;
}

spec_status_t launch_attention(AttnArgs a, int d, int dtype, const AttnPlan& plan, void* ws,
                               hipStream_t stream) {
  a.S = plan.S;
  a.SP = plan.S;
  a.dyn = 0;
  a.dyn_groups = plan.grid;
  int grid = plan.grid;
  const int units = a.B * a.Hkv;
  if (plan.S > 1 && dtype == SPEC_BF16 && d == 128 && a.mode == 0 && a.B >= 2 && a.B <= 64) {
    // several sequences: split what the lengths hold rather than the
    // capacity, so short sequences leave no empty workgroups and every
    // split is about as long (the partials are numbered split by split).
    // Text and top-K lists are short: there the extra round trip for the
    // lengths before the list is read costs more than the balance saves.
    a.dyn = 1;
  } else if (plan.S > 1 && dtype == SPEC_BF16 && d == 128) {
    // the pipelined kernel's waves write their own partials when that keeps
    // the merge small (phases per split as in PipeCfg) and the rows are few.
    // With 33-64 rows, twice the partial bytes cost the merge more than the
    // phase merge in LDS costs the split (the ragged paged text-anchored
    // batch, 56 rows: 19.7 us with one partial per split, 21.1 with two).
    const int nb = min(4, (a.R + 15) / 16);
    const int kp = (nb >= 3) ? 2 : 4 / nb;
    if (nb <= 2 && plan.S * kp <= plan.sp_max) a.SP = plan.S * kp;
  }
  a.chunk = plan.chunk;
  if (plan.S > 1) {
    a.part_acc = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + plan.off_acc);
    a.part_ml = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + plan.off_ml);
  } else {
    a.part_acc = nullptr;
    a.part_ml = nullptr;
  }
  if (grid == 0) return SPEC_OK;
  hipError_t e;
  mark_before_main(stream);
  if (plan.gather)
    e = (d == 64) ? launch_d<64, true>(a, dtype, grid, stream)
                  : launch_d<128, true>(a, dtype, grid, stream);
  else
    e = (d == 64) ? launch_d<64, false>(a, dtype, grid, stream)
                  : launch_d<128, false>(a, dtype, grid, stream);
  mark_after_main(stream);
  if (e != hipSuccess) return SPEC_ERR_HIP;
  if (plan.S > 1) {
    // balanced plans merge few partials per unit when the capacity plan has
    // few splits (a unit's balanced split count is about its share of them)
    if (a.dyn ? plan.S <= 2 * kMergeSmall : a.SP <= kMergeSmall) {
      const int blocks = units * ((a.R + kMergeSmallRows - 1) / kMergeSmallRows);
      const dim3 block(64 * kMergeSmallRows);
      if (d == 64)
        hipLaunchKernelGGL((attn_merge_small_kernel<64, false>), dim3(blocks), block, 0, stream, a);
      else if (a.dyn)
        hipLaunchKernelGGL((attn_merge_small_kernel<128, true>), dim3(blocks), block, 0, stream, a);
      else
        hipLaunchKernelGGL((attn_merge_small_kernel<128, false>), dim3(blocks), block, 0, stream, a);
    } else {
      const dim3 block(kMergeThreads);
      const bool vstat = !a.dyn && a.SP >= kMergeVecStats;
      const bool wide = (long)units * a.R >= kMergeWideRows;
      if (d == 64)
        hipLaunchKernelGGL((attn_merge_kernel<64, 1, false>), dim3(units * a.R), block, 0, stream, a);
      else if (wide && vstat)
        hipLaunchKernelGGL((attn_merge_kernel<128, 2, true>), dim3(units * a.R), block, 0, stream, a);
      else if (wide)
        hipLaunchKernelGGL((attn_merge_kernel<128, 2, false>), dim3(units * a.R), block, 0, stream, a);
      else if (vstat)
        hipLaunchKernelGGL((attn_merge_kernel<128, 1, true>), dim3(units * a.R * 2), block, 0, stream,
                           a);
      else
        hipLaunchKernelGGL((attn_merge_kernel<128, 1, false>), dim3(units * a.R * 2), block, 0, stream,
                           a);
    }
    if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
  }
  return SPEC_OK;
}

}  // namespace spec

// Top-K key selection for sparse draft attention (gfx950).
//
// Score (per sequence b, KV head g, key j < kv_len[b]):
//   qbar[c]  = q[h0][c] + q[h0+1][c] + ...   (fp64, heads of the group in order)
//   score_j  = (((0 + qbar[0]*k_j[0]) + qbar[1]*k_j[1]) + ...)   (fp64, c in
//              order, each product and each sum rounded separately)
// The evaluation order is fixed so the result is reproducible bit for bit by
// any implementation.  Keys are ranked by (score desc, index asc).
//
// topk_score_ring_kernel (bf16 keys): one workgroup of 8 waves per range of
//   a unit's keys; every wave streams its own 64-key tiles through an LDS
//   slot by DMA and runs one key's fp64 chain per lane while the next tile
//   is in flight.  It writes the score and adds the key to a per-unit
//   4096-bin histogram of a coarse monotone key (the top 12 bits of the
//   order-preserving bit pattern of float(score): sign, exponent, 3 mantissa
//   bits).  topk_score_kernel does the same for fp32 keys, 256 keys per
//   workgroup staged with plain loads.
// topk_select_kernel: one 1024-thread workgroup per unit.  From the
//   histogram it finds the bin holding the K-th key.  One pass over the
//   16-bit float keys (also written by the score kernel) sets an LDS
//   selection bit for every key above that bin and gathers the bin's keys as
//   candidates, whose exact scores are then fetched.  A second 4096-bin histogram over
//   the next 12 bits of the float key narrows the candidates to one sub-bin,
//   whose few keys are ranked by counting; that fixes the exact threshold
//   (score*, index*).  The winners' bits are set and the selected indices are
//   written in ascending order from the bits with one block scan.  Fallbacks
//   keep every case exact: a bitonic sort of the candidates when one sub-bin
//   holds many equal float keys, an exact radix select over the 64-bit keys
//   when the bin holds more candidates than LDS, and compaction straight from
//   the scores when the cache is longer than the LDS bit mask.
#include <math.h>
#include <string.h>

#include <algorithm>

#include "common.h"
#include "internal.h"

namespace spec {

namespace {

constexpr int kHistBins = 4096;
constexpr int kScoreKeys = 256;   // keys per score workgroup
constexpr int kCandMax = 4096;    // candidates sortable in LDS
constexpr int kSelBatch = 16;     // scores in flight per thread in the selection passes
constexpr int kSelWords = 4;      // 16-byte words of 16-bit keys in flight per thread

struct TopkArgs {
  const void* q;
  const void* k;
  const int32_t* kv_len;
  const int32_t* page_table;
  int32_t max_pages, page_shift;
  int32_t B, Hq, Hkv, G, max_len, top_k;
  int32_t splits;       // key ranges per unit (streaming score pass)
  double* scores;       // [U, max_len]
  uint16_t* key16;      // [U, max_len] top 16 bits of the ordered float key
  uint32_t* hist;       // [U, kHistBins]
  int32_t* sel_idx;     // [U, top_k]
};

__device__ __forceinline__ size_t topk_row(const TopkArgs& a, int b, int g, int pos) {
  if (a.page_shift >= 0) {
    const int page = a.page_table[(size_t)b * a.max_pages + (pos >> a.page_shift)];
    const int slot = pos & ((1 << a.page_shift) - 1);
    return (((size_t)page * a.Hkv + g) << a.page_shift) + slot;
  }
  return ((size_t)b * a.Hkv + g) * (size_t)a.max_len + pos;
}

// Order-preserving 64-bit key of a double; -0 is folded onto +0.
__device__ __forceinline__ uint64_t order_key64(double x) {
  if (x == 0.0) x = 0.0;
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Order-preserving 32-bit key of float(score) (round to nearest: monotone
// non-decreasing in the score); -0 is folded onto +0.
__device__ __forceinline__ uint32_t fine_key32(double x) {
  float f = (float)x;
  if (f == 0.f) f = 0.f;
  const uint32_t u = __float_as_uint(f);
  return (u >> 31) ? ~u : (u | 0x80000000u);
}

// Coarse histogram bin: the top 12 bits of that key (sign, exponent, 3
// mantissa bits).
__device__ __forceinline__ uint32_t coarse_bin(double x) { return fine_key32(x) >> 20; }

template <int D, bool BF16>
__global__ __launch_bounds__(256) void topk_score_kernel(TopkArgs a) {
  constexpr int ROW_B = BF16 ? D * 2 : D * 4;       // bytes per key row
  constexpr int PITCH = ROW_B + 8;                  // padded LDS pitch
  __shared__ __align__(16) unsigned char krows[kScoreKeys * PITCH];
  __shared__ double qbar[D];
  // two 16-bit bin counters per word (a tile has at most 256 keys), so the
  // workgroup fits twice per CU's LDS
  __shared__ uint32_t hist[kHistBins / 2];
  __shared__ size_t rowidx[kScoreKeys];

  const int tiles = (a.max_len + kScoreKeys - 1) / kScoreKeys;
  const int u = blockIdx.x / tiles, tile = blockIdx.x - (blockIdx.x / tiles) * tiles;
  const int b = u / a.Hkv, g = u - b * a.Hkv;
  const int L = ld_uniform(a.kv_len, b);
  const int j0 = tile * kScoreKeys;
  // The group's query values are requested in batches of 8 heads (clamped,
  // unconditional loads: all in flight at once) before anything waits,
  // then summed in head order.
  constexpr int QB = 8;
  float qv[QB];
  const int c = min((int)threadIdx.x, D - 1);
#pragma unroll
  for (int k = 0; k < QB; ++k) {
    const size_t qi = ((size_t)b * a.Hq + g * a.G + min(k, a.G - 1)) * D + c;   // q: [B, 1, Hq, D]
    qv[k] = BF16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(a.q)[qi])
                 : reinterpret_cast<const float*>(a.q)[qi];
  }
  if (j0 >= L) return;
  const int nk = min(kScoreKeys, L - j0);

  for (int i = threadIdx.x; i < kHistBins / 2; i += blockDim.x) hist[i] = 0;
  if (threadIdx.x < D) {
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < QB; ++k)
      if (k < a.G) s = add_rn(s, (double)qv[k]);
    for (int h0 = QB; h0 < a.G; h0 += QB) {   // groups of more than 8 heads
      float qw[QB];
#pragma unroll
      for (int k = 0; k < QB; ++k) {
        const size_t qi = ((size_t)b * a.Hq + g * a.G + min(h0 + k, a.G - 1)) * D + c;
        qw[k] = BF16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(a.q)[qi])
                     : reinterpret_cast<const float*>(a.q)[qi];
      }
#pragma unroll
      for (int k = 0; k < QB; ++k)
        if (h0 + k < a.G) s = add_rn(s, (double)qw[k]);
    }
    qbar[threadIdx.x] = s;
  }
  // resolve the tile's rows once (page table lookups), then stage the K rows
  // (ROW_B/16 chunks of 16 bytes per key) with a batch of loads in flight
  if ((int)threadIdx.x < nk) rowidx[threadIdx.x] = topk_row(a, b, g, j0 + threadIdx.x);
  __syncthreads();
  constexpr int CH = ROW_B / 16;
  constexpr int PB = 16;                                   // loads in flight per thread
  const unsigned char* kb = reinterpret_cast<const unsigned char*>(a.k);
  for (int e0 = 0; e0 < nk * CH; e0 += PB * 256) {
    u32x4_t v[PB];
#pragma unroll
    for (int k = 0; k < PB; ++k) {
      const int e = e0 + k * 256 + threadIdx.x;
      const int key = e / CH, ch = e - (e / CH) * CH;
      v[k] = (e < nk * CH) ? ld16(kb + rowidx[key] * ROW_B + ch * 16) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int k = 0; k < PB; ++k) {
      const int e = e0 + k * 256 + threadIdx.x;
      const int key = e / CH, ch = e - (e / CH) * CH;
      if (e < nk * CH) {
        uint2* dst = reinterpret_cast<uint2*>(krows + key * PITCH + ch * 16);   // 8-byte aligned
        dst[0] = make_uint2(v[k][0], v[k][1]);
        dst[1] = make_uint2(v[k][2], v[k][3]);
      }
    }
  }
  __syncthreads();

  const int key = threadIdx.x;
  if (key < nk) {
    double acc = 0.0;
    const unsigned char* row = krows + key * PITCH;
    if (BF16) {
      for (int c = 0; c < D; c += 4) {
        const uint2 w = *reinterpret_cast<const uint2*>(row + c * 2);
        const double k0 = (double)__uint_as_float(w.x << 16);
        const double k1 = (double)__uint_as_float(w.x & 0xFFFF0000u);
        const double k2 = (double)__uint_as_float(w.y << 16);
        const double k3 = (double)__uint_as_float(w.y & 0xFFFF0000u);
        acc = add_rn(acc, mul_rn(qbar[c], k0));
        acc = add_rn(acc, mul_rn(qbar[c + 1], k1));
        acc = add_rn(acc, mul_rn(qbar[c + 2], k2));
        acc = add_rn(acc, mul_rn(qbar[c + 3], k3));
      }
    } else {
      for (int c = 0; c < D; c += 2) {
        const float2 w = *reinterpret_cast<const float2*>(row + c * 4);
        acc = add_rn(acc, mul_rn(qbar[c], (double)w.x));
        acc = add_rn(acc, mul_rn(qbar[c + 1], (double)w.y));
      }
    }
    a.scores[(size_t)u * a.max_len + j0 + key] = acc;
    const uint32_t k32 = fine_key32(acc);
    a.key16[(size_t)u * a.max_len + j0 + key] = (uint16_t)(k32 >> 16);
    const uint32_t bin = k32 >> 20;
    atomicAdd(&hist[bin >> 1], (bin & 1u) ? 0x10000u : 1u);
  }
  __syncthreads();
  uint32_t* gh = a.hist + (size_t)u * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x)
    if (const uint32_t c = (hist[i >> 1] >> (16 * (i & 1))) & 0xFFFFu) atomicAdd(&gh[i], c);
}

// Streaming score pass for bf16 keys.  The unit's length is cut on the
// device into at most a.splits ranges of whole rounds of 8 64-key tiles;
// range s is workgroup (u, s).  Wave w takes the range's tiles w, w + 8, ... through a private
// LDS slot.  The DMA stores chunk c of tile row r at chunk position
// c ^ (r % CH), so the lanes of a quarter-wave, each reading its own key's
// row, address distinct banks.  A lane copies its row to registers; the
// slot then takes the next tile's DMA, and the fp64 chain runs while that is
// in flight.  Only this wave reads and refills its slot, so its own waits
// order the two: no workgroup barrier inside the loop.
constexpr int kRingWaves = 8;
constexpr int kRingTile = 64;   // keys per wave tile (one per lane)

template <int D>
__global__ __launch_bounds__(kRingWaves * 64, 1) void topk_score_ring_kernel(TopkArgs a) {
  constexpr int ROW_B = D * 2;               // bytes per key row
  constexpr int CH = ROW_B / 16;             // 16-byte chunks per row
  constexpr int RPI = 64 / CH;               // rows per 1 KB DMA instruction
  constexpr int NI = kRingTile / RPI;        // DMA instructions per tile
  constexpr int SLOT = kRingTile * ROW_B;
  __shared__ __align__(16) unsigned char slots[kRingWaves * SLOT];
  __shared__ __align__(16) double qbar[D];
  __shared__ uint32_t hist[kHistBins];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int u = blockIdx.x / a.splits, s = blockIdx.x - (blockIdx.x / a.splits) * a.splits;
  const int b = u / a.Hkv, g = u - b * a.Hkv;
  const int L = ld_uniform(a.kv_len, b);
  // ranges of whole rounds of wave tiles (every wave the same number of
  // tiles): 512 keys at 25,512 keys x 4 units, not 448 with one wave idle
  // (top-K 31.7 -> 31.5 us; 4 x 32,768: 53.6 -> 53.3)
  constexpr int kRound = kRingTile * kRingWaves;
  const int per = ((L + a.splits - 1) / a.splits + kRound - 1) / kRound * kRound;
  const int t_beg = s * per, t_end = min(L, t_beg + per);
  const int n_tiles = t_end > t_beg ? (t_end - t_beg + kRingTile - 1) / kRingTile : 0;
  const int my_tiles = n_tiles > wave ? (n_tiles - wave + kRingWaves - 1) / kRingWaves : 0;
  lds_u8_t* const slot_l = (lds_u8_t*)(slots + wave * SLOT);
  const uint32_t slot_lds = (uint32_t)(size_t)slot_l;
  const unsigned char* kb = reinterpret_cast<const unsigned char*>(a.k);
  const int rr = lane / CH, cpos = lane % CH;   // DMA lane: row within the instruction, chunk slot

  // DMA of wave tile i: instruction j brings rows RPI*j .. RPI*j + RPI-1
  // (keys past the range repeat its last key; their scores are not kept).
  auto issue = [&](int i) {
    const int k0 = t_beg + (wave + i * kRingWaves) * kRingTile;
    const size_t mine = topk_row(a, b, g, min(k0 + lane, t_end - 1));
    const uint32_t lo = (uint32_t)mine, hi = (uint32_t)(mine >> 32);
    // Every row address first: each DMA statement is a compiler memory
    // barrier.  A contiguous cache's rows are arithmetic; a paged cache's
    // come from the lanes that looked them up, by shuffles.
    const unsigned char* src[NI];
    if (a.page_shift < 0) {
      const size_t base = ((size_t)b * a.Hkv + g) * (size_t)a.max_len;
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int r = RPI * j + rr;
        src[j] = kb + (base + (size_t)min(k0 + r, t_end - 1)) * ROW_B + 16 * (cpos ^ (r % CH));
      }
    } else {
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int r = RPI * j + rr;
        const size_t row = (size_t)__shfl(lo, r) | ((size_t)__shfl(hi, r) << 32);
        src[j] = kb + row * ROW_B + 16 * (cpos ^ (r % CH));
      }
    }
#pragma unroll
    for (int j = 0; j < NI; ++j) dma16(src[j], slot_lds + (uint32_t)(j * 1024));
  };
  if (my_tiles > 0) issue(0);

  // group query sum, fp64 in head order (the first tile is already in flight)
  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) hist[i] = 0;
  if (threadIdx.x < D) {   // heads requested 8 at a time (clamped), then added in order
    const uint16_t* qh = reinterpret_cast<const uint16_t*>(a.q) +
                         ((size_t)b * a.Hq + g * a.G) * D + threadIdx.x;
    double q = 0.0;
    for (int h0 = 0; h0 < a.G; h0 += 8) {
      float qv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) qv[k] = bf16_bits_to_f32(qh[(size_t)min(h0 + k, a.G - 1) * D]);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (h0 + k < a.G) q = add_rn(q, (double)qv[k]);
    }
    qbar[threadIdx.x] = q;
  }
  __syncthreads();

  double* const sc = a.scores + (size_t)u * a.max_len;
  uint16_t* const k16 = a.key16 + (size_t)u * a.max_len;
  for (int i = 0; i < my_tiles; ++i) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");      // this wave's tile i is in LDS
    u32x4_t kr[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c)
      kr[c] = *reinterpret_cast<const u32x4_t*>(slots + wave * SLOT + lane * ROW_B +
                                                16 * (c ^ (lane % CH)));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");    // the slot is free again
    if (i + 1 < my_tiles) issue(i + 1);
    double acc = 0.0;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = kr[c][e];
        acc = add_rn(acc, mul_rn(qbar[8 * c + 2 * e], (double)__uint_as_float(w << 16)));
        acc = add_rn(acc, mul_rn(qbar[8 * c + 2 * e + 1],
                                       (double)__uint_as_float(w & 0xFFFF0000u)));
      }
    }
    const int key = t_beg + (wave + i * kRingWaves) * kRingTile + lane;
    if (key < t_end) {
      sc[key] = acc;
      const uint32_t k32 = fine_key32(acc);
      k16[key] = (uint16_t)(k32 >> 16);
      atomicAdd(&hist[k32 >> 20], 1u);
    }
  }
  __syncthreads();
  if (n_tiles > 0) {
    uint32_t* gh = a.hist + (size_t)u * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x)
      if (const uint32_t c = hist[i]) atomicAdd(&gh[i], c);
  }
}

// Block-wide exclusive prefix sum of one value per thread (at most 64
// waves); every thread of the block calls it.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wsum,
                                                         uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_prefix_sum(v);             // inclusive, within the wave
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  // every wave scans the waves' sums itself (one LDS read, one DPP scan)
  const int nw = (int)(blockDim.x >> 6);
  const uint32_t wp = wave_prefix_sum(lane < nw ? wsum[lane] : 0u);
  const uint32_t before =
      wave > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)wp, wave - 1) : 0u;
  if (threadIdx.x == 0) *total = (uint32_t)__builtin_amdgcn_readlane((int)wp, 63);
  __syncthreads();   // wsum is read by every wave before the next scan writes it
  return before + x - v;
}

__device__ __forceinline__ bool cand_before(uint64_t ka, int ia, uint64_t kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);   // (score desc, index asc)
}

// Inverse of order_key64 (for -0 folded onto +0 it returns +0).
__device__ __forceinline__ double key64_to_double(uint64_t k) {
  const uint64_t u = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
  return __longlong_as_double((long long)u);
}

constexpr int kMaskKeys = 131072;   // keys whose selection bits fit LDS
constexpr int kSmall = 1024;        // boundary sub-bin sizes ranked by counting

__global__ __launch_bounds__(1024) void topk_select_kernel(TopkArgs a) {
  __shared__ uint64_t ckey[kCandMax];
  __shared__ int32_t cidx[kCandMax];
  __shared__ uint32_t selmask[kMaskKeys / 32];   // bit j: key j is selected
  __shared__ uint32_t fh[kHistBins];             // second-level histogram of the candidates
  __shared__ uint16_t small[kSmall];             // candidates of the boundary sub-bin
  __shared__ uint32_t wsum[16];
  __shared__ uint32_t s_total, s_ncand, s_bin, s_above, s_nsmall;
  __shared__ uint64_t s_thr_key;
  __shared__ int32_t s_thr_idx;
  __shared__ uint32_t dh[256];

  const int u = blockIdx.x;
  const int b = u / a.Hkv;
  const int K = a.top_k;
  const double* sc = a.scores + (size_t)u * a.max_len;
  int32_t* out = a.sel_idx + (size_t)u * K;
  uint32_t* gh = a.hist + (size_t)u * kHistBins;
  const uint16_t* k16 = a.key16 + (size_t)u * a.max_len;
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6;

  // Requested together with the length, since neither depends on it: this
  // thread's histogram bins (descending order) and its first batch of 16-bit
  // keys (indices clamped to the row's capacity; slots at or past the length
  // are masked where the keys are used).  Rows of a multiple of 8 keys start
  // on 16-byte boundaries (the workspace is 256-byte aligned) and are read as
  // 16-byte words of 8 keys, kSelWords per thread per round; other rows are
  // read key by key, kSelBatch per thread per round.
  const bool vec = (a.max_len & 7) == 0;
  uint32_t c4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c4[i] = gh[kHistBins - 1 - (tid * 4 + i)];
  const u32x4_t* w16 = reinterpret_cast<const u32x4_t*>(k16);
  u32x4_t kw[kSelWords];
  uint32_t kv[kSelBatch];
  if (vec) {
#pragma unroll
    for (int k = 0; k < kSelWords; ++k) kw[k] = w16[min(k * nt + tid, (a.max_len >> 3) - 1)];
  } else {
#pragma unroll
    for (int k = 0; k < kSelBatch; ++k) kv[k] = k16[min(k * nt + tid, a.max_len - 1)];
  }
  const int L = ld_uniform(a.kv_len, b);

  if (K >= L) {
    for (int j = tid; j < K; j += nt) out[j] = (j < L) ? j : -1;
    for (int i = tid; i < kHistBins; i += nt) gh[i] = 0;
    return;
  }
  const bool use_mask = L <= kMaskKeys;

  // (a) boundary bin of the coarse histogram: highest bin whose suffix count
  //     reaches K.  Thread t owns bins [4t, 4t+4); counts scanned from the top.
  if (tid == 0) {
    s_bin = 0;
    s_above = 0;
  }
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) mine += c4[i];
  const uint32_t before = block_exclusive_scan(mine, wsum, &s_total);
  {
    uint32_t run = before;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (run < (uint32_t)K && run + c4[i] >= (uint32_t)K) {
        s_bin = kHistBins - 1 - (tid * 4 + i);
        s_above = run;
      }
      run += c4[i];
    }
  }
  if (tid == 0) s_ncand = 0;
  __syncthreads();
  const uint32_t bstar = s_bin;
  int need = K - (int)s_above;                           // 1..count(bstar)

  // (b) one pass over the 16-bit keys (a quarter of the score bytes; one
  //     workgroup streams them all): keys above the boundary bin set their
  //     selection bit, keys in it join the candidate list
  if (vec) {
    // thread: 8 consecutive keys per word, whose selection bits are one byte
    // of the mask; every byte of the mask words below L is written (zero
    // past L).  A wave scan of the per-thread candidate counts places them.
    const int nw = (L + 7) >> 3;
    const int nwm = use_mask ? ((L + 31) >> 5) * 4 : nw;
    uint8_t* selb = reinterpret_cast<uint8_t*>(selmask);
    for (int c0 = 0; c0 < nwm; c0 += nt * kSelWords) {
      if (c0 > 0) {
#pragma unroll
        for (int k = 0; k < kSelWords; ++k) kw[k] = w16[min(c0 + k * nt + tid, nw - 1)];
      }
      // Branch-free unsigned arithmetic on the 16-bit keys (a compare per
      // key would go through a scalar mask and a select, a VALU -> SALU ->
      // VALU chain per key): a key's coarse bin (its top 12 bits) lies above
      // bstar iff the key exceeds gt_key, and equals bstar iff key - eq_key
      // is below 16; keys at or past L are masked once per word.
      const uint32_t gt_key = (bstar << 4) | 15u, eq_key = bstar << 4;
      uint32_t cmask[kSelWords];
      uint32_t cnt = 0;
#pragma unroll
      for (int k = 0; k < kSelWords; ++k) {
        const int c = c0 + k * nt + tid;
        const uint32_t wd[4] = {kw[k][0], kw[k][1], kw[k][2], kw[k][3]};
        const int rem = L - c * 8;                     // keys of this word below L
        const uint32_t vmask = rem >= 8 ? 0xFFu : (1u << max(rem, 0)) - 1u;
        uint32_t am = 0, cm = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t key = (wd[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
          am |= ((gt_key - key) >> 31) << e;                  // key > gt_key
          cm |= ((((key - eq_key) >> 4) - 1u) >> 31) << e;    // 0 <= key - eq_key < 16
        }
        am &= vmask;
        cm &= vmask;
        if (use_mask && c < nwm) selb[c] = (uint8_t)am;
        cmask[k] = cm;
        cnt += (uint32_t)__popc(cm);
      }
      const uint32_t incl = wave_prefix_sum(cnt);
      const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
      if (wtot) {
        uint32_t wbase = 0;
        if (lane == 0) wbase = atomicAdd(&s_ncand, wtot);
        uint32_t pos = (uint32_t)__builtin_amdgcn_readfirstlane((int)wbase) + incl - cnt;
#pragma unroll
        for (int k = 0; k < kSelWords; ++k) {
          uint32_t cm = cmask[k];
          const int c = c0 + k * nt + tid;
          while (cm) {
            const int e = __ffs(cm) - 1;
            cm &= cm - 1;
            if (pos < (uint32_t)kCandMax) cidx[pos] = c * 8 + e;
            ++pos;
          }
        }
      }
    }
  }
  for (int j0 = 0; !vec && j0 < L; j0 += nt * kSelBatch) {
    // unconditional loads from clamped indices: a guarded load would be
    // compiled as a branch with its own wait, one round trip per key
    if (j0 > 0) {
#pragma unroll
      for (int k = 0; k < kSelBatch; ++k) kv[k] = k16[min(j0 + k * nt + tid, L - 1)];
    }
    // ballots first, then one LDS reservation per wave for the whole batch
    uint64_t bcs[kSelBatch];
    uint32_t wtotal = 0;
#pragma unroll
    for (int k = 0; k < kSelBatch; ++k) {
      const int j = j0 + k * nt + tid;
      const uint32_t cb = kv[k] >> 4;
      const uint64_t ba = __builtin_amdgcn_ballot_w64(j < L && cb > bstar);
      bcs[k] = __builtin_amdgcn_ballot_w64(j < L && cb == bstar);
      wtotal += (uint32_t)__popcll(bcs[k]);
      if (use_mask && lane == 0) {
        const int w = (j0 + k * nt + wave * 64) >> 5;   // 64-aligned run of keys
        selmask[w] = (uint32_t)ba;
        selmask[w + 1] = (uint32_t)(ba >> 32);
      }
    }
    if (wtotal) {
      uint32_t wbase = 0;
      if (lane == 0) wbase = atomicAdd(&s_ncand, wtotal);
      wbase = (uint32_t)__builtin_amdgcn_readfirstlane((int)wbase);
      const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
      for (int k = 0; k < kSelBatch; ++k) {
        if ((bcs[k] >> lane) & 1ull) {
          const uint32_t pos = wbase + (uint32_t)__popcll(bcs[k] & below);
          if (pos < (uint32_t)kCandMax) cidx[pos] = j0 + k * nt + tid;
        }
        wbase += (uint32_t)__popcll(bcs[k]);
      }
    }
  }
  for (int i = tid; i < kHistBins; i += nt) fh[i] = 0;
  if (tid == 0) s_nsmall = 0;
  __syncthreads();
  const uint32_t ncand = s_ncand;
  if (ncand <= (uint32_t)kCandMax) {   // the candidates' exact scores, in one gather
    for (uint32_t i = tid; i < ncand; i += nt) ckey[i] = order_key64(sc[cidx[i]]);
    __syncthreads();
  }

  if (ncand <= (uint32_t)kCandMax) {
    need = max(1, min(need, (int)max(ncand, 1u)));        // guards a corrupted histogram
    // (c1) second level: the next 12 bits of the float key split the boundary
    //      bin; find the sub-bin holding the need-th candidate
    for (uint32_t i = tid; i < ncand; i += nt)
      atomicAdd(&fh[(fine_key32(key64_to_double(ckey[i])) >> 8) & 0xFFFu], 1u);
    __syncthreads();
    uint32_t f4[4];
    uint32_t fm = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f4[i] = fh[kHistBins - 1 - (tid * 4 + i)];
      fm += f4[i];
    }
    const uint32_t fbefore = block_exclusive_scan(fm, wsum, &s_total);
    {
      uint32_t run = fbefore;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (run < (uint32_t)need && run + f4[i] >= (uint32_t)need) {
          s_bin = kHistBins - 1 - (tid * 4 + i);
          s_above = run;
        }
        run += f4[i];
      }
    }
    __syncthreads();
    const uint32_t fbin = s_bin;
    const int need2 = need - (int)s_above;
    const uint32_t fcount = fh[fbin];
    if (fcount <= (uint32_t)kSmall) {
      // (c2) rank the sub-bin's candidates by counting
      for (uint32_t i = tid; i < ncand; i += nt)
        if (((fine_key32(key64_to_double(ckey[i])) >> 8) & 0xFFFu) == fbin)
          small[atomicAdd(&s_nsmall, 1u)] = (uint16_t)i;
      __syncthreads();
      const uint32_t m = s_nsmall;
      for (uint32_t i = tid; i < m; i += nt) {
        const uint64_t ki = ckey[small[i]];
        const int ii = cidx[small[i]];
        int rank = 0;
        for (uint32_t j = 0; j < m; ++j)
          rank += cand_before(ckey[small[j]], cidx[small[j]], ki, ii) ? 1 : 0;
        if (rank == need2 - 1) {
          s_thr_key = ki;
          s_thr_idx = ii;
        }
      }
    } else {
      // (c2') many equal float keys: bitonic sort of all candidates
      uint32_t n2 = 1;
      while (n2 < ncand) n2 <<= 1;
      for (uint32_t i = ncand + tid; i < n2; i += nt) {
        ckey[i] = 0;          // below every real key
        cidx[i] = 0x7fffffff;
      }
      __syncthreads();
      for (uint32_t size = 2; size <= n2; size <<= 1) {
        for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
          for (uint32_t t = tid; t < n2 / 2; t += nt) {
            const uint32_t lo = 2 * t - (t & (stride - 1));
            const uint32_t hi = lo + stride;
            const bool up = ((lo & size) == 0);   // "up" = (score desc, index asc) order
            const uint64_t kl = ckey[lo], kh = ckey[hi];
            const int il = cidx[lo], ih = cidx[hi];
            const bool swap = up ? cand_before(kh, ih, kl, il) : cand_before(kl, il, kh, ih);
            if (swap) {
              ckey[lo] = kh; ckey[hi] = kl;
              cidx[lo] = ih; cidx[hi] = il;
            }
          }
          __syncthreads();
        }
      }
      if (tid == 0) {
        s_thr_key = ckey[need - 1];
        s_thr_idx = cidx[need - 1];
      }
    }
    __syncthreads();
  } else {
    // Exact radix select on the 64-bit keys of the boundary bin, 8-bit digits
    // from the top; `rem` keys of the current prefix group are still needed.
    uint64_t prefix = 0, pmask = 0;
    int rem = need;
    for (int shift = 56; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += nt) dh[i] = 0;
      __syncthreads();
      for (int j = tid; j < L; j += nt) {
        const double s = sc[j];
        if (coarse_bin(s) != bstar) continue;
        const uint64_t kk = order_key64(s);
        if ((kk & pmask) == prefix) atomicAdd(&dh[(kk >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        uint32_t run = 0;
        int dsel = 0;
        for (int dgt = 255; dgt >= 0; --dgt) {
          if (run + dh[dgt] >= (uint32_t)rem) { dsel = dgt; break; }
          run += dh[dgt];
        }
        s_bin = (uint32_t)dsel;
        s_above = run;
      }
      __syncthreads();
      prefix |= (uint64_t)s_bin << shift;
      pmask |= 255ull << shift;
      rem -= (int)s_above;
      __syncthreads();
    }
    // every key equal to `prefix` ties; the lowest `rem` indices among them win
    uint32_t cnt_before = 0;
    int thr = -1;
    for (int j0 = 0; j0 < L && thr < 0; j0 += nt) {
      const int j = j0 + tid;
      const uint32_t f = (j < L && order_key64(sc[j]) == prefix) ? 1u : 0u;
      const uint32_t ex = block_exclusive_scan(f, wsum, &s_total);
      if (f && cnt_before + ex + 1 == (uint32_t)rem) s_thr_idx = j;
      __syncthreads();
      if (cnt_before + s_total >= (uint32_t)rem) thr = s_thr_idx;
      cnt_before += s_total;
      __syncthreads();
    }
    if (tid == 0) s_thr_key = prefix;
    __syncthreads();
  }
  const uint64_t tk = s_thr_key;
  const int ti = s_thr_idx;

  // (d) ordered compaction of the selected keys
  uint32_t base = 0;
  if (use_mask && ncand <= (uint32_t)kCandMax) {
    // the boundary bin's winners join the bits of the keys above it; then
    // thread t owns a contiguous run of mask words, so one scan orders all
    for (uint32_t i = tid; i < ncand; i += nt) {
      const uint64_t kk = ckey[i];
      const int j = cidx[i];
      if (kk > tk || (kk == tk && j <= ti)) atomicOr(&selmask[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
    const int nwords = (L + 31) >> 5;
    const int per = (nwords + nt - 1) / nt;
    const int w0 = min(nwords, tid * per), w1 = min(nwords, w0 + per);
    uint32_t cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += (uint32_t)__popc(selmask[w]);
    const uint32_t ex = block_exclusive_scan(cnt, wsum, &s_total);
    uint32_t pos = ex;
    for (int w = w0; w < w1; ++w) {
      uint32_t bits = selmask[w];
      while (bits) {
        const int k = __ffs(bits) - 1;
        bits &= bits - 1;
        if (pos < (uint32_t)K) out[pos] = (w << 5) + k;
        ++pos;
      }
    }
    base = s_total;
  } else {
    // long caches: rounds of 32-key runs per thread straight from the scores
    for (int r0 = 0; r0 < L; r0 += nt * 32) {
      const int jl = r0 + tid * 32;
      double sv[32];
#pragma unroll
      for (int k = 0; k < 32; ++k) sv[k] = sc[min(jl + k, L - 1)];   // clamped, unconditional
      uint32_t mask = 0;
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        const int j = jl + k;
        const uint64_t kk = order_key64(sv[k]);
        if (j < L && (kk > tk || (kk == tk && j <= ti))) mask |= 1u << k;
      }
      const uint32_t ex = block_exclusive_scan((uint32_t)__popc(mask), wsum, &s_total);
      uint32_t pos = base + ex;
      while (mask) {
        const int k = __ffs(mask) - 1;
        mask &= mask - 1;
        if (pos < (uint32_t)K) out[pos] = jl + k;
        ++pos;
      }
      base += s_total;
    }
  }
  for (int j = K - 1 - tid; j >= (int)base; j -= nt) out[j] = -1;   // base == K here
  // leave the histogram clean (last: stores count against the loads' waits)
  for (int i = tid; i < kHistBins; i += nt) gh[i] = 0;
}

// ---------------------------------------------- Sparse-to-Dense ranking ----
// Per key j < kv_len[b] of unit u: the mean attention of the text rows, i.e.
// the row blocks' partial sums (from std.hip) added in block order in fp64
// and divided by the row count (0 without text).  That mean goes to the
// caller's fp32 score array; the ranking key is the mean for visual
// positions and -inf for text positions, which are kept unconditionally and
// must never displace a visual one.  Keys, 16-bit float keys and the coarse
// histogram are laid out exactly as the selection kernel above expects.
__global__ __launch_bounds__(256) void std_score_kernel(StdArgs s, TopkArgs a, float* score_out) {
  __shared__ uint32_t hist[kHistBins / 2];
  __shared__ uint32_t text_bits[kScoreKeys / 32];
  const int tiles = (a.max_len + kScoreKeys - 1) / kScoreKeys;
  const int u = blockIdx.x / tiles, tile = blockIdx.x - (blockIdx.x / tiles) * tiles;
  const int b = u / a.Hkv;
  const int L = ld_uniform(a.kv_len, b);
  const int j0 = tile * kScoreKeys;
  if (j0 >= L) return;
  const int T = ld_uniform(s.text_len, b);
  const int nrb = (T * s.G + 127) / 128;
  for (int i = threadIdx.x; i < kHistBins / 2; i += blockDim.x) hist[i] = 0;
  if (threadIdx.x < kScoreKeys / 32) text_bits[threadIdx.x] = 0;
  __syncthreads();
  const int* text = s.text_idx + (size_t)b * s.t_max;
  for (int i = threadIdx.x; i < T; i += blockDim.x) {
    const int x = text[i] - j0;
    if (x >= 0 && x < kScoreKeys) atomicOr(&text_bits[x >> 5], 1u << (x & 31));
  }
  __syncthreads();
  const int j = j0 + (int)threadIdx.x;
  if (j < L) {
    const float* col = s.colsum + (size_t)u * s.RB * a.max_len + j;
    double sum = 0.0;
    for (int r0 = 0; r0 < nrb; r0 += 8) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = col[(size_t)min(r0 + i, nrb - 1) * a.max_len];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (r0 + i < nrb) sum += (double)v[i];
    }
    const double mean = T ? sum / (double)(T * s.G) : 0.0;
    if (score_out) score_out[(size_t)u * a.max_len + j] = (float)mean;
    const bool is_text = (text_bits[threadIdx.x >> 5] >> (threadIdx.x & 31)) & 1u;
    const double key = is_text ? -INFINITY : mean;
    a.scores[(size_t)u * a.max_len + j] = key;
    const uint32_t k32 = fine_key32(key);
    a.key16[(size_t)u * a.max_len + j] = (uint16_t)(k32 >> 16);
    const uint32_t bin = k32 >> 20;
    atomicAdd(&hist[bin >> 1], (bin & 1u) ? 0x10000u : 1u);
  }
  __syncthreads();
  uint32_t* gh = a.hist + (size_t)u * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x)
    if (const uint32_t c = (hist[i >> 1] >> (16 * (i & 1))) & 0xFFFFu) atomicAdd(&gh[i], c);
}

// First index in the ascending array x[0, n) whose value is >= v.
__device__ __forceinline__ int lower_bound(const int32_t* x, int n, int v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (x[mid] < v) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// The i-th (from 0) position that is not in the ascending, distinct list
// text[0, T): text[k] - k positions precede text[k] outside the list, a
// non-decreasing count, so the answer is i plus the number of k with
// text[k] - k <= i.
__device__ __forceinline__ int ith_outside(const int32_t* text, int T, int i) {
  int lo = 0, hi = T;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (text[mid] - mid <= i) lo = mid + 1;
    else hi = mid;
  }
  return i + lo;
}

// The selection without text positions, and the kept list: the ascending
// union of the selection and the text positions, each element placed at its
// own index plus its rank in the other list.  When the sequence has no more
// visual positions than K, every one of them is selected (the ranking then
// also picked text positions, which are replaced here) and the kept list is
// every position below kv_len.
__global__ __launch_bounds__(256) void std_list_kernel(StdArgs s, int K, int32_t* sel,
                                                       int32_t* keep, int32_t* keep_len) {
  const int W = K + s.t_max;
  const int per_u = (W + 255) / 256;
  const int u = blockIdx.x / per_u;
  const int item = (blockIdx.x - u * per_u) * 256 + (int)threadIdx.x;
  const int b = u / s.Hkv;
  const int L = ld_uniform(s.kv_len, b), T = ld_uniform(s.text_len, b);
  const int nvis = L - T;
  const int32_t* text = s.text_idx + (size_t)b * s.t_max;
  int32_t* su = sel + (size_t)u * K;
  int32_t* ku = keep ? keep + (size_t)u * W : nullptr;
  if (nvis <= K) {
    if (item < K) su[item] = (item < nvis) ? ith_outside(text, T, item) : -1;
    if (ku && item < W) ku[item] = (item < L) ? item : -1;
    if (keep_len && item == 0) keep_len[u] = L;
  } else {
    if (ku) {
      if (item < K) {
        const int v = su[item];
        ku[item + lower_bound(text, T, v)] = v;
      } else if (item < K + T) {
        const int i = item - K, x = text[i];
        ku[i + lower_bound(su, K, x)] = x;
      } else if (item < W) {
        ku[item] = -1;
      }
    }
    if (keep_len && item == 0) keep_len[u] = K + T;
  }
}

}  // namespace

StdRankPlan plan_std_rank(int units, int max_len, size_t scratch_off) {
  StdRankPlan p;
  const size_t hist_bytes = (size_t)units * kHistBins * sizeof(uint32_t);
  p.hist_in_sync = hist_bytes <= kSyncBytes;
  p.off_scores = align_up(scratch_off, 256);
  p.off_key16 = align_up(p.off_scores + (size_t)units * max_len * sizeof(double), 256);
  size_t end = align_up(p.off_key16 + (size_t)units * max_len * sizeof(uint16_t), 256);
  if (p.hist_in_sync) {
    p.off_hist = 0;
  } else {
    p.off_hist = end;
    end = align_up(end + hist_bytes, 256);
  }
  p.ws_bytes = end;
  return p;
}

spec_status_t launch_std_rank(const StdArgs& s, int top_k, int32_t* sel_idx, int32_t* keep_idx,
                              int32_t* keep_len, float* score, const StdRankPlan& plan, void* ws,
                              hipStream_t stream) {
  TopkArgs a;
  memset(&a, 0, sizeof(a));
  a.kv_len = s.kv_len;
  a.B = s.B;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.G = s.G;
  a.max_len = s.max_len;
  a.top_k = top_k;
  char* w = reinterpret_cast<char*>(ws);
  a.scores = reinterpret_cast<double*>(w + plan.off_scores);
  a.key16 = reinterpret_cast<uint16_t*>(w + plan.off_key16);
  a.hist = reinterpret_cast<uint32_t*>(w + plan.off_hist);
  a.sel_idx = sel_idx;
  const int units = s.B * s.Hkv;
  if (!plan.hist_in_sync) {
    const spec_status_t st =
        launch_zero(a.hist, (size_t)units * kHistBins * sizeof(uint32_t), stream);
    if (st != SPEC_OK) return st;
  }
  const int tiles = (s.max_len + kScoreKeys - 1) / kScoreKeys;
  hipLaunchKernelGGL(std_score_kernel, dim3(units * tiles), dim3(256), 0, stream, s, a, score);
  if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
  hipLaunchKernelGGL(topk_select_kernel, dim3(units), dim3(1024), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
  const int per_u = (top_k + s.t_max + 255) / 256;
  hipLaunchKernelGGL(std_list_kernel, dim3(units * per_u), dim3(256), 0, stream, s, top_k,
                     sel_idx, keep_idx, keep_len);
  if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
  return SPEC_OK;
}

TopkPlan plan_topk(int units, int max_len, int top_k, int rows, int d) {
  TopkPlan p;
  const size_t hist_bytes = (size_t)units * kHistBins * sizeof(uint32_t);
  p.hist_in_sync = hist_bytes <= kSyncBytes;
  p.off_scores = kSyncBytes;
  p.off_key16 = align_up(p.off_scores + (size_t)units * max_len * sizeof(double), 256);
  size_t end = align_up(p.off_key16 + (size_t)units * max_len * sizeof(uint16_t), 256);
  if (p.hist_in_sync) {
    p.off_hist = 0;
  } else {
    p.off_hist = end;
    end = align_up(end + hist_bytes, 256);
  }
  p.attn = plan_attention(units, top_k, rows, d, true, end);
  p.ws_bytes = p.attn.ws_bytes > end ? p.attn.ws_bytes : end;
  return p;
}

spec_status_t launch_topk_select(const AttnArgs& aa, int d, int dtype, int top_k,
                                 int32_t* sel_idx, const TopkPlan& plan, void* ws,
                                 hipStream_t stream) {
  TopkArgs a;
  memset(&a, 0, sizeof(a));
  a.q = aa.q;
  a.k = aa.k;
  a.kv_len = aa.kv_len;
  a.page_table = aa.page_table;
  a.max_pages = aa.max_pages;
  a.page_shift = aa.page_shift;
  a.B = aa.B;
  a.Hq = aa.Hq;
  a.Hkv = aa.Hkv;
  a.G = aa.G;
  a.max_len = aa.max_len;
  a.top_k = top_k;
  char* w = reinterpret_cast<char*>(ws);
  a.scores = reinterpret_cast<double*>(w + plan.off_scores);
  a.key16 = reinterpret_cast<uint16_t*>(w + plan.off_key16);
  a.hist = reinterpret_cast<uint32_t*>(w + plan.off_hist);
  a.sel_idx = sel_idx;
  const int units = a.B * a.Hkv;
  const int tiles = (a.max_len + kScoreKeys - 1) / kScoreKeys;
  if (!plan.hist_in_sync) {   // scratch holds arbitrary data; the select kernel clears it after use
    const spec_status_t st =
        launch_zero(a.hist, (size_t)units * kHistBins * sizeof(uint32_t), stream);
    if (st != SPEC_OK) return st;
  }
  const dim3 grid(units * tiles), block(256);
  mark_before_main(stream);
  if (dtype == SPEC_BF16) {
    // about one streaming workgroup per CU
    a.splits = std::max(1, device_cu_count() / units);
    const dim3 rgrid(units * a.splits), rblock(kRingWaves * 64);
    if (d == 64) hipLaunchKernelGGL((topk_score_ring_kernel<64>), rgrid, rblock, 0, stream, a);
    else hipLaunchKernelGGL((topk_score_ring_kernel<128>), rgrid, rblock, 0, stream, a);
  } else {
    if (d == 64) hipLaunchKernelGGL((topk_score_kernel<64, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((topk_score_kernel<128, false>), grid, block, 0, stream, a);
  }
  mark_after_main(stream);
  if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
  hipLaunchKernelGGL(topk_select_kernel, dim3(units), dim3(1024), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
  return SPEC_OK;
}

}  // namespace spec

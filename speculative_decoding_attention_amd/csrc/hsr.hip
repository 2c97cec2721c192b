// Hidden-state-reuse fusion FC on gfx950:
//   Y[M, D] = X[M, 2D] W^T,  X[r] = concat(E[r], H[r]),  W [D, 2D] bf16.
// The concatenation is never materialised: loaders read columns k < D from E
// and k >= D from H.
//
// Large M (the batched draft step): a tiled GEMM on the matrix cores
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation).  A workgroup owns a BM x BN
// output tile (BM = 32*MT rows of X, BN = 16*NT*WN rows of W) and a K range;
// its 2*WN waves form a 2 x WN grid of (16*MT) x (16*NT) blocks (eight waves:
// two per SIMD hide each other's LDS and MFMA latency).  K advances in
// 64-wide steps whose X and W slabs (BM and BN rows of 128 bytes) move from
// HBM to LDS by DMA into a ring of NS stages, so data in flight costs no
// registers.  Each 128-byte row keeps its 16-byte chunk c at slot
// c ^ ((row >> 1) & 7): two rows share a 256-byte bank line, so the 16 rows
// of a fragment read (one chunk each) land on 16 distinct bank groups.  Split-K partials are summed in split order
// by a second small kernel, so results are bitwise reproducible.
//
// Small M (one draft token at a time): a stream of W through HBM, below.
#include <string.h>

#include "common.h"
#include "internal.h"

namespace spec {

namespace {

constexpr int kGemmBK = 64;                // K per step (128 bytes of a row)
constexpr int kGemmRing = 160 * 1024;      // LDS ring bytes (all of it)
constexpr int kGemmWN = 4;                 // waves along N (2 x kGemmWN waves per workgroup)

struct HsrArgs {
  const uint16_t* e;
  const uint16_t* h;
  const uint16_t* w;
  void* y;
  float* part;       // [S, M, D] split-K partials (S > 1)
  int32_t M, D, out_bf16;
  int32_t tiles_m, tiles_n, S, ksteps;
};

template <int MT, int NT, int WN>
struct GemmCfg {
  static constexpr int WAVES = 2 * WN;                   // 2 x WN grid of waves
  static constexpr int BM = 32 * MT, BN = 16 * NT * WN;
  static constexpr int STAGE = (BM + BN) * 128;          // bytes of one K step
  static constexpr int NS = (kGemmRing / STAGE < 8) ? kGemmRing / STAGE : 8;   // ring depth
  static constexpr int INSTR = STAGE / 1024;             // 1 KB DMAs per step
  static constexpr int PER_WAVE = INSTR / WAVES;
  static_assert(INSTR % WAVES == 0 && NS >= 3 && NS - 2 <= 6, "ring shape");
  static_assert(PER_WAVE * (NS - 2) <= 63, "vmcnt range");
};

// DMA of K step `ks` (columns 64*ks..) of the tile's X rows m0.. and W rows
// n0.. into one ring stage.  Instruction j moves 8 rows of 128 bytes; X rows
// past M repeat row M-1 (their outputs are never stored).
template <int MT, int NT, int WN>
__device__ __forceinline__ void gemm_src(const HsrArgs& a, int m0, int n0, int ks, int wave,
                                         int lane, const unsigned char* (&src)[GemmCfg<MT, NT, WN>::PER_WAVE]) {
  using C = GemmCfg<MT, NT, WN>;
  const int k0 = ks * kGemmBK;
  const int sub = lane >> 3, slot = lane & 7;
#pragma unroll
  for (int jj = 0; jj < C::PER_WAVE; ++jj) {
    const int j = wave + C::WAVES * jj;
    const int row = 8 * (j < C::BM / 8 ? j : j - C::BM / 8) + sub;
    const int chunk = slot ^ ((row >> 1) & 7);
    const int k = k0 + 8 * chunk;
    if (j < C::BM / 8) {
      const int m = min(m0 + row, a.M - 1);
      const uint16_t* xr = (k0 < a.D) ? a.e + (size_t)m * a.D + k : a.h + (size_t)m * a.D + (k - a.D);
      src[jj] = reinterpret_cast<const unsigned char*>(xr);
    } else {
      src[jj] = reinterpret_cast<const unsigned char*>(a.w + (size_t)(n0 + row) * (2 * a.D) + k);
    }
  }
}

// Requests instructions [J0, J1) of a step whose addresses gemm_src computed.
template <int MT, int NT, int WN, int J0, int J1>
__device__ __forceinline__ void gemm_dma(const unsigned char* const (&src)[GemmCfg<MT, NT, WN>::PER_WAVE],
                                         uint32_t stage_lds, int wave) {
  using C = GemmCfg<MT, NT, WN>;
#pragma unroll
  for (int jj = J0; jj < J1; ++jj)
    dma16(src[jj], stage_lds + (uint32_t)((wave + C::WAVES * jj) * 1024));
}

template <int MT, int NT, int WN>
__device__ __forceinline__ void gemm_issue(const HsrArgs& a, int m0, int n0, int ks,
                                           uint32_t stage_lds, int wave, int lane) {
  using C = GemmCfg<MT, NT, WN>;
  const unsigned char* src[C::PER_WAVE];
  gemm_src<MT, NT, WN>(a, m0, n0, ks, wave, lane, src);
  gemm_dma<MT, NT, WN, 0, C::PER_WAVE>(src, stage_lds, wave);
}

template <int MT, int NT, int WN>
__global__ __launch_bounds__(128 * WN, 1) void hsr_mfma_kernel(HsrArgs a) {
  using C = GemmCfg<MT, NT, WN>;
  __shared__ __align__(16) unsigned char ring[kGemmRing];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, q4 = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;
  const int kswap = (wave >> 2) & 1;              // waves are dealt to SIMDs round-robin
  // work item = (tile_n, split, tile_m): the tile_m neighbours share the W
  // slab of the same K range and land on the same XCD
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int tm = item % a.tiles_m;
  const int rest = item / a.tiles_m;
  const int sk = rest % a.S;
  const int tn = rest / a.S;
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  const int ks0 = (int)(((long)sk * a.ksteps) / a.S), ks1 = (int)(((long)(sk + 1) * a.ksteps) / a.S);
  const int nsteps = ks1 - ks0;

  lds_u8_t* const ring_l = (lds_u8_t*)ring;
  const uint32_t ring_lds = (uint32_t)(size_t)ring_l;
  for (int j = 0; j < C::NS - 1 && j < nsteps; ++j)
    gemm_issue<MT, NT, WN>(a, m0, n0, ks0 + j, ring_lds + (uint32_t)(j * C::STAGE), wave, lane);

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int t = 0; t < nsteps; ++t) {
    wait_tiles_barrier<C::PER_WAVE, C::NS - 2>(nsteps - 1 - t);
    // The refill of step t - 1's slot is spread over this step's MFMAs: the
    // matrix cores keep working while the address unit takes the requests
    // (one 1 KB request per 16 clocks per CU), instead of every wave
    // stalling on a burst of requests between the barrier and its MFMAs.
    const bool refill = t + C::NS - 1 < nsteps;
    const uint32_t nxt = ring_lds + (uint32_t)(((t + C::NS - 1) % C::NS) * C::STAGE);
    const unsigned char* src[C::PER_WAVE];
    gemm_src<MT, NT, WN>(a, m0, n0, refill ? ks0 + t + C::NS - 1 : ks0, wave, lane, src);
    const unsigned char* st = ring + (t % C::NS) * C::STAGE;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {            // two 32-wide k steps of the MFMA
      // the two waves that share a SIMD (w and w + 4) take the halves in
      // opposite orders, so one's LDS reads overlap the other's MFMAs
      // instead of both waiting for the same reads after the barrier
      const int kk = kh ^ kswap;
      const int c = 4 * kk + q4;
      bf16x8_t af[MT], bfr[NT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = wm * 16 * MT + 16 * mt + r16;
        af[mt] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(st + row * 128 + ((c ^ ((row >> 1) & 7)) * 16)));
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int row = wn * 16 * NT + 16 * nt + r16;
        bfr[nt] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(st + C::BM * 128 + row * 128 +
                                                                 ((c ^ ((row >> 1) & 7)) * 16)));
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], bfr[nt], acc[mt][nt], 0, 0, 0);
      if (refill) {
        if (kh == 0) gemm_dma<MT, NT, WN, 0, C::PER_WAVE / 2>(src, nxt, wave);
        else gemm_dma<MT, NT, WN, C::PER_WAVE / 2, C::PER_WAVE>(src, nxt, wave);
      }
    }
  }

  // lane (r16, q4) of block (mt, nt) holds rows 4*q4+i, column r16
  const int rb = m0 + wm * 16 * MT + 4 * q4, cb = n0 + wn * 16 * NT + r16;
  if (a.S == 1) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = rb + 16 * mt + i;
          if (m < a.M) {
            const size_t oi = (size_t)m * a.D + cb + 16 * nt;
            if (a.out_bf16)
              reinterpret_cast<uint16_t*>(a.y)[oi] = (uint16_t)f32_to_bf16_bits(acc[mt][nt][i]);
            else
              reinterpret_cast<float*>(a.y)[oi] = acc[mt][nt][i];
          }
        }
    return;
  }
  // split-K: the partial goes to the workspace; hsr_reduce_kernel adds the
  // splits in order once every split has finished
  float* mine = a.part + (size_t)sk * a.M * a.D;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = rb + 16 * mt + i;
        if (m < a.M) mine[(size_t)m * a.D + cb + 16 * nt] = acc[mt][nt][i];
      }
}

// Y = sum over splits s = 0..S-1 (in order) of the partials; 4 consecutive
// outputs per thread, every split's load in flight at once.
__global__ __launch_bounds__(256) void hsr_reduce_kernel(HsrArgs a) {
  constexpr int SMAX = 8;
  const size_t n4 = (size_t)a.M * a.D / 4;
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n4) return;
  const size_t plane = (size_t)a.M * a.D;
  f32x4_t v[SMAX];
#pragma unroll
  for (int sp = 0; sp < SMAX; ++sp)   // clamped split index: no guarded loads
    v[sp] = *reinterpret_cast<const f32x4_t*>(a.part + (size_t)min(sp, a.S - 1) * plane + 4 * e);
  f32x4_t sum = v[0];
#pragma unroll
  for (int sp = 1; sp < SMAX; ++sp)
    if (sp < a.S) sum += v[sp];
  if (a.out_bf16) {
    const uint32_t lo = f32_to_bf16_bits(sum[0]) | (f32_to_bf16_bits(sum[1]) << 16);
    const uint32_t hi = f32_to_bf16_bits(sum[2]) | (f32_to_bf16_bits(sum[3]) << 16);
    reinterpret_cast<uint2*>(a.y)[e] = make_uint2(lo, hi);
  } else {
    reinterpret_cast<f32x4_t*>(a.y)[e] = sum;
  }
}

// One-row path (the per-draft-step case): the FC is a stream of
// W (2*D*D bf16) through HBM.  Each wave owns RW consecutive output columns
// (W rows) and requests U 16-byte chunks of each of them at once (for
// D = 3584 that is the whole row pair), before it waits for anything: the
// workgroup's X loads (M rows of [e;h]) go out first, so staging X in LDS
// overlaps the W stream.  Products of bf16 values are exact in fp32; each
// lane accumulates its chunks in order and the wave reduces by shuffles.
template <int MM, int RW, int U, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void hsr_gemv_kernel(HsrArgs a) {
  extern __shared__ __align__(16) unsigned char xs[];   // [MM][Kd] bf16
  constexpr int XPT = 4;                                 // X chunks per thread per pass
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Kd = 2 * a.D, chunks = Kd / 8;
  const int n0 = (blockIdx.x * WAVES + wave) * RW;
  const uint16_t* wr = a.w + (size_t)min(n0, a.D - 1) * Kd;
  float acc[RW][MM];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int m = 0; m < MM; ++m) acc[r][m] = 0.f;

  for (int cb = 0, pass = 0; cb < chunks; cb += 64 * U, ++pass) {   // uniform trip count
    const int c0 = cb + lane;
    // X: MM*chunks chunks, XPT per thread per pass, loaded before W so the
    // compiler's wait for them does not cover the W loads
    u32x4_t xv[XPT];
    const bool stage = (pass == 0);
    const int xper = WAVES * 64 * XPT;
    for (int e0 = 0; stage && e0 < MM * chunks; e0 += xper) {
#pragma unroll
      for (int k = 0; k < XPT; ++k) {
        const int e = e0 + k * WAVES * 64 + tid;
        const int m = e / chunks, c = e - (e / chunks) * chunks;
        xv[k] = u32x4_t{0, 0, 0, 0};
        if (e < MM * chunks && m < a.M) {
          const int kk = c * 8;
          xv[k] = ld16((kk < a.D) ? a.e + (size_t)m * a.D + kk
                                  : a.h + (size_t)m * a.D + (kk - a.D));
        }
      }
      if (e0 + xper < MM * chunks) {   // more X than one pass: store now
#pragma unroll
        for (int k = 0; k < XPT; ++k) {
          const int e = e0 + k * WAVES * 64 + tid;
          if (e < MM * chunks) *reinterpret_cast<u32x4_t*>(xs + (size_t)e * 16) = xv[k];
        }
      }
    }
    u32x4_t wv[U][RW];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        const int c = c0 + 64 * u;
        wv[u][r] = (c < chunks && n0 + r < a.D) ? ld16(wr + (size_t)r * Kd + c * 8)
                                                 : u32x4_t{0, 0, 0, 0};
      }
    if (stage) {
      // the last X pass is still in registers
      const int e0 = ((MM * chunks - 1) / xper) * xper;
#pragma unroll
      for (int k = 0; k < XPT; ++k) {
        const int e = e0 + k * WAVES * 64 + tid;
        if (e < MM * chunks) *reinterpret_cast<u32x4_t*>(xs + (size_t)e * 16) = xv[k];
      }
      __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 64 * u;
      if (c >= chunks) break;
#pragma unroll
      for (int m = 0; m < MM; ++m) {
        const u32x4_t x = *reinterpret_cast<const u32x4_t*>(xs + ((size_t)m * chunks + c) * 16);
        float xf[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          xf[2 * j] = __uint_as_float(x[j] << 16);
          xf[2 * j + 1] = __uint_as_float(x[j] & 0xFFFF0000u);
        }
#pragma unroll
        for (int r = 0; r < RW; ++r) {
          float sacc = acc[r][m];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            sacc = __builtin_fmaf(__uint_as_float(wv[u][r][j] << 16), xf[2 * j], sacc);
            sacc = __builtin_fmaf(__uint_as_float(wv[u][r][j] & 0xFFFF0000u), xf[2 * j + 1], sacc);
          }
          acc[r][m] = sacc;
        }
      }
    }
  }
  if (n0 >= a.D) return;
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      float v = acc[r][m];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
      acc[r][m] = v;
    }
  if (lane < RW * MM) {
    const int r = lane / MM, m = lane - (lane / MM) * MM;
    float v = 0.f;
#pragma unroll
    for (int rr = 0; rr < RW; ++rr)
#pragma unroll
      for (int mm = 0; mm < MM; ++mm)
        if (rr == r && mm == m) v = acc[rr][mm];
    if (m < a.M && n0 + r < a.D) {
      const size_t oi = (size_t)m * a.D + n0 + r;
      if (a.out_bf16)
        reinterpret_cast<uint16_t*>(a.y)[oi] = (uint16_t)f32_to_bf16_bits(v);
      else
        reinterpret_cast<float*>(a.y)[oi] = v;
    }
  }
}

struct HsrPlan {
  int MT, BN, tiles_m, tiles_n, S, ksteps;
  size_t ws_bytes;
};

HsrPlan plan_hsr(int m, int d) {
  HsrPlan p;
  p.MT = (m <= 64) ? 2 : 4;
  // Wide W tiles for the batched case: every N tile re-reads its X rows, so
  // BN = 256 halves the X traffic per output column against 128 (measured
  // 37 -> 34 us at M = 320, D = 3584, with six K splits).
  p.BN = (m > 64 && d % 256 == 0) ? 256 : (d % 128 == 0) ? 128 : 64;
  p.tiles_m = (m + 32 * p.MT - 1) / (32 * p.MT);
  p.tiles_n = d / p.BN;
  p.ksteps = 2 * d / kGemmBK;
  const long tiles = (long)p.tiles_m * p.tiles_n;
  const int cus = device_cu_count();
  // split K until the grid covers the CUs, at least 4 steps per split
  long S = (cus + tiles / 2) / tiles;
  S = S < 1 ? 1 : (S > 8 ? 8 : S);
  while (S > 1 && p.ksteps / S < 4) --S;
  p.S = (int)S;
  p.ws_bytes = (S > 1) ? kSyncBytes + align_up((size_t)S * m * d * sizeof(float), 256) : 0;
  return p;
}

}  // namespace

// Up to kGemvMaxM rows the W stream kernel is used (measured faster than the
// matrix-core tiles for one row; from two rows on the tiles win).
constexpr int kGemvMaxM = 1;

bool use_gemv(int m, int d_model) {
  return m <= kGemvMaxM && (size_t)4 * d_model <= 64 * 1024;   // X row in default dynamic LDS
}

size_t hsr_workspace(int m, int d_model) {
  if (use_gemv(m, d_model)) return 0;   // the stream kernel needs no workspace
  return plan_hsr(m, d_model).ws_bytes;
}

spec_status_t launch_hsr(const void* e, const void* h, const void* w, int m, int d_model, void* y,
                         int out_bf16, void* ws, hipStream_t stream) {
  if (use_gemv(m, d_model)) {
    HsrArgs a;
    memset(&a, 0, sizeof(a));
    a.e = reinterpret_cast<const uint16_t*>(e);
    a.h = reinterpret_cast<const uint16_t*>(h);
    a.w = reinterpret_cast<const uint16_t*>(w);
    a.y = y;
    a.M = m;
    a.D = d_model;
    a.out_bf16 = out_bf16;
    constexpr int RW = 1, U = 14, WV = 8;   // one W row per wave (measured best)
    const dim3 grid((d_model + WV * RW - 1) / (WV * RW)), block(WV * 64);
    static_assert(kGemvMaxM == 1, "one X row in LDS");
    mark_before_main(stream);
    hipLaunchKernelGGL((hsr_gemv_kernel<1, RW, U, WV>), grid, block, (size_t)4 * d_model, stream, a);
    mark_after_main(stream);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
  }
  const HsrPlan p = plan_hsr(m, d_model);
  HsrArgs a;
  a.e = reinterpret_cast<const uint16_t*>(e);
  a.h = reinterpret_cast<const uint16_t*>(h);
  a.w = reinterpret_cast<const uint16_t*>(w);
  a.y = y;
  a.part = (p.S > 1) ? reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + kSyncBytes) : nullptr;
  a.M = m;
  a.D = d_model;
  a.out_bf16 = out_bf16;
  a.tiles_m = p.tiles_m;
  a.tiles_n = p.tiles_n;
  a.S = p.S;
  a.ksteps = p.ksteps;
  const dim3 grid(p.tiles_m * p.tiles_n * p.S), block(128 * kGemmWN);
  constexpr int N64 = 64 / (16 * kGemmWN), N128 = 128 / (16 * kGemmWN);
  constexpr int N256 = 256 / (16 * kGemmWN);
  mark_before_main(stream);
  switch (p.MT * 1000 + p.BN) {
    case 4256: hipLaunchKernelGGL((hsr_mfma_kernel<4, N256, kGemmWN>), grid, block, 0, stream, a); break;
    case 2064: hipLaunchKernelGGL((hsr_mfma_kernel<2, N64, kGemmWN>), grid, block, 0, stream, a); break;
    case 2128: hipLaunchKernelGGL((hsr_mfma_kernel<2, N128, kGemmWN>), grid, block, 0, stream, a); break;
    case 4064: hipLaunchKernelGGL((hsr_mfma_kernel<4, N64, kGemmWN>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((hsr_mfma_kernel<4, N128, kGemmWN>), grid, block, 0, stream, a); break;
  }
  mark_after_main(stream);
  if (p.S > 1) {
    if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
    const size_t n4 = (size_t)m * d_model / 4;
    hipLaunchKernelGGL(hsr_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream,
                       a);
  }
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

}  // namespace spec

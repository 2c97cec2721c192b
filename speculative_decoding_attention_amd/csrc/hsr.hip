// Hidden-state-reuse fusion FC on the gfx950 matrix cores:
//   Y[M, D] = X[M, 2D] W^T,  X[r] = concat(E[r], H[r]),  W [D, 2D] bf16.
// The concatenation is never materialised: the A-operand loader reads
// columns k < D from E and k >= D from H.
//
// Tiling.  A workgroup (4 waves) owns a BM x BN output tile (BM = 16*MF
// rows, BN = 4 waves x 16*WNF columns) and a K-slice; split-K slices are
// summed by the last workgroup of each tile in split order, so results are
// bitwise reproducible.  Per 128-wide K block, the X rows of the tile are
// staged in LDS (shared by the 4 waves); each wave streams its own W rows
// straight from HBM into registers (W is read exactly once per M band and
// is the dominant byte stream), one block ahead of the MFMAs
// (v_mfma_f32_16x16x32_bf16; A = X rows, B = W rows, both K-contiguous).
#include <string.h>

#include "common.h"
#include "internal.h"

namespace spec {

namespace {

constexpr int kBK = 128;          // K block staged per iteration
constexpr int kAP = kBK * 2 + 16;  // LDS pitch (bytes) of one staged X row

struct HsrArgs {
  const uint16_t* e;
  const uint16_t* h;
  const uint16_t* w;
  void* y;
  float* part;       // [S, M, D] split-K partials (S > 1)
  uint32_t* tick;    // [tiles] arrival counters (S > 1), in the sync region
  int32_t M, D, out_bf16;
  int32_t tiles_m, tiles_n, S, k_slice;
};

template <int MF>
__device__ __forceinline__ void load_a_block(const HsrArgs& a, int m0, int k0, u32x4_t (&ra)[3],
                                             int tid) {
  // MF*16 rows x 128 k = MF*16*16 chunks of 16 B; 256 threads -> <= 3 chunks each (MF <= 3)
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    const int e = tid + c * 256;
    if (e < MF * 16 * 16) {
      const int r = e >> 4, ch = e & 15;
      const int row = m0 + r, k = k0 + ch * 8;
      if (row < a.M) {
        const uint16_t* src = (k < a.D) ? a.e + (size_t)row * a.D + k
                                        : a.h + (size_t)row * a.D + (k - a.D);
        ra[c] = ld16(src);
      } else {
        ra[c] = u32x4_t{0, 0, 0, 0};
      }
    }
  }
}

template <int MF>
__device__ __forceinline__ void store_a_block(unsigned char* buf, const u32x4_t (&ra)[3], int tid) {
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    const int e = tid + c * 256;
    if (e < MF * 16 * 16) {
      const int r = e >> 4, ch = e & 15;
      *reinterpret_cast<u32x4_t*>(buf + r * kAP + ch * 16) = ra[c];
    }
  }
}

template <int MF, int WNF>
__global__ __launch_bounds__(256) void hsr_gemm_kernel(HsrArgs a) {
  static_assert(MF * 16 * 16 <= 768, "A block must fit 3 chunks per thread");
  __shared__ __align__(16) unsigned char abuf[2][MF * 16 * kAP];
  __shared__ uint32_t s_tick;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, q4 = lane >> 4;
  // work item = (tile_n, split, tile_m): neighbours share W columns -> same XCD
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int tm = item % a.tiles_m;
  const int rest = item / a.tiles_m;
  const int sk = rest % a.S;
  const int tn = rest / a.S;
  const int m0 = tm * MF * 16;
  const int n0 = tn * (4 * WNF * 16) + wave * WNF * 16;
  const int kb0 = sk * a.k_slice, kb1 = kb0 + a.k_slice;
  const int Kd = 2 * a.D;

  f32x4_t acc[MF][WNF];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf)
#pragma unroll
    for (int wn = 0; wn < WNF; ++wn) acc[mf][wn] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // W rows of this lane: column n0 + 16*wn + r16, k offset 8*q4 within a 32-step
  const uint16_t* wrow[WNF];
#pragma unroll
  for (int wn = 0; wn < WNF; ++wn) wrow[wn] = a.w + (size_t)(n0 + 16 * wn + r16) * Kd + 8 * q4;

  u32x4_t ra[3];
  u32x4_t wb[2][kBK / 32][WNF];
  load_a_block<MF>(a, m0, kb0, ra, tid);
#pragma unroll
  for (int s = 0; s < kBK / 32; ++s)
#pragma unroll
    for (int wn = 0; wn < WNF; ++wn) wb[0][s][wn] = ld16(wrow[wn] + kb0 + 32 * s);
  store_a_block<MF>(abuf[0], ra, tid);
  __syncthreads();

  int cur = 0;
  for (int k0 = kb0; k0 < kb1; k0 += kBK) {
    const int kn = k0 + kBK;
    const bool more = kn < kb1;
    if (more) {
      load_a_block<MF>(a, m0, kn, ra, tid);
#pragma unroll
      for (int s = 0; s < kBK / 32; ++s)
#pragma unroll
        for (int wn = 0; wn < WNF; ++wn) wb[cur ^ 1][s][wn] = ld16(wrow[wn] + kn + 32 * s);
    }
    const unsigned char* ab = abuf[cur];
#pragma unroll
    for (int s = 0; s < kBK / 32; ++s) {
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) {
        const u32x4_t av =
            *reinterpret_cast<const u32x4_t*>(ab + (mf * 16 + r16) * kAP + (32 * s + 8 * q4) * 2);
#pragma unroll
        for (int wn = 0; wn < WNF; ++wn)
          acc[mf][wn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av),
                                                                as_bf16x8(wb[cur][s][wn]),
                                                                acc[mf][wn], 0, 0, 0);
      }
    }
    if (more) store_a_block<MF>(abuf[cur ^ 1], ra, tid);
    __syncthreads();
    cur ^= 1;
  }

  // acc[mf][wn][i] = Y[m0 + 16*mf + 4*q4 + i][n0 + 16*wn + r16]
  if (a.S == 1) {
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m0 + 16 * mf + 4 * q4 + i;
        if (row >= a.M) continue;
#pragma unroll
        for (int wn = 0; wn < WNF; ++wn) {
          const size_t oi = (size_t)row * a.D + n0 + 16 * wn + r16;
          if (a.out_bf16)
            reinterpret_cast<uint16_t*>(a.y)[oi] = (uint16_t)f32_to_bf16_bits(acc[mf][wn][i]);
          else
            reinterpret_cast<float*>(a.y)[oi] = acc[mf][wn][i];
        }
      }
    return;
  }
  // split-K: publish this slice, the last arrival sums all slices in order
  float* mine = a.part + (size_t)sk * a.M * a.D;
#pragma unroll
  for (int mf = 0; mf < MF; ++mf)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + 16 * mf + 4 * q4 + i;
      if (row >= a.M) continue;
#pragma unroll
      for (int wn = 0; wn < WNF; ++wn)
        st_agent(mine + (size_t)row * a.D + n0 + 16 * wn + r16, acc[mf][wn][i]);
    }
  block_stores_done();   // partials visible device-wide before the arrival (see st_agent)
  const int tile = tn * a.tiles_m + tm;
  if (tid == 0)
    s_tick = __hip_atomic_fetch_add(&a.tick[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (s_tick != (uint32_t)(a.S - 1)) return;
#pragma unroll
  for (int mf = 0; mf < MF; ++mf)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + 16 * mf + 4 * q4 + i;
      if (row >= a.M) continue;
#pragma unroll
      for (int wn = 0; wn < WNF; ++wn) {
        const size_t oi = (size_t)row * a.D + n0 + 16 * wn + r16;
        float sum = 0.f;
        for (int s = 0; s < a.S; ++s) {
          sum += ld_agent(a.part + (size_t)s * a.M * a.D + oi);
        }
        if (a.out_bf16)
          reinterpret_cast<uint16_t*>(a.y)[oi] = (uint16_t)f32_to_bf16_bits(sum);
        else
          reinterpret_cast<float*>(a.y)[oi] = sum;
      }
    }
  if (tid == 0) a.tick[tile] = 0u;
}


// Small-M path (M <= 8 rows, the per-draft-step case): the FC is a stream of
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
  int MF, WNF, tiles_m, tiles_n, S, k_slice;
  size_t off_tick, ws_bytes;
};

HsrPlan plan_hsr(int m, int d) {
  HsrPlan p;
  p.MF = (m <= 16) ? 1 : (m <= 32 ? 2 : 3);
  p.WNF = (m > 16 && d % 128 == 0) ? 2 : 1;
  p.tiles_m = (m + 16 * p.MF - 1) / (16 * p.MF);
  p.tiles_n = d / (64 * p.WNF);
  const int Kd = 2 * d;
  const int tiles = p.tiles_m * p.tiles_n;
  const int target = device_cu_count();
  int S = 1;
  while (S < 16 && tiles * S * 2 <= target + target / 8 && (Kd % (2 * S * kBK)) == 0) S *= 2;
  p.S = S;
  p.k_slice = Kd / S;
  // split-K only when tiles * S <= about 1.1 x CUs, so the counters always fit
  // the sync region; the finishing workgroup of a tile returns its counter to 0
  p.off_tick = 0;
  p.ws_bytes = (S > 1) ? kSyncBytes + align_up((size_t)S * m * d * sizeof(float), 256) : 0;
  return p;
}

}  // namespace

size_t hsr_workspace(int m, int d_model) {
  if (m <= 8 && (size_t)8 * 4 * d_model <= 160 * 1024) return 0;   // small-M path needs none
  return plan_hsr(m, d_model).ws_bytes;
}

constexpr int kGemvMaxM = 8;

spec_status_t launch_hsr(const void* e, const void* h, const void* w, int m, int d_model, void* y,
                         int out_bf16, void* ws, hipStream_t stream) {
  if (m <= kGemvMaxM && (size_t)kGemvMaxM * 4 * d_model <= 160 * 1024) {
    HsrArgs a;
    memset(&a, 0, sizeof(a));
    a.e = reinterpret_cast<const uint16_t*>(e);
    a.h = reinterpret_cast<const uint16_t*>(h);
    a.w = reinterpret_cast<const uint16_t*>(w);
    a.y = y;
    a.M = m;
    a.D = d_model;
    a.out_bf16 = out_bf16;
    constexpr int RW = 2, U = 14, WV = 8;
    const dim3 grid((d_model + WV * RW - 1) / (WV * RW)), block(WV * 64);
    const int mm = (m <= 1) ? 1 : (m <= 2) ? 2 : (m <= 4) ? 4 : 8;
    const size_t lds = (size_t)mm * 4 * d_model;
    switch (mm) {
      case 1: hipLaunchKernelGGL((hsr_gemv_kernel<1, RW, U, WV>), grid, block, lds, stream, a); break;
      case 2: hipLaunchKernelGGL((hsr_gemv_kernel<2, RW, U, WV>), grid, block, lds, stream, a); break;
      case 4: hipLaunchKernelGGL((hsr_gemv_kernel<4, RW, U, WV>), grid, block, lds, stream, a); break;
      default: {
        // more than the default 64 KiB of dynamic LDS: raise the limit once
        static bool raised = false;
        if (!raised) {
          if (hipFuncSetAttribute(reinterpret_cast<const void*>(&hsr_gemv_kernel<8, RW, U, WV>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize,
                                  8 * 4 * 5120) != hipSuccess)
            return SPEC_ERR_HIP;
          raised = true;
        }
        hipLaunchKernelGGL((hsr_gemv_kernel<8, RW, U, WV>), grid, block, lds, stream, a);
        break;
      }
    }
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
  }
  const HsrPlan p = plan_hsr(m, d_model);
  HsrArgs a;
  a.e = reinterpret_cast<const uint16_t*>(e);
  a.h = reinterpret_cast<const uint16_t*>(h);
  a.w = reinterpret_cast<const uint16_t*>(w);
  a.y = y;
  a.part = (p.S > 1) ? reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + kSyncBytes) : nullptr;
  a.tick = (p.S > 1) ? reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(ws) + p.off_tick)
                     : nullptr;
  a.M = m;
  a.D = d_model;
  a.out_bf16 = out_bf16;
  a.tiles_m = p.tiles_m;
  a.tiles_n = p.tiles_n;
  a.S = p.S;
  a.k_slice = p.k_slice;
  const dim3 grid(p.tiles_m * p.tiles_n * p.S), block(256);
  const int cfg = p.MF * 10 + p.WNF;
  switch (cfg) {
    case 11: hipLaunchKernelGGL((hsr_gemm_kernel<1, 1>), grid, block, 0, stream, a); break;
    case 21: hipLaunchKernelGGL((hsr_gemm_kernel<2, 1>), grid, block, 0, stream, a); break;
    case 22: hipLaunchKernelGGL((hsr_gemm_kernel<2, 2>), grid, block, 0, stream, a); break;
    case 31: hipLaunchKernelGGL((hsr_gemm_kernel<3, 1>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((hsr_gemm_kernel<3, 2>), grid, block, 0, stream, a); break;
  }
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

}  // namespace spec

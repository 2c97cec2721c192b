// Shared device helpers for the gfx950 kernels (wave64, MFMA, LDS).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spec {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: 256 CUs in 8 XCDs, one L2 each

// Workgroups are dealt round-robin to the XCDs (WG i runs on XCD i % 8).
// Remap so that each XCD gets a contiguous range of work items: neighbouring
// work (the splits of one (sequence, KV head) unit, the tiles of one GEMM
// row band) then shares that XCD's L2.
__device__ __forceinline__ int xcd_remap(int i, int n) {
  const int per = n / kXcds, rem = n % kXcds;
  const int x = i % kXcds, j = i / kXcds;
  return (x < rem) ? x * (per + 1) + j : rem * (per + 1) + (x - rem) * per + j;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round to nearest even (inputs are finite on every path that calls this).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// A wave-uniform load through the scalar unit (s_load, waited on with
// lgkmcnt).  A vector load's wait (vmcnt) retires in order, so waiting for a
// length loaded after DMA requests would also wait for all of those; a
// scalar load never does.  Only for data no kernel of the same launch writes
// (lengths, list sizes).  The index must be uniform across the wave.
__device__ __forceinline__ int ld_uniform(const int32_t* p, int i) {
  typedef const int32_t __attribute__((address_space(4)))* cptr_t;
  return ((cptr_t)p)[__builtin_amdgcn_readfirstlane(i)];
}

// fp64 product and sum, each rounded once to nearest even and never fused
// with a neighbour into an FMA (fixed-order chains that define a result bit
// for bit need both roundings; the compiler's default contraction, which
// also applies to the math header's __dmul_rn / __dadd_rn, would drop the
// product's).
__device__ __forceinline__ double mul_rn(double a, double b) {
#pragma clang fp contract(off)
  return a * b;
}
__device__ __forceinline__ double add_rn(double a, double b) {
#pragma clang fp contract(off)
  return a + b;
}

// 16-byte global load / store helpers.
__device__ __forceinline__ u32x4_t ld16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// Butterfly reductions across lanes l ^ 16 and l ^ 32 (the four 16-lane
// rows of a wave that hold the same MFMA output column).
// Inclusive prefix sum over the wave's 64 lanes by DPP: Hillis-Steele shifts
// within each 16-lane row, then the gfx9 row broadcasts of lane 15 (into
// rows 1 and 3) and lane 31 (into rows 2 and 3).  Each step is one VALU
// instruction; a shuffle step would be an LDS permute with its round trip.
// Every lane of the wave must be active.
__device__ __forceinline__ uint32_t wave_prefix_sum(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// The wave's sum, uniform (lane 63 of the prefix sum).
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_prefix_sum(x), 63);
}

// Across the four 16-lane rows of the wave (lanes l, l^16, l^32, l^48).  The
// gfx950 row swaps exchange rows in the VALU (a shuffle would be an LDS
// permute): after v_permlane16_swap of a value with itself, a lane's two
// results are its own value and its partner row's, in some order; the same
// holds for v_permlane32_swap one level up.  Combining the two is
// commutative, so every lane gets what the xor-16-then-32 order gives.
__device__ __forceinline__ float max_across_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_across_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ---------------------------------------------------------- LDS DMA ----
typedef __attribute__((address_space(3))) unsigned char lds_u8_t;

// One 1 KB DMA: each lane copies 16 bytes from its own address g to LDS at
// lds_byte_addr + 16*lane.  The LDS base goes through M0, which is set in the
// same statement; no code of this library keeps a value in M0.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_byte_addr) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_byte_addr);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(base) : "memory");
}

// Waits until at most N of this wave's DMA loads are outstanding, then a
// workgroup barrier; acts as a compiler memory barrier for LDS accesses.
template <int N>
__device__ __forceinline__ void wait_dma_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" :: "n"(N) : "memory");
}

// Waits until at most `later` tile groups of PER_WAVE DMA loads each are
// still outstanding for this wave (later clamped to [0, MAXL], so every
// vmcnt immediate is known at compile time), then a workgroup barrier.
template <int PER_WAVE, int MAXL>
__device__ __forceinline__ void wait_tiles_barrier(int later_tiles) {
  static_assert(PER_WAVE * MAXL <= 63, "vmcnt range");
  if constexpr (MAXL <= 0) {
    wait_dma_barrier<0>();
  } else {
    if (later_tiles >= MAXL)
      wait_dma_barrier<PER_WAVE * MAXL>();
    else
      wait_tiles_barrier<PER_WAVE, MAXL - 1>(later_tiles);
  }
}

}  // namespace spec

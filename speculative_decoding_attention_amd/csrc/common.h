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

// 16-byte global load / store helpers.
__device__ __forceinline__ u32x4_t ld16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// Butterfly reductions across lanes l ^ 16 and l ^ 32 (the four 16-lane
// rows of a wave that hold the same MFMA output column).
__device__ __forceinline__ float max_across_rows(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float sum_across_rows(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Device-wide hand-off between workgroups without cache flushes.  Each XCD
// has its own L2, so plain stores can sit in one XCD's L2 where another XCD
// cannot see them, and a release fence writes back that whole L2 (costly:
// tens of microseconds when every workgroup of a grid does it).  Instead the
// data handed off is stored and loaded at agent scope: such stores write
// through to the device-coherent level and complete (vmcnt) only once they
// are visible there, and such loads bypass the non-coherent caches.  The
// producer's waves wait for their own stores, meet at a workgroup barrier,
// and only then does thread 0 signal with an agent-scope atomic; the
// consumer reads the data only after it has seen the signal.
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __uint_as_float(__hip_atomic_load(const_cast<uint32_t*>(reinterpret_cast<const uint32_t*>(p)),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
// Every wave's agent-scope stores have completed when this returns.
__device__ __forceinline__ void block_stores_done() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
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

template <int PER_WAVE>
__device__ __forceinline__ void wait_tiles_barrier(int later_tiles) {
  switch (later_tiles) {
    case 0: wait_dma_barrier<0>(); break;
    case 1: wait_dma_barrier<PER_WAVE * 1>(); break;
    case 2: wait_dma_barrier<PER_WAVE * 2>(); break;
    case 3: wait_dma_barrier<PER_WAVE * 3>(); break;
    case 4: wait_dma_barrier<PER_WAVE * 4>(); break;
    case 5: wait_dma_barrier<PER_WAVE * 5>(); break;
    default: wait_dma_barrier<PER_WAVE * 6>(); break;
  }
}

}  // namespace spec

// Plain streaming read (gfx950): the reference rate every HBM-bound kernel
// of the library is compared with.  Each thread keeps eight 16-byte loads in
// flight over a grid-stride walk of the buffer; the workgroup folds what it
// read into one XOR word, so no load is dead and the caller can check that
// every byte was read exactly once (the XOR of the sink words is the XOR of
// the buffer's 32-bit words).
#include "common.h"
#include "internal.h"

namespace spec {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeLoads = 8;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4_t* p, size_t n16,
                                                                   uint32_t* sink) {
  __shared__ uint32_t red[kProbeThreads / 64];
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t x = 0;
  for (; i + (kProbeLoads - 1) * stride < n16; i += kProbeLoads * stride) {
    u32x4_t v[kProbeLoads];
#pragma unroll
    for (int k = 0; k < kProbeLoads; ++k) v[k] = p[i + k * stride];
#pragma unroll
    for (int k = 0; k < kProbeLoads; ++k) x ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = p[i];
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
    for (int w = 0; w < kProbeThreads / 64; ++w) y ^= red[w];
    sink[blockIdx.x] = y;
  }
}

}  // namespace

spec_status_t launch_read_probe(const void* p, size_t bytes, uint32_t* sink, hipStream_t stream) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(SPEC_READ_PROBE_SINK_WORDS), dim3(kProbeThreads), 0,
                     stream, reinterpret_cast<const u32x4_t*>(p), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

}  // namespace spec

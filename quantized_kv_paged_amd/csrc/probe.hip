// Streaming-read probe: the HBM read bandwidth this device reaches, the measured ceiling
// beside the nominal 8 TB/s that the decode kernels' KV-read rate is also compared with.
// Every thread XORs the 16-byte words of its grid-stride share of the buffer (kProbeUnroll
// independent nontemporal loads in flight per thread; each load instruction of a wave reads
// 1 KB of whole cache lines, which nontemporal loads stream past the caches); every block
// writes the XOR of its threads, so the host can check that each word was read exactly once.
#include "device_common.h"
#include "mlaq_kernels.h"

namespace mlaq {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* __restrict__ p, int64_t n,
                                                                   u32x4* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kProbeUnroll - 1) * stride < n; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int k = 0; k < kProbeUnroll; ++k) v[k] = __builtin_nontemporal_load(p + i + k * stride);
#pragma unroll
    for (int k = 0; k < kProbeUnroll; ++k) acc ^= v[k];
  }
  for (; i < n; i += stride) acc ^= __builtin_nontemporal_load(p + i);
  __shared__ u32x4 red[kProbeThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
#pragma unroll
  for (int s = kProbeThreads / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = red[0];
}

hipError_t launch_read_probe(const void* buf, int64_t words, void* partials, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4*>(buf), words, static_cast<u32x4*>(partials));
  return hipGetLastError();
}

}  // namespace mlaq

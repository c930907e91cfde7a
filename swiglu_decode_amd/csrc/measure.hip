// Measurement aid: a plain streaming read of device memory, the attainable
// HBM read rate that the fused kernels' rates are set beside.
#include <hip/hip_runtime.h>

#include "sgd_host.hpp"

namespace sgd {

constexpr int RS_UNROLL = 8;        // 16-byte loads in flight per thread
constexpr unsigned RS_BLOCKS = 8192;  // 32 workgroups of 256 threads per CU
constexpr uint32_t RS_NEVER = 0x7fc0a5a5u;

// Every thread reads 16-byte vectors grid-stride, RS_UNROLL at a time, and
// folds them into one word; the word is stored only when it equals a value
// the caller's data is not expected to produce, so the loads cannot be
// dropped and nothing but the sink word is ever written.
__global__ __launch_bounds__(256) void read_stream_kernel(const uint4* __restrict__ p, size_t n16,
                                                          uint32_t* sink) {
  const size_t nt = (size_t)gridDim.x * blockDim.x;
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (RS_UNROLL - 1) * nt < n16; i += RS_UNROLL * nt) {
    uint4 v[RS_UNROLL];
#pragma unroll
    for (int u = 0; u < RS_UNROLL; ++u) v[u] = p[i + u * nt];
#pragma unroll
    for (int u = 0; u < RS_UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += nt) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == RS_NEVER) sink[0] = acc;
}

int launch_read_stream(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(read_stream_kernel, dim3(RS_BLOCKS), dim3(256), 0, s, static_cast<const uint4*>(buf),
                     bytes / 16, sink);
  return hip_status(hipGetLastError());
}

}  // namespace sgd

// Decode-stack glue around the fused MLP: bf16 -> fp32 residual init,
// RMSNorm to bf16 (Zhang & Sennrich 2019, unit gain), residual add, the bf16
// output head (fp32 accumulation on the bf16 MFMA) and a per-row argmax.
// The argmax stands in for greedy token selection, the correctness gate of
// the Fish Audio X post "We Made Our Best Voice Model Free…", section
// "FP8 only works if quality survives".
#include "sgd_device.hpp"
#include "sgd_host.hpp"

namespace sgd {

typedef short v8s __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void bf16_to_f32_kernel(const uint16_t* __restrict__ x, size_t n,
                                                          float* __restrict__ h) {
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n; i += (size_t)gridDim.x * 256ull)
    h[i] = bf16_to_f32(x[i]);
}

// One workgroup per row; fp32 sum of squares reduced in a fixed order.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ h, int d, float eps,
                                                      uint16_t* __restrict__ x) {
  const int row = blockIdx.x;
  const float* hr = h + (size_t)row * d;
  float ss = 0.0f;
  for (int c = threadIdx.x; c < d; c += 256) ss = fmaf(hr[c], hr[c], ss);
  __shared__ float red[256];
  red[threadIdx.x] = ss;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  const float inv = 1.0f / sqrtf(red[0] / (float)d + eps);
  for (int c = threadIdx.x; c < d; c += 256) x[(size_t)row * d + c] = (uint16_t)f32_to_bf16(hr[c] * inv);
}

__global__ __launch_bounds__(256) void residual_kernel(float* __restrict__ h, const uint16_t* __restrict__ y,
                                                       size_t n) {
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n; i += (size_t)gridDim.x * 256ull)
    h[i] += bf16_to_f32(y[i]);
}

// Head: logits[M, N] = bf16(h)[M, K] W[N, K]^T.  One wavefront per 16
// output columns (one 16-row band of W) and all M rows (up to 8 m-tiles),
// using the 16x16x32 bf16 MFMA.  Operand order of that instruction: lane l
// holds row l % 16 and K elements 8*(l/16)..8*(l/16)+7 of a 32-wide step.
__global__ __launch_bounds__(256) void head_kernel(const float* __restrict__ h, int M, int K,
                                                   const uint16_t* __restrict__ w, int N,
                                                   float* __restrict__ out) {
  const int wid = (int)((blockIdx.x * 256u + threadIdx.x) >> 6);
  const int l = threadIdx.x & 63;
  if (wid >= N / 16) return;
  const int n0 = wid * 16;
  const int MT = (M + 15) / 16;
  v4f acc[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
  const uint16_t* wr = w + (size_t)(n0 + (l & 15)) * K + 8 * (l >> 4);
  for (int k = 0; k < K; k += 32) {
    const uint4 wv = *reinterpret_cast<const uint4*>(wr + k);
    v8s b;
    b[0] = (short)(wv.x & 0xFFFF); b[1] = (short)(wv.x >> 16);
    b[2] = (short)(wv.y & 0xFFFF); b[3] = (short)(wv.y >> 16);
    b[4] = (short)(wv.z & 0xFFFF); b[5] = (short)(wv.z >> 16);
    b[6] = (short)(wv.w & 0xFFFF); b[7] = (short)(wv.w >> 16);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      if (mt < MT) {
        const int row = mt * 16 + (l & 15);
        v8s a;
        if (row < M) {
          const float* hp = h + (size_t)row * K + k + 8 * (l >> 4);
#pragma unroll
          for (int e = 0; e < 8; ++e) a[e] = (short)f32_to_bf16(hp[e]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) a[e] = 0;
        }
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[mt], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    if (mt < MT) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = mt * 16 + 4 * (l >> 4) + r;
        if (row < M) out[(size_t)row * N + n0 + (l & 15)] = acc[mt][r];
      }
    }
  }
}

// One workgroup per row: first index of the maximum.
__global__ __launch_bounds__(256) void argmax_kernel(const float* __restrict__ logits, int N,
                                                     int32_t* __restrict__ out) {
  const int row = blockIdx.x;
  const float* lr = logits + (size_t)row * N;
  float best = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int c = threadIdx.x; c < N; c += 256) {
    const float v = lr[c];
    if (v > best) {
      best = v;
      bi = c;
    }
  }
  __shared__ float sv[256];
  __shared__ int si[256];
  sv[threadIdx.x] = best;
  si[threadIdx.x] = bi;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      const float v2 = sv[threadIdx.x + o];
      const int i2 = si[threadIdx.x + o];
      if (v2 > sv[threadIdx.x] || (v2 == sv[threadIdx.x] && i2 < si[threadIdx.x])) {
        sv[threadIdx.x] = v2;
        si[threadIdx.x] = i2;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) out[row] = si[0];
}

static unsigned grid_for(size_t n) {
  size_t b = (n + 255) / 256;
  return (unsigned)(b > 4096 ? 4096 : (b == 0 ? 1 : b));
}

int launch_bf16_to_f32(const uint16_t* x, int M, int d, float* h, hipStream_t s) {
  const size_t n = (size_t)M * d;
  hipLaunchKernelGGL(bf16_to_f32_kernel, dim3(grid_for(n)), dim3(256), 0, s, x, n, h);
  return hip_status(hipGetLastError());
}

int launch_rmsnorm(const float* h, int M, int d, float eps, uint16_t* x, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(M), dim3(256), 0, s, h, d, eps, x);
  return hip_status(hipGetLastError());
}

int launch_residual_add(float* h, const uint16_t* y, int M, int d, hipStream_t s) {
  const size_t n = (size_t)M * d;
  hipLaunchKernelGGL(residual_kernel, dim3(grid_for(n)), dim3(256), 0, s, h, y, n);
  return hip_status(hipGetLastError());
}

int launch_head(const float* h, int M, int K, const uint16_t* w, int N, float* out, hipStream_t s) {
  const unsigned blocks = (unsigned)((N / 16 + 3) / 4);
  hipLaunchKernelGGL(head_kernel, dim3(blocks), dim3(256), 0, s, h, M, K, w, N, out);
  return hip_status(hipGetLastError());
}

int launch_argmax(const float* logits, int M, int N, int32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(argmax_kernel, dim3(M), dim3(256), 0, s, logits, N, out);
  return hip_status(hipGetLastError());
}

}  // namespace sgd

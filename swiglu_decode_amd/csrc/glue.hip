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

// Elementwise kernels over n = M*d elements, d a multiple of 128: four
// elements per thread (16-byte fp32 and 8-byte bf16 accesses).
__global__ __launch_bounds__(256) void bf16_to_f32_kernel(const uint16_t* __restrict__ x, size_t n4,
                                                          float* __restrict__ h) {
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256ull) {
    const uint2 v = reinterpret_cast<const uint2*>(x)[i];
    reinterpret_cast<float4*>(h)[i] =
        make_float4(bf16_to_f32(v.x & 0xFFFFu), bf16_to_f32(v.x >> 16), bf16_to_f32(v.y & 0xFFFFu), bf16_to_f32(v.y >> 16));
  }
}

__global__ __launch_bounds__(256) void residual_kernel(float* __restrict__ h, const uint16_t* __restrict__ y,
                                                       size_t n4) {
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256ull) {
    const uint2 v = reinterpret_cast<const uint2*>(y)[i];
    float4 a = reinterpret_cast<float4*>(h)[i];
    a.x += bf16_to_f32(v.x & 0xFFFFu);
    a.y += bf16_to_f32(v.x >> 16);
    a.z += bf16_to_f32(v.y & 0xFFFFu);
    a.w += bf16_to_f32(v.y >> 16);
    reinterpret_cast<float4*>(h)[i] = a;
  }
}

// One workgroup per row.  Each thread takes the row's 16-byte chunks t,
// t + 256, ... with up to four loads in flight; its sum of squares is an
// fma chain in that order, reduced over the wavefront by a fixed butterfly
// and over the four wavefronts in index order.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ h, int d, float eps,
                                                      uint16_t* __restrict__ x) {
  const int row = blockIdx.x;
  const float4* hr = reinterpret_cast<const float4*>(h + (size_t)row * d);
  const int n4 = d >> 2, t = threadIdx.x;
  float ss = 0.0f;
  for (int c0 = t; c0 < n4; c0 += 4 * 256) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = c0 + 256 * u < n4 ? hr[c0 + 256 * u] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ss = fmaf(v[u].x, v[u].x, ss);
      ss = fmaf(v[u].y, v[u].y, ss);
      ss = fmaf(v[u].z, v[u].z, ss);
      ss = fmaf(v[u].w, v[u].w, ss);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, WAVE);
  __shared__ float red[4];
  if ((t & 63) == 0) red[t >> 6] = ss;
  __syncthreads();
  const float inv = 1.0f / sqrtf((((red[0] + red[1]) + red[2]) + red[3]) / (float)d + eps);
  uint2* xr = reinterpret_cast<uint2*>(x + (size_t)row * d);
  for (int c0 = t; c0 < n4; c0 += 4 * 256) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = c0 + 256 * u < n4 ? hr[c0 + 256 * u] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (c0 + 256 * u < n4)
        xr[c0 + 256 * u] = make_uint2(f32_to_bf16(v[u].x * inv) | (f32_to_bf16(v[u].y * inv) << 16),
                                      f32_to_bf16(v[u].z * inv) | (f32_to_bf16(v[u].w * inv) << 16));
  }
}

// The residual add and the next block's RMSNorm in one pass over a row:
// h += y, then x = bf16(h / sqrt(mean(h^2) + eps)).  The arithmetic is that
// of residual_kernel followed by rmsnorm_kernel (the same fp32 add per
// element, the same chunk order of the sum of squares and the same
// reduction), so the results are bit-identical to the two calls.  The
// first pass forms h + y to sum its squares; the second forms it again and
// stores both h and x.
__global__ __launch_bounds__(256) void residual_rmsnorm_kernel(float* __restrict__ h,
                                                               const uint16_t* __restrict__ y, int d, float eps,
                                                               uint16_t* __restrict__ x) {
  const int row = blockIdx.x;
  float4* hr = reinterpret_cast<float4*>(h + (size_t)row * d);
  const uint2* yr = reinterpret_cast<const uint2*>(y + (size_t)row * d);
  const int n4 = d >> 2, t = threadIdx.x;
  auto added = [&](int c) {
    const float4 a = hr[c];
    const uint2 v = yr[c];
    return make_float4(a.x + bf16_to_f32(v.x & 0xFFFFu), a.y + bf16_to_f32(v.x >> 16),
                       a.z + bf16_to_f32(v.y & 0xFFFFu), a.w + bf16_to_f32(v.y >> 16));
  };
  float ss = 0.0f;
  for (int c0 = t; c0 < n4; c0 += 4 * 256) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = c0 + 256 * u < n4 ? added(c0 + 256 * u) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ss = fmaf(v[u].x, v[u].x, ss);
      ss = fmaf(v[u].y, v[u].y, ss);
      ss = fmaf(v[u].z, v[u].z, ss);
      ss = fmaf(v[u].w, v[u].w, ss);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, WAVE);
  __shared__ float red[4];
  if ((t & 63) == 0) red[t >> 6] = ss;
  __syncthreads();  // (also orders every thread's first-pass reads of h before any store to it)
  const float inv = 1.0f / sqrtf((((red[0] + red[1]) + red[2]) + red[3]) / (float)d + eps);
  uint2* xr = reinterpret_cast<uint2*>(x + (size_t)row * d);
  for (int c0 = t; c0 < n4; c0 += 4 * 256) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = c0 + 256 * u < n4 ? added(c0 + 256 * u) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (c0 + 256 * u < n4) {
        hr[c0 + 256 * u] = v[u];
        xr[c0 + 256 * u] = make_uint2(f32_to_bf16(v[u].x * inv) | (f32_to_bf16(v[u].y * inv) << 16),
                                      f32_to_bf16(v[u].z * inv) | (f32_to_bf16(v[u].w * inv) << 16));
      }
  }
}

// Head: logits[M, N] = bf16(h)[M, K] W[N, K]^T on the 16x16x32 bf16 MFMA.
// One workgroup per 16 output columns (one 16-row band of W) and all M rows
// (up to MTM m-tiles).  Its four wavefronts take the 32-wide k-steps q, q+4,
// ... with U steps' loads in flight at a time, and their partial sums are
// added in wavefront order at the end.  Operand order of the instruction:
// lane l holds row l % 16 and K elements 8*(l/16)..8*(l/16)+7 of a step.
template <int MTM, int U>
__global__ __launch_bounds__(256) void head_kernel(const float* __restrict__ h, int M, int K,
                                                   const uint16_t* __restrict__ w, int N,
                                                   float* __restrict__ out) {
  const int n0 = blockIdx.x * 16;
  const int q = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int KS = K / 32;
  v4f acc[MTM];
#pragma unroll
  for (int mt = 0; mt < MTM; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
  const uint16_t* wr = w + (size_t)(n0 + (l & 15)) * K + 8 * (l >> 4);
  const int hk = 8 * (l >> 4);
  for (int j0 = q; j0 < KS; j0 += 4 * U) {
    uint4 wv[U];
    float4 hv[U][MTM][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ks = j0 + 4 * u;
      const bool ok = ks < KS;
      wv[u] = ok ? *reinterpret_cast<const uint4*>(wr + 32 * ks) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int mt = 0; mt < MTM; ++mt) {
        const int row = mt * 16 + (l & 15);
        if (ok && row < M) {
          const float4* hp = reinterpret_cast<const float4*>(h + (size_t)row * K + 32 * ks + hk);
          hv[u][mt][0] = hp[0];
          hv[u][mt][1] = hp[1];
        } else {
          hv[u][mt][0] = hv[u][mt][1] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j0 + 4 * u >= KS) break;
      v8s b;
      b[0] = (short)(wv[u].x & 0xFFFF); b[1] = (short)(wv[u].x >> 16);
      b[2] = (short)(wv[u].y & 0xFFFF); b[3] = (short)(wv[u].y >> 16);
      b[4] = (short)(wv[u].z & 0xFFFF); b[5] = (short)(wv[u].z >> 16);
      b[6] = (short)(wv[u].w & 0xFFFF); b[7] = (short)(wv[u].w >> 16);
#pragma unroll
      for (int mt = 0; mt < MTM; ++mt) {
        if (mt * 16 < M) {
          const float4 p = hv[u][mt][0], r = hv[u][mt][1];
          v8s a;
          a[0] = (short)f32_to_bf16(p.x); a[1] = (short)f32_to_bf16(p.y);
          a[2] = (short)f32_to_bf16(p.z); a[3] = (short)f32_to_bf16(p.w);
          a[4] = (short)f32_to_bf16(r.x); a[5] = (short)f32_to_bf16(r.y);
          a[6] = (short)f32_to_bf16(r.z); a[7] = (short)f32_to_bf16(r.w);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[mt], 0, 0, 0);
        }
      }
    }
  }
  __shared__ v4f red[4][MTM][64];
#pragma unroll
  for (int mt = 0; mt < MTM; ++mt) red[q][mt][l] = acc[mt];
  __syncthreads();
  if (q != 0) return;
#pragma unroll
  for (int mt = 0; mt < MTM; ++mt) {
    if (mt * 16 < M) {
      const v4f sum = ((red[0][mt][l] + red[1][mt][l]) + red[2][mt][l]) + red[3][mt][l];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = mt * 16 + 4 * (l >> 4) + r;
        if (row < M) out[(size_t)row * N + n0 + (l & 15)] = sum[r];
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
  const size_t n4 = (size_t)M * d / 4;
  hipLaunchKernelGGL(bf16_to_f32_kernel, dim3(grid_for(n4)), dim3(256), 0, s, x, n4, h);
  return hip_status(hipGetLastError());
}

int launch_rmsnorm(const float* h, int M, int d, float eps, uint16_t* x, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(M), dim3(256), 0, s, h, d, eps, x);
  return hip_status(hipGetLastError());
}

int launch_residual_add(float* h, const uint16_t* y, int M, int d, hipStream_t s) {
  const size_t n4 = (size_t)M * d / 4;
  hipLaunchKernelGGL(residual_kernel, dim3(grid_for(n4)), dim3(256), 0, s, h, y, n4);
  return hip_status(hipGetLastError());
}

int launch_residual_rmsnorm(float* h, const uint16_t* y, int M, int d, float eps, uint16_t* x, hipStream_t s) {
  hipLaunchKernelGGL(residual_rmsnorm_kernel, dim3(M), dim3(256), 0, s, h, y, d, eps, x);
  return hip_status(hipGetLastError());
}

int launch_head(const float* h, int M, int K, const uint16_t* w, int N, float* out, hipStream_t s) {
  const dim3 grid((unsigned)(N / 16));
  if (M <= 64)
    hipLaunchKernelGGL((head_kernel<4, 4>), grid, dim3(256), 0, s, h, M, K, w, N, out);
  else
    hipLaunchKernelGGL((head_kernel<8, 2>), grid, dim3(256), 0, s, h, M, K, w, N, out);
  return hip_status(hipGetLastError());
}

int launch_argmax(const float* logits, int M, int N, int32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(argmax_kernel, dim3(M), dim3(256), 0, s, logits, N, out);
  return hip_status(hipGetLastError());
}

}  // namespace sgd

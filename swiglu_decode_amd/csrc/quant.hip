// Weight quantize + pack, unpack, and activation quantization kernels.
//
// Block format (128x128 weight tiles, fp32 scale amax/448) and MX format
// (1x32 E8M0 scales along K): fish.audio blog "Cómo hicimos que nuestra API
// de texto a voz sea gratuita…", section "Estrategia de cuantización FP8";
// Fish Audio X post "We Made Our Best Voice Model Free…", section "Custom
// kernels for the shapes TTS actually uses".  The packed layout is the
// library's own (stated in swiglu_decode.h); it is what the streaming GEMM
// reads with two 16-byte loads per lane per 16x128 tile.
#include "sgd_device.hpp"
#include "sgd_host.hpp"

namespace sgd {

// Pack one 16-byte run of 16 codes given as 8 dwords of bf16 pairs already
// converted to code pairs (low byte first).
__device__ __forceinline__ uint4 pack16(const uint32_t (&c)[8]) {
  uint4 r;
  r.x = c[0] | (c[1] << 16);
  r.y = c[2] | (c[3] << 16);
  r.z = c[4] | (c[5] << 16);
  r.w = c[6] | (c[7] << 16);
  return r;
}

// ---------------------------------------------------------------------------
// Block format: one 256-thread workgroup per 128x128 tile (nb, kb).  Thread t
// owns row t/2 of the tile and its 64-column half t%2; that half of the row
// lands in four 16-byte lane slots of one 1024-byte half of a packed tile.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_block_kernel(const uint16_t* __restrict__ w, int K,
                                                         uint8_t* __restrict__ codes,
                                                         float* __restrict__ scales) {
  const int kb = blockIdx.x, nb = blockIdx.y, KT = K >> 7;
  const int t = threadIdx.x, r = t >> 1, half = t & 1;
  const uint4* src = reinterpret_cast<const uint4*>(w + (size_t)(nb * 128 + r) * K + kb * 128 + half * 64);
  uint4 raw[8];
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    raw[i] = src[i];
    const uint32_t d[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      am = fmaxf(am, fabsf(bf16_to_f32(d[e] & 0xFFFFu)));
      am = fmaxf(am, fabsf(bf16_to_f32(d[e] >> 16)));
    }
  }
  __shared__ float red[4];
  am = wave_max(am);
  if ((t & 63) == 0) red[t >> 6] = am;
  __syncthreads();
  const float s = block_scale(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
  uint8_t* tile = codes + ((size_t)(nb * 8 + (r >> 4)) * KT + kb) * 2048 + half * 1024;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t c[8];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t d[4] = {raw[2 * q + i].x, raw[2 * q + i].y, raw[2 * q + i].z, raw[2 * q + i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        c[4 * i + e] = e4m3_encode(bf16_to_f32(d[e] & 0xFFFFu) / s) |
                       (e4m3_encode(bf16_to_f32(d[e] >> 16) / s) << 8);
    }
    *reinterpret_cast<uint4*>(tile + ((r & 15) + 16 * q) * 16) = pack16(c);
  }
  if (t == 0) scales[nb * KT + kb] = s;
}

// ---------------------------------------------------------------------------
// MX format: one wavefront per (16-row band j, k-tile t), t running over the
// padded range [0, 4*ceil(KT/4)).  Lane l = r + 16b owns row r of the band
// and 32-column block b of the tile, which is exactly the scale slot lane l
// feeds to the matrix instruction.  Its 32 codes go to lane slots r+16(2(b%2))
// and r+16(2(b%2)+1) of tile half b/2.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_mx_kernel(const uint16_t* __restrict__ w, int N, int K,
                                                      uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales) {
  const int KT = K >> 7, KG = (KT + 3) >> 2, TT = 4 * KG;
  const int wid = (int)((blockIdx.x * 256u + threadIdx.x) >> 6);
  const int l = threadIdx.x & 63;
  if (wid >= (N >> 4) * TT) return;
  const int j = wid / TT, t = wid % TT;
  const int r = l & 15, b = l >> 4;
  uint8_t* sp = scales + ((size_t)(j * KG + (t >> 2)) * 64 + l) * 4 + (t & 3);
  if (t >= KT) {  // padding slot of the last k-tile group
    *sp = 0;
    return;
  }
  const uint4* src = reinterpret_cast<const uint4*>(w + (size_t)(j * 16 + r) * K + t * 128 + b * 32);
  uint4 raw[4];
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    raw[i] = src[i];
    const uint32_t d[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      am = fmaxf(am, fabsf(bf16_to_f32(d[e] & 0xFFFFu)));
      am = fmaxf(am, fabsf(bf16_to_f32(d[e] >> 16)));
    }
  }
  const int X = mx_exponent(am);
  *sp = (uint8_t)(X + 127);
  const float m = pow2_neg(X);
  uint8_t* tile = codes + ((size_t)j * KT + t) * 2048 + (b >> 1) * 1024;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    uint32_t c[8];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 v = raw[2 * hh + i];
      const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        c[4 * i + e] = e4m3_encode(bf16_to_f32(d[e] & 0xFFFFu) * m) |
                       (e4m3_encode(bf16_to_f32(d[e] >> 16) * m) << 8);
    }
    *reinterpret_cast<uint4*>(tile + (r + 16 * (2 * (b & 1) + hh)) * 16) = pack16(c);
  }
}

// ---------------------------------------------------------------------------
// Unpack: one wavefront per packed tile (j, t); lane l moves its two 16-byte
// runs back to row 16j + l%16, columns 128t + 16(l/16) and +64.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void unpack_kernel(int fmt, const uint8_t* __restrict__ codes,
                                                     const void* __restrict__ scales, int N, int K,
                                                     uint8_t* __restrict__ out,
                                                     void* __restrict__ out_scales) {
  const int KT = K >> 7, KG = (KT + 3) >> 2;
  const int wid = (int)((blockIdx.x * 256u + threadIdx.x) >> 6);
  const int l = threadIdx.x & 63;
  if (wid >= (N >> 4) * KT) return;
  const int j = wid / KT, t = wid % KT;
  const uint8_t* tile = codes + (size_t)wid * 2048;
  const int row = j * 16 + (l & 15), q = l >> 4;
  uint8_t* dst = out + (size_t)row * K + t * 128 + 16 * q;
  *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(tile + l * 16);
  *reinterpret_cast<uint4*>(dst + 64) = *reinterpret_cast<const uint4*>(tile + 1024 + l * 16);
  if (fmt == FMT_MX) {
    const uint8_t* s = static_cast<const uint8_t*>(scales);
    static_cast<uint8_t*>(out_scales)[(size_t)row * (K >> 5) + 4 * t + q] =
        s[((size_t)(j * KG + (t >> 2)) * 64 + l) * 4 + (t & 3)];
  } else if ((j & 7) == 0 && l == 0) {
    const float* s = static_cast<const float*>(scales);
    static_cast<float*>(out_scales)[(j >> 3) * KT + t] = s[(j >> 3) * KT + t];
  }
}

// ---------------------------------------------------------------------------
// Activation quantization (logical output layout): one wavefront per
// (row, 128-column group); lane l handles columns 2l and 2l+1.
// ---------------------------------------------------------------------------
template <int FMT>
__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                        uint8_t* __restrict__ codes,
                                                        void* __restrict__ scales) {
  const int KG = K >> 7;
  const int wid = (int)((blockIdx.x * 256u + threadIdx.x) >> 6);
  const int l = threadIdx.x & 63;
  if (wid >= M * KG) return;
  const int row = wid / KG, g = wid % KG;
  const size_t off = (size_t)row * K + g * 128 + 2 * l;
  const uint32_t pr = *reinterpret_cast<const uint32_t*>(x + off);
  float sf;
  uint32_t se;
  const uint32_t c = quant_pair<FMT>(bf16_to_f32(pr & 0xFFFFu), bf16_to_f32(pr >> 16), &sf, &se);
  *reinterpret_cast<uint16_t*>(codes + off) = (uint16_t)c;
  if (FMT == FMT_BLOCK) {
    if (l == 0) static_cast<float*>(scales)[(size_t)row * KG + g] = sf;
  } else if ((l & 15) == 0) {
    static_cast<uint8_t*>(scales)[(size_t)row * (K >> 5) + 4 * g + (l >> 4)] = (uint8_t)se;
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* p, size_t n) {
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n; i += (size_t)gridDim.x * 256ull)
    p[i] = make_uint4(0, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static inline unsigned blocks_for_waves(size_t waves) { return (unsigned)((waves + 3) / 4); }

int launch_pack_weight(int fmt, const uint16_t* w, int N, int K, void* codes, void* scales,
                       hipStream_t s) {
  if (fmt == FMT_BLOCK) {
    hipLaunchKernelGGL(pack_block_kernel, dim3(K / 128, N / 128), dim3(256), 0, s, w, K,
                       static_cast<uint8_t*>(codes), static_cast<float*>(scales));
  } else {
    const int KG = (K / 128 + 3) / 4;
    hipLaunchKernelGGL(pack_mx_kernel, dim3(blocks_for_waves((size_t)(N / 16) * 4 * KG)), dim3(256),
                       0, s, w, N, K, static_cast<uint8_t*>(codes), static_cast<uint8_t*>(scales));
  }
  return hip_status(hipGetLastError());
}

int launch_unpack_weight(int fmt, const uint8_t* codes, const void* scales, int N, int K,
                         uint8_t* out_codes, void* out_scales, hipStream_t s) {
  hipLaunchKernelGGL(unpack_kernel, dim3(blocks_for_waves((size_t)(N / 16) * (K / 128))), dim3(256),
                     0, s, fmt, codes, scales, N, K, out_codes, out_scales);
  return hip_status(hipGetLastError());
}

int launch_quantize_act(int fmt, const uint16_t* x, int M, int K, uint8_t* codes, void* scales,
                        hipStream_t s) {
  const dim3 grid(blocks_for_waves((size_t)M * (K / 128)));
  if (fmt == FMT_BLOCK)
    hipLaunchKernelGGL(quant_act_kernel<FMT_BLOCK>, grid, dim3(256), 0, s, x, M, K, codes, scales);
  else
    hipLaunchKernelGGL(quant_act_kernel<FMT_MX>, grid, dim3(256), 0, s, x, M, K, codes, scales);
  return hip_status(hipGetLastError());
}

int launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 16;
  if (n == 0) return SGD_OK;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<uint4*>(p), n);
  return hip_status(hipGetLastError());
}

}  // namespace sgd

// The activations' fp8 workspace layout and the in-kernel quantizer of a
// 32-element block, shared by the persistent streaming kernel and the tiled
// large-M GEMM.
#pragma once

#include "sgd_device.hpp"

namespace sgd {

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ---------------------------------------------------------------------------
// Layout of the fp8 activations the kernels write to the workspace (Q(x) and
// Q(a), M rows of K codes): m-tile by m-tile.  m-tile t holds rows
// 16t..16t+Mt-1 (Mt = min(16, M - 16t)) as K/16 segments of 16 columns, each
// segment the Mt rows' 16 codes in row order.  The 16 rows x 16 columns one
// quarter-wavefront of an operand load needs are then 256 contiguous bytes,
// and one load instruction of a whole wavefront reads 1 KB in one piece
// (row-major rows K bytes apart would put the 16 rows of every load on 16
// different cache lines, all in the same L2 channel when K is a multiple of
// 4 KB).  A 128-column group of an m-tile is 128*Mt contiguous bytes.
// MX scales alike: m-tile t holds, per 128-column k-tile, the Mt rows' four
// E8M0 bytes (one dword per row).
__device__ __forceinline__ uint32_t act_tile_rows(int M, int row) { return (uint32_t)min(16, M - (row & ~15)); }
__device__ __forceinline__ uint32_t act_code_off(int M, int K, int row, int col) {
  return (uint32_t)(row & ~15) * (uint32_t)K + (uint32_t)(col >> 4) * 16u * act_tile_rows(M, row) +
         (uint32_t)(row & 15) * 16u + (uint32_t)(col & 15);
}
__device__ __forceinline__ uint32_t act_scale_off(int M, int K, int row, int kt) {
  return (uint32_t)(row & ~15) * (uint32_t)(K >> 5) + (uint32_t)kt * 4u * act_tile_rows(M, row) +
         (uint32_t)(row & 15) * 4u;
}

// Quantize one 32-element block held by one lane (one row, 32 consecutive
// columns): the 32 E4M3 codes in element order (8 dwords) and the block's
// scale.  Block format: the scale covers a 128-column group, whose 4 blocks
// sit in 4 consecutive lanes that are all active (amax over the group);
// returned in *sf.  MX: the E8M0 byte of this block, in *se.  E4M3
// conversion in hardware after clamping to +-448 (round to nearest even,
// checked against the integer encoder over 6.8e8 fp32 patterns on gfx950).
template <int FMT>
__device__ __forceinline__ void quant_block32(const float (&v)[32], uint32_t (&cw)[8], float* sf, uint32_t* se) {
  float am = 0.0f;
#pragma unroll
  for (int e = 0; e < 32; ++e) am = fmaxf(am, fabsf(v[e]));
  float mul = 1.0f, s = 1.0f;
  if (FMT == FMT_BLOCK) {
    am = fmaxf(am, __shfl_xor(am, 1, WAVE));
    am = fmaxf(am, __shfl_xor(am, 2, WAVE));
    s = block_scale(am);
  } else {
    const int X = mx_exponent(am);
    mul = pow2_neg(X);
    *se = (uint32_t)(X + 127);
  }
  *sf = s;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float q[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float t = FMT == FMT_BLOCK ? v[4 * c + e] / s : v[4 * c + e] * mul;
      q[e] = __builtin_amdgcn_fmed3f(t, -E4M3_MAX, E4M3_MAX);
    }
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w, true);
    cw[c] = (uint32_t)w;
  }
}

// The four E8M0 bytes of the lanes 4q..4q+3 packed into one word (lane 4q's
// byte lowest), valid in every lane of the four.
__device__ __forceinline__ uint32_t pack4_lanes(uint32_t e) {
  const int base = lane_id() & ~3;
  return __shfl(e, base, WAVE) | (__shfl(e, base + 1, WAVE) << 8) | (__shfl(e, base + 2, WAVE) << 16) |
         (__shfl(e, base + 3, WAVE) << 24);
}

// SiLU(g) * u in fp32 (the MLP's gate nonlinearity times the up projection).
__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

}  // namespace sgd

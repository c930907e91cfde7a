// Device-side helpers shared by the gfx950 kernels: bf16 / E4M3 / E8M0
// conversions, wavefront reductions, the 128-element group quantizer and
// the scaled fp8 MFMA wrapper.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgd {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

enum : int { FMT_BLOCK = 1, FMT_MX = 2 };

constexpr int WAVE = 64;
constexpr float E4M3_MAX = 448.0f;

// ---------------------------------------------------------------------------
// bf16
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round-to-nearest-even fp32 -> bf16 bits (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------
// E4M3 (OCP OFP8): round to nearest, ties to even, saturate at +-448.
// Integer formulation on the fp32 bit pattern: for |v| >= 2^-6 keep the top
// 3 mantissa bits with round-half-even on the 20 dropped bits (a carry moves
// into the exponent by itself) and rebias the exponent from 127 to 7; below
// 2^-6 the codes are the integers round(|v| * 2^9) of the subnormal grid.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;  // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu; // |v| >= 448 (and inf): saturate
  if (a >= 0x3C800000u) {                    // |v| >= 2^-6: normal code
    uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    return sign | ((r >> 20) - ((127u - 7u) << 3));
  }
  float f = __uint_as_float(a) * 512.0f;     // exact: scaling by 2^9
  return sign | (uint32_t)__builtin_rintf(f);
}

// ---------------------------------------------------------------------------
// Scale rules
// ---------------------------------------------------------------------------
// 128x128 / 1x128 block scale: fl32(amax / 448), 1 for an all-zero group.
// hipcc's default fp32 division is correctly rounded (IEEE).
__device__ __forceinline__ float block_scale(float amax) {
  return amax == 0.0f ? 1.0f : amax / E4M3_MAX;
}

// MX (OCP MX v1.0) shared exponent X = floor(log2(amax)) - 8, clamped to
// [-127, 127]; -127 for amax == 0.  floor(log2) comes from the exponent
// field (subnormals: from the position of the leading mantissa bit).
__device__ __forceinline__ int mx_exponent(float amax) {
  uint32_t b = __float_as_uint(amax) & 0x7FFFFFFFu;
  if (b == 0) return -127;
  int e = (int)(b >> 23);
  int fl = e ? e - 127 : (31 - __clz((int)b)) - 149;
  int X = fl - 8;
  return X < -127 ? -127 : (X > 127 ? 127 : X);
}

// 2^-X as an fp32 value, for X in [-127, 119] (exponent field 127 - X).
__device__ __forceinline__ float pow2_neg(int X) { return __uint_as_float((uint32_t)(127 - X) << 23); }

// 2^X as an fp32 value for X in [-126, 127]; 2^-127 (the E8M0 byte 0) is the
// fp32 subnormal 0x00400000.
__device__ __forceinline__ float pow2_pos(int X) {
  return X >= -126 ? __uint_as_float((uint32_t)(X + 127) << 23) : __uint_as_float(0x00400000u);
}

// Value of an E4M3 code (finite codes; the NaN codes are never produced).
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (c & 0x80u) ? -mag : mag;
}

// ---------------------------------------------------------------------------
// Wavefront reductions (wave64)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}
// max over aligned groups of 16 lanes
__device__ __forceinline__ float seg16_max(float v) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}

// ---------------------------------------------------------------------------
// Quantize one 128-element group of a row with one wavefront: lane l holds
// elements 2l and 2l+1.  BLOCK: one fp32 scale for the whole group.
// MX: lanes 16b..16b+15 form 32-element block b (b = 0..3), one E8M0 byte
// each.  Returns the two codes packed in the low 16 bits (element 2l in the
// low byte).  *scale_f (BLOCK) / *scale_e (MX, this lane's block) are set.
// ---------------------------------------------------------------------------
template <int FMT>
__device__ __forceinline__ uint32_t quant_pair(float v0, float v1, float* scale_f, uint32_t* scale_e) {
  float am = fmaxf(fabsf(v0), fabsf(v1));
  if (FMT == FMT_BLOCK) {
    float s = block_scale(wave_max(am));
    *scale_f = s;
    return e4m3_encode(v0 / s) | (e4m3_encode(v1 / s) << 8);
  } else {
    int X = mx_exponent(seg16_max(am));
    *scale_e = (uint32_t)(X + 127);
    float m = pow2_neg(X);
    return e4m3_encode(v0 * m) | (e4m3_encode(v1 * m) << 8);
  }
}

// ---------------------------------------------------------------------------
// Scaled fp8 MFMA 16x16x128.  Operand order (measured on gfx950): lane l
// holds row/column l % 16 with K = 16*(l/16)+[0,16) in bytes 0..15 and
// K = 64+16*(l/16)+[0,16) in bytes 16..31; the E8M0 scale of lane l applies
// to row/column l % 16, 32-wide K block l / 16.  D: lane l holds column
// l % 16, rows 4*(l/16)+r in element r.
// ---------------------------------------------------------------------------
__device__ __forceinline__ v4f mfma_f8(v8i a, v8i b, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ v8i make_v8i(uint4 lo, uint4 hi) {
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

// ---------------------------------------------------------------------------
// Cross-workgroup communication.
//
// L2 is per XCD and not coherent across XCDs; the agent-scope fences of the
// language memory model write back / invalidate a whole L2 each, which costs
// far too much when issued per work item.  Instead:
//  * every intermediate another workgroup reads is written with agent-
//    coherent (sc1, write-through) stores, and a producer waits for all its
//    stores to complete (s_waitcnt vmcnt(0)) before it arrives on a counter
//    or raises a flag with an atomic;
//  * small per-group data (scales, fp32 partial sums, the SwiGLU output) is
//    read back with agent-coherent (sc1) loads;
//  * the large activation operands are read with ordinary cached loads: each
//    such region is written once per launch, read only after its flag, and
//    laid out so that no 128-byte line straddles two groups, so no cache can
//    hold a stale copy of it (caches are invalidated at kernel boundaries).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void st_coherent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_coherent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ uint64_t ld_coherent(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory operation this wavefront issued has completed.
__device__ __forceinline__ void drain_memory() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Spin (whole wavefront) until *p >= target.  The signal fence keeps the
// compiler from moving later loads above the poll; the hardware issues them
// only after the poll's value has been compared.
__device__ __forceinline__ void wait_geq(const uint32_t* p, uint32_t target) {
  while (load_agent(p) < target) __builtin_amdgcn_s_sleep(4);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Buffer resource over [base, base + bytes); loads through it with the sc1
// cache policy are agent-coherent, and offsets past `bytes` read as zero.
constexpr int AUX_SC1 = 16;
// Cache-policy bit of a non-temporal (streaming) access.
constexpr int AUX_NT = 2;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ v4f ld_coherent_v4f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX_SC1));
}
typedef unsigned v4u __attribute__((ext_vector_type(4)));
// 16-byte agent-coherent (write-through) store through a buffer resource.
__device__ __forceinline__ void st_coherent_b128(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 v) {
  const v4u d = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(d, r, off, 0, AUX_SC1);
}
__device__ __forceinline__ uint32_t ld_coherent_u8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, AUX_SC1);
}
__device__ __forceinline__ uint32_t ld_coherent_u32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX_SC1);
}

// ---------------------------------------------------------------------------
// Copies from memory straight into LDS (no register receives data).  Written
// as the instructions themselves so that the compiler does not wait for them
// before unrelated work; a kernel that uses them waits for its copies itself
// (lds_copies_left: loads complete in issue order).
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) uint8_t lds_u8;
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_u8*)p;
}
// 1 KB: lane l's 16 bytes at buffer offset voff land at LDS byte m0 + 16*l.
__device__ __forceinline__ void lds_copy1k(__amdgpu_buffer_rsrc_t r, uint32_t m0, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(r) : "memory", "m0");
}
// 256 bytes: lane l's dword at buffer offset voff lands at LDS byte m0 + 4*l.
__device__ __forceinline__ void lds_copy256(__amdgpu_buffer_rsrc_t r, uint32_t m0, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(r) : "memory", "m0");
}
// As lds_copy256, agent-coherent (sc1): for small data other workgroups wrote.
__device__ __forceinline__ void lds_copy256_sc1(__amdgpu_buffer_rsrc_t r, uint32_t m0, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen sc1 lds" ::"s"(m0), "v"(voff), "s"(r) : "memory", "m0");
}
// Wait until at most N of this wavefront's memory loads are in flight.
template <int N>
__device__ __forceinline__ void lds_copies_left() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace sgd

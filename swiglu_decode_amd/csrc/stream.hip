// The weight-streaming scaled-FP8 GEMM and the single-launch fused SwiGLU MLP.
//
// What is computed (Fish Audio X post "We Made Our Best Voice Model Free…",
// section "Custom kernels for the shapes TTS actually uses"; fish.audio blog
// "Cómo hicimos que nuestra API de texto a voz sea gratuita…", sections
// "Resultados de benchmark del kernel" and "Qué hay en código abierto"):
//   scaled GEMM:  y = Q(x) W^T
//   fused MLP:    y = Q( silu(Q(x) Wg^T) * (Q(x) Wu^T) ) Wd^T
// with Q the per-row activation quantizer of the weights' format (1x128 fp32
// groups against 128x128 fp32 weight tiles, or 1x32 E8M0 on both operands),
// fp32 accumulation and a bf16 result.
//
// How (gfx950 design).  At decode shapes (M <= 128) every weight byte is used
// by at most 128 rows, so the work is a stream of HBM weight bytes into the
// 16x16x128 scaled fp8 MFMA.  One persistent kernel walks a queue of work
// items taken in ticket order:
//   XQ  items  quantize x into the workspace (rows padded to 16 with zeros);
//   GU  items  (MLP only) one 16-column slice of ffn: gate and up tiles over
//              all of d, split over the 4 wavefronts of the workgroup, reduced
//              in LDS, a = silu(g) * u written as fp32; the last of the 8 items
//              of a 128-column group re-quantizes that group and raises its
//              ready flag;
//   DN  items  32 output columns x one K chunk of the second GEMM (down
//              projection, or the plain GEMM's weight), split over the
//              wavefronts; chunks of one column tile are summed in a fixed
//              order by the last chunk to finish, then rounded to bf16.
// Each wavefront keeps a ring of P k-tiles of weights (two 16-byte loads per
// lane per 16x128 tile, fully coalesced) in flight.  Weight loads of an item
// are issued before its dependency wait, so HBM stays busy while a consumer
// waits for its producer.  Items depend only on items with smaller tickets,
// tickets are handed out in order, and a workgroup only ever waits on items
// already taken by running workgroups, so the queue cannot deadlock.  The
// last workgroup to leave resets every counter, so the next call (or graph
// replay) starts from a zeroed control block.
#include "sgd_device.hpp"
#include "sgd_host.hpp"

#include <mutex>

namespace sgd {

constexpr int NW = 4;       // wavefronts per workgroup
constexpr int NTD = 2;      // 16-row weight tiles per DN item
constexpr int XQ_GPI = 32;  // 128-wide groups per XQ item

struct StreamArgs {
  int M, Mpad, mlp;
  const uint16_t* x;
  int K1;                    // columns of x
  const uint8_t* wg;         // gate / up packed codes [F, K1] (MLP)
  const void* sg;
  const uint8_t* wu;
  const void* su;
  int F;
  const uint8_t* w2;         // second GEMM weight [N, K2]
  const void* s2;
  int N, K2;
  uint16_t* y;               // [M, N]
  uint32_t* ctrl;
  uint8_t* xq;               // [Mpad, K1] fp8 codes (plain GEMM)
  uint16_t* xb;              // [Mpad, K1] bf16 widened quantized x (MLP; MX scale folded in)
  void* xs;                  // block: fp32 [K1/128][Mpad]; mx: u8 [Mpad][K1/32]
  float* a32;                // [M, F]
  uint8_t* aq;               // [Mpad, F]
  void* as;                  // block: fp32 [F/128][Mpad]; mx: u8 [Mpad][F/32]
  float* ypart;              // [n_kc, M, N]
  int n_xq, n_gu, n_dt, n_kc, ktc, total;
  int off_grp, off_ready, off_ycnt;
};

// Wavefront index within the workgroup, as a scalar (uniform) value so that
// branches on it are scalar branches.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Per-workgroup LDS state: the ticket broadcast, a flag broadcast, and what
// this workgroup has already seen of its producers (so a consumer whose
// inputs are known to be ready enters the pipeline without a global poll).
struct WgState {
  uint32_t ticket, flag;
  uint32_t xq_seen;          // x quantization complete
  uint32_t grp_seen[8];      // bit g: ffn group g re-quantized (ffn <= 32768)
};

__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// Control block layout (uint32 words).
constexpr int C_TICKET = 0, C_DONE = 1, C_XQ = 2, C_HDR = 16;

// ---------------------------------------------------------------------------
// The per-wavefront streaming loop.
//   acc[nb][mt] += sum over k-tiles kt0..kt0+nk-1 of A(mt, kt) x B(nb, kt)^T
// B(nb, kt): the packed tile at bt[nb] + k*2048 (k = kt - kt0).
// A(mt, kt): rows 16mt..16mt+15 of a row-major [Mpad, Kd] code matrix.
// ---------------------------------------------------------------------------
template <int MT, int NB, int FMT, int P>
struct Streamer {
  const uint8_t* bt[NB];     // packed tile (nb, kt0), lane offset included
  const uint8_t* bshared[NB];  // same tile without the lane offset (filler loads)
  const uint8_t* ashared;    // row 0 of the A matrix at kt0 (filler loads)
  const float* bsf[NB];      // block: weight-scale row of tile band nb, indexed by kt
  const uint32_t* bsm[NB];   // mx: packed scale dwords of n-tile nb for this lane, + (kt/4)*64
  const uint8_t* arow;       // A: lane's row (l%16) in m-tile 0, + 16*(l/16)
  size_t a_mt_stride;        // 16 * Kd
  __amdgpu_buffer_rsrc_t asr; // activation scales (agent-coherent loads)
  uint32_t as_off;           // lane's byte offset in it (block: 16*(l/16); mx: row*(Kd/32) + l/16)
  uint32_t as_kt_stride;     // block: 4*Mpad; mx: 4
  uint32_t as_mt_stride;     // block: 64; mx: 16*Kd/32
  int kt0, nk;

  v8i B[P][NB];
  v8i A[P][MT];
  float SWb[P][NB];
  v4f SXb[P][MT];
  uint32_t SWm[P][NB];
  uint32_t SXm[P][MT];

  __device__ __forceinline__ void load_b(int slot_unused, int k, v8i (&b)[NB], float (&swb)[NB],
                                         uint32_t (&swm)[NB]) {
    (void)slot_unused;
    const bool ok = k < nk;
    const int kt = kt0 + (ok ? k : 0);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint8_t* p = ok ? bt[nb] + (size_t)k * 2048 : bshared[nb];
      b[nb] = make_v8i(*reinterpret_cast<const uint4*>(p), *reinterpret_cast<const uint4*>(p + 1024));
      if (FMT == FMT_BLOCK)
        swb[nb] = bsf[nb][kt];
      else
        swm[nb] = bsm[nb][(kt >> 2) * 64];  // byte kt % 4 is selected at use
    }
  }
  __device__ __forceinline__ void load_a(int k, v8i (&a)[MT], v4f (&sxb)[MT], uint32_t (&sxm)[MT]) {
    const bool ok = k < nk;
    const int kt = kt0 + (ok ? k : 0);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint8_t* p = ok ? arow + mt * a_mt_stride + (size_t)kt * 128 : ashared;
      a[mt] = make_v8i(*reinterpret_cast<const uint4*>(p), *reinterpret_cast<const uint4*>(p + 64));
      const uint32_t so = as_off + (uint32_t)kt * as_kt_stride + (uint32_t)mt * as_mt_stride;
      if (FMT == FMT_BLOCK)
        sxb[mt] = ld_coherent_v4f(asr, so);
      else
        sxm[mt] = ld_coherent_u8(asr, so);
    }
  }

  // Software pipeline over the wavefront's k-tiles.  The steady-state loop
  // consumes slot s and refills it with the tile P steps ahead; every load in
  // it is unconditional (past the last tile a slot is refilled from an
  // address all lanes share, one cache line), so the hardware load counter
  // sees the same pattern on every iteration and each consumer waits only
  // for its own slot.  The prologue either issues the ring in that same
  // order (dependency already known satisfied: `ready()` reads LDS only) or
  // issues the weight loads, waits for the producer, loads the activations
  // and drains, so the loop is entered either in the steady-state pattern or
  // with nothing in flight.
  template <class Ready, class Wait>
  __device__ __forceinline__ void run(v4f (&acc)[NB][MT], Ready ready, Wait wait) {
    if (nk <= 0) return;
    if (ready()) {
#pragma unroll
      for (int s = 0; s < P; ++s) {
        load_b(s, s, B[s], SWb[s], SWm[s]);
        load_a(s, A[s], SXb[s], SXm[s]);
      }
    } else {
#pragma unroll
      for (int s = 0; s < P; ++s) load_b(s, s, B[s], SWb[s], SWm[s]);
      wait();
#pragma unroll
      for (int s = 0; s < P; ++s) load_a(s, A[s], SXb[s], SXm[s]);
      __builtin_amdgcn_s_waitcnt(0);
    }
    int base = 0;
    for (; base + P <= nk; base += P) {
#pragma unroll
      for (int s = 0; s < P; ++s) {
        step(s, base + s, acc);
        load_b(s, base + s + P, B[s], SWb[s], SWm[s]);
        load_a(base + s + P, A[s], SXb[s], SXm[s]);
      }
    }
#pragma unroll
    for (int s = 0; s < P; ++s)
      if (base + s < nk) step(s, base + s, acc);
  }

  __device__ __forceinline__ void step(int s, int k, v4f (&acc)[NB][MT]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (FMT == FMT_BLOCK) {
          const v4f z = {0.f, 0.f, 0.f, 0.f};
          const v4f t = mfma_f8(A[s][mt], B[s][nb], z, 127, 127);
          acc[nb][mt] += t * (SXb[s][mt] * SWb[s][nb]);
        } else {
          const int sw = (int)(SWm[s][nb] >> (8 * ((kt0 + k) & 3)));
          acc[nb][mt] = mfma_f8(A[s][mt], B[s][nb], acc[nb][mt], (int)SXm[s][mt], sw);
        }
      }
    }
  }
};

template <int MT>
struct Depth { static constexpr int P = MT <= 2 ? 4 : 2; };

// ---------------------------------------------------------------------------
// The gate/up variant of the streaming loop.  The fp8 matrix instruction sums
// its products in groups of 8 with only ~13 bits kept below the largest
// product of a group (measured on gfx950), a ~1e-5 relative error that is
// harmless in a final output but flips fp8 codes when the result is
// re-quantized.  So the gate/up GEMM widens its fp8 operands to bf16 (exact:
// E4M3 values fit in bf16; for MX the power-of-two scale is folded in, also
// exactly) and runs the bf16 16x16x32 instruction, whose sums are fp32
// accurate.  Weights arrive packed exactly as for the fp8 path; activations
// come pre-widened (xb).  Operand order: value i of the lane's 32-byte run
// goes to element i%8 of instruction i/8, for both operands.
// ---------------------------------------------------------------------------
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v8bf widen8(uint32_t d0, uint32_t d1, float scale) {
  const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, scale, false);
  const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, scale, true);
  const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, scale, false);
  const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, scale, true);
  v8bf r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ v8bf as_v8bf(uint4 u) { return __builtin_bit_cast(v8bf, u); }

template <int MT, int NB, int FMT, int P>
struct StreamerBf16 {
  const uint8_t* bt[NB];       // packed tile (nb, kt0), lane offset included
  const uint8_t* bshared[NB];  // same tile without the lane offset (filler loads)
  const float* bsf[NB];        // block: weight-scale row of tile band nb, indexed by kt
  const uint32_t* bsm0[NB];    // mx: scale dwords of (row, block q/2), + (kt/4)*64
  const uint32_t* bsm1[NB];    // mx: scale dwords of (row, block 2+q/2)
  const uint16_t* arow;        // A: lane's row in m-tile 0 of xb, + 16*(l/16)
  const uint16_t* ashared;     // row 0 of xb (filler loads)
  size_t a_mt_stride;          // 16 * Kd (elements)
  const float* asf;            // block: act scales + 4*(l/16), indexed kt*Mpad + 16*mt
  int Mpad;
  int kt0, nk;

  v8i B[P][NB];
  uint4 A[P][MT][4];
  float SWb[P][NB];
  v4f SXb[P][MT];
  uint32_t SW0[P][NB], SW1[P][NB];

  __device__ __forceinline__ void load_b(int k, v8i (&b)[NB], float (&swb)[NB], uint32_t (&sw0)[NB],
                                         uint32_t (&sw1)[NB]) {
    const bool ok = k < nk;
    const int kt = kt0 + (ok ? k : 0);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint8_t* p = ok ? bt[nb] + (size_t)k * 2048 : bshared[nb];
      b[nb] = make_v8i(*reinterpret_cast<const uint4*>(p), *reinterpret_cast<const uint4*>(p + 1024));
      if (FMT == FMT_BLOCK) {
        swb[nb] = bsf[nb][kt];
      } else {
        sw0[nb] = bsm0[nb][(kt >> 2) * 64];
        sw1[nb] = bsm1[nb][(kt >> 2) * 64];
      }
    }
  }
  __device__ __forceinline__ void load_a(int k, uint4 (&a)[MT][4], v4f (&sxb)[MT]) {
    const bool ok = k < nk;
    const int kt = kt0 + (ok ? k : 0);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint16_t* p = ok ? arow + mt * a_mt_stride + (size_t)kt * 128 : ashared;
      const uint4* q = reinterpret_cast<const uint4*>(p);
      a[mt][0] = q[0];
      a[mt][1] = q[1];
      a[mt][2] = q[8];   // + 64 elements
      a[mt][3] = q[9];
      if (FMT == FMT_BLOCK) sxb[mt] = *reinterpret_cast<const v4f*>(asf + (size_t)kt * Mpad + 16 * mt);
    }
  }

  __device__ __forceinline__ void step(int s, int k, v4f (&acc)[NB][MT]) {
    const int sh = 8 * ((kt0 + k) & 3);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float s0 = 1.0f, s1 = 1.0f;
      if (FMT == FMT_MX) {
        s0 = pow2_pos((int)((SW0[s][nb] >> sh) & 0xFFu) - 127);
        s1 = pow2_pos((int)((SW1[s][nb] >> sh) & 0xFFu) - 127);
      }
      v8bf b[4];
      b[0] = widen8((uint32_t)B[s][nb][0], (uint32_t)B[s][nb][1], s0);
      b[1] = widen8((uint32_t)B[s][nb][2], (uint32_t)B[s][nb][3], s0);
      b[2] = widen8((uint32_t)B[s][nb][4], (uint32_t)B[s][nb][5], s1);
      b[3] = widen8((uint32_t)B[s][nb][6], (uint32_t)B[s][nb][7], s1);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (FMT == FMT_BLOCK) {
          v4f t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < 4; ++i) t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(A[s][mt][i]), b[i], t, 0, 0, 0);
          acc[nb][mt] += t * (SXb[s][mt] * SWb[s][nb]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[nb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(A[s][mt][i]), b[i], acc[nb][mt], 0, 0, 0);
        }
      }
    }
  }

  // Same pipeline discipline as Streamer::run.
  template <class Ready, class Wait>
  __device__ __forceinline__ void run(v4f (&acc)[NB][MT], Ready ready, Wait wait) {
    if (nk <= 0) return;
    if (ready()) {
#pragma unroll
      for (int s = 0; s < P; ++s) {
        load_b(s, B[s], SWb[s], SW0[s], SW1[s]);
        load_a(s, A[s], SXb[s]);
      }
    } else {
#pragma unroll
      for (int s = 0; s < P; ++s) load_b(s, B[s], SWb[s], SW0[s], SW1[s]);
      wait();
#pragma unroll
      for (int s = 0; s < P; ++s) load_a(s, A[s], SXb[s]);
      __builtin_amdgcn_s_waitcnt(0);
    }
    int base = 0;
    for (; base + P <= nk; base += P) {
#pragma unroll
      for (int s = 0; s < P; ++s) {
        step(s, base + s, acc);
        load_b(base + s + P, B[s], SWb[s], SW0[s], SW1[s]);
        load_a(base + s + P, A[s], SXb[s]);
      }
    }
#pragma unroll
    for (int s = 0; s < P; ++s)
      if (base + s < nk) step(s, base + s, acc);
  }
};

template <int MT>
struct DepthBf16 { static constexpr int P = MT <= 1 ? 3 : (MT <= 2 ? 2 : 1); };

// ---------------------------------------------------------------------------
// XQ item: quantize 128-wide groups [i*XQ_GPI, ...) of the padded x.
// ---------------------------------------------------------------------------
// Store one quantized 128-column group of one row with agent-coherent 32-bit
// stores: codes (lane l holds elements 2l, 2l+1; even lanes write four) and
// the group's scale(s) (block: one fp32 in [K/128][Mpad]; MX: four E8M0
// bytes, one per 32-column block, as one word of [Mpad][K/32]).
template <int FMT>
__device__ __forceinline__ void store_group(uint8_t* codes_at_group, uint32_t c, float sf, uint32_t se,
                                            float* sbl_at, uint8_t* smx_at) {
  const int l = threadIdx.x & 63;
  const uint32_t up = __shfl_down(c, 1, WAVE);
  if ((l & 1) == 0) st_coherent(reinterpret_cast<uint32_t*>(codes_at_group + 2 * l), (c & 0xFFFFu) | (up << 16));
  if (FMT == FMT_BLOCK) {
    if (l == 0) st_coherent(sbl_at, sf);
  } else {
    const uint32_t e1 = __shfl(se, 16, WAVE), e2 = __shfl(se, 32, WAVE), e3 = __shfl(se, 48, WAVE);
    if (l == 0) st_coherent(reinterpret_cast<uint32_t*>(smx_at), se | (e1 << 8) | (e2 << 16) | (e3 << 24));
  }
}

// ---------------------------------------------------------------------------
// XQ item: quantize 128-wide groups [i*XQ_GPI, ...) of the padded x.
// ---------------------------------------------------------------------------
template <int FMT>
__device__ void item_xq(const StreamArgs& a, int i) {
  const int w = wave_id(), l = threadIdx.x & 63;
  const int KG = a.K1 >> 7;
  const int G = a.Mpad * KG;
  const int g0 = i * XQ_GPI, g1 = min(G, g0 + XQ_GPI);
  for (int g = g0 + w; g < g1; g += NW) {
    const int row = g / KG, kg = g % KG;
    const size_t off = (size_t)row * a.K1 + kg * 128 + 2 * l;
    uint32_t c = 0, se = 0;
    float sf = 1.0f;
    if (row < a.M) {
      const uint32_t pr = *reinterpret_cast<const uint32_t*>(a.x + off);
      c = quant_pair<FMT>(bf16_to_f32(pr & 0xFFFFu), bf16_to_f32(pr >> 16), &sf, &se);
    }
    float* sbl = static_cast<float*>(a.xs) + (size_t)kg * a.Mpad + row;
    uint8_t* smx = static_cast<uint8_t*>(a.xs) + (size_t)row * (a.K1 >> 5) + 4 * kg;
    if (a.mlp) {
      // exact bf16 of the dequantized value (block: code value, its fp32
      // group scale applied after the MFMA; MX: code value times 2^X)
      const float m = FMT == FMT_BLOCK ? 1.0f : pow2_pos((int)se - 127);
      const uint32_t lo = f32_to_bf16(e4m3_decode(c & 0xFFu) * m);
      const uint32_t hi = f32_to_bf16(e4m3_decode(c >> 8) * m);
      st_coherent(reinterpret_cast<uint32_t*>(a.xb + off), lo | (hi << 16));
      if (FMT == FMT_BLOCK) {
        if (l == 0) st_coherent(sbl, sf);
      }
    } else {
      store_group<FMT>(a.xq + (off - 2 * l), c, sf, se, sbl, smx);
    }
  }
  drain_memory();
  __syncthreads();
  if (threadIdx.x == 0) atomic_add_agent(&a.ctrl[C_XQ], 1);
}

// Re-quantize 128-column group g of a32 into aq / as (all Mpad rows).
template <int FMT>
__device__ void requant_group(const StreamArgs& a, int g) {
  const int w = wave_id(), l = threadIdx.x & 63;
  for (int row = w; row < a.Mpad; row += NW) {
    uint32_t c = 0, se = 0;
    float sf = 1.0f;
    if (row < a.M) {
      const float* src = a.a32 + (size_t)row * a.F + g * 128 + 2 * l;
      c = quant_pair<FMT>(ld_coherent(src), ld_coherent(src + 1), &sf, &se);
    }
    store_group<FMT>(a.aq + (size_t)row * a.F + g * 128, c, sf, se,
                     static_cast<float*>(a.as) + (size_t)g * a.Mpad + row,
                     static_cast<uint8_t*>(a.as) + (size_t)row * (a.F >> 5) + 4 * g);
  }
}

// Fill the A-operand pointers of a Streamer for a row-major [Mpad, Kd] code
// matrix (filler loads read the wavefront's own first k-tile, which is ready)
// with scales in the internal layouts.
template <class S, int FMT>
__device__ __forceinline__ void set_a(S& st, const uint8_t* codes, const void* scales, int Kd, int Mpad,
                                      int kt0) {
  const int l = threadIdx.x & 63;
  st.arow = codes + (size_t)(l & 15) * Kd + 16 * (l >> 4);
  st.ashared = codes + (size_t)kt0 * 128;
  st.a_mt_stride = (size_t)16 * Kd;
  const uint32_t bytes = FMT == FMT_BLOCK ? (uint32_t)(Kd >> 7) * Mpad * 4 : (uint32_t)Mpad * (Kd >> 5);
  st.asr = make_rsrc(scales, bytes);
  if (FMT == FMT_BLOCK) {
    st.as_off = 16 * (l >> 4);
    st.as_kt_stride = 4 * Mpad;
    st.as_mt_stride = 64;
  } else {
    st.as_off = (uint32_t)(l & 15) * (Kd >> 5) + (l >> 4);
    st.as_kt_stride = 4;
    st.as_mt_stride = 16 * (Kd >> 5);
  }
}

// Fill the B-operand pointers of stream nb for weight n-tile jn of a packed
// [N, Kd] weight.
template <class S, int FMT>
__device__ __forceinline__ void set_b(S& st, int nb, const uint8_t* codes, const void* scales, int jn,
                                      int Kd, int kt0) {
  const int l = threadIdx.x & 63;
  const int KT = Kd >> 7, KG = (KT + 3) >> 2;
  st.bshared[nb] = codes + ((size_t)jn * KT + kt0) * 2048;
  st.bt[nb] = st.bshared[nb] + l * 16;
  if (FMT == FMT_BLOCK)
    st.bsf[nb] = static_cast<const float*>(scales) + (size_t)(jn >> 3) * KT;
  else
    st.bsm[nb] = static_cast<const uint32_t*>(scales) + (size_t)jn * KG * 64 + l;
}

// Write this wavefront's accumulators to LDS (waves 1..3); wave 0 keeps its
// own in registers and adds the others after the barrier.
template <int NB, int MT>
__device__ __forceinline__ void reduce_to_wave0(v4f (&acc)[NB][MT], v4f* red) {
  const int w = wave_id(), l = threadIdx.x & 63;
  if (w > 0) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) red[(((w - 1) * NB + nb) * MT + mt) * 64 + l] = acc[nb][mt];
  }
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int ww = 0; ww < NW - 1; ++ww)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nb][mt] += red[((ww * NB + nb) * MT + mt) * 64 + l];
  }
}

// ---------------------------------------------------------------------------
// GU item j: 16 ffn columns, gate and up over all of d.
// ---------------------------------------------------------------------------
template <int MT, int FMT>
__device__ void item_gu(const StreamArgs& a, int j, v4f* red, WgState& ws) {
  const int w = wave_id(), l = threadIdx.x & 63;
  const int KT = a.K1 >> 7;
  const int KTw = (KT + NW - 1) / NW;
  const int kt0 = min(KT, w * KTw);
  const int nk = min(KT, kt0 + KTw) - kt0;
  StreamerBf16<MT, 2, FMT, DepthBf16<MT>::P> st;
  st.kt0 = kt0;
  st.nk = nk;
  {
    const int KG = (KT + 3) >> 2;
    const uint8_t* wc[2] = {a.wg, a.wu};
    const void* wsc[2] = {a.sg, a.su};
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      st.bshared[nb] = wc[nb] + ((size_t)j * KT + kt0) * 2048;
      st.bt[nb] = st.bshared[nb] + l * 16;
      if (FMT == FMT_BLOCK) {
        st.bsf[nb] = static_cast<const float*>(wsc[nb]) + (size_t)(j >> 3) * KT;
      } else {
        const uint32_t* base = static_cast<const uint32_t*>(wsc[nb]) + (size_t)j * KG * 64 + (l & 15);
        st.bsm0[nb] = base + 16 * ((l >> 4) >> 1);
        st.bsm1[nb] = base + 16 * (2 + ((l >> 4) >> 1));
      }
    }
    st.arow = a.xb + (size_t)(l & 15) * a.K1 + 16 * (l >> 4);
    st.ashared = a.xb + (size_t)kt0 * 128;
    st.a_mt_stride = (size_t)16 * a.K1;
    st.Mpad = a.Mpad;
    if (FMT == FMT_BLOCK) st.asf = static_cast<const float*>(a.xs) + 4 * (l >> 4);
  }
  v4f acc[2][MT];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nb][mt] = v4f{0.f, 0.f, 0.f, 0.f};
  const uint32_t* xq_done = &a.ctrl[C_XQ];
  const uint32_t n_xq = (uint32_t)a.n_xq;
  st.run(
      acc, [&]() { return uniform(*(volatile uint32_t*)&ws.xq_seen) != 0; },
      [&]() {
        wait_geq(xq_done, n_xq);
        ws.xq_seen = 1;
      });
  reduce_to_wave0<2, MT>(acc, red);
  if (w == 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = mt * 16 + 4 * (l >> 4) + r;
        if (row < a.M) {
          const float g = acc[0][mt][r], u = acc[1][mt][r];
          st_coherent(a.a32 + (size_t)row * a.F + j * 16 + (l & 15), g / (1.0f + expf(-g)) * u);
        }
      }
    drain_memory();
  }
  __syncthreads();
  const int grp = j >> 3;
  if (threadIdx.x == 0) ws.flag = (atomic_add_agent(&a.ctrl[a.off_grp + grp], 1) == 7u);
  __syncthreads();
  if (ws.flag) {
    requant_group<FMT>(a, grp);
    drain_memory();
    __syncthreads();
    if (threadIdx.x == 0) {
      store_agent(&a.ctrl[a.off_grp + grp], 0u);
      store_agent(&a.ctrl[a.off_ready + grp], 1u);
    }
  }
}

// ---------------------------------------------------------------------------
// DN item: NTD*16 output columns x one K chunk of the second GEMM.
// ---------------------------------------------------------------------------
template <int MT, int FMT>
__device__ void item_dn(const StreamArgs& a, int i, v4f* red, WgState& ws) {
  const int w = wave_id(), l = threadIdx.x & 63;
  const int kc = i / a.n_dt, dt = i % a.n_dt;
  const int KT2 = a.K2 >> 7;
  const int kbeg = kc * a.ktc, kend = min(KT2, kbeg + a.ktc);
  const int KTw = (kend - kbeg + NW - 1) / NW;
  const int kt0 = min(kend, kbeg + w * KTw);
  const int nk = min(kend, kt0 + KTw) - kt0;
  Streamer<MT, NTD, FMT, Depth<MT>::P> st;
  st.kt0 = kt0;
  st.nk = nk;
#pragma unroll
  for (int s = 0; s < NTD; ++s) set_b<decltype(st), FMT>(st, s, a.w2, a.s2, dt * NTD + s, a.K2, kt0);
  if (a.mlp)
    set_a<decltype(st), FMT>(st, a.aq, a.as, a.F, a.Mpad, kt0);
  else
    set_a<decltype(st), FMT>(st, a.xq, a.xs, a.K1, a.Mpad, kt0);
  v4f acc[NTD][MT];
#pragma unroll
  for (int nb = 0; nb < NTD; ++nb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nb][mt] = v4f{0.f, 0.f, 0.f, 0.f};
  if (a.mlp) {
    const uint32_t* ready = &a.ctrl[a.off_ready];
    auto seen = [&](int g) { return (uniform(*(volatile uint32_t*)&ws.grp_seen[g >> 5]) >> (g & 31)) & 1u; };
    st.run(
        acc,
        [&]() {
          bool ok = true;
          for (int kt = kt0; kt < kt0 + nk; ++kt) ok = ok && seen(kt);
          return ok;
        },
        [&]() {
          for (int kt = kt0; kt < kt0 + nk; ++kt) {
            if (!seen(kt)) {
              wait_geq(&ready[kt], 1u);
              if ((threadIdx.x & 63) == 0) atomicOr(&ws.grp_seen[kt >> 5], 1u << (kt & 31));
            }
          }
        });
  } else {
    const uint32_t* xq_done = &a.ctrl[C_XQ];
    const uint32_t n_xq = (uint32_t)a.n_xq;
    st.run(
        acc, [&]() { return uniform(*(volatile uint32_t*)&ws.xq_seen) != 0; },
        [&]() {
          wait_geq(xq_done, n_xq);
          ws.xq_seen = 1;
        });
  }
  reduce_to_wave0<NTD, MT>(acc, red);
  if (w == 0) {
#pragma unroll
    for (int s = 0; s < NTD; ++s)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = mt * 16 + 4 * (l >> 4) + r;
          const int col = (dt * NTD + s) * 16 + (l & 15);
          if (row < a.M) {
            if (a.n_kc == 1)
              a.y[(size_t)row * a.N + col] = (uint16_t)f32_to_bf16(acc[s][mt][r]);
            else
              st_coherent(a.ypart + ((size_t)kc * a.M + row) * a.N + col, acc[s][mt][r]);
          }
        }
    if (a.n_kc > 1) drain_memory();
  }
  if (a.n_kc == 1) return;
  __syncthreads();
  if (threadIdx.x == 0)
    ws.flag = (atomic_add_agent(&a.ctrl[a.off_ycnt + dt], 1) == (uint32_t)(a.n_kc - 1));
  __syncthreads();
  if (ws.flag) {
    constexpr int COLS = NTD * 16;
    for (int e = threadIdx.x; e < a.M * COLS; e += NW * 64) {
      const int row = e / COLS, col = dt * COLS + e % COLS;
      float v = 0.0f;
      for (int c = 0; c < a.n_kc; ++c) v += ld_coherent(a.ypart + ((size_t)c * a.M + row) * a.N + col);
      a.y[(size_t)row * a.N + col] = (uint16_t)f32_to_bf16(v);
    }
    if (threadIdx.x == 0) store_agent(&a.ctrl[a.off_ycnt + dt], 0u);
  }
}

// ---------------------------------------------------------------------------
// The persistent kernel.
// ---------------------------------------------------------------------------
template <int MT, int FMT>
__global__ __launch_bounds__(NW * 64, (MT >= 8 ? 1 : 2)) void stream_kernel(StreamArgs a) {
  __shared__ v4f red[(NW - 1) * 2 * MT * 64];
  __shared__ WgState ws;
  if (threadIdx.x == 0) {
    ws.xq_seen = 0;
    for (int k = 0; k < 8; ++k) ws.grp_seen[k] = 0;
  }
  __syncthreads();
  int ticket = blockIdx.x;
  while (ticket < a.total) {
    // take the next ticket now; its latency overlaps this item
    uint32_t next = 0;
    if (threadIdx.x == 0) next = gridDim.x + atomic_add_agent(&a.ctrl[C_TICKET], 1);
    if (ticket < a.n_xq)
      item_xq<FMT>(a, ticket);
    else if (ticket < a.n_xq + a.n_gu)
      item_gu<MT, FMT>(a, ticket - a.n_xq, red, ws);
    else
      item_dn<MT, FMT>(a, ticket - a.n_xq - a.n_gu, red, ws);
    __syncthreads();
    if (threadIdx.x == 0) ws.ticket = next;
    __syncthreads();
    ticket = (int)uniform(ws.ticket);
  }
  if (threadIdx.x == 0) {
    if (atomic_add_agent(&a.ctrl[C_DONE], 1) == gridDim.x - 1) {
      // Every workgroup has taken its last ticket: reset the control block.
      const int n = a.off_ycnt + a.n_dt;
      for (int k = C_HDR; k < n; ++k) store_agent(&a.ctrl[k], 0u);
      store_agent(&a.ctrl[C_XQ], 0u);
      store_agent(&a.ctrl[C_TICKET], 0u);
      store_agent(&a.ctrl[C_DONE], 0u);
    }
  }
}

// ---------------------------------------------------------------------------
// host side: plan, workspace layout, launch
// ---------------------------------------------------------------------------
namespace {

struct Plan {
  int MT, Mpad;
  int n_xq, n_gu, n_dt, n_kc, ktc, total;
  int off_grp, off_ready, off_ycnt, ctrl_words;
  size_t off_xq, off_xs, off_a32, off_aq, off_as, off_ypart, bytes;  // off_xq: xq (GEMM) or xb (MLP)
};

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

int mt_for(int M) { return M <= 16 ? 1 : M <= 32 ? 2 : M <= 64 ? 4 : 8; }

Plan make_plan(int fmt, int M, int K1, int F, int N, int K2, bool mlp) {
  Plan p{};
  p.MT = mt_for(M);
  p.Mpad = 16 * p.MT;
  p.n_xq = (p.Mpad * (K1 / 128) + XQ_GPI - 1) / XQ_GPI;
  p.n_gu = mlp ? F / 16 : 0;
  p.n_dt = N / (16 * NTD);
  const int KT2 = K2 / 128;
  // K chunk of a DN item: about as many weight bytes as a GU item
  // (2 * 16 * d), and at least 4 k-tiles per chunk.
  int ktc = mlp ? K1 / 128 : KT2;
  if (!mlp) {
    // plain GEMM: split K so that there are enough items to fill the chip
    const int want_items = 1024;
    int chunks = (want_items + p.n_dt - 1) / p.n_dt;
    if (chunks > KT2 / 4) chunks = KT2 / 4 > 0 ? KT2 / 4 : 1;
    ktc = (KT2 + chunks - 1) / chunks;
  }
  if (ktc < 4) ktc = 4;
  if (ktc > KT2) ktc = KT2;
  p.ktc = ktc;
  p.n_kc = (KT2 + ktc - 1) / ktc;
  p.total = p.n_xq + p.n_gu + p.n_dt * p.n_kc;
  const int ng = mlp ? F / 128 : 0;
  p.off_grp = C_HDR;
  p.off_ready = p.off_grp + ng;
  p.off_ycnt = p.off_ready + ng;
  p.ctrl_words = p.off_ycnt + p.n_dt;
  size_t o = align256((size_t)p.ctrl_words * 4);
  p.off_xq = o;
  o = align256(o + (size_t)p.Mpad * K1 * (mlp ? 2 : 1));
  p.off_xs = o;
  o = align256(o + (fmt == FMT_BLOCK ? (size_t)(K1 / 128) * p.Mpad * 4 : (size_t)p.Mpad * (K1 / 32)));
  p.off_a32 = o;
  if (mlp) o = align256(o + (size_t)M * F * 4);
  p.off_aq = o;
  if (mlp) o = align256(o + (size_t)p.Mpad * F);
  p.off_as = o;
  if (mlp) o = align256(o + (fmt == FMT_BLOCK ? (size_t)(F / 128) * p.Mpad * 4 : (size_t)p.Mpad * (F / 32)));
  p.off_ypart = o;
  if (p.n_kc > 1) o = align256(o + (size_t)p.n_kc * M * N * 4);
  p.bytes = o;
  return p;
}

template <int MT, int FMT>
const void* kernel_ptr() { return reinterpret_cast<const void*>(&stream_kernel<MT, FMT>); }

const void* pick_kernel(int MT, int fmt) {
  if (fmt == FMT_BLOCK) {
    switch (MT) {
      case 1: return kernel_ptr<1, FMT_BLOCK>();
      case 2: return kernel_ptr<2, FMT_BLOCK>();
      case 4: return kernel_ptr<4, FMT_BLOCK>();
      default: return kernel_ptr<8, FMT_BLOCK>();
    }
  }
  switch (MT) {
    case 1: return kernel_ptr<1, FMT_MX>();
    case 2: return kernel_ptr<2, FMT_MX>();
    case 4: return kernel_ptr<4, FMT_MX>();
    default: return kernel_ptr<8, FMT_MX>();
  }
}

// Resident workgroups per device for each kernel variant (queried once).
struct Occupancy {
  std::mutex mu;
  int cus[64] = {0};
  int per_cu[64][2][4] = {};
};
Occupancy g_occ;

int resident_blocks(const void* kern, int MT, int fmt, int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return SGD_EHIP;
  const int fi = fmt == FMT_BLOCK ? 0 : 1;
  const int mi = MT == 1 ? 0 : MT == 2 ? 1 : MT == 4 ? 2 : 3;
  std::lock_guard<std::mutex> lock(g_occ.mu);
  if (g_occ.cus[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return SGD_EHIP;
    g_occ.cus[dev] = cus;
  }
  if (g_occ.per_cu[dev][fi][mi] == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, NW * 64, 0) != hipSuccess || nb <= 0)
      return SGD_EHIP;
    g_occ.per_cu[dev][fi][mi] = nb;
  }
  *out = g_occ.cus[dev] * g_occ.per_cu[dev][fi][mi];
  return SGD_OK;
}

}  // namespace

size_t stream_workspace_bytes(int fmt, int M, int K1, int F, int N, int K2, bool mlp) {
  return make_plan(fmt, M, K1, F, N, K2, mlp).bytes;
}

int launch_stream(const Problem& pr, hipStream_t s) {
  const bool mlp = pr.gate != nullptr;
  const int F = mlp ? pr.gate->N : 0;
  const Plan p = make_plan(pr.fmt, pr.M, pr.K1, F, pr.w2->N, pr.w2->K, mlp);
  StreamArgs a{};
  a.M = pr.M;
  a.Mpad = p.Mpad;
  a.mlp = mlp ? 1 : 0;
  a.x = pr.x;
  a.K1 = pr.K1;
  if (mlp) {
    a.wg = static_cast<const uint8_t*>(pr.gate->codes);
    a.sg = pr.gate->scales;
    a.wu = static_cast<const uint8_t*>(pr.up->codes);
    a.su = pr.up->scales;
  }
  a.F = F;
  a.w2 = static_cast<const uint8_t*>(pr.w2->codes);
  a.s2 = pr.w2->scales;
  a.N = pr.w2->N;
  a.K2 = pr.w2->K;
  a.y = pr.y;
  uint8_t* ws = static_cast<uint8_t*>(pr.ws);
  a.ctrl = reinterpret_cast<uint32_t*>(ws);
  a.xq = ws + p.off_xq;
  a.xb = reinterpret_cast<uint16_t*>(ws + p.off_xq);
  a.xs = ws + p.off_xs;
  a.a32 = reinterpret_cast<float*>(ws + p.off_a32);
  a.aq = ws + p.off_aq;
  a.as = ws + p.off_as;
  a.ypart = reinterpret_cast<float*>(ws + p.off_ypart);
  a.n_xq = p.n_xq;
  a.n_gu = p.n_gu;
  a.n_dt = p.n_dt;
  a.n_kc = p.n_kc;
  a.ktc = p.ktc;
  a.total = p.total;
  a.off_grp = p.off_grp;
  a.off_ready = p.off_ready;
  a.off_ycnt = p.off_ycnt;

  const void* kern = pick_kernel(p.MT, pr.fmt);
  int resident = 0;
  int rc = resident_blocks(kern, p.MT, pr.fmt, &resident);
  if (rc != SGD_OK) return rc;
  // Workgroups are dispatched in index order, so the first (static) tickets
  // and every later (atomic) ticket reach workgroups that are already
  // running: a wait only ever targets an item that is being worked on.
  int grid = resident < p.total ? resident : p.total;
  if (grid < 1) grid = 1;
  void* args[] = {&a};
  return hip_status(hipLaunchKernel(kern, dim3(grid), dim3(NW * 64), args, 0, s));
}

}  // namespace sgd

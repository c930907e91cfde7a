// Large-M (prefill) path: the scaled fp8 GEMM as a compute-bound tiled
// kernel, for M beyond the decode shapes of the streaming kernel.  The pages'
// second benchmark family (fish.audio blog, section "Resultados de benchmark
// del kernel": the MLP at M from 1 to 4096 and square MXFP8 GEMMs from 1024^3
// to 16384^3) is this regime: arithmetic intensity ~M flop per weight byte,
// far above the HBM ridge, so the matrix cores set the pace.
//
// Operands.  Both are arrays of 2 KB tiles in the operand order of
// v_mfma_scale_f32_16x16x128_f8f6f4 (lane l = r + 16q: row r, columns
// 16q..16q+15 at byte 16l and 64+16q.. at 1024 + 16l):
//   * the packed weight, tile (n-block j, k-tile t) at (j*K/128 + t)*2048;
//   * the activations in the workspace layout with every m-tile full
//     (M padded to Mpad = 16*ceil(M/16) zero rows): tile (m-tile i, k-tile t)
//     at i*16*K + t*2048.
// So a workgroup copies whole tiles from memory to LDS and each wavefront
// reads its operands with two 16-byte LDS reads per tile.
//
// Kernel.  A workgroup computes a BM x BN block of C = Q(x) W^T over all of
// K, k-tile by k-tile through NSTG LDS stages: while the matrix cores work on
// stage kt, k-tiles kt+1 .. kt+NSTG-1 are on their way into the other stages
// by direct memory-to-LDS loads (no registers), the operand tiles and their
// scales alike, and one barrier per k-tile hands a stage over.  With two
// stages the copies' latency, not the matrix cores, set the pace (measured:
// 1.1 PFLOP/s at 8192^3; three stages of 256 x 128 give 1.7).  Wavefront
// (wm, wn) owns TM m-tiles x TN n-blocks.  MX: the E8M0 scales go into the
// instruction; block format: the unscaled product of each k-tile is added
// with the row's activation scale times the weight block's scale, as in the
// streaming kernel.
#include "sgd_act.hpp"
#include "sgd_device.hpp"
#include "sgd_host.hpp"

namespace sgd {

namespace {

constexpr uint32_t OOB_T = 0x80000000u;  // a buffer offset past every buffer's end
constexpr int KSPLIT_CUS = 256;          // compute units a split-K launch aims to fill

struct TileArgs {
  const uint8_t* a;  // Q(x) codes, full m-tiles [Mpad/16][K/128][2048]
  const void* as;    // block: fp32 [K/128][Mpad]; mx: [Mpad/16][K/128][16] dwords
  int Mpad, K;
  const uint8_t* w;  // packed weight [N/16][K/128][2048]
  const void* ws;    // packed weight scales
  int N;
  void* c;           // [M, N] bf16 or fp32 (row-major)
  int M;             // rows of C stored
  uint32_t a_bytes, as_bytes, w_bytes, ws_bytes;
  int tiles_m;       // blocks along M (the grid is tiles_m x blocks along N, times ksplit)
  int ksplit;        // K ranges: range r writes fp32 partial sums at c + r*M*N (OUT 1), summed by a second kernel
};

__device__ __forceinline__ int uni_t(int v) { return __builtin_amdgcn_readfirstlane(v); }

// LDS stage of the tiled GEMM: the k-tile's AT activation tiles and BT weight
// tiles (2 KB each, A first), then the scales: 64 bytes per m-tile (mx: the
// rows' E8M0 bytes of the k-tile's four 32-column blocks, row-major; block:
// the 16 rows' fp32 scales), then 256 bytes per n-tile (mx: the dword of 4
// k-tiles of each lane's row, as packed; block: one fp32 per 128-row weight
// block of the workgroup).
template <int AT, int BT>
__host__ __device__ constexpr int tile_stage_bytes() { return (AT + BT) * 2048 + AT * 64 + BT * 256; }
constexpr int TRASH_BYTES = 256;  // where the copies that only pad the per-wavefront count land

template <int FMT, int WGM, int WGN, int TM, int TN, int NSTG, int OUT>
__global__ __launch_bounds__(64 * WGM * WGN) void tile_gemm_kernel(TileArgs p) {
  constexpr int AT = WGM * TM, BT = WGN * TN;  // A and B tiles of one k-tile
  constexpr int NW = WGM * WGN;
  constexpr int CH = 2 * (AT + BT) / NW;       // 1 KB tile halves each wavefront copies per stage
  static_assert(2 * (AT + BT) % NW == 0, "stage halves");
  static_assert(AT % 4 == 0 && BT % 8 == 0, "scale copies");
  constexpr int SC = AT / 4 + (FMT == FMT_MX ? BT : 1);  // 256-byte scale copies per stage
  constexpr int SCH = (SC + NW - 1) / NW;                 // per wavefront (padded)
  constexpr int OPS = CH + SCH;                           // copies per wavefront per stage
  constexpr int SB = tile_stage_bytes<AT, BT>();
  static_assert(NSTG >= 2, "stages");
  extern __shared__ __align__(16) uint8_t lds[];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8*)lds;
  const uint32_t trash = lds0 + (uint32_t)(NSTG * SB);
  const int l = lane_id(), wv = uni_t((int)(threadIdx.x >> 6));
  const int wm = wv % WGM, wn = wv / WGM;
  const int nblk = (int)gridDim.x / p.ksplit;
  const int kr = (int)blockIdx.x / nblk, blk = (int)blockIdx.x - kr * nblk;
  const int bm = blk % p.tiles_m, bn = blk / p.tiles_m;
  const int KTall = p.K >> 7;
  // this block's k-tiles [k0, KT)
  const int k0 = (int)(((long long)kr * KTall) / p.ksplit), KT = (int)(((long long)(kr + 1) * KTall) / p.ksplit);
  const int mt0 = bm * AT, nb0 = bn * BT;  // first m-tile / n-block of the block
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, p.a_bytes), rw = make_rsrc(p.w, p.w_bytes);
  const __amdgpu_buffer_rsrc_t ras = make_rsrc(p.as, p.as_bytes), rws = make_rsrc(p.ws, p.ws_bytes);
  const int MTA = p.Mpad >> 4, NBW = p.N >> 4;

  // ---- stage copy: k-tile kt into stage buffer b.  Wavefront wv copies tile
  // halves wv, wv + NW, ... and scale blocks wv, wv + NW, ...; every
  // wavefront issues exactly OPS copies (k-tiles past K, tiles past the
  // matrices and the padding read zeros), so that the number of copies in
  // flight behind a stage is the same for all ----
  auto copy_stage = [&](int kt, int b) {
    const uint32_t base = lds0 + (uint32_t)(b * SB);
    const bool in = kt < KT;
    const uint32_t ukt = in ? (uint32_t)kt : 0u;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int h = wv + NW * i, t = h >> 1, half = h & 1;
      const uint32_t m0 = base + (uint32_t)(t * 2048 + half * 1024);
      const uint32_t lo = (uint32_t)half * 1024u + (uint32_t)l * 16u;
      if (t < AT) {
        const int mt = mt0 + t;
        lds_copy1k(ra, m0, in && mt < MTA ? (uint32_t)mt * 16u * (uint32_t)p.K + ukt * 2048u + lo : OOB_T);
      } else {
        const int nb = nb0 + t - AT;
        lds_copy1k(rw, m0, in && nb < NBW ? ((uint32_t)nb * (uint32_t)KTall + ukt) * 2048u + lo : OOB_T);
      }
    }
    const uint32_t sbase = base + (uint32_t)((AT + BT) * 2048);
#pragma unroll
    for (int i = 0; i < SCH; ++i) {
      const int c = wv + NW * i;
      if (c < AT / 4) {
        // m-tiles mt0 + 4c .. +3: lane l carries (m-tile 4c + l/16, dword l%16)
        const int mt = mt0 + 4 * c + (l >> 4);
        const bool ok = in && mt < MTA;
        const uint32_t o = FMT == FMT_MX
                               ? (uint32_t)mt * 16u * (uint32_t)(p.K >> 5) + ukt * 64u + (uint32_t)(l & 15) * 4u
                               : (ukt * (uint32_t)p.Mpad + (uint32_t)mt * 16u + (uint32_t)(l & 15)) * 4u;
        lds_copy256(ras, sbase + (uint32_t)(c * 256), ok ? o : OOB_T);
      } else if (c < SC) {
        const uint32_t dst = sbase + (uint32_t)(AT * 64 + (c - AT / 4) * 256);
        if (FMT == FMT_MX) {
          const int nb = nb0 + c - AT / 4;
          const uint32_t KG = (uint32_t)(KTall + 3) >> 2;
          const uint32_t o = ((uint32_t)nb * KG + (ukt >> 2)) * 256u + (uint32_t)l * 4u;
          lds_copy256(rws, dst, in && nb < NBW ? o : OOB_T);
        } else {
          // lane j: the scale of the workgroup's j-th 128-row weight block
          const int wblk = (nb0 >> 3) + l;
          const bool ok = in && l < BT / 8 && wblk * 8 < NBW;
          lds_copy256(rws, dst, ok ? ((uint32_t)wblk * (uint32_t)KTall + ukt) * 4u : OOB_T);
        }
      } else {
        lds_copy256(ras, trash, OOB_T);
      }
    }
  };

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // NSTG - 1 stages in flight ahead of the one being multiplied; one barrier
  // per k-tile both publishes stage kt (every wavefront has waited for its
  // own copies of it) and frees stage kt - 1 for the copy of kt + NSTG - 1
#pragma unroll
  for (int b = 0; b < NSTG - 1; ++b) copy_stage(k0 + b, b);
  for (int kt = k0; kt < KT; ++kt) {
    const int j0 = kt - k0;  // (stage index: the range's own position)
    lds_copies_left<(NSTG - 2) * OPS>();
    __syncthreads();
    copy_stage(kt + NSTG - 1, (j0 + NSTG - 1) % NSTG);
    const uint8_t* st = lds + (j0 % NSTG) * SB;
    const uint8_t* ssa = st + (AT + BT) * 2048;
    const uint8_t* ssb = ssa + AT * 64;
    v8i av[TM];
    uint32_t xa[TM];
    v4f xb[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int ti = wm * TM + i;
      const uint8_t* t = st + ti * 2048 + l * 16;
      av[i] = make_v8i(*reinterpret_cast<const uint4*>(t), *reinterpret_cast<const uint4*>(t + 1024));
      if (FMT == FMT_MX)
        xa[i] = (uint32_t)ssa[ti * 64 + (l & 15) * 4 + (l >> 4)];
      else
        xb[i] = *reinterpret_cast<const v4f*>(ssa + ti * 64 + 16 * (l >> 4));
    }
    const int sh = 8 * (kt & 3);
    const float wbs = FMT == FMT_MX ? 1.0f : reinterpret_cast<const float*>(ssb)[(wn * TN) >> 3];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const uint8_t* t = st + (AT + wn * TN + j) * 2048 + l * 16;
      const v8i bv = make_v8i(*reinterpret_cast<const uint4*>(t), *reinterpret_cast<const uint4*>(t + 1024));
      const uint32_t wsd = FMT == FMT_MX ? reinterpret_cast<const uint32_t*>(ssb)[(wn * TN + j) * 64 + l] : 0u;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if (FMT == FMT_MX) {
          acc[i][j] = mfma_f8(av[i], bv, acc[i][j], (int)xa[i], (int)(wsd >> sh));
        } else {
          const v4f z = {0.f, 0.f, 0.f, 0.f};
          const v4f t4 = mfma_f8(av[i], bv, z, 127, 127);
          acc[i][j] += t4 * (xb[i] * wbs);
        }
      }
    }
  }
  lds_copies_left<0>();  // (the fillers' copies: nothing may be in flight at exit)

  // ---- epilogue: rows < M, columns < N ----
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = (nb0 + wn * TN + j) * 16 + (l & 15);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int row = (mt0 + wm * TM + i) * 16 + 4 * (l >> 4) + rr;
        if (row < p.M && col < p.N) {
          const size_t o = (size_t)row * p.N + col;
          if (OUT == 1)
            static_cast<float*>(p.c)[(size_t)kr * p.M * p.N + o] = acc[i][j][rr];
          else
            static_cast<uint16_t*>(p.c)[o] = (uint16_t)f32_to_bf16(acc[i][j][rr]);
        }
      }
    }
}

// Q(x) of bf16 x [M, K] in the workspace layout with full m-tiles (rows
// M..Mpad-1 quantized as zeros): one wavefront per (m-tile, 128-column
// group), one lane per (row, 32-column block), the streaming kernel's
// quantizer.
template <int FMT>
__global__ __launch_bounds__(256) void act_tiles_kernel(const uint16_t* __restrict__ x, int M, int K, int Mpad,
                                                        uint8_t* __restrict__ codes, void* __restrict__ scales) {
  const int nmt = Mpad >> 4, ng = K >> 7;
  const long long wave = ((long long)blockIdx.x * 256 + threadIdx.x) >> 6;
  if (wave >= (long long)nmt * ng) return;
  const int g = (int)(wave / nmt), mt = (int)(wave - (long long)g * nmt);
  const int l = lane_id(), row = mt * 16 + (l >> 2), j = l & 3;
  float v[32];
  if (row < M) {
    const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)row * K + g * 128 + 32 * j);
    uint4 w[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) w[c] = src[c];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t ww[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * c + 2 * e] = bf16_to_f32(ww[e] & 0xFFFFu);
        v[8 * c + 2 * e + 1] = bf16_to_f32(ww[e] >> 16);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e) v[e] = 0.0f;
  }
  uint32_t cw[8], se = 0;
  float sf = 1.0f;
  quant_block32<FMT>(v, cw, &sf, &se);
  const size_t off = (size_t)mt * 16 * K + (size_t)(g * 128 + 32 * j) / 16 * 256 + (size_t)(l >> 2) * 16;
  *reinterpret_cast<uint4*>(codes + off) = make_uint4(cw[0], cw[1], cw[2], cw[3]);
  *reinterpret_cast<uint4*>(codes + off + 256) = make_uint4(cw[4], cw[5], cw[6], cw[7]);
  if (FMT == FMT_BLOCK) {
    // (padded rows: zero scales, like the streaming kernel's layout)
    if (j == 0) static_cast<float*>(scales)[(size_t)g * Mpad + row] = row < M ? sf : 0.0f;
  } else {
    const uint32_t e4 = pack4_lanes(se);
    if (j == 0)
      reinterpret_cast<uint32_t*>(scales)[(size_t)mt * 16 * (K >> 5) / 4 + (size_t)g * 16 + (l >> 2)] = e4;
  }
}

// y [M, N] bf16 = the sum of the S fp32 partials [S][M][N] (in range order),
// four elements per lane.
__global__ __launch_bounds__(256) void ksum_kernel(const float* __restrict__ part, int S, long long n,
                                                   uint16_t* __restrict__ y) {
  const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  float4 v = *reinterpret_cast<const float4*>(part + i);
  for (int r = 1; r < S; ++r) {
    const float4 w = *reinterpret_cast<const float4*>(part + (size_t)r * n + i);
    v.x += w.x;
    v.y += w.y;
    v.z += w.z;
    v.w += w.w;
  }
  const uint32_t lo = f32_to_bf16(v.x) | (f32_to_bf16(v.y) << 16), hi = f32_to_bf16(v.z) | (f32_to_bf16(v.w) << 16);
  *reinterpret_cast<uint2*>(y + i) = make_uint2(lo, hi);
}

template <int FMT, int WGM, int WGN, int TM, int TN, int NSTG, int OUT>
int launch_tile_cfg(TileArgs p, hipStream_t s) {
  constexpr int BM = WGM * TM * 16, BN = WGN * TN * 16;
  constexpr size_t lds = (size_t)NSTG * tile_stage_bytes<WGM * TM, WGN * TN>() + TRASH_BYTES;
  static_assert(lds <= 163840, "LDS of one workgroup");
  p.tiles_m = (p.Mpad + BM - 1) / BM;
  const long long grid = (long long)p.tiles_m * ((p.N + BN - 1) / BN) * p.ksplit;
  auto k = tile_gemm_kernel<FMT, WGM, WGN, TM, TN, NSTG, OUT>;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) !=
      hipSuccess)
    return SGD_EHIP;
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(64 * WGM * WGN), lds, s, p);
  return hip_status(hipGetLastError());
}

template <int FMT, int OUT>
int launch_tile_gemm_fmt(const TileArgs& a, bool big, hipStream_t s) {
  if (big) return launch_tile_cfg<FMT, 4, 2, 4, 4, 3, OUT>(a, s);  // 256 x 128 blocks, 8 wavefronts of 64 x 64, 3 stages
  return launch_tile_cfg<FMT, 2, 2, 4, 4, 4, OUT>(a, s);           // 128 x 128 blocks, 4 wavefronts of 64 x 64, 4 stages
}

}  // namespace

size_t act_tiles_codes_bytes(int M, int K) { return (size_t)((M + 15) / 16) * 16 * (size_t)K; }
size_t act_tiles_scales_bytes(int fmt, int M, int K) {
  const size_t Mpad = (size_t)((M + 15) / 16) * 16;
  return fmt == FMT_BLOCK ? (size_t)(K / 128) * Mpad * 4 : Mpad * (size_t)(K / 32);
}

int launch_act_tiles(int fmt, const uint16_t* x, int M, int K, uint8_t* codes, void* scales, hipStream_t s) {
  const int Mpad = (M + 15) / 16 * 16;
  const long long waves = (long long)(Mpad / 16) * (K / 128);
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (fmt == FMT_BLOCK)
    hipLaunchKernelGGL(act_tiles_kernel<FMT_BLOCK>, grid, dim3(256), 0, s, x, M, K, Mpad, codes, scales);
  else
    hipLaunchKernelGGL(act_tiles_kernel<FMT_MX>, grid, dim3(256), 0, s, x, M, K, Mpad, codes, scales);
  return hip_status(hipGetLastError());
}

// C [M, N] (bf16, or fp32 when out_f32) = Q(A) W^T for Q(A) in the full-tile
// workspace layout of Mpad >= M rows.  With `part` (fp32, part_bytes) and a
// bf16 C that the 128 x 128 blocks alone would spread over fewer workgroups
// than compute units: K is split into S ranges (S blocks per compute unit
// at most, at least 16 k-tiles each), whose fp32 partial sums go to `part`
// and are added by a second kernel.
int launch_tile_gemm(int fmt, const uint8_t* a, const void* as, int M, int K, const sgd_weight* w, void* c,
                     bool out_f32, hipStream_t s, float* part, size_t part_bytes) {
  TileArgs p{};
  p.a = a;
  p.as = as;
  p.Mpad = (M + 15) / 16 * 16;
  p.K = K;
  p.w = static_cast<const uint8_t*>(w->codes);
  p.ws = w->scales;
  p.N = w->N;
  p.c = c;
  p.M = M;
  p.a_bytes = (uint32_t)act_tiles_codes_bytes(M, K);
  p.as_bytes = (uint32_t)act_tiles_scales_bytes(fmt, M, K);
  p.w_bytes = (uint32_t)((size_t)w->N * (size_t)K);
  p.ws_bytes = (uint32_t)sgd_packed_scales_bytes(fmt, w->N, K);
  // the big blocks when they still give at least one per compute unit
  const long long big_blocks = (long long)((p.Mpad + 255) / 256) * ((p.N + 127) / 128);
  const bool big = big_blocks >= 256;
  p.ksplit = 1;
  if (!big && !out_f32 && part) {
    const long long blocks = (long long)((p.Mpad + 127) / 128) * ((p.N + 127) / 128);
    int S = (int)(KSPLIT_CUS / blocks);
    if (S > (K / 128) / 16) S = (K / 128) / 16;
    while (S > 1 && (size_t)S * (size_t)M * (size_t)p.N * 4u > part_bytes) --S;
    if (S > 1) {
      p.ksplit = S;
      p.c = part;
      const int rc = fmt == FMT_BLOCK ? launch_tile_gemm_fmt<FMT_BLOCK, 1>(p, false, s)
                                      : launch_tile_gemm_fmt<FMT_MX, 1>(p, false, s);
      if (rc) return rc;
      const long long n = (long long)M * p.N;  // (a multiple of 4: N is of 128)
      hipLaunchKernelGGL(ksum_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, s, part, S, n,
                         static_cast<uint16_t*>(c));
      return hip_status(hipGetLastError());
    }
  }
  if (fmt == FMT_BLOCK)
    return out_f32 ? launch_tile_gemm_fmt<FMT_BLOCK, 1>(p, big, s) : launch_tile_gemm_fmt<FMT_BLOCK, 0>(p, big, s);
  return out_f32 ? launch_tile_gemm_fmt<FMT_MX, 1>(p, big, s) : launch_tile_gemm_fmt<FMT_MX, 0>(p, big, s);
}

}  // namespace sgd

// Paged decode attention over an MXFP8 K/V cache with grouped query heads:
// the other half of a decode step next to the MLP.  fish.audio blog "Cómo
// hicimos que nuestra API de texto a voz sea gratuita…", section "Qué hay en
// código abierto": an MXFP8 FlashAttention whose modes include paged decode
// with native GQA through a stride-0 K/V broadcast (the query heads of a
// group read their group's K/V once, nothing is replicated per head).
//
// Cache.  Each token's K and V vectors (head_dim 128, per KV head) are
// quantized on their own in 1x32 MX blocks along head_dim when written.
// Pages hold 16 token slots; per (page, KV head) 2112 bytes:
//   K: a 16 x 128 tile in the operand order of the scaled fp8 matrix
//      instruction (lane l = r + 16q: slot r, dims 16q.. and 64+16q..), then
//      64 scale bytes, byte l = (slot l % 16, block l / 16): the instruction's
//      scale operand, one byte per lane;
//   V: lane l = (d % 16) + 16 (r / 4) holds 32 bytes, byte 4n + r % 4 the code
//      of (slot r, dim 16n + d % 16): per 16-dim block n one dword of four
//      consecutive slots, the operand order of a 16x16x16 bf16 matrix
//      instruction's A operand (V^T, dims x slots); then byte
//      16 (r / 4) + 4b + r % 4 = the scale of (slot r, block b), the 16 bytes
//      of one lane group together.
//
// Decode.  A workgroup takes one (sequence, KV head) and one of S splits of
// the sequence's pages (with one split, workgroups are matched to pairs in
// order of length, so that the compute units get similar shares); its four
// wavefronts take every fourth page of the split, RING pages in flight each.
// Per page one 16x16x128 MX-scaled fp8 product gives the scores of the
// page's 16 slots against all (up to 16) query heads of the group, the K
// tile being the shared operand (the stride-0 broadcast); the online softmax
// (fp32, exp2, scores pre-multiplied by sm_scale * log2 e) is updated; then
// o^T += V^T p^T on the bf16 matrix instruction: V's E4M3 codes widened exactly to bf16,
// its per-(slot, block) scale folded into p (rounded to bf16) by ldexp.  The
// products are taken transposed so that p and the softmax rescale never
// cross lanes through LDS.
// The four wavefronts' states are merged in LDS into the split's partial
// (row max, row sum, unnormalized o); a second kernel merges the splits and
// writes bf16.  The work is HBM-bound: one pass over the sequence's K and V.
#include "sgd_act.hpp"
#include "sgd_device.hpp"
#include "sgd_host.hpp"

namespace sgd {

namespace {

constexpr int HD = 128;               // head_dim
constexpr int PSLOTS = 16;            // token slots per page
constexpr int PAGE_BYTES = 2112;      // per (page, KV head)
constexpr int MAXG = 16;              // query heads per KV head
constexpr int RING = 2;               // pages in flight per wavefront (3, 4 and 6 measured no faster)
constexpr int MAXB_ORDER = 256;      // batches up to this size take workgroups in order of length
constexpr int MAXCHUNK = 1024;        // pages of one split (their ids are staged in LDS)
constexpr float LOG2E = 1.4426950408889634f;

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));

struct AttnArgs {
  const uint16_t* q;   // [B, Hq, 128] bf16
  const uint8_t* kc;   // [n_pages, Hkv, 2112]
  const uint8_t* vc;
  const int32_t* bt;   // [B, max_pages]
  const int32_t* lens; // [B]
  int B, Hq, Hkv, G, max_pages, n_pages, S, chunk;  // chunk: pages per split
  float qk_scale;      // sm_scale * log2(e)
  float* part;         // [B * Hkv * S][G][2 + 128]: row max (log2 units), row sum, o
  uint16_t* out;       // [B, Hq, 128] bf16
};


// ---------------------------------------------------------------------------
// cache write: one lane per (token, KV head, 32-dim block)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kv_write_kernel(int kind, const uint16_t* __restrict__ x,
                                                       const int32_t* __restrict__ slots, int n, int Hkv,
                                                       uint8_t* __restrict__ cache, int n_pages) {
  const long long lane_all = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long vec = lane_all >> 2;
  const int j = (int)(lane_all & 3);
  if (vec >= (long long)n * Hkv) return;  // (whole groups of four lanes: vec is shared by them)
  const int t = (int)(vec / Hkv), h = (int)(vec - (long long)t * Hkv);
  const int slot = slots[t];
  const bool ok = slot >= 0 && slot < n_pages * PSLOTS;  // (invalid slots are skipped)
  float v[32];
  const uint4* src = reinterpret_cast<const uint4*>(x + vec * HD + 32 * j);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint4 w = src[c];
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[8 * c + 2 * e] = bf16_to_f32(ww[e] & 0xFFFFu);
      v[8 * c + 2 * e + 1] = bf16_to_f32(ww[e] >> 16);
    }
  }
  uint32_t cw[8], se = 0;
  float sf = 1.0f;
  quant_block32<FMT_MX>(v, cw, &sf, &se);
  if (!ok) return;
  const int page = slot / PSLOTS, r = slot - page * PSLOTS;
  uint8_t* base = cache + ((size_t)page * Hkv + h) * PAGE_BYTES;
  if (kind == 0) {
    // dims 32j..32j+31 are 16-dim segments 2j and 2j+1; segment s sits at
    // half s / 4, lane r + 16 (s % 4)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int s = 2 * j + u;
      *reinterpret_cast<uint4*>(base + (s >> 2) * 1024 + (r + 16 * (s & 3)) * 16) =
          make_uint4(cw[4 * u], cw[4 * u + 1], cw[4 * u + 2], cw[4 * u + 3]);
    }
    base[2048 + r + 16 * j] = (uint8_t)se;
  } else {
    // dim d = 32j + 4k + e (byte e of cw[k]): lane (d % 16) + 16 (r / 4),
    // byte 4 (d / 16) + r % 4
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 32 * j + 4 * k + e;
        base[32 * ((d & 15) + 16 * (r >> 2)) + 4 * (d >> 4) + (r & 3)] = (uint8_t)(cw[k] >> (8 * e));
      }
    base[2048 + 16 * (r >> 2) + 4 * j + (r & 3)] = (uint8_t)se;
  }
}

// ---------------------------------------------------------------------------
// decode: one workgroup per (sequence, KV head, split), four wavefronts
// ---------------------------------------------------------------------------
struct AttnLds {
  uint8_t qt[2048];           // the group's quantized queries as the A operand tile (rows >= G zero)
  uint8_t qs[64];             // their scale bytes, byte l = (head l % 16, block l / 16)
  float m[4][MAXG], l[4][MAXG];
  float o[4][MAXG][HD];
  int ids[MAXCHUNK];          // physical pages of this split
  int len[256];               // sequence lengths (for the work order)
};

// (four wavefronts per SIMD: 118 registers, no spills; 3 per SIMD measured 5 % slower)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void attn_decode_kernel(AttnArgs a) {
  __shared__ AttnLds L;
  const int l = lane_id(), wv = (int)(threadIdx.x >> 6);
  const int S = a.S;
  const int split = blockIdx.x % S;
  int bh = blockIdx.x / S;
  const int Tmax = a.max_pages * PSLOTS;
  if (S == 1 && a.B <= MAXB_ORDER) {
    // Work order by length: workgroup w < half takes the w-th longest
    // (sequence, KV head) pair and workgroup half + w the w-th shortest.
    // When every workgroup is resident, w and half + w tend to share a
    // compute unit, which then holds about twice the mean length.
    for (int t = threadIdx.x; t < a.B; t += 256) {
      const int v = a.lens[t];
      L.len[t] = v < 0 ? 0 : (v > Tmax ? Tmax : v);
    }
    __syncthreads();
    for (int t = threadIdx.x; t < a.B; t += 256) {
      const int lt = L.len[t];
      int rank = 0;
      for (int u = 0; u < a.B; ++u) rank += (L.len[u] > lt || (L.len[u] == lt && u < t)) ? 1 : 0;
      L.ids[rank] = t;  // (sequences by length, longest first; ties by index)
    }
    __syncthreads();
    const int n = a.B * a.Hkv, half = (n + 1) / 2;
    const int r = bh < half ? bh : n - 1 - (bh - half);
    bh = L.ids[r / a.Hkv] * a.Hkv + r % a.Hkv;
    __syncthreads();  // (the page ids below overwrite the order)
  }
  const int b = bh / a.Hkv, kvh = bh - b * a.Hkv;
  const int G = a.G;
  int T = a.lens[b];
  T = T < 0 ? 0 : (T > Tmax ? Tmax : T);
  const int npages = (T + PSLOTS - 1) / PSLOTS;
  const int p0 = split * a.chunk, p1 = min(npages, p0 + a.chunk);

  // the group's queries, quantized (MX, 32-dim blocks) into the A tile
  for (int i = threadIdx.x; i < 2048 / 16; i += 256) reinterpret_cast<uint4*>(L.qt)[i] = make_uint4(0u, 0u, 0u, 0u);
  if (threadIdx.x < 64) L.qs[threadIdx.x] = 127u;  // (rows >= G: zero codes, unit scale)
  // the split's page ids, staged once (so that no load of the page loop
  // depends on another load)
  for (int i = p0 + (int)threadIdx.x; i < p1; i += 256) L.ids[i - p0] = a.bt[(size_t)b * a.max_pages + i];
  __syncthreads();
  if (wv == 0 && l < 4 * G) {  // (lanes of a head are four consecutive ones, all active)
    const int g = l >> 2, j = l & 3;
    const uint4* src = reinterpret_cast<const uint4*>(a.q + ((size_t)b * a.Hq + (size_t)kvh * G + g) * HD + 32 * j);
    float v[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 w = src[c];
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * c + 2 * e] = bf16_to_f32(ww[e] & 0xFFFFu);
        v[8 * c + 2 * e + 1] = bf16_to_f32(ww[e] >> 16);
      }
    }
    uint32_t cw[8], se = 0;
    float sf = 1.0f;
    quant_block32<FMT_MX>(v, cw, &sf, &se);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int s = 2 * j + u;
      *reinterpret_cast<uint4*>(L.qt + (s >> 2) * 1024 + (g + 16 * (s & 3)) * 16) =
          make_uint4(cw[4 * u], cw[4 * u + 1], cw[4 * u + 2], cw[4 * u + 3]);
    }
    L.qs[g + 16 * j] = (uint8_t)se;
  }
  __syncthreads();
  const v8i qa = make_v8i(*reinterpret_cast<const uint4*>(L.qt + l * 16),
                          *reinterpret_cast<const uint4*>(L.qt + 1024 + l * 16));
  const int qsc = L.qs[l];

  // Everything is computed transposed, so that no value crosses lanes
  // through LDS: the scores as K Q^T (slots x heads), whose accumulator
  // layout (lane l: head l % 16, slots 4(l/16)..+3) is the B operand layout
  // of p^T in o^T = V^T p^T, and o^T's (lane l: head l % 16, dims
  // 16n + 4(l/16) + rr) keeps each head's rescale in its own lanes.  Per lane:
  // the running max and sum of head l % 16 (alike in its four lane groups).
  const int q4 = 4 * (l >> 4);
  float mh = -INFINITY, lh = 0.0f;
  v4f o[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) o[n] = v4f{0.f, 0.f, 0.f, 0.f};

  const uint32_t cache_bytes = (uint32_t)a.n_pages * (uint32_t)a.Hkv * (uint32_t)PAGE_BYTES;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.kc, cache_bytes), rv = make_rsrc(a.vc, cache_bytes);
  struct Slot {
    v8i k;
    uint32_t ks;
    uint4 v0, v1;
    uint4 vs;
  } R[RING];
  auto issue = [&](int u, int p) {
    uint32_t base = 0x80000000u;  // (past the cache: reads zero)
    if (p < p1) {
      const int phys = L.ids[p - p0];
      if (phys >= 0 && phys < a.n_pages) base = ((uint32_t)phys * (uint32_t)a.Hkv + (uint32_t)kvh) * PAGE_BYTES;
    }
    const bool in = base != 0x80000000u;
    R[u].k = make_v8i(__builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, in ? base + l * 16 : base, 0, AUX_NT)),
                      __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, in ? base + 1024 + l * 16 : base, 0, AUX_NT)));
    R[u].ks = __builtin_amdgcn_raw_buffer_load_b8(rk, in ? base + 2048 + l : base, 0, 0);
    R[u].v0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, in ? base + l * 32 : base, 0, AUX_NT));
    R[u].v1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, in ? base + l * 32 + 16 : base, 0, AUX_NT));
    R[u].vs = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, in ? base + 2048 + 16 * (l >> 4) : base, 0, 0));  // (this lane group's slots)
  };
  // Each page is taken on its own: its scores, one online-softmax update,
  // then o^T += V^T p^T; its slot is refilled with the page RING steps ahead
  // right after, so the loads of the next RING - 1 pages stay in flight
  // while a page is worked on.
  auto page_step = [&](int u, int pg) {
    // scores (log2 units): slots 4(l/16)+j of page pg against head l % 16
    const v4f z = {0.f, 0.f, 0.f, 0.f};
    const v4f sc = mfma_f8(R[u].k, qa, z, (int)R[u].ks, qsc);
    float sv[4], mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool live = pg * PSLOTS + q4 + j < T;
      sv[j] = live ? sc[j] * a.qk_scale : -INFINITY;
      mx = fmaxf(mx, sv[j]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(mh, mx);  // (finite: slot 0 of the page is live)
    const float al = exp2f(mh - mn);
    float pr[4], sm = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pr[j] = sv[j] == -INFINITY ? 0.0f : exp2f(sv[j] - mn);
      sm += pr[j];
    }
    sm += __shfl_xor(sm, 16, 64);
    sm += __shfl_xor(sm, 32, 64);
    lh = lh * al + sm;
    mh = mn;
#pragma unroll
    for (int n = 0; n < 8; ++n) o[n] *= al;
    // o^T += V^T p^T on the matrix unit: A = V's codes (dim 16n + l % 16,
    // slots 4(l/16)..+3), B = p (head l % 16, the same slots) times V's
    // scale of (slot, 32-dim block), one operand per block.  Slots past the
    // length have p = 0 and zeroed codes (a stale slot may hold NaN codes).
    const uint32_t vsw[4] = {R[u].vs.x, R[u].vs.y, R[u].vs.z, R[u].vs.w};
    v4s pb[4];
#pragma unroll
    for (int bk = 0; bk < 4; ++bk) {
      v4bf t;
#pragma unroll
      for (int j = 0; j < 4; ++j) t[j] = (__bf16)__builtin_amdgcn_ldexpf(pr[j], (int)((vsw[bk] >> (8 * j)) & 0xFFu) - 127);
      pb[bk] = __builtin_bit_cast(v4s, t);
    }
    const int live = T - (pg * PSLOTS + q4);  // slots of this lane group within the length
    const uint32_t keep = live >= 4 ? 0xFFFFFFFFu : live <= 0 ? 0u : (0xFFFFFFFFu >> (8 * (4 - live)));
    const uint32_t vw[8] = {R[u].v0.x, R[u].v0.y, R[u].v0.z, R[u].v0.w, R[u].v1.x, R[u].v1.y, R[u].v1.z, R[u].v1.w};
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const uint32_t w = vw[n] & keep;
      const v2bf b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
      const v2bf b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
      const v4bf av = {b0[0], b0[1], b1[0], b1[1]};
      o[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4s, av), pb[n >> 1], o[n], 0, 0, 0);
    }
  };
  int p = p0 + wv;
#pragma unroll
  for (int u = 0; u < RING; ++u) issue(u, p + 4 * u);
  for (; p < p1; p += 4 * RING) {
#pragma unroll
    for (int u = 0; u < RING; ++u) {
      const int pg = p + 4 * u;
      if (pg < p1) page_step(u, pg);
      issue(u, pg + 4 * RING);
    }
  }

  // merge the four wavefronts into the split's partial
  const int h = l & 15;
  if (l < 16) {
    L.m[wv][h] = mh;
    L.l[wv][h] = lh;
  }
  if (h < G) {
#pragma unroll
    for (int n = 0; n < 8; ++n)
      *reinterpret_cast<v4f*>(&L.o[wv][h][16 * n + q4]) = o[n];
  }
  __syncthreads();
  float* part = a.part + (size_t)blockIdx.x * G * (2 + HD);
  for (int i = threadIdx.x; i < G * HD; i += 256) {
    const int g = i / HD, dd = i - g * HD;
    float M = L.m[0][g];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, L.m[w][g]);
    float acc = 0.0f, sum = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = L.m[w][g] == -INFINITY ? 0.0f : exp2f(L.m[w][g] - M);
      acc += L.o[w][g][dd] * f;
      sum += L.l[w][g] * f;
    }
    if (S == 1) {
      // one split: the output itself (the merge kernel's arithmetic for a
      // single partial; a sequence of length 0 gives zeros)
      const float inv = sum > 0.0f ? 1.0f / sum : 0.0f;
      a.out[((size_t)b * a.Hq + (size_t)kvh * G + g) * HD + dd] = (uint16_t)f32_to_bf16(acc * inv);
      continue;
    }
    part[g * (2 + HD) + 2 + dd] = acc;
    if (dd == 0) {
      part[g * (2 + HD)] = M;
      part[g * (2 + HD) + 1] = sum;
    }
  }
}

// The splits of each (sequence, query head) merged: one wavefront each, two
// dims per lane.  A sequence of length 0 gives zeros.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const long long wave = ((long long)blockIdx.x * 256 + threadIdx.x) >> 6;
  if (wave >= (long long)a.B * a.Hq) return;
  const int l = lane_id();
  const int b = (int)(wave / a.Hq), h = (int)(wave - (long long)b * a.Hq);
  const int kvh = h / a.G, g = h - kvh * a.G;
  const size_t stride = (size_t)a.G * (2 + HD);
  const float* base = a.part + ((size_t)b * a.Hkv + kvh) * a.S * stride + (size_t)g * (2 + HD);
  float M = -INFINITY;
  for (int s = 0; s < a.S; ++s) M = fmaxf(M, base[s * stride]);
  float o0 = 0.0f, o1 = 0.0f, sum = 0.0f;
  if (M != -INFINITY) {
    for (int s = 0; s < a.S; ++s) {
      const float m = base[s * stride];
      if (m == -INFINITY) continue;
      const float f = exp2f(m - M);
      sum += base[s * stride + 1] * f;
      o0 += base[s * stride + 2 + 2 * l] * f;
      o1 += base[s * stride + 2 + 2 * l + 1] * f;
    }
  }
  const float inv = sum > 0.0f ? 1.0f / sum : 0.0f;
  const uint32_t w = f32_to_bf16(o0 * inv) | (f32_to_bf16(o1 * inv) << 16);
  reinterpret_cast<uint32_t*>(a.out + ((size_t)b * a.Hq + h) * HD)[l] = w;
}

int attn_splits(int B, int Hkv, int max_pages) {
  // about 512 workgroups (two per compute unit; four fit, and every split
  // adds a prologue, a merge and the second kernel: measured at batch 64 with
  // 8 KV heads, 1 split 86 us, 2 splits 91-93, 4 splits 95-97, 8 splits 101),
  // splits of at least 8 pages (128 tokens) and at most MAXCHUNK
  int s = (512 + B * Hkv - 1) / (B * Hkv);
  const int by_len = (max_pages + 7) / 8;
  if (s > by_len) s = by_len;
  if (s > 64) s = 64;
  const int need = (max_pages + MAXCHUNK - 1) / MAXCHUNK;
  if (s < need) s = need;
  return s < 1 ? 1 : s;
}

}  // namespace

size_t attn_workspace_bytes(int B, int Hq, int Hkv, int max_pages) {
  const int S = attn_splits(B, Hkv, max_pages);
  return (size_t)B * Hkv * S * (size_t)(Hq / Hkv) * (2 + HD) * sizeof(float);
}

int launch_kv_write(int kind, const uint16_t* x, const int32_t* slots, int n, int Hkv, uint8_t* cache, int n_pages,
                    hipStream_t s) {
  const long long lanes = (long long)n * Hkv * 4;
  hipLaunchKernelGGL(kv_write_kernel, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, s, kind, x, slots, n, Hkv,
                     cache, n_pages);
  return hip_status(hipGetLastError());
}

int launch_paged_decode(const uint16_t* q, const uint8_t* kc, const uint8_t* vc, int n_pages, const int32_t* bt,
                        int max_pages, const int32_t* lens, int B, int Hq, int Hkv, float sm_scale, uint16_t* out,
                        void* ws, hipStream_t s) {
  AttnArgs a{};
  a.q = q;
  a.kc = kc;
  a.vc = vc;
  a.bt = bt;
  a.lens = lens;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.max_pages = max_pages;
  a.n_pages = n_pages;
  a.S = attn_splits(B, Hkv, max_pages);
  a.chunk = (max_pages + a.S - 1) / a.S;
  a.qk_scale = sm_scale * LOG2E;
  a.part = static_cast<float*>(ws);
  a.out = out;
  const dim3 grid((unsigned)(B * Hkv * a.S));
  hipLaunchKernelGGL(attn_decode_kernel, grid, dim3(256), 0, s, a);
  int rc = hip_status(hipGetLastError());
  if (rc || a.S == 1) return rc;  // (one split: the decode kernel wrote the output)
  const long long waves = (long long)B * Hq;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, a);
  return hip_status(hipGetLastError());
}

}  // namespace sgd

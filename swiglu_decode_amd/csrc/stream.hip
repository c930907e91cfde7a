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
// How (gfx950).  At decode shapes (M <= 128) the work is a stream of HBM
// weight bytes into the matrix cores, and the time goes to keeping that
// stream full and to the few points where workgroups must wait for each
// other.  One persistent kernel, one workgroup per compute unit, a static
// schedule:
//   * A weight "band" is 16 rows of ffn for gate and up together (GU), or 32
//     output columns of the second GEMM (DN: the down projection, or the
//     plain GEMM's weight).  A band's k-tiles are cut into chunks of P
//     k-tiles; each phase's chunks are dealt to workgroups in equal
//     contiguous ranges, and within a workgroup round-robin to its streaming
//     wavefronts.
//   * Streaming wavefronts only load and multiply.  Each keeps a ring of P
//     slots (two 16x128 weight tiles with their scales and the matching
//     activation tile) in flight; a chunk's refills load the next chunk.  At
//     the end of a band each streaming wavefront hands its partial sums to
//     the workgroup's sync wavefront through LDS and goes on streaming: it
//     never waits for memory writes.
//   * The sync wavefront does everything that crosses workgroups: it
//     quantizes its share of x, sums the streaming wavefronts' partials,
//     combines the split-K partials of a band shared with a neighbouring
//     workgroup (the last to arrive sums all of them in workgroup order, so
//     results do not depend on timing), applies SiLU(gate)*up, re-quantizes
//     each finished 128-column group of the product, raises the flags the
//     second GEMM waits on, and writes the output.
// Flags are written once per XCD (eight copies) so that at most the
// workgroups of one XCD poll a cache line.  Every wait is on work that some
// workgroup does before waiting itself, and all workgroups are resident
// (the grid never exceeds what fits at once), so the waits always end.
// Flags hold the number of the launch that raised them, and each counter is
// zeroed by its last arriver, so the next launch (or graph replay) finds the
// control block ready without a clearing pass at the end of this one.
#include "sgd_act.hpp"
#include "sgd_device.hpp"
#include "sgd_host.hpp"

#include <mutex>

namespace sgd {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));


// Per row-tile count MT (M rows padded to 16*MT): streaming wavefronts per
// workgroup, ring depth (= k-tiles per chunk), LDS partial-sum slots.
template <int MT>
struct Cfg {
  static constexpr int NS = MT >= 4 ? 3 : 7;
  // (one row tile: 2 k-tiles per chunk measured 0.1-0.5 us faster than 4,
  // with fewer bytes queued in HBM ahead of each synchronisation)
  static constexpr int P = MT == 4 ? 4 : 2;
  static constexpr int NSLOT = MT >= 8 ? 1 : 2;
  static constexpr int NWAVE = NS + 1;
  // ring slots (= k-tiles per chunk) of the MLP's second GEMM (deeper rings,
  // that would prefetch a workgroup's whole share of it while Q(a) is not
  // ready, measured slower: their traffic competes with the last gate/up
  // loads, which are on the critical path)
  static constexpr int PD = P;
  // Gate/up with the activations staged in LDS (row tiles of 64 and 128
  // rows, when every workgroup holds at most NS whole bands): each streaming
  // wavefront owns one band over all of K with a PG-deep weight ring, and
  // the sync wavefront stages Q(x) one k-tile at a time into DA LDS stages
  // that all streaming wavefronts read.
  static constexpr bool KS = MT >= 4;
  static constexpr int PG = 8;
  static constexpr int DA = 4;
  // k-tiles of Q(x) the sync wavefront keeps in flight while staging (their
  // copies within the 63 loads a wavefront can track, and fewer than DA)
  static constexpr int LD = 3;
  // Staged gate/up on the scaled fp8 matrix instruction instead of widening
  // to bf16 (format FMT; see gu_f8).
  template <int FMT>
  static constexpr bool gu_f8() {
    // With one wavefront per SIMD the widening and the bf16 products (2,600
    // cycles per k-tile against 1,024 of matrix work at 128 rows) paced the
    // loop as much as the staging did; fp8 products take a quarter of that.
    // Their coarser sums move the error against the oracle from 1.7e-3 to
    // 2.0-2.2e-3 at 64-128 rows.  Block-scaled weights at 64 rows (the
    // 24-layer decode stack) keep the widened products: there the fp8 sums
    // put the stack's logits outside the spread of equally valid results
    // (depth 1: 1.9e-3 against 5.4e-4).  (The outlier widths, ffn = 13824,
    // hold more bands than the staged schedule takes: bf16 path.)
    return MT >= 8 || (MT >= 4 && FMT == FMT_MX);
  }
};

// One LDS stage of staged gate/up activations: per m-tile the 2 KB operand
// tile in lane order (lane l's 32 bytes at l*16 and 1024 + l*16), then the
// k-tile's row scales (block: fp32 per row; mx: the dword of a row's four
// E8M0 bytes), 16*MT entries of 4 bytes.
template <int MT>
__host__ __device__ constexpr int ks_stage_bytes() { return MT * 2048 + MT * 64; }

struct Phase {
  int KT;       // k-tiles of the weight's K
  int CPB;      // chunks per band, ceil(KT / P)
  int nbands;   // GU: ffn / 16; DN: N / 32
  int nchunks;  // nbands * CPB
  int nwg;      // workgroups the chunks are dealt to
  int nunits;   // ranges are dealt in units of upc chunks: nunits * upc = nchunks
  int upc;      // (upc = CPB: whole bands, no band shared by two workgroups; 1: chunks)
};

struct Args {
  int M, Mpad, mlp;
  const uint16_t* x;         // [M, K1] bf16
  int K1;
  const uint8_t* wg;         // gate / up packed codes [F, K1] (MLP)
  const void* sg;
  const uint8_t* wu;
  const void* su;
  int F;
  const uint8_t* w2;         // second GEMM weight [N, K2]
  const void* s2;
  int N, K2;
  uint16_t* y;               // [M, N] bf16 (when y32 and h_out are null)
  float* y32;                // [M, N] fp32 output instead, or null
  // Decode block (the MLP with its RMSNorm prologue and residual epilogue):
  // x = bf16(RMSNorm(h_in)) is formed in the kernel and the output is
  // h_out = fl32(h_in + bf16(y)) instead of y.  Null for the plain MLP.
  const float* h_in;         // [M, K1] fp32 residual stream
  float* h_out;              // [M, N] fp32, not overlapping h_in
  float eps;
  int row_stash;             // the dynamic LDS holds a row of h_in (K1 floats) for the prologue
  int row_parts;             // workgroups that share a row's prologue
  uint32_t* ctrl;
  uint8_t* xa;               // codes of Q(x) [M, K1]
  void* xs;                  // x scales: block fp32 [K1/128][Mpad]; mx u8 [M][K1/32]
  float* a32;                // [M, F] silu(g) * u
  uint8_t* aq;               // [M, F] codes of Q(a)
  void* as;                  // block fp32 [F/128][Mpad]; mx u8 [M][F/32]
  float* gpart;              // split-K partials of shared GU bands: [G][2 sides] slots
  float* dpart;              // split-K partials of shared DN bands: [G][2 sides] slots
  float* amax;               // staged gate/up: [F/16][Mpad] each band's per-row max |a| over its 16 columns
  uint32_t scale_bytes_g, scale_bytes_2;  // packed weight-scale sizes
  int G;                     // workgroups in the grid
  int n_pairs, n_items;      // x quantization: (k-group, row tile) pairs, dealt into items
  int ngroups;               // F / 128
  int ks;                    // gate/up with LDS-staged activations (Cfg::KS variants)
  int keep_a;                // staged gate/up: also store a for inspection
  uint64_t budget;           // longest a wait may spin, in ticks of the 100 MHz real-time counter
  Phase gu, dn;
};

// Control block (32-bit words).  Page r (r < NREP) holds XCD copy r of the
// x-quantization flags and of the group-ready flags.
constexpr int C_DONE = 0;
// Launches completed on this control block.  Flags are raised with the
// current launch's number (C_EPOCH + 1) rather than 1, so they never need
// clearing; every counter is zeroed by its own last arriver.  The last
// workgroup then only advances C_EPOCH and zeroes C_DONE.
constexpr int C_EPOCH = 64;
// A wait that spins longer than Args::budget gives up: it adds one to C_ERR
// (sticky until the workspace is cleared; the host reads it) and stores the
// launch number in C_ERR_EP, which ends every other wait of that launch at
// once.  The launch then runs to its end on whatever data it has, so every
// wavefront exits normally; its outputs are invalid.
constexpr int C_ERR = CTRL_ERR_WORD, C_ERR_EP = CTRL_ERR_WORD + 1;
constexpr int PAGE0 = 1024, PAGE_WORDS = 1024, NREP = 8;
constexpr int PG_XQ = 0, PG_RDY = 512;
constexpr int C_GCNT = PAGE0 + NREP * PAGE_WORDS;  // arrivals of 16-column bands per group
constexpr int C_GPCNT = C_GCNT + 512;              // arrivals on shared GU bands
constexpr int C_DPCNT = C_GPCNT + 2048;            // arrivals on shared DN bands
constexpr int CTRL_WORDS = 65536;
constexpr size_t CTRL_BYTES = (size_t)CTRL_WORDS * 4;
static_assert(CTRL_BYTES == CONTROL_BLOCK_BYTES, "control block size");
constexpr int MAX_ITEMS = 512, MAX_GROUPS = 512, MAX_GBANDS = 2048;
// staged gate/up: flag of band b (its row maxima are published), the last words
constexpr int C_BFLAG = CTRL_WORDS - MAX_GBANDS;
// Workgroups a grid may have; the workspace holds two partial-sum slots for each.
constexpr int MAX_WG = 512;
constexpr uint32_t OOB = 0x80000000u;  // a buffer offset past every buffer's end

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
// This launch's number (flags raised in it hold this value).
__device__ __forceinline__ uint32_t launch_epoch(const Args& a) { return load_agent(&a.ctrl[C_EPOCH]) + 1u; }

// ---------------------------------------------------------------------------
// static schedule
// ---------------------------------------------------------------------------
__device__ __forceinline__ int range_start(const Phase& ph, int W) {
  return (int)(((long long)W * ph.nunits) / ph.nwg) * ph.upc;
}
// The workgroup whose range holds chunk c.
__device__ __forceinline__ int owner_wg(const Phase& ph, int c) {
  int W = (int)(((long long)c * ph.nwg) / ph.nchunks);
  while (W + 1 < ph.nwg && range_start(ph, W + 1) <= c) ++W;
  return W;
}
// Which of its two partial slots workgroup W uses for band b (0: the band
// its range starts in, 1: the band it ends in).
__device__ __forceinline__ int band_side(const Phase& ph, int W, int b) {
  return b == range_start(ph, W) / ph.CPB ? 0 : 1;
}

struct ChunkPos {
  int ok;    // a real chunk (else every load is a filler)
  int band;
  int kt0;   // first k-tile
};

template <int P>
__device__ __forceinline__ ChunkPos chunk_pos(const Phase& ph, int c, int c1) {
  ChunkPos p{0, 0, 0};
  if (c < c1) {
    p.ok = 1;
    p.band = c / ph.CPB;
    p.kt0 = (c - p.band * ph.CPB) * P;
  }
  return p;
}

// ---------------------------------------------------------------------------
// LDS shared by a workgroup's wavefronts
// ---------------------------------------------------------------------------
template <int MT, int NS, int NSLOT>
struct Lds {
  v4f part[NSLOT][NS][2][MT][64];  // per band: each streaming wavefront's accumulators
  uint32_t arrived[NSLOT];         // streaming wavefronts that filled the slot
  uint32_t consumed;               // band events the sync wavefront has taken
  uint32_t xq_ok;                  // Q(x) complete
  uint32_t rdy[MAX_GROUPS / 32];   // bit g: group g of Q(a) (k-tile g of the second GEMM) is ready
  uint32_t a_ready;                // staged gate/up: k-tiles of Q(x) staged so far
  uint32_t prog[NS];               // staged gate/up: k-tiles each streaming wavefront has used
  uint32_t gu_left;                // streaming wavefronts done with gate/up (band finishing included)
  uint32_t abort;                  // a wait of this workgroup gave up: every other wait ends at once
  float red[4];                    // decode-block prologue: the four wavefront sums of squares
};

__device__ __forceinline__ uint32_t lds_load(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_store(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// ---------------------------------------------------------------------------
// Bounded waiting.  Every spin of the kernel carries a Guard: the
// workgroup's LDS abort word and the launch's budget.  A wait whose budget
// runs out (workgroups that are not all resident at once, e.g. beside another
// persistent launch) gives up: it records the failure in the control block
// (C_ERR, C_ERR_EP) and in the abort word, and returns.  After that every
// wait of the workgroup, and every cross-workgroup wait of the launch,
// returns at once, so the kernel always runs to its end.
// ---------------------------------------------------------------------------
struct Guard {
  uint32_t* abort;  // LDS
  uint32_t* ctrl;
  uint64_t budget;  // ticks of the 100 MHz real-time counter
  uint32_t ep;      // this launch's number
};

__device__ __forceinline__ void give_up(const Guard& g) {
  if (lane_id() == 0) {
    lds_store(g.abort, 1u);
    atomic_add_agent(g.ctrl + C_ERR, 1u);
    store_agent(g.ctrl + C_ERR_EP, g.ep);
  }
}

// Checked every 16th pass of a spin that polls LDS: true when the wait must
// end (the workgroup gave up, or this wait outlived the budget; t0 is taken
// on the first check).
__device__ __forceinline__ bool must_stop(const Guard& g, uint32_t& pass, uint64_t& t0) {
  if ((++pass & 15u) != 0u) return false;
  if (lds_load(g.abort)) return true;
  const uint64_t t = wall_clock64();
  if (t0 == 0) t0 = t;
  if (t - t0 > g.budget) {
    give_up(g);
    return true;
  }
  return false;
}

__device__ __forceinline__ void lds_wait_geq(const Guard& g, const uint32_t* p, uint32_t target) {
  uint32_t pass = 0;
  uint64_t t0 = 0;
  while (lds_load(p) < target) {
    if (must_stop(g, pass, t0)) return;
    __builtin_amdgcn_s_sleep(1);
  }
}

// ---------------------------------------------------------------------------
// Streaming wavefront
// ---------------------------------------------------------------------------
// LDS copy of Q(x) (used when it fits): codes [Mpad][K1 + 16] (rows padded
// by 16 bytes so the 16 rows of an operand load fall in distinct banks), then
// the scales: block fp32 [K1/128][Mpad]; mx E8M0 [Mpad][K1/32].
__host__ __device__ constexpr int xl_row_stride(int K1) { return K1 + 16; }
__host__ __device__ constexpr int xl_scale_offset(int Mpad, int K1) { return Mpad * (K1 + 16); }
__host__ __device__ constexpr int xl_bytes(int fmt, int Mpad, int K1) {
  return xl_scale_offset(Mpad, K1) + (fmt == FMT_BLOCK ? (K1 / 128) * Mpad * 4 : Mpad * (K1 / 32));
}

// One wavefront's ring of P slots: weights of stream 0/1 and their scale
// words (block: fp32 bits in S0; mx: S0/S1 = dwords holding this lane's two
// 32-column-block scales for gate/up, its own scale slot for the second
// GEMM), fp8 activations (one 32-byte operand per m-tile) and their scales
// (block: rows 4*(l/16)..+3 as v4f; mx, in X0: gate/up: the dword of the
// four 32-column-block scales of this lane's row, second GEMM: this lane's
// own block scale byte).  Each phase has a ring of its own.
// The three phases a streaming wavefront runs: the MLP's gate/up product,
// the MLP's second GEMM (activations: Q(a)), and the plain GEMM (Q(x)).
constexpr int PK_GU = 0, PK_DN = 1, PK_GEMM = 2;

template <int MT, int P>
struct Ring {
  v8i RB[P][2];
  uint32_t S0[P][2], S1[P][2];
  v8i RA[P][MT];
  v4f XB[P][MT];
  uint32_t X0[P][MT];
};

template <int MT, int FMT>
__device__ void finish_gu_band(const Args& a, int b, v4f (&s)[2][MT], uint32_t ep);
struct Guard;
template <int MT, int FMT>
__device__ void finish_gu_band_staged(const Args& a, int b, v4f (&s)[2][MT], uint32_t ep, const Guard& gd);

template <int MT, int FMT, int P, int XL>
struct Streamer {
  const Args& a;
  const int q;  // index among the workgroup's streaming wavefronts
  const uint8_t* lx;  // LDS copy of Q(x) (XL)
  const Guard gd;
  // buffer resources of the current phase
  __amdgpu_buffer_rsrc_t rw0, rw1, rs0, rs1, rx, rxs;
  // lane constants
  uint32_t lo16;                   // l * 16
  uint32_t mo_gu0, mo_gu1, mo_dn;  // mx weight-scale lane offsets (bytes)
  uint32_t xsh;                    // mx gate/up: bit offset of this lane's first block scale in X0
  uint32_t xs_lane;                // block format: activation-scale lane offset (bytes)

  __device__ Streamer(const Args& args, int wq, const uint8_t* lds_x, const Guard& g)
      : a(args), q(wq), lx(lds_x), gd(g) {
    const int l = lane_id();
    lo16 = (uint32_t)l * 16u;
    mo_gu0 = ((uint32_t)(l & 15) + 16u * (uint32_t)((l >> 4) >> 1)) * 4u;
    mo_gu1 = ((uint32_t)(l & 15) + 16u * (2u + (uint32_t)((l >> 4) >> 1))) * 4u;
    mo_dn = (uint32_t)l * 4u;
    // gate/up lanes use blocks (l/16)/2 and 2 + (l/16)/2 of their k-tile
    xsh = 8u * (uint32_t)((l >> 4) >> 1);
    xs_lane = 16u * (uint32_t)(l >> 4);
  }

  template <int PK>
  __device__ __forceinline__ void make_resources() {
    const bool gu = PK == PK_GU;
    const uint32_t KT1 = (uint32_t)(a.K1 >> 7);
    const uint32_t xs_bytes = FMT == FMT_BLOCK ? KT1 * (uint32_t)a.Mpad * 4u : (uint32_t)a.M * (KT1 * 4u);
    if (gu) {
      const uint32_t bytes_g = (uint32_t)a.F * (uint32_t)a.K1;
      rw0 = make_rsrc(a.wg, bytes_g);
      rw1 = make_rsrc(a.wu, bytes_g);
      rs0 = make_rsrc(a.sg, a.scale_bytes_g);
      rs1 = make_rsrc(a.su, a.scale_bytes_g);
      rx = make_rsrc(a.xa, (uint32_t)a.M * (uint32_t)a.K1);
      rxs = make_rsrc(a.xs, xs_bytes);
    } else {
      rw0 = rw1 = make_rsrc(a.w2, (uint32_t)a.N * (uint32_t)a.K2);
      rs0 = rs1 = make_rsrc(a.s2, a.scale_bytes_2);
      if (PK == PK_DN) {
        rx = make_rsrc(a.aq, (uint32_t)a.M * (uint32_t)a.F);
        rxs = make_rsrc(a.as, FMT == FMT_BLOCK ? (uint32_t)(a.F >> 7) * (uint32_t)a.Mpad * 4u
                                              : (uint32_t)a.M * (uint32_t)(a.F >> 5));
      } else {
        rx = make_rsrc(a.xa, (uint32_t)a.M * (uint32_t)a.K1);
        rxs = make_rsrc(a.xs, xs_bytes);
      }
    }
  }

  static __device__ __forceinline__ uint4 ld4(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
  }
  // Weight codes are read once per launch: non-temporal loads, so that the
  // stream does not evict what is reused (the kernel's code, the scales, the
  // activations and the control block) from L2 and the Infinity Cache.  Those
  // misses would otherwise wait behind the weight stream in the HBM queues
  // (measured: 37.4 -> 34.8 us at M=1, d=4096 MXFP8).
  static __device__ __forceinline__ uint4 ld4_stream(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, AUX_NT));
  }

  // ---- loads of one ring slot (unconditional: fillers read past the end) ----
  template <bool GU, class Rg, bool F8 = false>
  __device__ __forceinline__ void load_b(Rg& R, int s, const ChunkPos& cp, int KT, int k) {
    const int kt_ = cp.kt0 + k;
    const bool ok = cp.ok && kt_ < KT;
    const uint32_t kt = ok ? (uint32_t)kt_ : 0u;
    const uint32_t n0 = GU ? (uint32_t)cp.band : 2u * (uint32_t)cp.band;
    const uint32_t n1 = GU ? (uint32_t)cp.band : 2u * (uint32_t)cp.band + 1u;
    const uint32_t uKT = (uint32_t)KT;
    const uint32_t t0 = ok ? (n0 * uKT + kt) * 2048u + lo16 : OOB;
    const uint32_t t1 = ok ? (n1 * uKT + kt) * 2048u + lo16 : OOB;
    R.RB[s][0] = make_v8i(ld4_stream(rw0, t0), ld4_stream(rw0, t0 + 1024u));
    R.RB[s][1] = make_v8i(ld4_stream(rw1, t1), ld4_stream(rw1, t1 + 1024u));
    if (FMT == FMT_BLOCK) {
      const uint32_t o0 = ok ? ((n0 >> 3) * uKT + kt) * 4u : OOB;
      const uint32_t o1 = ok ? ((n1 >> 3) * uKT + kt) * 4u : OOB;
      R.S0[s][0] = __builtin_amdgcn_raw_buffer_load_b32(rs0, o0, 0, 0);
      R.S0[s][1] = __builtin_amdgcn_raw_buffer_load_b32(rs1, o1, 0, 0);
    } else {
      const uint32_t KG = (uKT + 3u) >> 2;
      const uint32_t g0 = (n0 * KG + (kt >> 2)) * 256u;
      const uint32_t g1 = (n1 * KG + (kt >> 2)) * 256u;
      if (GU && !F8) {
        R.S0[s][0] = __builtin_amdgcn_raw_buffer_load_b32(rs0, ok ? g0 + mo_gu0 : OOB, 0, 0);
        R.S1[s][0] = __builtin_amdgcn_raw_buffer_load_b32(rs0, ok ? g0 + mo_gu1 : OOB, 0, 0);
        R.S0[s][1] = __builtin_amdgcn_raw_buffer_load_b32(rs1, ok ? g1 + mo_gu0 : OOB, 0, 0);
        R.S1[s][1] = __builtin_amdgcn_raw_buffer_load_b32(rs1, ok ? g1 + mo_gu1 : OOB, 0, 0);
      } else {
        R.S0[s][0] = __builtin_amdgcn_raw_buffer_load_b32(rs0, ok ? g0 + mo_dn : OOB, 0, 0);
        R.S0[s][1] = __builtin_amdgcn_raw_buffer_load_b32(rs1, ok ? g1 + mo_dn : OOB, 0, 0);
      }
    }
  }

  template <int PK, int PP, int MLO = 0, int MHI = MT>
  __device__ __forceinline__ void load_a(Ring<MT, PP>& R, int s, const ChunkPos& cp, int KT, int k) {
    constexpr bool GU = PK == PK_GU;
    const int kt_ = cp.kt0 + k;
    const bool ok = cp.ok && kt_ < KT;
    const uint32_t kt = ok ? (uint32_t)kt_ : 0u;
    const uint32_t Kd = PK == PK_DN ? (uint32_t)a.F : (uint32_t)a.K1;
    if (XL && PK != PK_DN) {
      // Q(x) from LDS (fillers read k-tile 0 and are never used)
      const int l = lane_id();
      const int rs = xl_row_stride(a.K1);
      const uint8_t* sc = lx + xl_scale_offset(16 * MT, a.K1);
#pragma unroll
      for (int mt = MLO; mt < MHI; ++mt) {
        const uint8_t* p = lx + (mt * 16 + (l & 15)) * rs + kt * 128 + 16 * (l >> 4);
        R.RA[s][mt] = make_v8i(*reinterpret_cast<const uint4*>(p), *reinterpret_cast<const uint4*>(p + 64));
        if (FMT == FMT_BLOCK) {
          R.XB[s][mt] = *reinterpret_cast<const v4f*>(sc + (kt * (16 * MT) + 16 * mt + 4 * (l >> 4)) * 4);
        } else {
          const uint8_t* e = sc + (mt * 16 + (l & 15)) * (a.K1 >> 5) + 4 * kt;
          R.X0[s][mt] = GU ? *reinterpret_cast<const uint32_t*>(e) : (uint32_t)e[l >> 4];
        }
      }
      return;
    }
    // workspace layout: m-tiles of 16-column segments (act_code_off); lanes
    // whose row is past M read zeros
    const uint32_t r = (uint32_t)(lane_id() & 15), g = (uint32_t)(lane_id() >> 4);
#pragma unroll
    for (int mt = MLO; mt < MHI; ++mt) {
      const int Mt = min(16, a.M - 16 * mt);
      const bool v = ok && (int)r < Mt;
      const uint32_t uMt = (uint32_t)max(Mt, 0);
      const uint32_t o = v ? (uint32_t)mt * 16u * Kd + (kt * 8u + g) * 16u * uMt + r * 16u : OOB;
      R.RA[s][mt] = make_v8i(ld4(rx, o), ld4(rx, v ? o + 64u * uMt : OOB));
      if (FMT == FMT_BLOCK) {
        const uint32_t so = xs_lane + (kt * (uint32_t)a.Mpad + 16u * (uint32_t)mt) * 4u;
        R.XB[s][mt] = ld_coherent_v4f(rxs, ok ? so : OOB);
      } else {
        const uint32_t so = (uint32_t)mt * 16u * (Kd >> 5) + kt * 4u * uMt + r * 4u;
        R.X0[s][mt] = GU ? ld_coherent_u32(rxs, v ? so : OOB) : ld_coherent_u8(rxs, v ? so + g : OOB);
      }
    }
  }

  // ---- one k-step ------------------------------------------------------------
  static __device__ __forceinline__ v8bf widen8(uint32_t d0, uint32_t d1, float scale) {
    const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, scale, false);
    const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, scale, true);
    const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, scale, false);
    const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, scale, true);
    v8bf v;
    v[0] = p0[0]; v[1] = p0[1]; v[2] = p1[0]; v[3] = p1[1];
    v[4] = p2[0]; v[5] = p2[1]; v[6] = p3[0]; v[7] = p3[1];
    return v;
  }

  // Gate/up: fp8 widened to bf16 (exact; MX scale folded in), bf16 MFMA.  The
  // fp8 matrix instruction sums its products in groups of 8 keeping only
  // ~13 bits below the largest product of a group (measured on gfx950); that
  // ~1e-5 relative error would flip fp8 codes of the re-quantized product,
  // while the bf16 instruction's sums are fp32-accurate.
  template <int PP>
  __device__ __forceinline__ void step_gu(Ring<MT, PP>& R, int s, int sa, int kt, v4f (&acc)[2][MT]) {
    const int sh = 8 * (kt & 3);
    v8bf av[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float s0 = 1.0f, s1 = 1.0f;
      if (FMT == FMT_MX) {
        s0 = pow2_pos((int)((R.X0[sa][mt] >> xsh) & 0xFFu) - 127);
        s1 = pow2_pos((int)((R.X0[sa][mt] >> (xsh + 16u)) & 0xFFu) - 127);
      }
      const v8i x = R.RA[sa][mt];
      av[mt][0] = widen8((uint32_t)x[0], (uint32_t)x[1], s0);
      av[mt][1] = widen8((uint32_t)x[2], (uint32_t)x[3], s0);
      av[mt][2] = widen8((uint32_t)x[4], (uint32_t)x[5], s1);
      av[mt][3] = widen8((uint32_t)x[6], (uint32_t)x[7], s1);
    }
    v8bf b[2][4];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float s0 = 1.0f, s1 = 1.0f;
      if (FMT == FMT_MX) {
        s0 = pow2_pos((int)((R.S0[s][nb] >> sh) & 0xFFu) - 127);
        s1 = pow2_pos((int)((R.S1[s][nb] >> sh) & 0xFFu) - 127);
      }
      const v8i w = R.RB[s][nb];
      b[nb][0] = widen8((uint32_t)w[0], (uint32_t)w[1], s0);
      b[nb][1] = widen8((uint32_t)w[2], (uint32_t)w[3], s0);
      b[nb][2] = widen8((uint32_t)w[4], (uint32_t)w[5], s1);
      b[nb][3] = widen8((uint32_t)w[6], (uint32_t)w[7], s1);
    }
    // 32-deep steps outermost: consecutive matrix instructions feed
    // independent accumulators (each accumulator's own order is unchanged)
    if (FMT == FMT_BLOCK) {
      v4f t[2][MT];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) t[nb][mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) t[nb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt][i], b[nb][i], t[nb][mt], 0, 0, 0);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[nb][mt] += t[nb][mt] * (R.XB[sa][mt] * __uint_as_float(R.S0[s][nb]));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            acc[nb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt][i], b[nb][i], acc[nb][mt], 0, 0, 0);
    }
  }

  // Second GEMM: scaled fp8 MFMA (MX scales in the instruction).
  template <int PP, int MLO = 0, int MHI = MT>
  __device__ __forceinline__ void step_dn(Ring<MT, PP>& R, int s, int sa, int kt, v4f (&acc)[2][MT]) {
    const int sh = 8 * (kt & 3);
#pragma unroll
    for (int mt = MLO; mt < MHI; ++mt) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const v8i av = R.RA[sa][mt];
        if (FMT == FMT_BLOCK) {
          const v4f z = {0.f, 0.f, 0.f, 0.f};
          const v4f t = mfma_f8(av, R.RB[s][nb], z, 127, 127);
          acc[nb][mt] += t * (R.XB[sa][mt] * __uint_as_float(R.S0[s][nb]));
        } else {
          acc[nb][mt] = mfma_f8(av, R.RB[s][nb], acc[nb][mt], (int)R.X0[sa][mt], (int)(R.S0[s][nb] >> sh));
        }
      }
    }
  }

  // Second GEMM, one ring slot: the matrix instructions of m-tile group g
  // (NG groups), then that group's refill loads for the next chunk, so the
  // refills go out while the matrix unit works through the rest
  template <int PK, int PP, int G, int NG>
  __device__ __forceinline__ void dn_slot(Ring<MT, PP>& R, int s, int kt, int KT, const ChunkPos& np,
                                          v4f (&acc)[2][MT]) {
    constexpr int LO = G * MT / NG, HI = (G + 1) * MT / NG;
    if (kt < KT) step_dn<PP, LO, HI>(R, s, s, kt, acc);
    load_a<PK, PP, LO, HI>(R, s, np, KT, s);
    if constexpr (G + 1 < NG) dn_slot<PK, PP, G + 1, NG>(R, s, kt, KT, np, acc);
  }

  // Staged gate/up: the weights of band `band` at k-tile kt (ring slot s)
  // times every m-tile of the LDS stage, in the arithmetic of step_gu.
  template <class Rg>
  __device__ __forceinline__ void step_gu_staged(Rg& R, int s, int kt, const uint8_t* st, v4f (&acc)[2][MT]) {
    const int l = lane_id();
    const int sh = 8 * (kt & 3);
    v8bf b[2][4];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float s0 = 1.0f, s1 = 1.0f;
      if (FMT == FMT_MX) {
        s0 = pow2_pos((int)((R.S0[s][nb] >> sh) & 0xFFu) - 127);
        s1 = pow2_pos((int)((R.S1[s][nb] >> sh) & 0xFFu) - 127);
      }
      const v8i w = R.RB[s][nb];
      b[nb][0] = widen8((uint32_t)w[0], (uint32_t)w[1], s0);
      b[nb][1] = widen8((uint32_t)w[2], (uint32_t)w[3], s0);
      b[nb][2] = widen8((uint32_t)w[4], (uint32_t)w[5], s1);
      b[nb][3] = widen8((uint32_t)w[6], (uint32_t)w[7], s1);
    }
    const uint8_t* sc = st + MT * 2048;
    v8bf av[MT][4];
    v4f xb[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const v8i x = make_v8i(*reinterpret_cast<const uint4*>(st + mt * 2048 + l * 16),
                             *reinterpret_cast<const uint4*>(st + mt * 2048 + 1024 + l * 16));
      float s0 = 1.0f, s1 = 1.0f;
      xb[mt] = v4f{1.f, 1.f, 1.f, 1.f};
      if (FMT == FMT_MX) {
        const uint32_t e = reinterpret_cast<const uint32_t*>(sc)[mt * 16 + (l & 15)];
        s0 = pow2_pos((int)((e >> xsh) & 0xFFu) - 127);
        s1 = pow2_pos((int)((e >> (xsh + 16u)) & 0xFFu) - 127);
      } else {
        xb[mt] = *reinterpret_cast<const v4f*>(sc + (16 * mt + 4 * (l >> 4)) * 4);
      }
      av[mt][0] = widen8((uint32_t)x[0], (uint32_t)x[1], s0);
      av[mt][1] = widen8((uint32_t)x[2], (uint32_t)x[3], s0);
      av[mt][2] = widen8((uint32_t)x[4], (uint32_t)x[5], s1);
      av[mt][3] = widen8((uint32_t)x[6], (uint32_t)x[7], s1);
    }
    // (matrix instructions ordered as in step_gu)
    if (FMT == FMT_BLOCK) {
      v4f t[2][MT];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) t[nb][mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) t[nb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt][i], b[nb][i], t[nb][mt], 0, 0, 0);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[nb][mt] += t[nb][mt] * (xb[mt] * __uint_as_float(R.S0[s][nb]));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            acc[nb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt][i], b[nb][i], acc[nb][mt], 0, 0, 0);
    }
  }

  // Staged gate/up on the scaled fp8 matrix instruction (weights and Q(x)
  // straight from their codes, MX scales in the instruction; block scales
  // applied per k-tile as in step_dn).
  template <class Rg>
  __device__ __forceinline__ void step_gu_staged_f8(Rg& R, int s, int kt, const uint8_t* st, v4f (&acc)[2][MT]) {
    const int l = lane_id();
    const int sh = 8 * (kt & 3);
    const uint8_t* sc = st + MT * 2048;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const v8i x = make_v8i(*reinterpret_cast<const uint4*>(st + mt * 2048 + l * 16),
                             *reinterpret_cast<const uint4*>(st + mt * 2048 + 1024 + l * 16));
      if (FMT == FMT_MX) {
        const uint32_t e = reinterpret_cast<const uint32_t*>(sc)[mt * 16 + (l & 15)];
        const int sa = (int)((e >> (8u * (uint32_t)(l >> 4))) & 0xFFu);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[nb][mt] = mfma_f8(x, R.RB[s][nb], acc[nb][mt], sa, (int)(R.S0[s][nb] >> sh));
      } else {
        const v4f xb = *reinterpret_cast<const v4f*>(sc + (16 * mt + 4 * (l >> 4)) * 4);
        const v4f z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const v4f t = mfma_f8(x, R.RB[s][nb], z, 127, 127);
          acc[nb][mt] += t * (xb * __uint_as_float(R.S0[s][nb]));
        }
      }
    }
  }

  // Staged gate/up for this wavefront's band (the q-th of the workgroup's
  // whole bands, if it has one): all k-tiles in order, the activations from
  // the LDS stages, then the band's SiLU, write-out and group accounting.
  template <int NS, int NSLOT>
  __device__ __forceinline__ void run_gu_staged(Lds<MT, NS, NSLOT>& L, const uint8_t* stages) {
    constexpr int PG = Cfg<MT>::PG, DA = Cfg<MT>::DA, SB = ks_stage_bytes<MT>();
    const Phase& ph = a.gu;
    const int W = blockIdx.x;
    if (W >= ph.nwg) return;
    const int band = range_start(ph, W) / ph.CPB + q;
    if (band >= range_start(ph, W + 1) / ph.CPB) return;
    const int KT = ph.KT;
    const uint32_t ep = launch_epoch(a);
    make_resources<PK_GU>();
    constexpr bool F8 = Cfg<MT>::template gu_f8<FMT>();
    struct {
      v8i RB[PG][2];
      uint32_t S0[PG][2], S1[PG][2];
    } R;
    const ChunkPos cp{1, band, 0};
#pragma unroll
    for (int s = 0; s < 2; ++s) load_b<true, decltype(R), F8>(R, s, cp, KT, s);
    // the rest once Q(x) exists: a full prefetch at launch would delay the
    // x quantization and its cross-workgroup flags (measured)
    lds_wait_geq(gd, &L.xq_ok, 1u);
#pragma unroll
    for (int s = 2; s < PG; ++s) load_b<true, decltype(R), F8>(R, s, cp, KT, s);
    v4f acc[2][MT];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[nb][mt] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < KT; k0 += PG) {
#pragma unroll
      for (int s = 0; s < PG; ++s) {
        const int kt = k0 + s;
        if (kt < KT) {
          lds_wait_geq(gd, &L.a_ready, (uint32_t)(kt + 1));
          if (F8)
            step_gu_staged_f8(R, s, kt, stages + (kt % DA) * SB, acc);
          else
            step_gu_staged(R, s, kt, stages + (kt % DA) * SB, acc);
          if (lane_id() == 0) lds_store(&L.prog[q], (uint32_t)(kt + 1));
        }
        load_b<true, decltype(R), F8>(R, s, cp, KT, kt + PG);  // past K: a filler
      }
    }
    finish_gu_band_staged<MT, FMT>(a, band, acc, ep, gd);
  }

  // Wait until the groups of Q(a) that chunk cp reads are ready (its k-tiles
  // lie in one word of the mask: PP divides 32 and k-tiles start at multiples of PP).
  template <int PP, int NS, int NSLOT>
  __device__ __forceinline__ void wait_groups(Lds<MT, NS, NSLOT>& L, const ChunkPos& cp, int KT) const {
    if (!cp.ok) return;
    const int n = min(PP, KT - cp.kt0);
    const uint32_t need = ((1u << n) - 1u) << (cp.kt0 & 31);
    const uint32_t* w = &L.rdy[cp.kt0 >> 5];
    uint32_t pass = 0;
    uint64_t t0 = 0;
    while ((lds_load(w) & need) != need) {
      if (must_stop(gd, pass, t0)) return;
      __builtin_amdgcn_s_sleep(1);
    }
  }

  // Hand this wavefront's sums for band event k to the sync wavefront.
  template <int NS, int NSLOT>
  __device__ __forceinline__ void publish(Lds<MT, NS, NSLOT>& L, int k, v4f (&acc)[2][MT]) {
    const int slot = k % NSLOT;
    if (k >= NSLOT) lds_wait_geq(gd, &L.consumed, (uint32_t)(k - NSLOT + 1));
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) L.part[slot][q][nb][mt][lane_id()] = acc[nb][mt];
    if (lane_id() == 0)
      __hip_atomic_fetch_add(&L.arrived[slot], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  }

  // Stream this workgroup's chunks of one phase.  The ring is filled with the
  // weights of this wavefront's first chunk before `between()` runs (the
  // workgroup-wide x quantization, when there is one; every wavefront calls
  // it exactly once), and with activations after it.
  template <int PK, int PP, int NS, int NSLOT, class Between>
  __device__ __forceinline__ void run_phase(Lds<MT, NS, NSLOT>& L, int& k, Between between) {
    constexpr bool GU = PK == PK_GU;
    const Phase& ph = GU ? a.gu : a.dn;
    const int W = blockIdx.x;
    if (!(W < ph.nwg && range_start(ph, W) < range_start(ph, W + 1))) {
      between();
      return;
    }
    const int c0 = range_start(ph, W), c1 = range_start(ph, W + 1);
    const int KT = ph.KT;
    int c = c0 + q;
    make_resources<PK>();
    Ring<MT, PP> R;
    ChunkPos cp = chunk_pos<PP>(ph, c, c1);
#pragma unroll
    for (int s = 0; s < PP; ++s) load_b<GU>(R, s, cp, KT, s);
    between();
    // activations only once they exist (the LDS copy of Q(x) already does;
    // Q(a) chunk by chunk, as its groups become ready)
    if (PK != PK_DN) {
      if (!XL) lds_wait_geq(gd, &L.xq_ok, 1u);
    } else {
      wait_groups<PP>(L, cp, KT);
    }
#pragma unroll
    for (int s = 0; s < PP; ++s) load_a<PK>(R, s, cp, KT, s);
    const int bf = c0 / ph.CPB, bl = (c1 - 1) / ph.CPB;
    for (int b = bf; b <= bl; ++b) {
      const int hi = min(c1, (b + 1) * ph.CPB);
      v4f acc[2][MT];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nb][mt] = v4f{0.f, 0.f, 0.f, 0.f};
      while (c < hi) {
        const int cn = c + NS;
        const ChunkPos np = chunk_pos<PP>(ph, cn, c1);
        if (PK == PK_DN) wait_groups<PP>(L, np, KT);
#pragma unroll
        for (int s = 0; s < PP; ++s) {
          const int kt = cp.kt0 + s;
          if (GU || MT < 4) {
            if (kt < KT) {
              if (GU)
                step_gu(R, s, s, kt, acc);
              else
                step_dn(R, s, s, kt, acc);
            }
            load_b<GU>(R, s, np, KT, s);
            load_a<PK>(R, s, np, KT, s);
          } else {
            dn_slot<PK, PP, 0, 2>(R, s, kt, KT, np, acc);
            load_b<GU>(R, s, np, KT, s);
          }
        }
        c = cn;
        cp = np;
      }
      publish(L, k++, acc);
    }
  }
};

// ---------------------------------------------------------------------------
// Sync wavefront
// ---------------------------------------------------------------------------
// Block-format scales live in [groups][Mpad]; rows M..Mpad-1 hold zero.
__device__ __forceinline__ void zero_pad_scales(float* col_of_group, int M, int Mpad) {
  const int l = lane_id();
  if (l >= M && l < Mpad) st_coherent(col_of_group + l, 0.0f);
  if (l + 64 >= M && l + 64 < Mpad) st_coherent(col_of_group + l + 64, 0.0f);
}

__device__ __forceinline__ void bf16x32_to_f32(const uint4 (&w)[4], float (&v)[32]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t ww[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[8 * c + 2 * e] = bf16_to_f32(ww[e] & 0xFFFFu);
      v[8 * c + 2 * e + 1] = bf16_to_f32(ww[e] >> 16);
    }
  }
}

// All wavefronts of a workgroup quantize x into LDS (layout above): one lane
// per (row, 32-column block).  The loads of a lane's first four blocks are
// issued before the wavefront's first weight loads, so waiting for them does
// not wait for the weights (the load counter completes in issue order).
// Rows M..Mpad-1 become zero codes with zero scales.
template <int FMT>
struct XqLocal {
  static constexpr int U = 4;  // blocks per lane whose loads go first
  uint4 raw[U][4];

  __device__ __forceinline__ void load(const Args& a) {
    const int nb = a.K1 >> 5, T = a.M * nb;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = (int)threadIdx.x + u * (int)blockDim.x;
      if (i < T) {
        const int r = i / nb, j = i - r * nb;
        const uint4* src = reinterpret_cast<const uint4*>(a.x + (size_t)r * a.K1 + 32 * j);
#pragma unroll
        for (int c = 0; c < 4; ++c) raw[u][c] = src[c];
      }
    }
  }

  static __device__ __forceinline__ void quant_block(const Args& a, uint8_t* lx, int Mpad, int i,
                                                     const uint4 (&w)[4]) {
    const int nb = a.K1 >> 5;
    const int r = i / nb, j = i - r * nb;
    uint8_t* sc = lx + xl_scale_offset(Mpad, a.K1);
    float v[32];
    bf16x32_to_f32(w, v);
    uint32_t cw[8], se = 0;
    float sf = 1.0f;
    quant_block32<FMT>(v, cw, &sf, &se);
    if (FMT == FMT_BLOCK) {
      if ((j & 3) == 0) reinterpret_cast<float*>(sc)[(j >> 2) * Mpad + r] = sf;
    } else {
      sc[r * nb + j] = (uint8_t)se;
    }
    uint4* dst = reinterpret_cast<uint4*>(lx + r * xl_row_stride(a.K1) + 32 * j);
    dst[0] = make_uint4(cw[0], cw[1], cw[2], cw[3]);
    dst[1] = make_uint4(cw[4], cw[5], cw[6], cw[7]);
  }

  __device__ __forceinline__ void finish(const Args& a, uint8_t* lx, int Mpad) {
    const int nb = a.K1 >> 5, T = a.M * nb, nt = blockDim.x, t = threadIdx.x;
    // (T is a multiple of 4, so the 4 lanes of a block group agree on i < T)
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (t + u * nt < T) quant_block(a, lx, Mpad, t + u * nt, raw[u]);
    for (int i = t + U * nt; i < T; i += nt) {
      const int r = i / nb, j = i - r * nb;
      const uint4* src = reinterpret_cast<const uint4*>(a.x + (size_t)r * a.K1 + 32 * j);
      uint4 w[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) w[c] = src[c];
      quant_block(a, lx, Mpad, i, w);
    }
    // padded rows
    const int rs = xl_row_stride(a.K1);
    const int nz = (Mpad - a.M) * rs / 16;
    uint4* z = reinterpret_cast<uint4*>(lx + a.M * rs);
    for (int e = t; e < nz; e += nt) z[e] = make_uint4(0u, 0u, 0u, 0u);
    uint8_t* sc = lx + xl_scale_offset(Mpad, a.K1);
    if (FMT == FMT_BLOCK) {
      const int pad = Mpad - a.M;
      for (int e = t; e < (a.K1 >> 7) * pad; e += nt)
        reinterpret_cast<float*>(sc)[(e / pad) * Mpad + a.M + e % pad] = 0.0f;
    } else {
      for (int e = t; e < (Mpad - a.M) * nb; e += nt) sc[a.M * nb + e] = 0u;
    }
  }
};

// Quantize x into the workspace for one item: its (128-column group,
// 16-row tile) pairs, one lane per (row, 32-column block).
template <int FMT>
__device__ __forceinline__ void xq_item(const Args& a, int item) {
  const int l = lane_id();
  const int MTa = a.Mpad >> 4;
  const int p0 = (int)(((long long)item * a.n_pairs) / a.n_items);
  const int p1 = (int)(((long long)(item + 1) * a.n_pairs) / a.n_items);
  const __amdgpu_buffer_rsrc_t rxa = make_rsrc(a.xa, (uint32_t)a.M * (uint32_t)a.K1);
  for (int p = p0; p < p1; ++p) {
    const int kg = p / MTa, mt = p - kg * MTa;
    const int row = mt * 16 + (l >> 2), j = l & 3;
    float* sbl = static_cast<float*>(a.xs) + (size_t)kg * a.Mpad;
    if (row < a.M) {  // the 4 lanes of a row agree
      const uint4* src = reinterpret_cast<const uint4*>(a.x + (size_t)row * a.K1 + kg * 128 + 32 * j);
      uint4 w[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) w[c] = src[c];
      float v[32];
      bf16x32_to_f32(w, v);
      uint32_t cw[8], se = 0;
      float sf = 1.0f;
      quant_block32<FMT>(v, cw, &sf, &se);
      const uint32_t off = act_code_off(a.M, a.K1, row, kg * 128 + 32 * j);
      st_coherent_b128(rxa, off, make_uint4(cw[0], cw[1], cw[2], cw[3]));
      st_coherent_b128(rxa, off + 16u * act_tile_rows(a.M, row), make_uint4(cw[4], cw[5], cw[6], cw[7]));
      if (FMT == FMT_BLOCK) {
        if (j == 0) st_coherent(sbl + row, sf);
      } else {
        const uint32_t e4 = pack4_lanes(se);
        if (j == 0)
          st_coherent(reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(a.xs) + act_scale_off(a.M, a.K1, row, kg)), e4);
      }
    }
    if (FMT == FMT_BLOCK && mt == MTa - 1) zero_pad_scales(sbl, a.M, a.Mpad);
  }
}

// Block-format scales of the padded rows M..Mpad-1 of every group of Q(x): zero.
__device__ __forceinline__ void zero_pad_x_scales(const Args& a) {
  const int pad = a.Mpad - a.M, KT1 = a.K1 >> 7;
  for (int e = lane_id(); e < KT1 * pad; e += 64)
    st_coherent(static_cast<float*>(a.xs) + (size_t)(e / pad) * a.Mpad + a.M + e % pad, 0.0f);
}

// Re-quantize 128-column group g of a = silu(g)*u (fp32, written by other
// workgroups: read agent-coherently), one lane per (row, 32-column block),
// U blocks per lane at a time with all their loads issued first (one memory
// round trip per U blocks).
template <int FMT, int U>
__device__ __forceinline__ void requant_group(const Args& a, int g) {
  const int l = lane_id();
  const __amdgpu_buffer_rsrc_t r32 = make_rsrc(a.a32, (uint32_t)a.M * (uint32_t)a.F * 4u);
  const __amdgpu_buffer_rsrc_t raq = make_rsrc(a.aq, (uint32_t)a.M * (uint32_t)a.F);
  const int n = a.M * 4;  // (a multiple of 4: the 4 lanes of a row agree on i < n)
  for (int i0 = l; i0 < n; i0 += 64 * U) {
    float vv[U][32];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + 64 * u;
      const uint32_t base = ((uint32_t)(i >> 2) * (uint32_t)a.F + (uint32_t)(g * 128 + 32 * (i & 3))) * 4u;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const v4f t = ld_coherent_v4f(r32, i < n ? base + 16u * c : OOB);
        vv[u][4 * c] = t[0];
        vv[u][4 * c + 1] = t[1];
        vv[u][4 * c + 2] = t[2];
        vv[u][4 * c + 3] = t[3];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + 64 * u;
      if (i >= n) break;
      const int r = i >> 2, j = i & 3;
      const uint32_t col = (uint32_t)(g * 128 + 32 * j);
      uint32_t cw[8], se = 0;
      float sf = 1.0f;
      quant_block32<FMT>(vv[u], cw, &sf, &se);
      const uint32_t off = act_code_off(a.M, a.F, r, (int)col);
      st_coherent_b128(raq, off, make_uint4(cw[0], cw[1], cw[2], cw[3]));
      st_coherent_b128(raq, off + 16u * act_tile_rows(a.M, r), make_uint4(cw[4], cw[5], cw[6], cw[7]));
      if (FMT == FMT_BLOCK) {
        if (j == 0) st_coherent(static_cast<float*>(a.as) + (size_t)g * a.Mpad + r, sf);
      } else {
        const uint32_t e4 = pack4_lanes(se);
        if (j == 0)
          st_coherent(reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(a.as) + act_scale_off(a.M, a.F, r, g)), e4);
      }
    }
  }
  if (FMT == FMT_BLOCK) zero_pad_scales(static_cast<float*>(a.as) + (size_t)g * a.Mpad, a.M, a.Mpad);
}


// Raise flag i of every XCD copy of a flag array (lanes 0..NREP-1, one each).
__device__ __forceinline__ void raise_flag(uint32_t* ctrl, int page_off, int i, uint32_t ep) {
  const int l = lane_id();
  if (l < NREP) store_agent(&ctrl[PAGE0 + l * PAGE_WORDS + page_off + i], ep);
}

// The decode block's RMSNorm prologue: x = bf16(h / sqrt(mean(h^2) + eps))
// (unit gain), quantized into the workspace as xq_item does, by every
// wavefront of a workgroup before they take up their roles.  Item i is part
// i % P of the 128-column groups of row i / P (P = row_parts; M * P items
// dealt over the n_items workgroups); each item forms its row's whole sum of
// squares.  That sum follows the standalone RMSNorm kernel's order exactly:
// 256 partial sums, partial t (lane t % 64 of wavefront t / 64, the first
// four wavefronts) taking the 16-byte chunks t, t + 256, t + 512, t + 768,
// t + 1024, ... in one fma chain; a butterfly over each wavefront's 64; the
// four wavefront sums added in order.  So x is bit-identical to that
// kernel's output.  With `stash` (LDS for K1 floats) the row read for the
// sum of squares is kept for the quantization pass.  Ends with every
// wavefront's stores drained and the workgroup's flag raised.
template <int FMT>
__device__ __forceinline__ void block_prologue(const Args& a, float* red, float* stash, uint32_t ep) {
  const int l = lane_id(), wv = (int)(threadIdx.x >> 6), nw = (int)(blockDim.x >> 6);
  const int W = blockIdx.x, P = a.row_parts;
  const int d = a.K1, n4 = d >> 2, ng = d >> 7;
  const __amdgpu_buffer_rsrc_t rxa = make_rsrc(a.xa, (uint32_t)a.M * (uint32_t)a.K1);
  for (int i = W; i < a.M * P; i += a.n_items) {
    const int row = i / P, part = i - row * P;
    const int jb = 4 * ((part * ng) / P), je = 4 * (((part + 1) * ng) / P);  // this part's 32-column blocks
    const __amdgpu_buffer_rsrc_t rh = make_rsrc(a.h_in + (size_t)row * d, (uint32_t)d * 4u);
    if (wv < 4) {
      float ss = 0.0f;
      for (int c0 = 64 * wv + l; c0 < n4 + 64 * wv + l; c0 += 1024) {
        // (chunks past the row are zeros, which leave the chain unchanged)
        v4f v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = c0 + 256 * u;
          v[u] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rh, c < n4 ? (uint32_t)c * 16u : OOB, 0, 0));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = c0 + 256 * u;
          if (stash && c < n4) *reinterpret_cast<v4f*>(stash + 4 * c) = v[u];
#pragma unroll
          for (int e = 0; e < 4; ++e) ss = fmaf(v[u][e], v[u][e], ss);
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, WAVE);
      if (l == 0) red[wv] = ss;
    }
    __syncthreads();
    const float inv = 1.0f / sqrtf((((red[0] + red[1]) + red[2]) + red[3]) / (float)d + a.eps);
    // one lane per 32-column block over the whole workgroup (jb, je and the
    // steps are multiples of 4: the four lanes of a 128-column group agree)
    for (int j0 = jb + 64 * wv; j0 < je; j0 += 64 * nw) {
      const int j = j0 + l;
      if (j < je) {
        float v[32];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const v4f t = stash ? *reinterpret_cast<const v4f*>(stash + 4 * (8 * j + c))
                              : __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rh, (uint32_t)(8 * j + c) * 16u, 0, 0));
#pragma unroll
          for (int e = 0; e < 4; ++e) v[4 * c + e] = bf16_to_f32(f32_to_bf16(t[e] * inv));
        }
        uint32_t cw[8], se = 0;
        float sf = 1.0f;
        quant_block32<FMT>(v, cw, &sf, &se);
        const uint32_t off = act_code_off(a.M, a.K1, row, 32 * j);
        st_coherent_b128(rxa, off, make_uint4(cw[0], cw[1], cw[2], cw[3]));
        st_coherent_b128(rxa, off + 16u * act_tile_rows(a.M, row), make_uint4(cw[4], cw[5], cw[6], cw[7]));
        if (FMT == FMT_BLOCK) {
          if ((j & 3) == 0) st_coherent(static_cast<float*>(a.xs) + (size_t)(j >> 2) * a.Mpad + row, sf);
        } else {
          const uint32_t e4 = pack4_lanes(se);
          if ((j & 3) == 0)
            st_coherent(reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(a.xs) + act_scale_off(a.M, a.K1, row, j >> 2)), e4);
        }
      }
    }
    __syncthreads();  // (the stash and the partial sums are free for the next item)
  }
  if (FMT == FMT_BLOCK && W == 0 && wv == 0) zero_pad_x_scales(a);
  drain_memory();
  __syncthreads();  // every wavefront's stores have completed
  if (wv == 0 && W < a.n_items) raise_flag(a.ctrl, PG_XQ, W, ep);
}

// A cross-workgroup wait has lasted one more pass: true when it must end
// (some wait of this launch gave up, as err_ep shows, or this one outlived the
// budget).
__device__ __forceinline__ bool must_stop_global(const Guard& g, uint32_t err_ep, uint64_t& t0) {
  if (err_ep == g.ep) {
    if (lane_id() == 0) lds_store(g.abort, 1u);
    return true;
  }
  const uint64_t t = wall_clock64();
  if (t0 == 0) t0 = t;
  if (t - t0 > g.budget) {
    give_up(g);
    return true;
  }
  return false;
}

// Spin until flags [0, n) of this XCD's copy are all raised in this launch.
__device__ __forceinline__ void wait_flags(const Guard& g, const uint32_t* flags, int n) {
  const int l = lane_id();
  uint64_t t0 = 0;
  for (;;) {
    // (every flag's load issued before any is compared: one round trip a pass)
    bool ok = true;
    for (int i = l; i < n; i += 64) ok &= load_agent(flags + i) == g.ep;
    const uint32_t err_ep = load_agent(g.ctrl + C_ERR_EP);
    if (__all(ok)) break;
    if (must_stop_global(g, err_ep, t0)) break;
    __builtin_amdgcn_s_sleep(8);
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Poll the group-ready flags of groups [g0, g1) until all are set, copying
// each 32-group word into the workgroup's LDS mask as its flags rise (flags
// only rise during a launch, so every copy only adds bits).
template <int MT, int NS, int NSLOT>
__device__ __forceinline__ void mirror_ready(const Guard& gd, Lds<MT, NS, NSLOT>& L, const uint32_t* flags, int g0,
                                             int g1) {
  const int l = lane_id();
  const int a0 = g0 & ~31;
  uint64_t t0 = 0;
  for (;;) {
    bool all = true;
    const uint32_t err_ep = load_agent(gd.ctrl + C_ERR_EP);
    for (int i0 = a0; i0 < g1; i0 += 64) {
      const int i = i0 + l;
      const bool in = i >= g0 && i < g1;
      const bool r = in && load_agent(flags + i) == gd.ep;
      const uint64_t bal = __ballot(r);
      all = all && __all(r || !in);
      if (l == 0) {
        lds_store(&L.rdy[i0 >> 5], (uint32_t)bal);
        if (i0 + 32 < g1) lds_store(&L.rdy[(i0 >> 5) + 1], (uint32_t)(bal >> 32));
      }
    }
    if (all) break;
    if (must_stop_global(gd, err_ep, t0)) break;
    __builtin_amdgcn_s_sleep(4);
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Split-K partials of shared bands, slot (workgroup W, side).  Up to two row
// tiles: [2][M][16] fp32, rows < M only (one row costs two stores).  More:
// the sync wavefront's sums in their register layout, [2][MT][64 lanes] x
// v4f, so that each lane moves 16 bytes per (n-block, m-tile).
template <int MT>
__device__ __forceinline__ uint32_t part_slot_bytes() { return 2u * MT * 64u * 16u; }
template <int MT>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(const Args& a, const float* part) {
  return make_rsrc(part, (uint32_t)a.G * 2u * part_slot_bytes<MT>());
}

// Sum of the split-K partials of a shared band over its workgroups, in
// workgroup order (all of one workgroup's loads in flight together).
template <int MT>
__device__ __forceinline__ void sum_shared(const Args& a, const Phase& ph, const float* part, int b,
                                           v4f (&s)[2][MT]) {
  const int l = lane_id();
  const __amdgpu_buffer_rsrc_t r = part_rsrc<MT>(a, part);
  const int w0 = owner_wg(ph, b * ph.CPB), w1 = owner_wg(ph, b * ph.CPB + ph.CPB - 1);
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) s[nb][mt] = v4f{0.f, 0.f, 0.f, 0.f};
  if (MT <= 2) {
    for (int w = w0; w <= w1; ++w) {
      const float* base = part + ((size_t)w * 2 + band_side(ph, w, b)) * 2 * a.M * 16;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int row = min(mt * 16 + 4 * (l >> 4) + rr, a.M - 1);
            s[nb][mt][rr] += ld_coherent(base + ((size_t)nb * a.M + row) * 16 + (l & 15));
          }
    }
    return;
  }
  for (int w = w0; w <= w1; ++w) {
    const uint32_t base = ((uint32_t)w * 2u + (uint32_t)band_side(ph, w, b)) * part_slot_bytes<MT>();
    v4f t[2][MT];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) t[nb][mt] = ld_coherent_v4f(r, base + (uint32_t)(((nb * MT + mt) * 64 + l) * 16));
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) s[nb][mt] += t[nb][mt];
  }
}

// Store this workgroup's sums of shared band b and arrive; true if this was
// the last workgroup of the band (all partials are then visible).
template <int MT>
__device__ __forceinline__ bool arrive_shared(const Args& a, const Phase& ph, float* part, uint32_t* cnt, int b,
                                              const v4f (&s)[2][MT], int nsh) {
  const int l = lane_id();
  const int side = band_side(ph, blockIdx.x, b);
  if (MT <= 2) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int row = mt * 16 + 4 * (l >> 4) + rr;
          if (row < a.M)
            st_coherent(part + ((((size_t)blockIdx.x * 2 + side) * 2 + nb) * a.M + row) * 16 + (l & 15),
                        s[nb][mt][rr]);
        }
  } else {
    const __amdgpu_buffer_rsrc_t r = part_rsrc<MT>(a, part);
    const uint32_t base = ((uint32_t)blockIdx.x * 2u + (uint32_t)side) * part_slot_bytes<MT>();
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        st_coherent_b128(r, base + (uint32_t)(((nb * MT + mt) * 64 + l) * 16), __builtin_bit_cast(uint4, s[nb][mt]));
  }
  drain_memory();
  uint32_t old = 0;
  if (l == 0) old = atomic_add_agent(cnt + b, 1u);
  const bool last = uni((int)old) == nsh - 1;
  if (last && l == 0) store_agent(cnt + b, 0u);  // (the counter's last use in this launch)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return last;
}

template <int MT, int NS, int NSLOT>
__device__ __forceinline__ void take_event(const Guard& gd, Lds<MT, NS, NSLOT>& L, int k, v4f (&s)[2][MT]) {
  const int slot = k % NSLOT;
  lds_wait_geq(gd, &L.arrived[slot], (uint32_t)NS);
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      v4f v = L.part[slot][0][nb][mt][lane_id()];
#pragma unroll
      for (int w = 1; w < NS; ++w) v += L.part[slot][w][nb][mt][lane_id()];
      s[nb][mt] = v;
    }
  if (lane_id() == 0) {
    lds_store(&L.arrived[slot], 0u);
    lds_store(&L.consumed, (uint32_t)(k + 1));
  }
}

template <int MT, int FMT>
__device__ void finish_gu_band(const Args& a, int b, v4f (&s)[2][MT], uint32_t ep) {
  const int l = lane_id();
  const Phase& ph = a.gu;
  const int nsh = owner_wg(ph, b * ph.CPB + ph.CPB - 1) - owner_wg(ph, b * ph.CPB) + 1;
  if (nsh > 1) {
    if (!arrive_shared<MT>(a, ph, a.gpart, a.ctrl + C_GPCNT, b, s, nsh)) return;
    sum_shared<MT>(a, ph, a.gpart, b, s);
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int row = mt * 16 + 4 * (l >> 4) + rr;
      if (row < a.M) st_coherent(a.a32 + (size_t)row * a.F + b * 16 + (l & 15), silu_mul(s[0][mt][rr], s[1][mt][rr]));
    }
  drain_memory();
  const int grp = b >> 3;
  uint32_t old = 0;
  if (l == 0) old = atomic_add_agent(&a.ctrl[C_GCNT + grp], 1u);
  if (uni((int)old) != 7) return;
  if (l == 0) store_agent(&a.ctrl[C_GCNT + grp], 0u);  // (its last use in this launch)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  // (MX: several blocks per lane at a time; the block format measured
  // faster with one)
  requant_group<FMT, (FMT == FMT_MX ? (MT < 4 ? MT : 4) : 1)>(a, grp);
  drain_memory();
  raise_flag(a.ctrl, PG_RDY, grp, ep);
}

// End of band b of the staged gate/up, whose streaming wavefront owns the
// whole band (so every band has an owner that reaches this point without
// waiting on any other band).  The band re-quantizes its own 16 columns of
// a = silu(g)*u from registers; the bands of one quantization block
// exchange only their per-row maxima |a| (MX: the pair 2j, 2j+1 of a
// 32-column block; block format: the 8 bands of a 128-column group).  The
// codes and scales equal those of requant_group over the same fp32 values:
// the block maximum does not depend on the order it is taken in, and each
// code depends only on its value and the block's scale.  a itself is
// stored afterwards, off the critical path, for inspection only.
template <int MT, int FMT>
__device__ void finish_gu_band_staged(const Args& a, int b, v4f (&s)[2][MT], uint32_t ep, const Guard& gd) {
  const int l = lane_id(), c = l & 15, g4 = l >> 4;
  float h[MT][4], am[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      h[mt][rr] = silu_mul(s[0][mt][rr], s[1][mt][rr]);
      am[mt][rr] = fabsf(h[mt][rr]);
    }
  // row maxima over the band's 16 columns (the 16 lanes of a row group)
#pragma unroll
  for (int off = 1; off < 16; off <<= 1)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) am[mt][rr] = fmaxf(am[mt][rr], __shfl_xor(am[mt][rr], off, WAVE));
  // publish them (lane c < 4 of a row group: row 4*g4 + c), then the flag
  float* amx = a.amax + (size_t)b * a.Mpad;
  if (c < 4) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const float v = c == 0 ? am[mt][0] : c == 1 ? am[mt][1] : c == 2 ? am[mt][2] : am[mt][3];
      st_coherent(amx + mt * 16 + 4 * g4 + c, v);
    }
  }
  drain_memory();
  if (l == 0) store_agent(&a.ctrl[C_BFLAG + b], ep);
  // the block's maxima: lane c reads band b0 + c % NB of its rows
  constexpr int NB = FMT == FMT_MX ? 2 : 8;
  const int b0 = b & ~(NB - 1);
  wait_flags(gd, a.ctrl + C_BFLAG + b0, NB);
  const float* src = a.amax + (size_t)(b0 + (c & (NB - 1))) * a.Mpad;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) am[mt][rr] = ld_coherent(src + mt * 16 + 4 * g4 + rr);
#pragma unroll
  for (int off = 1; off < NB; off <<= 1)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) am[mt][rr] = fmaxf(am[mt][rr], __shfl_xor(am[mt][rr], off, WAVE));
  // codes of this band's 16 columns: lane (c, g4) codes rows 4*g4 + rr of
  // column c; a 4x4 byte transpose within each lane quad gives lane
  // 4j + i the codes of row 4*g4 + i, columns 4j..4j+3 (one dword)
  const __amdgpu_buffer_rsrc_t raq = make_rsrc(a.aq, (uint32_t)a.M * (uint32_t)a.F);
  const __amdgpu_buffer_rsrc_t ras =
      make_rsrc(a.as, FMT == FMT_BLOCK ? (uint32_t)(a.F >> 7) * (uint32_t)a.Mpad * 4u : (uint32_t)a.M * (uint32_t)(a.F >> 5));
  const int i = c & 3, quad = l & ~3;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    uint32_t d = 0, sv = 0;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      float t;
      if (FMT == FMT_BLOCK) {
        const float sc = block_scale(am[mt][rr]);
        t = h[mt][rr] / sc;
        if (rr == i) sv = __float_as_uint(sc);
      } else {
        const int X = mx_exponent(am[mt][rr]);
        t = h[mt][rr] * pow2_neg(X);
        if (rr == i) sv = (uint32_t)(X + 127);
      }
      const float q = __builtin_amdgcn_fmed3f(t, -E4M3_MAX, E4M3_MAX);
      d |= ((uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q, q, 0, false) & 0xFFu) << (8 * rr);
    }
    uint32_t e = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) e |= ((__shfl(d, quad + k, WAVE) >> (8 * i)) & 0xFFu) << (8 * k);
    const int row = mt * 16 + 4 * g4 + i;
    if (row < a.M) {
      const uint32_t off = act_code_off(a.M, a.F, row, b * 16 + 4 * (c >> 2));
      __builtin_amdgcn_raw_buffer_store_b32(e, raq, off, 0, AUX_SC1);
      // the block's scale, once per row: lanes c < 4 of the band that writes it
      if (c < 4) {
        if (FMT == FMT_BLOCK) {
          if ((b & 7) == 0) __builtin_amdgcn_raw_buffer_store_b32(sv, ras, ((uint32_t)(b >> 3) * (uint32_t)a.Mpad + (uint32_t)row) * 4u, 0, AUX_SC1);
        } else if ((b & 1) == 0) {
          __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sv, ras, act_scale_off(a.M, a.F, row, b >> 3) + (uint32_t)((b >> 1) & 3), 0, AUX_SC1);
        }
      }
    }
  }
  if (FMT == FMT_BLOCK && (b & 7) == 0) zero_pad_scales(static_cast<float*>(a.as) + (size_t)(b >> 3) * a.Mpad, a.M, a.Mpad);
  drain_memory();
  const int grp = b >> 3;
  uint32_t old = 0;
  if (l == 0) old = atomic_add_agent(&a.ctrl[C_GCNT + grp], 1u);
  if (uni((int)old) == 7) {
    if (l == 0) store_agent(&a.ctrl[C_GCNT + grp], 0u);  // (its last use in this launch)
    raise_flag(a.ctrl, PG_RDY, grp, ep);
  }
  // a, for inspection only (nothing in this launch reads it)
  if (a.keep_a) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int row = mt * 16 + 4 * g4 + rr;
        if (row < a.M) a.a32[(size_t)row * a.F + b * 16 + c] = h[mt][rr];
      }
  }
}

// BLK: the decode block's residual epilogue (h_out = h_in + bf16(y)); a
// separate instantiation, so that the plain MLP carries none of its code.
template <int MT, bool BLK>
__device__ __forceinline__ void finish_dn_band(const Args& a, int b, v4f (&s)[2][MT]) {
  const int l = lane_id();
  const Phase& ph = a.dn;
  // decode block: the residual stream's values of this band, loaded ahead of
  // the split-K combine's round trips (up to 64 rows: at 128 the registers
  // would spill, and they are loaded at the store instead)
  constexpr bool PRE = BLK && MT <= 4;
  float hv[2][PRE ? MT : 1][4];
  if (PRE) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int row = mt * 16 + 4 * (l >> 4) + rr;
          hv[nb][PRE ? mt : 0][rr] = row < a.M ? a.h_in[(size_t)row * a.N + b * 32 + nb * 16 + (l & 15)] : 0.0f;
        }
  }
  const int nsh = owner_wg(ph, b * ph.CPB + ph.CPB - 1) - owner_wg(ph, b * ph.CPB) + 1;
  if (nsh > 1) {
    if (!arrive_shared<MT>(a, ph, a.dpart, a.ctrl + C_DPCNT, b, s, nsh)) return;
    sum_shared<MT>(a, ph, a.dpart, b, s);
  }
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int row = mt * 16 + 4 * (l >> 4) + rr;
        if (row < a.M) {
          const size_t o = (size_t)row * a.N + b * 32 + nb * 16 + (l & 15);
          if (BLK)  // residual epilogue: the bf16 output added to the fp32 stream
            a.h_out[o] = (PRE ? hv[nb][PRE ? mt : 0][rr] : a.h_in[o]) + bf16_to_f32(f32_to_bf16(s[nb][mt][rr]));
          else if (a.y32)
            a.y32[o] = s[nb][mt][rr];
          else
            a.y[o] = (uint16_t)f32_to_bf16(s[nb][mt][rr]);
        }
      }
}

// Staged gate/up: copy Q(x) (workspace, m-tile order) into the LDS stages
// one k-tile at a time, for the nst streaming wavefronts that hold a band.
// The copies go from memory straight into LDS (2*MT 1 KB copies of codes and
// MT/4 256-byte copies of row scales per k-tile, OPS in all), LD k-tiles in
// flight; stage kt % DA is refilled once every one of those wavefronts has
// used k-tile kt - DA.  No register holds the data, and this wavefront issues
// no other loads meanwhile, so it waits for exactly the copies of the oldest
// k-tile (register-held copies left the compiler waiting for nearly all of
// them, which cut the staging to about one k-tile in flight).
template <int MT, int FMT, int NS, int NSLOT>
__device__ __forceinline__ void stage_activations(const Guard& gd, const Args& a, Lds<MT, NS, NSLOT>& L,
                                                  uint8_t* stages, int nst) {
  constexpr int DA = Cfg<MT>::DA, SB = ks_stage_bytes<MT>(), LD = Cfg<MT>::LD;
  constexpr int NSC = (16 * MT + 63) / 64;  // 256-byte scale copies (one dword per row)
  constexpr int OPS = 2 * MT + NSC;
  static_assert(LD * OPS <= 63 && LD < DA, "copies in flight");
  const int l = lane_id();
  const uint32_t r = (uint32_t)(l & 15), g = (uint32_t)(l >> 4);
  const int KT = a.gu.KT;
  const uint32_t KT1 = (uint32_t)(a.K1 >> 7);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.xa, (uint32_t)a.M * (uint32_t)a.K1);
  const __amdgpu_buffer_rsrc_t rxs =
      make_rsrc(a.xs, FMT == FMT_BLOCK ? KT1 * (uint32_t)a.Mpad * 4u : (uint32_t)a.M * (KT1 * 4u));
  const uint32_t lds_st = lds_addr(stages);
  auto copy = [&](int kt) {
    const uint32_t base = lds_st + (uint32_t)((kt % DA) * SB);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int Mt = min(16, a.M - 16 * mt);
      const bool v = (int)r < Mt;
      const uint32_t uMt = (uint32_t)max(Mt, 0);
      const uint32_t o = (uint32_t)mt * 16u * (uint32_t)a.K1 + ((uint32_t)kt * 8u + g) * 16u * uMt + r * 16u;
      lds_copy1k(rx, base + (uint32_t)(mt * 2048), v ? o : OOB);
      lds_copy1k(rx, base + (uint32_t)(mt * 2048 + 1024), v ? o + 64u * uMt : OOB);
    }
    // entry e (row e % 16 of m-tile e / 16): lane l of copy j carries e = 64 j + l
#pragma unroll
    for (int j = 0; j < NSC; ++j) {
      const int e = 64 * j + l;
      uint32_t off = OOB;
      if (e >= 16 * MT) {
      } else if (FMT == FMT_BLOCK) {
        off = ((uint32_t)kt * (uint32_t)a.Mpad + (uint32_t)e) * 4u;
      } else {
        const int mt = e >> 4, rr = e & 15;
        const int Mt = min(16, a.M - 16 * mt);
        if (rr < Mt) off = (uint32_t)mt * 16u * KT1 * 4u + (uint32_t)kt * 4u * (uint32_t)Mt + (uint32_t)rr * 4u;
      }
      lds_copy256_sc1(rxs, base + (uint32_t)(MT * 2048 + 256 * j), off);
    }
  };
  auto stage_free = [&](int kt) {
    if (kt >= DA)
      for (int w = 0; w < nst; ++w) lds_wait_geq(gd, &L.prog[w], (uint32_t)(kt - DA + 1));
  };
  for (int t = 0; t < LD && t < KT; ++t) {
    stage_free(t);
    copy(t);
  }
  for (int kt = 0; kt < KT; ++kt) {
    // copies issued after k-tile kt's: those of the next min(LD - 1, KT - 1 - kt) k-tiles
    const int after = min(LD - 1, KT - 1 - kt);
    if (after >= 3)
      lds_copies_left<(LD >= 4 ? 3 : 0) * OPS>();
    else if (after == 2)
      lds_copies_left<(LD >= 3 ? 2 : 0) * OPS>();
    else if (after == 1)
      lds_copies_left<OPS>();
    else
      lds_copies_left<0>();
    if (l == 0) lds_store(&L.a_ready, (uint32_t)(kt + 1));
    if (kt + LD < KT) {
      stage_free(kt + LD);
      copy(kt + LD);
    }
  }
}

template <int MT, int FMT, int XL, bool BLK, int NS, int NSLOT>
__device__ __forceinline__ void sync_wave(const Args& a, Lds<MT, NS, NSLOT>& L, uint8_t* stages) {
  const int l = lane_id();
  const int W = blockIdx.x;
  const int rep = W & (NREP - 1);
  const uint32_t* page = a.ctrl + PAGE0 + rep * PAGE_WORDS;
  const uint32_t ep = launch_epoch(a);
  const Guard gd{&L.abort, a.ctrl, a.budget, ep};
  if (!XL) {
    // quantize this workgroup's share of x, then wait for everyone's
    // (the decode block's prologue has run already, flag included)
    if (W < a.n_items && !BLK) {
      xq_item<FMT>(a, W);
      drain_memory();
      raise_flag(a.ctrl, PG_XQ, W, ep);
    }
    wait_flags(gd, page + PG_XQ, a.n_items);
    if (l == 0) lds_store(&L.xq_ok, 1u);
  }

  int k = 0;
  if (a.mlp && W < a.gu.nwg) {
    const Phase& ph = a.gu;
    const int c0 = range_start(ph, W), c1 = range_start(ph, W + 1);
    if (Cfg<MT>::KS && a.ks) {
      // the streaming wavefronts finish their own bands
      const int nst = min((c1 - c0) / ph.CPB, NS);
      if (nst > 0) stage_activations<MT, FMT>(gd, a, L, stages, nst);
    } else if (c0 < c1) {
      for (int b = c0 / ph.CPB; b <= (c1 - 1) / ph.CPB; ++b) {
        v4f s[2][MT];
        take_event(gd, L, k++, s);
        finish_gu_band<MT, FMT>(a, b, s, ep);
      }
    }
  }
  if (W < a.dn.nwg) {
    const Phase& ph = a.dn;
    const int c0 = range_start(ph, W), c1 = range_start(ph, W + 1);
    if (c0 < c1) {
      if (a.mlp) {
        // groups (k-tiles of the second GEMM) this workgroup's chunks read
        int g0 = 0, g1 = ph.KT;
        if (c0 / ph.CPB == (c1 - 1) / ph.CPB) {
          g0 = (c0 % ph.CPB) * Cfg<MT>::PD;
          g1 = min(ph.KT, ((c1 - 1) % ph.CPB) * Cfg<MT>::PD + Cfg<MT>::PD);
        }
        mirror_ready(gd, L, page + PG_RDY, g0, g1);
      }
      for (int b = c0 / ph.CPB; b <= (c1 - 1) / ph.CPB; ++b) {
        v4f s[2][MT];
        take_event(gd, L, k++, s);
        finish_dn_band<MT, BLK>(a, b, s);
      }
    }
  }
  // leave once the streaming wavefronts are done with gate/up (in the staged
  // variant they finish bands themselves, and those flag and counter updates
  // must precede this workgroup's arrival); the last workgroup advances the
  // launch number
  if (a.mlp) lds_wait_geq(gd, &L.gu_left, (uint32_t)NS);
  drain_memory();
  uint32_t old = 0;
  if (l == 0) old = atomic_add_agent(&a.ctrl[C_DONE], 1u);
  if (uni((int)old) != a.G - 1) return;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (ep == 0xFFFFFFFFu) {
    // the launch number is about to wrap: clear every flag (flags of earlier
    // launches could otherwise match a later number)
    for (int i = l; i < NREP * PAGE_WORDS; i += 64) store_agent(&a.ctrl[PAGE0 + i], 0u);
    for (int i = l; i < MAX_GBANDS; i += 64) store_agent(&a.ctrl[C_BFLAG + i], 0u);
    if (l == 0) store_agent(&a.ctrl[C_ERR_EP], 0u);
  }
  if (l == 0) {
    store_agent(&a.ctrl[C_EPOCH], ep == 0xFFFFFFFFu ? 0u : ep);
    store_agent(&a.ctrl[C_DONE], 0u);
  }
}

// ---------------------------------------------------------------------------
// The persistent kernel: wavefront 0 syncs, the others stream.
// ---------------------------------------------------------------------------
// XL: Q(x) is built in LDS by every workgroup (no cross-workgroup wait
// before the first product); otherwise it is built once in the workspace.
// MLP: 0 the plain GEMM, 1 the fused MLP, 2 the decode block (the fused MLP
// with its RMSNorm prologue and residual epilogue); separate kernels, so that
// each gets its own register allocation.
template <int MT, int FMT, int XL, int MLP>
__global__ __launch_bounds__(64 * Cfg<MT>::NWAVE, 1) void stream_kernel(Args a) {
  using C = Cfg<MT>;
  static_assert(MLP != 2 || !XL, "the decode block quantizes x into the workspace");
  __shared__ Lds<MT, C::NS, C::NSLOT> L;
  extern __shared__ __align__(16) uint8_t lds_x[];
  const int wv = uni((int)(threadIdx.x >> 6));
  if (threadIdx.x == 0) {
    for (int i = 0; i < C::NSLOT; ++i) L.arrived[i] = 0u;
    L.consumed = 0u;
    L.xq_ok = XL ? 1u : 0u;
    for (int i = 0; i < MAX_GROUPS / 32; ++i) L.rdy[i] = 0u;
    L.a_ready = 0u;
    for (int i = 0; i < C::NS; ++i) L.prog[i] = 0u;
    L.gu_left = 0u;
    L.abort = 0u;
  }
  __syncthreads();
  if (MLP == 2)
    block_prologue<FMT>(a, L.red, a.row_stash ? reinterpret_cast<float*>(lds_x) : nullptr, launch_epoch(a));
  if (wv == 0) {
    if (XL) {
      XqLocal<FMT> xq;
      xq.load(a);
      xq.finish(a, lds_x, 16 * MT);
      __syncthreads();
    }
    sync_wave<MT, FMT, XL, MLP == 2>(a, L, lds_x);
  } else {
    const Guard gd{&L.abort, a.ctrl, a.budget, launch_epoch(a)};
    Streamer<MT, FMT, C::P, XL> st(a, wv - 1, lds_x, gd);
    int k = 0;
    XqLocal<FMT> xq;
    if (XL) {
      // x's loads first: the first product waits for them; the first weight
      // slots go out right behind them (at 16 rows, 128 KB of x per
      // workgroup, waiting for x before issuing them cost 0.5 us)
      xq.load(a);
    }
    // the first weights are in flight while x is quantized
    auto quantize_x = [&]() {
      if (XL) {
        xq.finish(a, lds_x, 16 * MT);
        __syncthreads();
      }
    };
    auto nothing = []() {};
    if (MLP) {
      if (C::KS && a.ks)
        st.run_gu_staged(L, lds_x);
      else
        st.template run_phase<PK_GU, C::P>(L, k, quantize_x);
      if (lane_id() == 0) __hip_atomic_fetch_add(&L.gu_left, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      st.template run_phase<PK_DN, C::PD>(L, k, nothing);
    } else {
      st.template run_phase<PK_GEMM, C::P>(L, k, quantize_x);
    }
  }
}

// ---------------------------------------------------------------------------
// Standalone SwiGLU + re-quantization (the middle launch of the unfused
// pipeline: gate/up GEMM, this, down GEMM, with the intermediates in HBM).
// gu [M, 2F] fp32 holds g in columns [0, F) and u in [F, 2F).  One
// wavefront per (128-column group, 16-row tile), one lane per (row,
// 32-column block), the arithmetic of the fused kernel's band finish and
// group re-quantization: a = silu(g) * u in fp32, then quant_block32.  Q(a)
// is written in the workspace layout (codes m-tile by m-tile; block scales
// [F/128][Mpad] with padded rows zero; MX scales per m-tile and k-tile).
// ---------------------------------------------------------------------------
template <int FMT>
__global__ __launch_bounds__(256) void swiglu_quant_kernel(const float* __restrict__ gu, int M, int F, int Mpad,
                                                           uint8_t* __restrict__ aq, void* __restrict__ as) {
  const int nmt = (M + 15) >> 4;
  const int wave = (int)((blockIdx.x * 256u + threadIdx.x) >> 6);
  if (wave >= (F >> 7) * nmt) return;
  const int g = wave / nmt, mt = wave - g * nmt;
  const int l = lane_id(), row = mt * 16 + (l >> 2), j = l & 3;
  if (row < M) {  // (the 4 lanes of a row agree)
    const float4* pg = reinterpret_cast<const float4*>(gu + (size_t)row * 2 * F + g * 128 + 32 * j);
    const float4* pu = reinterpret_cast<const float4*>(gu + (size_t)row * 2 * F + F + g * 128 + 32 * j);
    float v[32];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float4 x = pg[c], y = pu[c];
      v[4 * c] = silu_mul(x.x, y.x);
      v[4 * c + 1] = silu_mul(x.y, y.y);
      v[4 * c + 2] = silu_mul(x.z, y.z);
      v[4 * c + 3] = silu_mul(x.w, y.w);
    }
    uint32_t cw[8], se = 0;
    float sf = 1.0f;
    quant_block32<FMT>(v, cw, &sf, &se);
    const uint32_t off = act_code_off(M, F, row, g * 128 + 32 * j);
    *reinterpret_cast<uint4*>(aq + off) = make_uint4(cw[0], cw[1], cw[2], cw[3]);
    *reinterpret_cast<uint4*>(aq + off + 16u * act_tile_rows(M, row)) = make_uint4(cw[4], cw[5], cw[6], cw[7]);
    if (FMT == FMT_BLOCK) {
      if (j == 0) static_cast<float*>(as)[(size_t)g * Mpad + row] = sf;
    } else {
      const uint32_t e4 = pack4_lanes(se);
      if (j == 0) *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(as) + act_scale_off(M, F, row, g)) = e4;
    }
  }
  if (FMT == FMT_BLOCK && mt == 0) {
    float* col = static_cast<float*>(as) + (size_t)g * Mpad;
    if (l >= M && l < Mpad) col[l] = 0.0f;
    if (l + 64 >= M && l + 64 < Mpad) col[l + 64] = 0.0f;
  }
}

// ---------------------------------------------------------------------------
// host side: plan, workspace layout, launch
// ---------------------------------------------------------------------------
namespace {

struct Plan {
  int ok;
  int ks;  // staged gate/up
  int MT, Mpad, G, n_pairs, n_items, ngroups;
  Phase gu, dn;
  size_t off_xa, off_xs, off_a32, off_aq, off_as, off_gpart, off_dpart, off_amax, bytes;
};

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }
int mt_for(int M) { return M <= 16 ? 1 : M <= 32 ? 2 : M <= 64 ? 4 : 8; }
int cfg_ns(int MT) { return MT == 1 ? Cfg<1>::NS : MT == 2 ? Cfg<2>::NS : MT == 4 ? Cfg<4>::NS : Cfg<8>::NS; }
int cfg_p(int MT) { return MT == 1 ? Cfg<1>::P : MT == 2 ? Cfg<2>::P : MT == 4 ? Cfg<4>::P : Cfg<8>::P; }
int cfg_pd(int MT) { return MT == 1 ? Cfg<1>::PD : MT == 2 ? Cfg<2>::PD : MT == 4 ? Cfg<4>::PD : Cfg<8>::PD; }
int cfg_nwave(int MT) { return cfg_ns(MT) + 1; }

// Chunks are dealt in equal contiguous ranges: of whole bands when `whole`
// (over as few workgroups as give the same number of bands to each), else
// of chunks (over enough workgroups to keep every streaming wavefront busy).
Phase make_phase(int KT, int nbands, int P, int NS, int G, bool whole) {
  Phase ph{};
  ph.KT = KT;
  ph.CPB = (KT + P - 1) / P;
  ph.nbands = nbands;
  ph.nchunks = nbands * ph.CPB;
  ph.nunits = whole ? nbands : ph.nchunks;
  ph.upc = whole ? ph.CPB : 1;
  if (whole) {
    const int per = (nbands + G - 1) / G;
    ph.nwg = (nbands + per - 1) / per;
  } else {
    const int nwg = ph.nchunks / NS;
    ph.nwg = nwg < 1 ? 1 : (nwg > G ? G : nwg);
    // Rather S workgroups per band (ranges that never straddle a band: one
    // band event, one split-K combine, and only that band's k-range of Q(a)
    // to wait for), for the smallest S that needs fewer rounds of chunks per
    // streaming wavefront than the plain split.
    const int rounds = ((ph.nchunks + ph.nwg - 1) / ph.nwg + NS - 1) / NS;
    for (int S = 1; S <= G / nbands && S <= ph.CPB; ++S) {
      if (((ph.CPB + S - 1) / S + NS - 1) / NS < rounds) {
        ph.nwg = nbands * S;
        break;
      }
    }
  }
  return ph;
}

Plan make_plan(int fmt, int M, int K1, int F, int N, int K2, bool mlp, int G) {
  Plan p{};
  p.MT = mt_for(M);
  p.Mpad = 16 * p.MT;
  p.G = G;
  const int P = cfg_p(p.MT), NS = cfg_ns(p.MT);
  const int KT1 = K1 / 128;
  p.n_pairs = KT1 * p.MT;
  p.n_items = p.n_pairs < G ? p.n_pairs : G;
  if (p.n_items > MAX_ITEMS) p.n_items = MAX_ITEMS;
  p.ngroups = mlp ? F / 128 : 0;
  // gate/up: whole bands when splitting would give a workgroup fewer than
  // two bands (then most bands would be shared, and each shared band costs
  // a round trip through memory at its end)
  if (mlp) p.gu = make_phase(KT1, F / 16, P, NS, G, F / 16 < 2 * G);
  // staged gate/up: whole bands over every workgroup, at most NS each
  const int nb = F / 16, wks = nb < G ? nb : G;
  p.ks = 0;
  if (mlp && p.MT >= 4 && (nb + wks - 1) / wks <= NS) {
    p.gu = make_phase(KT1, nb, P, NS, G, true);
    p.gu.nwg = wks;
    p.ks = 1;
  }
  p.dn = make_phase(K2 / 128, N / 32, mlp ? cfg_pd(p.MT) : P, NS, G, false);
  p.ok = p.ngroups <= MAX_GROUPS && (!mlp || F / 16 <= MAX_GBANDS) && N / 32 <= C_BFLAG - C_DPCNT;
  size_t o = CTRL_BYTES;
  p.off_xa = o;
  o = align256(o + (size_t)M * K1);
  p.off_xs = o;
  o = align256(o + (fmt == FMT_BLOCK ? (size_t)KT1 * p.Mpad * 4 : (size_t)M * (K1 / 32)));
  const size_t part = (size_t)MAX_WG * 2 * 2 * p.Mpad * 16 * 4;  // two slots of [2][Mpad][16] fp32 each
  p.off_a32 = o;
  if (mlp) o = align256(o + (size_t)M * F * 4);
  p.off_aq = o;
  if (mlp) o = align256(o + (size_t)M * F);
  p.off_as = o;
  if (mlp) o = align256(o + (fmt == FMT_BLOCK ? (size_t)(F / 128) * p.Mpad * 4 : (size_t)M * (F / 32)));
  p.off_gpart = o;
  if (mlp) o = align256(o + part);
  p.off_dpart = o;
  o = align256(o + part);
  // (whether gate/up is staged depends on the grid; the layout does not)
  p.off_amax = o;
  if (mlp && p.MT >= 4) o = align256(o + (size_t)(F / 16) * p.Mpad * 4);
  p.bytes = o;
  return p;
}

template <int MT, int FMT, int XL, int MLP>
const void* kernel_ptr() { return reinterpret_cast<const void*>(&stream_kernel<MT, FMT, XL, MLP>); }

// Kernel variants: (MT, XL) in (1,0) (1,1) (2,0) (2,1) (4,0) (8,0), each for
// the plain GEMM (kind 0) and for the MLP (kind 1); the decode block (kind 2)
// at MT 1, 2, 4, 8 with XL = 0.
constexpr int NVAR = 16;
int var_index(int MT, int XL, int kind) {
  const int mi = MT == 1 ? 0 : MT == 2 ? 1 : MT == 4 ? 2 : 3;
  if (kind == 2) return 12 + mi;
  return (MT == 1 ? XL : MT == 2 ? 2 + XL : MT == 4 ? 4 : 5) + (kind ? 6 : 0);
}

template <int FMT, int MLP>
const void* pick_fmt(int vi) {
  if constexpr (MLP == 2) {
    switch (vi - 12) {
      case 0: return kernel_ptr<1, FMT, 0, 2>();
      case 1: return kernel_ptr<2, FMT, 0, 2>();
      case 2: return kernel_ptr<4, FMT, 0, 2>();
      default: return kernel_ptr<8, FMT, 0, 2>();
    }
  } else {
    switch (vi % 6) {
      case 0: return kernel_ptr<1, FMT, 0, MLP>();
      case 1: return kernel_ptr<1, FMT, 1, MLP>();
      case 2: return kernel_ptr<2, FMT, 0, MLP>();
      case 3: return kernel_ptr<2, FMT, 1, MLP>();
      case 4: return kernel_ptr<4, FMT, 0, MLP>();
      default: return kernel_ptr<8, FMT, 0, MLP>();
    }
  }
}
const void* pick_kernel(int MT, int fmt, int XL, int kind) {
  const int vi = var_index(MT, XL, kind);
  if (fmt == FMT_BLOCK)
    return kind == 2 ? pick_fmt<FMT_BLOCK, 2>(vi) : kind ? pick_fmt<FMT_BLOCK, 1>(vi) : pick_fmt<FMT_BLOCK, 0>(vi);
  return kind == 2 ? pick_fmt<FMT_MX, 2>(vi) : kind ? pick_fmt<FMT_MX, 1>(vi) : pick_fmt<FMT_MX, 0>(vi);
}

constexpr int LDS_PER_WG = 163840;  // gfx950: 160 KB of LDS per workgroup
size_t static_lds(int MT) {
  switch (MT) {
    case 1: return sizeof(Lds<1, Cfg<1>::NS, Cfg<1>::NSLOT>);
    case 2: return sizeof(Lds<2, Cfg<2>::NS, Cfg<2>::NSLOT>);
    case 4: return sizeof(Lds<4, Cfg<4>::NS, Cfg<4>::NSLOT>);
    default: return sizeof(Lds<8, Cfg<8>::NS, Cfg<8>::NSLOT>);
  }
}
// LDS stages of the staged gate/up (the MLP variants with Cfg::KS).
int ks_dyn(int MT, bool mlp) {
  if (!mlp) return 0;
  return MT == 4 ? Cfg<4>::DA * ks_stage_bytes<4>() : MT == 8 ? Cfg<8>::DA * ks_stage_bytes<8>() : 0;
}
// Q(x) goes to LDS when it fits beside the partial-sum slots (with margin).
bool use_xl(int fmt, int MT, int K1) {
  if (MT > 2) return false;
  return static_lds(MT) + (size_t)xl_bytes(fmt, 16 * MT, K1) + 1024 <= (size_t)LDS_PER_WG;
}

// Workgroups resident at once on the current device for each kernel variant
// (queried once per device): the grid, so that every workgroup runs
// concurrently with every other.
struct Occupancy {
  std::mutex mu;
  int cus[64] = {0};
  int per_cu[64][2][NVAR] = {};
};
Occupancy g_occ;

// The XL variants may use up to all LDS the static part leaves; the
// occupancy is taken at that maximum, so it holds for any smaller use.
int grid_size(int MT, int fmt, int XL, int kind, int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return SGD_EHIP;
  const int fi = fmt == FMT_BLOCK ? 0 : 1;
  const int vi = var_index(MT, XL, kind);
  std::lock_guard<std::mutex> lock(g_occ.mu);
  if (g_occ.cus[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return SGD_EHIP;
    g_occ.cus[dev] = cus;
  }
  if (g_occ.per_cu[dev][fi][vi] == 0) {
    const void* kern = pick_kernel(MT, fmt, XL, kind);
    const int dyn = XL ? LDS_PER_WG - (int)static_lds(MT) : ks_dyn(MT, kind != 0);
    // (any variant may be launched with up to all the LDS its static part
    // leaves: the decode block's row stash)
    if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_PER_WG - (int)static_lds(MT)) !=
        hipSuccess)
      return SGD_EHIP;
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, 64 * cfg_nwave(MT), (size_t)dyn) != hipSuccess ||
        nb <= 0)
      return SGD_EHIP;
    g_occ.per_cu[dev][fi][vi] = nb;
  }
  *out = g_occ.cus[dev] * g_occ.per_cu[dev][fi][vi];
  return SGD_OK;
}

}  // namespace

size_t stream_workspace_bytes(int fmt, int M, int K1, int F, int N, int K2, bool mlp) {
  // the layout does not depend on the grid (partial slots are sized for MAX_WG)
  const Plan p = make_plan(fmt, M, K1, F, N, K2, mlp, MAX_WG);
  return p.ok ? p.bytes : 0;
}

int act_mtile_pad(int M) { return 16 * mt_for(M); }

int launch_swiglu_quantize(int fmt, const float* gu, int M, int F, uint8_t* aq, void* as, hipStream_t s) {
  const int Mpad = 16 * mt_for(M);
  const size_t waves = (size_t)(F / 128) * (size_t)((M + 15) / 16);
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (fmt == FMT_BLOCK)
    hipLaunchKernelGGL(swiglu_quant_kernel<FMT_BLOCK>, grid, dim3(256), 0, s, gu, M, F, Mpad, aq, as);
  else
    hipLaunchKernelGGL(swiglu_quant_kernel<FMT_MX>, grid, dim3(256), 0, s, gu, M, F, Mpad, aq, as);
  return hip_status(hipGetLastError());
}

// The same for Mrows (a multiple of 16) rows in the full-tile layout: block
// scales [F/128][Mrows].
int launch_swiglu_quantize_tiles(int fmt, const float* gu, int Mrows, int F, uint8_t* aq, void* as, hipStream_t s) {
  const size_t waves = (size_t)(F / 128) * (size_t)(Mrows / 16);
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (fmt == FMT_BLOCK)
    hipLaunchKernelGGL(swiglu_quant_kernel<FMT_BLOCK>, grid, dim3(256), 0, s, gu, Mrows, F, Mrows, aq, as);
  else
    hipLaunchKernelGGL(swiglu_quant_kernel<FMT_MX>, grid, dim3(256), 0, s, gu, Mrows, F, Mrows, aq, as);
  return hip_status(hipGetLastError());
}

int stream_workspace_layout(int fmt, int M, int K1, int F, size_t (&off)[5]) {
  const Plan p = make_plan(fmt, M, K1, F, K1, F, true, MAX_WG);
  if (!p.ok) return SGD_EDIM;
  off[0] = p.off_xa;
  off[1] = p.off_xs;
  off[2] = p.off_a32;
  off[3] = p.off_aq;
  off[4] = p.off_as;
  return SGD_OK;
}

int launch_stream(const Problem& pr, hipStream_t s) {
  const bool mlp = pr.gate != nullptr;
  const int F = mlp ? pr.gate->N : 0;
  const int MT = mt_for(pr.M);
  // (activations given already quantized are read from the caller's
  // buffers; the decode block quantizes x into the workspace, row by row)
  const int plain_xl = !pr.xq_in && use_xl(pr.fmt, MT, pr.K1) ? 1 : 0;
  const int XL = plain_xl && !pr.h_in ? 1 : 0;
  // (the decode block runs on the grid of the plain MLP's kernel: the same
  // split of the work, so the same sums, bit for bit)
  int G = 0;
  int rc = grid_size(MT, pr.fmt, plain_xl, mlp ? 1 : 0, &G);
  if (rc != SGD_OK) return rc;
  if (pr.h_in) {
    // the block's own kernel must fit one workgroup per compute unit
    int Gb = 0;
    rc = grid_size(MT, pr.fmt, 0, 2, &Gb);
    if (rc != SGD_OK) return rc;
  }
  if (pr.h_in && !plain_xl) {
    // one workgroup per compute unit, which the row stash always leaves room for
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return SGD_EHIP;
    const int cus = g_occ.cus[dev];
    if (G > cus) G = cus;
  }
  if (G > MAX_WG) G = MAX_WG;
  const Plan p = make_plan(pr.fmt, pr.M, pr.K1, F, pr.w2->N, pr.w2->K, mlp, G);
  if (!p.ok) return SGD_EDIM;
  Args a{};
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
    a.scale_bytes_g = (uint32_t)sgd_packed_scales_bytes(pr.fmt, F, pr.K1);
  }
  a.F = F;
  a.w2 = static_cast<const uint8_t*>(pr.w2->codes);
  a.s2 = pr.w2->scales;
  a.N = pr.w2->N;
  a.K2 = pr.w2->K;
  a.scale_bytes_2 = (uint32_t)sgd_packed_scales_bytes(pr.fmt, a.N, a.K2);
  a.y = pr.y;
  a.y32 = pr.y32;
  a.h_in = pr.h_in;
  a.h_out = pr.h_out;
  a.eps = pr.eps;
  size_t dyn = XL ? (size_t)((xl_bytes(pr.fmt, p.Mpad, pr.K1) + 15) & ~15) : (size_t)ks_dyn(p.MT, mlp);
  if (pr.h_in) {
    // the prologue's row stash, where it fits beside the static LDS (the
    // dynamic LDS is otherwise unused until the prologue is done)
    const size_t row = (size_t)pr.K1 * 4;
    if (static_lds(p.MT) + (row > dyn ? row : dyn) + 1024 <= (size_t)LDS_PER_WG) {
      a.row_stash = 1;
      if (row > dyn) dyn = row;
    }
  }
  uint8_t* ws = static_cast<uint8_t*>(pr.ws);
  a.ctrl = reinterpret_cast<uint32_t*>(ws);
  a.xa = ws + p.off_xa;
  a.xs = ws + p.off_xs;
  a.a32 = reinterpret_cast<float*>(ws + p.off_a32);
  a.aq = ws + p.off_aq;
  a.as = ws + p.off_as;
  a.gpart = reinterpret_cast<float*>(ws + p.off_gpart);
  a.dpart = reinterpret_cast<float*>(ws + p.off_dpart);
  a.amax = reinterpret_cast<float*>(ws + p.off_amax);
  a.G = G;
  a.n_pairs = p.n_pairs;
  a.n_items = XL ? 0 : p.n_items;
  if (pr.h_in) {
    // the prologue's items: rows, each split into row_parts shares of its
    // 128-column groups, as few as give every lane of a workgroup at most one
    // 32-column block (each share reads the whole row for its sum of squares)
    const int ng = pr.K1 / 128, lanes = 64 * cfg_nwave(MT);
    int parts = (4 * ng + lanes - 1) / lanes;
    if (parts > G / pr.M) parts = G / pr.M;
    if (parts < 1) parts = 1;
    a.row_parts = parts;
    a.n_items = pr.M * parts < G ? pr.M * parts : G;
  }
  if (pr.xq_in) {
    // nothing to quantize: Q(x) is the caller's, in the workspace layout
    a.xa = const_cast<uint8_t*>(pr.xq_in);
    a.xs = const_cast<void*>(pr.xs_in);
    a.n_items = 0;
  }
  a.ngroups = p.ngroups;
  a.ks = p.ks;
  a.keep_a = keep_intermediates() ? 1 : 0;
  a.budget = wait_budget_ticks();
  a.gu = p.gu;
  a.dn = p.dn;
  void* args[] = {&a};
  const int kind = pr.h_in ? 2 : mlp ? 1 : 0;
  return hip_status(hipLaunchKernel(pick_kernel(p.MT, pr.fmt, XL, kind), dim3(G), dim3(64 * cfg_nwave(p.MT)), args, dyn, s));
}

}  // namespace sgd

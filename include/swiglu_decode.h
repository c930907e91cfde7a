/*
 * swiglu_decode.h -- C ABI of the decode-shape FP8 SwiGLU MLP library for
 * AMD Instinct MI355X (gfx950).
 *
 * What it computes.  The layer is the SwiGLU MLP of a decoder ("activation,
 * gate multiplication, down projection"; Fish Audio X post "We Made Our Best
 * Voice Model Free. Here's the GPU Math Behind It.", section "Custom kernels
 * for the shapes TTS actually uses"):
 *
 *     y = ( silu(x Wg^T) * (x Wu^T) ) Wd^T,   silu(g) = g / (1 + exp(-g))
 *
 * at decode shapes (1 <= M <= 128 rows), with FP8 E4M3 weights and
 * activations in one of two scaling formats (same X post section; fish.audio
 * blog "Cómo hicimos que nuestra API de texto a voz sea gratuita…", sections
 * "Estrategia de cuantización FP8" and "Qué hay en código abierto"):
 *
 *   SGD_FMT_BLOCK128  one fp32 scale per 128x128 weight tile and per 1x128
 *                     activation group; s = amax / 448, code = E4M3(v / s).
 *   SGD_FMT_MX32      one E8M0 power-of-two scale per 1x32 block along K on
 *                     both operands (OCP MX v1.0), 2^X with
 *                     X = floor(log2(amax)) - 8, code = E4M3(v * 2^-X).
 *
 * E4M3 conversion rounds to nearest with ties to even and saturates at
 * +-448.  The activation quantization, both GEMMs, SiLU(gate)*up and the
 * re-quantization of that product run in ONE kernel launch
 * (sgd_fused_swiglu_mlp); the blog's section "Resultados de benchmark del
 * kernel" fuses activation quantization with the scale packing and the
 * SwiGLU prologue with the down GEMM's activation quantization.
 *
 * Conventions shared by every call:
 *   - Pointers to tensors are DEVICE pointers owned by the caller; bf16 is
 *     passed as uint16_t bit patterns.  Matrices are row-major.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously; nothing synchronises the host.
 *   - The library never allocates or frees memory and keeps no per-call
 *     global state (its one process-wide setting is the wait budget below),
 *     so calls can be captured into a hipGraph.
 *   - Errors detected on the host (bad argument, shape, alignment, size)
 *     are returned as a negative sgd_status and NOTHING is launched.  A
 *     launch failure returns SGD_EHIP.  Faults inside a kernel surface on
 *     the caller's next stream synchronisation, as for any HIP kernel.
 *   - Tensors whose pointer must be 16-byte aligned: bf16 x / W / y, fp8
 *     codes, workspaces.  Scale arrays: 4-byte aligned.
 */
#ifndef SWIGLU_DECODE_H
#define SWIGLU_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
enum {
  SGD_OK = 0,
  SGD_EINVAL = -1,     /* null pointer, non-positive size, M out of range   */
  SGD_EALIGN = -2,     /* a pointer is not aligned as documented            */
  SGD_EDIM = -3,       /* a dimension is not a multiple of its tile size    */
  SGD_EWORKSPACE = -4, /* workspace missing or smaller than required        */
  SGD_EFMT = -5,       /* unknown format, or operands of different formats  */
  SGD_EHIP = -6,       /* the HIP runtime refused a launch or a query       */
  SGD_ETIMEOUT = -7    /* a persistent kernel's wait gave up (see below)    */
};

/* ---- formats ----------------------------------------------------------- */
enum { SGD_FMT_BLOCK128 = 1, SGD_FMT_MX32 = 2 };

#define SGD_MAX_M 128 /* largest row count of sgd_scaled_gemm / fused MLP */
#define SGD_MAX_M_LARGE 65536 /* largest row count of the large-M (prefill) path */

/*
 * A packed (pre-shuffled) FP8 weight W [N, K] in nn.Linear orientation
 * (y = x W^T).  `codes` and `scales` are device buffers of
 * sgd_packed_codes_bytes / sgd_packed_scales_bytes bytes written by
 * sgd_quantize_pack_weight.  N and K are multiples of 128.
 *
 * Packed code layout: 16x128 tiles, tile (j, t) at byte (j*(K/128) + t)*2048;
 * element (r, c) of a tile at byte h*1024 + lane*16 + b with h = c/64,
 * q = (c%64)/16, b = c%16, lane = r + 16*q (the operand order of the
 * 16x16x128 fp8 MFMA: lane l owns row l%16).
 * Scales: BLOCK128 -> fp32 [N/128, K/128] row-major.  MX32 -> E8M0 bytes;
 * for row band j and k-tile group g (4 k-tiles) 256 bytes at
 * (j*ceil(K/512) + g)*256, byte lane*4 + i = scale of row 16j + lane%16,
 * 32-column block 4*(4g+i) + lane/16; bytes past K are zero.
 */
typedef struct sgd_weight {
  int32_t fmt;        /* SGD_FMT_BLOCK128 or SGD_FMT_MX32 */
  int32_t N;          /* output features (rows of W)       */
  int32_t K;          /* input features (columns of W)     */
  int32_t reserved;   /* must be 0                         */
  const void* codes;  /* packed E4M3 codes, device          */
  const void* scales; /* packed scales, device              */
} sgd_weight;

/* Human-readable name of a status code (static string, never NULL). */
const char* sgd_status_str(int status);

/* ABI version of this header (bumped on incompatible change). */
int sgd_abi_version(void);

/* ---- sizes ------------------------------------------------------------- */
/* Bytes of the packed codes / packed scales of an N x K weight; 0 if the
 * format or a dimension is invalid.  Every weight of this library has N and
 * K positive multiples of 128, each at most 2^20, and N*K < 2^31 (the
 * streaming kernels address a weight with 32-bit offsets). */
size_t sgd_packed_codes_bytes(int fmt, int N, int K);
size_t sgd_packed_scales_bytes(int fmt, int N, int K);

/*
 * Quantize a bf16 weight W [N, K] (row-major) and write it in the packed
 * layout.  One launch.  BLOCK128: amax over each 128x128 tile, s = amax/448
 * (IEEE fp32 division; s = 1 for an all-zero tile), codes E4M3(w / s).
 * MX32: per row, per 32 columns, E8M0 X = floor(log2 amax) - 8 (E = 0 for
 * an all-zero block), codes E4M3(w * 2^-X).  Passage: fish.audio blog,
 * section "Estrategia de cuantización FP8" (128x128 block and 1x32 UE8M0
 * microscaling) and the X post section "Custom kernels for the shapes TTS
 * actually uses".  The output is bit-identical to the plain definition.
 * Errors: SGD_EFMT, SGD_EINVAL (null, N/K <= 0 or > 2^20), SGD_EDIM (N or K
 * not a multiple of 128, or N*K >= 2^31), SGD_EALIGN.
 */
int sgd_quantize_pack_weight(int fmt, const uint16_t* w_bf16, int N, int K,
                             void* codes_out, void* scales_out, void* stream);

/*
 * Inverse of the packing (for inspection and tests): codes_rowmajor [N, K]
 * uint8 and scales in logical layout (BLOCK128 fp32 [N/128, K/128];
 * MX32 uint8 [N, K/32]).  Errors as sgd_quantize_pack_weight.
 */
int sgd_unpack_weight(const sgd_weight* w, uint8_t* codes_rowmajor,
                      void* scales_logical, void* stream);

/*
 * Per-row activation quantization of x [M, K] bf16 along K: BLOCK128 groups
 * of 128 (fp32 scales [M, K/128]) or MX32 blocks of 32 (E8M0 [M, K/32]),
 * same rules as the weights.  This is the prologue the fused kernels run
 * internally (fish.audio blog, section "Resultados de benchmark del kernel":
 * activation quantization and UE8M0 scale packing in one launch).
 * 1 <= M <= 65536; K a positive multiple of 128.
 */
int sgd_quantize_act(int fmt, const uint16_t* x_bf16, int M, int K,
                     uint8_t* codes, void* scales, void* stream);

/* ---- workspaces -------------------------------------------------------- */
/*
 * The GEMM and MLP kernels need a device workspace for the quantized
 * activations, the SwiGLU intermediate, split-K partial sums, per-row maxima
 * exchanged while re-quantizing (M > 32) and synchronisation counters.  Its first 256 KB are a control block that must
 * be zero-filled ONCE after allocation (sgd_workspace_clear or any fill
 * kernel); every call that completes leaves it ready for the next (counters
 * zero, flags holding the number of the launch that raised them), so one
 * workspace can serve calls of any shape that fit in it.  After a call that
 * did not complete (a device fault, or SGD_ETIMEOUT from sgd_workspace_status),
 * clear it again.  Calls that share a workspace must not overlap (serialise
 * them on one stream).  Size in bytes; 0 on invalid arguments (weight limits
 * as for sgd_packed_codes_bytes; ffn <= 32768 for the MLP).  The size does
 * not depend on the device.
 *
 * Persistent kernels.  sgd_scaled_gemm and sgd_fused_swiglu_mlp launch one
 * workgroup per compute unit, and their workgroups wait for each other, so
 * all of them must be resident at once: do not run a second such launch (or
 * any kernel that holds compute units for long) concurrently on the same
 * device.  Every wait is bounded: one that spins longer than the wait budget
 * gives up, the launch then runs to its end without waiting (its outputs are
 * invalid) and the workspace records the failure, which
 * sgd_workspace_status reports.
 */
size_t sgd_gemm_workspace_bytes(int fmt, int M, int N, int K);
size_t sgd_mlp_workspace_bytes(int fmt, int M, int d, int ffn);

/*
 * Where sgd_fused_swiglu_mlp keeps its intermediates in the workspace, for
 * inspection and tests (the layout belongs to this ABI version).  Writes
 * five byte offsets into `offsets` (host array of 5):
 *   [0] Q(x) codes, [1] Q(x) scales, [2] a = silu(g)*u, fp32 [M, ffn]
 *   row-major, [3] Q(a) codes, [4] Q(a) scales.
 * Codes are stored m-tile by m-tile: rows 16t..16t+Mt-1 (Mt = min(16,
 * M-16t)) form K/16 segments of 16 columns, each segment the Mt rows' 16
 * codes in row order (K = d for Q(x), ffn for Q(a)).  BLOCK128 scales: fp32
 * [K/128][Mpad] (Mpad = M rounded up to 16, 32, 64 or 128; padded rows
 * zero).  MX32 scales: m-tile t holds, per 128-column k-tile, the Mt rows'
 * four E8M0 bytes (one dword per row, 32-column blocks in order).  Q(x) is
 * written to the workspace only when it does not fit in LDS (in practice
 * M > 32, or a very wide d); Q(a) always; a always at M <= 32 and otherwise
 * only with sgd_set_keep_intermediates(1).  Returns SGD_OK or
 * SGD_EINVAL (shape or format invalid, or offsets NULL).
 */
int sgd_mlp_workspace_layout(int fmt, int M, int d, int ffn, size_t* offsets);

/* Zero-fill `bytes` bytes of `workspace` with a fill kernel (no memset
 * node, so it is safe to capture).  bytes must be a multiple of 16. */
int sgd_workspace_clear(void* workspace, size_t bytes, void* stream);

/* Set the wait budget of the persistent kernels: the longest any one of
 * their cross-workgroup waits may spin before the launch gives up, in
 * microseconds (0 restores the default of 1 s).  A process-wide setting read
 * when a call is launched (a captured graph keeps the value of its capture).
 * Returns the previous budget. */
uint32_t sgd_set_wait_budget_us(uint32_t us);

/* Keep the SwiGLU intermediate for inspection: when nonzero, fused MLP and
 * decode-block calls also store a = silu(g)*u (fp32) in the workspace where
 * sgd_mlp_workspace_layout says, also on the path (M > 32) whose re-
 * quantization works from registers and does not otherwise store it.  For
 * tests and debugging; it costs store bandwidth.  Process-wide, read when a
 * call is launched (a captured graph keeps the value of its capture); 0 by
 * default.  Returns the previous setting. */
int sgd_set_keep_intermediates(int keep);

/* Whether any launch on `workspace` gave up a wait since the workspace was
 * last cleared: SGD_OK, or SGD_ETIMEOUT (then the outputs of the call(s)
 * concerned are invalid; clear the workspace before reusing it).
 * SYNCHRONISES `stream` and reads one word of the control block to the host,
 * so it is a diagnostic, not for graph capture.  Errors: SGD_EINVAL (null),
 * SGD_EALIGN, SGD_EHIP. */
int sgd_workspace_status(const void* workspace, void* stream);

/* ---- the hot path ------------------------------------------------------ */
/*
 * y [M, N] bf16 = Q(x) * W^T: x [M, K] bf16 is quantized per row in W's
 * format, multiplied by the packed weight with fp32 accumulation on the
 * MFMA units, and rounded to bf16 (nearest-even).  One launch.  Passage:
 * fish.audio blog, section "Qué hay en código abierto" (FP8 GEMM with 1x128
 * activation x 128x128 weight blocks, and MXFP8 1x32 UE8M0).
 * 1 <= M <= SGD_MAX_M.  Errors: SGD_EINVAL, SGD_EALIGN, SGD_EDIM, SGD_EFMT,
 * SGD_EWORKSPACE (ws_bytes < sgd_gemm_workspace_bytes).
 */
int sgd_scaled_gemm(const uint16_t* x_bf16, int M, const sgd_weight* w,
                    uint16_t* y_bf16, void* workspace, size_t ws_bytes,
                    void* stream);

/*
 * y [M, d] bf16 = SwiGLU MLP of x [M, d] bf16 with packed gate [ffn, d],
 * up [ffn, d] and down [d, ffn] weights, all in one format.  ONE launch:
 * quantize x; g = Q(x) Wg^T and u = Q(x) Wu^T in fp32; a = silu(g) * u in
 * fp32; re-quantize a per row along ffn in the same format; y = Q(a) Wd^T
 * in fp32; round to bf16.  The intermediates stay in the workspace (on-chip
 * caches in practice) and never round-trip through a separate launch.
 * 1 <= M <= SGD_MAX_M; d and ffn multiples of 128.  Errors as
 * sgd_scaled_gemm, plus SGD_EFMT when the three weights differ in format
 * and SGD_EDIM when their shapes do not chain.
 */
int sgd_fused_swiglu_mlp(const uint16_t* x_bf16, int M, const sgd_weight* gate,
                         const sgd_weight* up, const sgd_weight* down,
                         uint16_t* y_bf16, void* workspace, size_t ws_bytes,
                         void* stream);

/*
 * The fused SwiGLU MLP for callers that cannot allocate device memory (code
 * under graph capture that may not call hipMalloc, tight serving loops,
 * harnesses that forbid allocation): the same computation and kernel as
 * sgd_fused_swiglu_mlp, with the workspace taken from a fixed array of
 * SGD_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it
 * runs on until the process ends (device-side static memory; no hipMalloc,
 * hipFree or allocating library call is made).  The caller passes inputs and
 * outputs as for sgd_fused_swiglu_mlp.  Shapes whose workspace
 * (sgd_mlp_workspace_bytes) exceeds the array return SGD_EWORKSPACE; every
 * M <= 128 with d <= 16384 and ffn <= 32768 fits.  The first call on a device
 * zero-fills the array's control block with a kernel on `stream`.  All calls
 * on one GPU share its array and it keeps the last call's contents: calls
 * that overlap on one GPU (two streams, two threads) race and must be
 * serialised by the caller, also against each other's graph replays.  A
 * wait that gives up (see the wait budget) leaves that call's output
 * invalid with no status to query; use the workspace entry point where that
 * matters.  Errors as sgd_fused_swiglu_mlp.
 */
#define SGD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int sgd_fused_swiglu_mlp_noalloc(const uint16_t* x_bf16, int M, const sgd_weight* gate,
                                 const sgd_weight* up, const sgd_weight* down,
                                 uint16_t* y_bf16, void* stream);

/*
 * One pre-RMSNorm residual decode block in ONE launch: the fused SwiGLU MLP
 * with its RMSNorm prologue and residual epilogue,
 *   h_out = fl32( h_in + bf16( MLP( bf16( h_in / sqrt(mean(h_in^2) + eps) ) ) ) )
 * per row (unit-gain RMSNorm, Zhang & Sennrich 2019; MLP as
 * sgd_fused_swiglu_mlp).  The kernel forms x = bf16(RMSNorm(h_in)) itself,
 * bit-identical to sgd_rmsnorm_bf16, and adds the bf16 MLP output to h_in in
 * fp32 as sgd_residual_add does, so the result is bit-identical to
 * sgd_rmsnorm_bf16 + sgd_fused_swiglu_mlp + sgd_residual_add.  A decode step
 * of L blocks is then L launches (plus the head), which a caller captures as
 * one graph: the serving context of the fish.audio blog, sections "Qué hay en
 * código abierto" (graph-capture safety) and "Hardware y adquisición" (decode
 * batches up to 64 under graph capture).
 * h_in, h_out [M, d] fp32, 16-byte aligned; h_out must not overlap h_in
 * (SGD_EINVAL), so a stack alternates two buffers.  0 <= eps <= 1.  Weights,
 * workspace (sgd_mlp_workspace_bytes) and errors as sgd_fused_swiglu_mlp.
 */
int sgd_fused_swiglu_block(const float* h_in, int M, const sgd_weight* gate,
                           const sgd_weight* up, const sgd_weight* down, float eps,
                           float* h_out, void* workspace, size_t ws_bytes,
                           void* stream);

/* ---- large-M (prefill) path: compute-bound tiled GEMMs ------------------ */
/*
 * The pages' second benchmark family (fish.audio blog, section "Resultados
 * de benchmark del kernel": the SwiGLU MLP at M from 1 to 4096, and square
 * MXFP8 GEMMs from 1024^3 to 16384^3), where the arithmetic intensity (about
 * M flop per weight byte) puts the matrix cores, not HBM, on the critical
 * path.  Same quantization, weights and arithmetic as the decode path (the
 * scaled fp8 MFMA with fp32 accumulation), in an LDS-tiled kernel: blocks
 * of 256x128 (128x128 when that gives fewer blocks than compute units) of
 * the output over all of K, two LDS stages.  Several launches each; no
 * persistent waits.  Their workspaces keep no state between calls and leave
 * the first 256 KB (a persistent call's control block) untouched, so one
 * workspace may serve both paths when the calls are serialised.
 */

/* Workspace of sgd_scaled_gemm_large: Q(x) in 16-row tiles.  0 for an
 * unsupported shape (M > SGD_MAX_M_LARGE, N or K not multiples of 128, or
 * 16*ceil(M/16)*K >= 2^31). */
size_t sgd_gemm_large_workspace_bytes(int fmt, int M, int N, int K);

/* y [M, N] bf16 = Q(x) W^T for x [M, K] bf16, any 1 <= M <= SGD_MAX_M_LARGE:
 * the result of sgd_scaled_gemm (fish.audio blog, section "Qué hay en código
 * abierto"), up to the order of the fp32 sums.  Two launches (quantize x,
 * tiled GEMM).  Errors as sgd_scaled_gemm, workspace
 * sgd_gemm_large_workspace_bytes. */
int sgd_scaled_gemm_large(const uint16_t* x_bf16, int M, const sgd_weight* w,
                          uint16_t* y_bf16, void* workspace, size_t ws_bytes,
                          void* stream);

/* Workspace of sgd_swiglu_mlp_prefill: Q(x), the fp32 gate/up products of
 * 16*ceil(M/16) rows and Q(a).  0 for an unsupported shape. */
size_t sgd_mlp_prefill_workspace_bytes(int fmt, int M, int d, int ffn);

/* y [M, d] bf16 = SwiGLU MLP of x [M, d] bf16 for large M (the arithmetic of
 * sgd_fused_swiglu_mlp, fish.audio blog, section "Qué hay en código
 * abierto"; X post, section "Custom kernels for the shapes TTS actually
 * uses"): quantize x; [g | u] = Q(x) [Wg; Wu]^T in fp32 (tiled GEMM);
 * a = silu(g) * u re-quantized per row; y = Q(a) Wd^T (tiled GEMM).  Four
 * launches, intermediates in the workspace.  gate_up is the stacked
 * [2*ffn, d] weight (gate rows first, as sgd_scaled_gemm_f32 of the
 * unfused pipeline reads it); down is [d, ffn].  1 <= M <= SGD_MAX_M_LARGE.
 * Errors: SGD_EINVAL, SGD_EALIGN, SGD_EDIM (shapes that do not chain or are
 * unsupported), SGD_EFMT, SGD_EWORKSPACE. */
int sgd_swiglu_mlp_prefill(const uint16_t* x_bf16, int M, const sgd_weight* gate_up,
                           const sgd_weight* down, uint16_t* y_bf16, void* workspace,
                           size_t ws_bytes, void* stream);

/* ---- paged decode attention over an MXFP8 K/V cache -------------------- */
/*
 * The other half of a decode step (fish.audio blog, section "Qué hay en
 * código abierto": MXFP8 FlashAttention, paged decode with native GQA through
 * a stride-0 K/V broadcast; section "Resultados de benchmark del kernel" for
 * its measurement).  head_dim is 128.
 *
 * Cache: pages of 16 token slots; per (page, KV head) 2112 bytes, so a cache
 * is [n_pages][Hkv][2112] bytes (16-byte aligned).  Each token's K and V
 * vectors are quantized on their own in 1x32 MX blocks along head_dim (E4M3,
 * E8M0 scale) when written.
 *   K: bytes 0..2047: the 16 x 128 operand tile of the slots (lane l = r + 16q
 *      holds slot r, dims 16q..16q+15 at bytes 16l.. and dims 64+16q..
 *      at 1024 + 16l..); bytes 2048 + l: scale of (slot l % 16, block l / 16).
 *   V: byte 32l + 4n + (r % 4), l = (d % 16) + 16 (r / 4): code of
 *      (slot r, dim d = 16n + d % 16), n < 8 (each lane's 32 bytes hold four
 *      consecutive slots of its dims); byte 2048 + 16 (r / 4) + 4b + r % 4:
 *      scale of (slot r, block b).
 * Slot s of a sequence's token t is page block_table[b][t / 16], slot t % 16.
 */

/* Bytes of one cache (K or V): n_pages * Hkv * 2112, or 0 when that reaches 2^31. */
size_t sgd_kv_cache_bytes(int n_pages, int Hkv);

/* Quantize and write n tokens' vectors x [n, Hkv, head_dim] bf16 into a cache
 * (kind 0: K layout, 1: V layout) at slots[i] = page * 16 + offset (int32).
 * Slots outside [0, n_pages * 16) are skipped.  head_dim must be 128.
 * Errors: SGD_EINVAL, SGD_EDIM, SGD_EALIGN. */
int sgd_kv_cache_write(int kind, const uint16_t* x_bf16, const int32_t* slots, int n, int Hkv,
                       int head_dim, uint8_t* cache, int n_pages, void* stream);

/* Workspace of sgd_paged_decode_attention (per-split partial results), or 0
 * for unsupported sizes. */
size_t sgd_paged_attention_workspace_bytes(int B, int Hq, int Hkv, int max_pages);

/* out [B, Hq, 128] bf16 = softmax(sm_scale * q' K'^T) V' per sequence b and
 * query head h over the sequence's seq_lens[b] tokens, q' the query quantized
 * like the cache (MX, 32-dim blocks), query head h reading KV head
 * h / (Hq / Hkv) (Hq a multiple of Hkv, at most 16 query heads per KV head).
 * block_table [B, max_pages] int32 gives each sequence's physical pages;
 * lengths are clamped to [0, max_pages * 16], a length of 0 gives zeros, and
 * table entries outside [0, n_pages) read zeros (their values are then
 * undefined, never an access out of bounds).  Two launches (page splits in
 * parallel, then their merge).  Errors: SGD_EINVAL, SGD_EDIM (head_dim !=
 * 128), SGD_EALIGN (q, caches, out 16-byte; table, lengths 4-byte),
 * SGD_EWORKSPACE. */
int sgd_paged_decode_attention(const uint16_t* q_bf16, const uint8_t* k_cache,
                               const uint8_t* v_cache, int n_pages, const int32_t* block_table,
                               int max_pages, const int32_t* seq_lens, int B, int Hq, int Hkv,
                               int head_dim, float sm_scale, uint16_t* out_bf16, void* workspace,
                               size_t ws_bytes, void* stream);

/* ---- the unfused pipeline (three launches, intermediates in HBM) -------- */
/*
 * The same MLP as sgd_fused_swiglu_mlp in three launches whose intermediates
 * go through HBM, the launch-per-step form the fused kernel replaces (Fish
 * Audio X post, section "Custom kernels for the shapes TTS actually uses":
 * separate launches for activation, gate multiplication and down projection,
 * each writing to and reading from HBM; fish.audio blog, section "Resultados
 * de benchmark del kernel", fusing the SwiGLU prologue into the down GEMM's
 * activation quantization):
 *   1. gu [M, 2*ffn] fp32 = Q(x) [Wg; Wu]^T          sgd_scaled_gemm_f32
 *      (one packed weight [2*ffn, d]: the packed gate followed by the packed
 *      up, codes after codes and scales after scales, is the packing of the
 *      stacked matrix, since both layouts run band by band);
 *   2. Q(a), a = silu(g) * u                         sgd_swiglu_quantize
 *   3. y = Q(a) Wd^T                                 sgd_scaled_gemm_q
 *
 * Activations in the WORKSPACE LAYOUT (the layout sgd_mlp_workspace_layout
 * documents): codes M*K bytes stored m-tile by m-tile; scales of
 * sgd_act_scales_bytes bytes (BLOCK128: fp32 [K/128][Mpad], Mpad = M
 * rounded up to 16, 32, 64 or 128, padded rows zero; MX32: per m-tile and
 * 128-column k-tile one dword of four E8M0 bytes per row).
 */

/* y [M, N] fp32 = Q(x) W^T: sgd_scaled_gemm with an fp32 output (16-byte
 * aligned).  Same workspace and errors. */
int sgd_scaled_gemm_f32(const uint16_t* x_bf16, int M, const sgd_weight* w,
                        float* y_f32, void* workspace, size_t ws_bytes,
                        void* stream);

/* Bytes of the scales of M x K activations in the workspace layout; 0 when
 * invalid (1 <= M <= SGD_MAX_M, K a positive multiple of 128). */
size_t sgd_act_scales_bytes(int fmt, int M, int K);

/* From gu [M, 2*ffn] fp32 (g in columns [0, ffn), u in [ffn, 2*ffn)):
 * a = silu(g) * u in fp32, quantized per row along ffn in `fmt` (the rules
 * of sgd_quantize_act) into codes aq [M*ffn] and scales `as`, workspace
 * layout.  One launch.  1 <= M <= SGD_MAX_M; ffn a multiple of 128.  gu
 * and aq 16-byte aligned, as 4-byte aligned.  Errors: SGD_EFMT, SGD_EINVAL,
 * SGD_EDIM, SGD_EALIGN. */
int sgd_swiglu_quantize(int fmt, const float* gu, int M, int ffn, uint8_t* aq,
                        void* as, void* stream);

/* y [M, N] bf16 = Q(x) W^T with Q(x) given already quantized in W's format
 * (codes xq [M*K] and scales xs in the workspace layout), fp32 accumulation.
 * Same workspace (sgd_gemm_workspace_bytes) and errors as sgd_scaled_gemm;
 * xq 16-byte aligned, xs 4-byte aligned. */
int sgd_scaled_gemm_q(const uint8_t* xq, const void* xs, int M,
                      const sgd_weight* w, uint16_t* y_bf16, void* workspace,
                      size_t ws_bytes, void* stream);

/* ---- decode-stack glue (pre-RMSNorm residual blocks + output head) ----- */
/* These calls serve the 24-block decode-stack workload only (24 pre-RMSNorm
 * residual SwiGLU blocks at d=2560, ffn=9728, then a bf16 output head and a
 * per-row argmax).  The pages describe the MLP, not the layers around it:
 * no passage defines these operations; each comment states the definition
 * used.  Errors: SGD_EINVAL (null pointer, M or shape out of range),
 * SGD_EALIGN, SGD_EDIM. */
/* h [M, d] fp32 <- x [M, d] bf16 (exact widening).  d multiple of 128. */
int sgd_bf16_to_f32(const uint16_t* x_bf16, int M, int d, float* h, void* stream);

/* x [M, d] bf16 = bf16( h / sqrt(mean(h^2) + eps) ) per row, unit gain
 * (Zhang & Sennrich 2019, RMSNorm).  d multiple of 128. */
int sgd_rmsnorm_bf16(const float* h, int M, int d, float eps, uint16_t* x_bf16,
                     void* stream);

/* h [M, d] fp32 += y [M, d] bf16 (the residual add). */
int sgd_residual_add(float* h, const uint16_t* y_bf16, int M, int d, void* stream);

/* The residual add and the next block's RMSNorm in one launch: h += y, then
 * x = bf16( h / sqrt(mean(h^2) + eps) ) per row, unit gain.  Bit-identical
 * to sgd_residual_add followed by sgd_rmsnorm_bf16 (one pass less over h and
 * one launch less between two blocks).  h [M, d] fp32 is updated in place;
 * y, x [M, d] bf16; all 16-byte aligned; d multiple of 128.  x must not
 * overlap h or y. */
int sgd_residual_rmsnorm_bf16(float* h, const uint16_t* y_bf16, int M, int d, float eps,
                              uint16_t* x_bf16, void* stream);

/* logits [M, N] fp32 = bf16(h) [M, K] * W^T with W [N, K] bf16 row-major,
 * fp32 accumulation (the bf16 output head).  h is fp32 and is rounded to
 * bf16 (nearest-even) on load.  M <= 128, N and K multiples of 128. */
int sgd_head_logits(const float* h, int M, int K, const uint16_t* w_bf16, int N,
                    float* logits, void* stream);

/* out[m] = argmax_n logits[m, n] (lowest index among equal maxima). */
int sgd_argmax_rows(const float* logits, int M, int N, int32_t* out, void* stream);

/* ---- measurement aid ---------------------------------------------------- */
/*
 * Read `bytes` bytes of device memory at `buf` once, as a plain streaming
 * read (16-byte loads, grid-stride, 8192 workgroups of 256 threads), and
 * write nothing but possibly the one word at `sink` (device, caller-owned).
 * Timing it gives the attainable HBM read rate of the device, the context
 * for the hot path's achieved rates (a weight stream is a read stream).
 * buf 16-byte aligned, bytes a multiple of 16, sink 4-byte aligned.
 * Errors: SGD_EINVAL (null pointer, bytes == 0), SGD_EALIGN.
 */
int sgd_read_stream(const void* buf, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SWIGLU_DECODE_H */

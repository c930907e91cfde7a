// C ABI entry points: host-side validation, then one launch on the caller's
// stream.  Nothing is launched when validation fails.
#include "sgd_host.hpp"

#include <stdint.h>

#include <atomic>

using namespace sgd;

namespace {

constexpr int ABI_VERSION = 2;
constexpr int MAX_DIM = 1 << 20;
// The streaming kernels address a weight's codes with 32-bit offsets and use
// offset 2^31 as their past-the-end filler, so a weight holds fewer than 2^31
// codes.
constexpr size_t MAX_WEIGHT_BYTES = size_t(1) << 31;
// The persistent kernels' wait budget (sgd_set_wait_budget_us).
constexpr uint32_t DEFAULT_WAIT_BUDGET_US = 1000000;
std::atomic<uint32_t> g_wait_budget_us{DEFAULT_WAIT_BUDGET_US};
// Whether fused calls keep a = silu(g)*u in the workspace (sgd_set_keep_intermediates).
std::atomic<int> g_keep_intermediates{0};

inline bool fmt_ok(int fmt) { return fmt == SGD_FMT_BLOCK128 || fmt == SGD_FMT_MX32; }
inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool al4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// N, K of a weight: positive multiples of 128 within range, fewer than 2^31
// elements in all.
int check_nk(int N, int K) {
  if (N <= 0 || K <= 0 || N > MAX_DIM || K > MAX_DIM) return SGD_EINVAL;
  if ((N % 128) || (K % 128)) return SGD_EDIM;
  if ((size_t)N * (size_t)K >= MAX_WEIGHT_BYTES) return SGD_EDIM;
  return SGD_OK;
}

int check_weight(const sgd_weight* w) {
  if (!w) return SGD_EINVAL;
  if (!fmt_ok(w->fmt)) return SGD_EFMT;
  if (w->reserved != 0) return SGD_EINVAL;
  int rc = check_nk(w->N, w->K);
  if (rc) return rc;
  if (!w->codes || !w->scales) return SGD_EINVAL;
  if (!al16(w->codes) || !al4(w->scales)) return SGD_EALIGN;
  return SGD_OK;
}

}  // namespace

namespace sgd {
uint64_t wait_budget_ticks() { return (uint64_t)g_wait_budget_us.load(std::memory_order_relaxed) * 100u; }
bool keep_intermediates() { return g_keep_intermediates.load(std::memory_order_relaxed) != 0; }

int check_mlp_args(const uint16_t* x_bf16, int M, const sgd_weight* gate, const sgd_weight* up,
                   const sgd_weight* down, const uint16_t* y_bf16) {
  int rc;
  if ((rc = check_weight(gate)) || (rc = check_weight(up)) || (rc = check_weight(down))) return rc;
  if (gate->fmt != up->fmt || gate->fmt != down->fmt) return SGD_EFMT;
  const int d = gate->K, F = gate->N;
  if (up->N != F || up->K != d || down->N != d || down->K != F) return SGD_EDIM;
  if (F > 32768) return SGD_EINVAL;
  if (!x_bf16 || !y_bf16 || M <= 0 || M > SGD_MAX_M) return SGD_EINVAL;
  if (!al16(x_bf16) || !al16(y_bf16)) return SGD_EALIGN;
  return SGD_OK;
}
}  // namespace sgd

extern "C" {

const char* sgd_status_str(int status) {
  switch (status) {
    case SGD_OK: return "ok";
    case SGD_EINVAL: return "invalid argument (null pointer, size or row count out of range)";
    case SGD_EALIGN: return "pointer not aligned as required";
    case SGD_EDIM: return "dimension not a multiple of its tile size, or shapes do not chain";
    case SGD_EWORKSPACE: return "workspace missing or too small";
    case SGD_EFMT: return "unknown format or mixed formats";
    case SGD_EHIP: return "HIP runtime error";
    case SGD_ETIMEOUT:
      return "a cross-workgroup wait of a persistent kernel gave up (workgroups not resident at once); "
             "outputs of that call are invalid and the workspace must be cleared";
    default: return "unknown status";
  }
}

int sgd_abi_version(void) { return ABI_VERSION; }

size_t sgd_packed_codes_bytes(int fmt, int N, int K) {
  if (!fmt_ok(fmt) || check_nk(N, K) != SGD_OK) return 0;
  return (size_t)N * (size_t)K;
}

size_t sgd_packed_scales_bytes(int fmt, int N, int K) {
  if (!fmt_ok(fmt) || check_nk(N, K) != SGD_OK) return 0;
  if (fmt == SGD_FMT_BLOCK128) return (size_t)(N / 128) * (size_t)(K / 128) * 4;
  const size_t kg = ((size_t)K / 128 + 3) / 4;
  return (size_t)(N / 16) * kg * 256;
}

int sgd_quantize_pack_weight(int fmt, const uint16_t* w_bf16, int N, int K, void* codes_out,
                             void* scales_out, void* stream) {
  if (!fmt_ok(fmt)) return SGD_EFMT;
  int rc = check_nk(N, K);
  if (rc) return rc;
  if (!w_bf16 || !codes_out || !scales_out) return SGD_EINVAL;
  if (!al16(w_bf16) || !al16(codes_out) || !al4(scales_out)) return SGD_EALIGN;
  return launch_pack_weight(fmt, w_bf16, N, K, codes_out, scales_out, as_stream(stream));
}

int sgd_unpack_weight(const sgd_weight* w, uint8_t* codes_rowmajor, void* scales_logical, void* stream) {
  int rc = check_weight(w);
  if (rc) return rc;
  if (!codes_rowmajor || !scales_logical) return SGD_EINVAL;
  if (!al16(codes_rowmajor) || !al4(scales_logical)) return SGD_EALIGN;
  return launch_unpack_weight(w->fmt, static_cast<const uint8_t*>(w->codes), w->scales, w->N, w->K,
                              codes_rowmajor, scales_logical, as_stream(stream));
}

int sgd_quantize_act(int fmt, const uint16_t* x_bf16, int M, int K, uint8_t* codes, void* scales,
                     void* stream) {
  if (!fmt_ok(fmt)) return SGD_EFMT;
  if (M <= 0 || M > 65536 || K <= 0 || K > MAX_DIM) return SGD_EINVAL;
  if (K % 128) return SGD_EDIM;
  if (!x_bf16 || !codes || !scales) return SGD_EINVAL;
  if (!al16(x_bf16) || !al16(codes) || !al4(scales)) return SGD_EALIGN;
  return launch_quantize_act(fmt, x_bf16, M, K, codes, scales, as_stream(stream));
}

size_t sgd_gemm_workspace_bytes(int fmt, int M, int N, int K) {
  if (!fmt_ok(fmt) || M <= 0 || M > SGD_MAX_M || check_nk(N, K) != SGD_OK) return 0;
  return stream_workspace_bytes(fmt, M, K, 0, N, K, false);
}

size_t sgd_mlp_workspace_bytes(int fmt, int M, int d, int ffn) {
  if (!fmt_ok(fmt) || M <= 0 || M > SGD_MAX_M || check_nk(ffn, d) != SGD_OK) return 0;
  if (ffn > 32768) return 0;
  return stream_workspace_bytes(fmt, M, d, ffn, d, ffn, true);
}

int sgd_mlp_workspace_layout(int fmt, int M, int d, int ffn, size_t* offsets) {
  if (!offsets || sgd_mlp_workspace_bytes(fmt, M, d, ffn) == 0) return SGD_EINVAL;
  size_t off[5];
  const int rc = stream_workspace_layout(fmt, M, d, ffn, off);
  if (rc != SGD_OK) return rc;
  for (int i = 0; i < 5; ++i) offsets[i] = off[i];
  return SGD_OK;
}

int sgd_workspace_clear(void* workspace, size_t bytes, void* stream) {
  if (!workspace || bytes == 0) return SGD_EINVAL;
  if (!al16(workspace) || (bytes % 16)) return SGD_EALIGN;
  return launch_fill_zero(workspace, bytes, as_stream(stream));
}

int sgd_set_keep_intermediates(int keep) { return g_keep_intermediates.exchange(keep ? 1 : 0, std::memory_order_relaxed); }

uint32_t sgd_set_wait_budget_us(uint32_t us) {
  return g_wait_budget_us.exchange(us == 0 ? DEFAULT_WAIT_BUDGET_US : us, std::memory_order_relaxed);
}

int sgd_workspace_status(const void* workspace, void* stream) {
  if (!workspace) return SGD_EINVAL;
  if (!al16(workspace)) return SGD_EALIGN;
  if (hipStreamSynchronize(as_stream(stream)) != hipSuccess) return SGD_EHIP;
  uint32_t gave_up = 0;
  if (hipMemcpy(&gave_up, static_cast<const uint32_t*>(workspace) + CTRL_ERR_WORD, sizeof(gave_up),
                hipMemcpyDeviceToHost) != hipSuccess)
    return SGD_EHIP;
  return gave_up ? SGD_ETIMEOUT : SGD_OK;
}

int sgd_read_stream(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes == 0) return SGD_EINVAL;
  if (!al16(buf) || (bytes % 16) || (reinterpret_cast<uintptr_t>(sink) & 3)) return SGD_EALIGN;
  return launch_read_stream(buf, bytes, sink, as_stream(stream));
}

int sgd_scaled_gemm(const uint16_t* x_bf16, int M, const sgd_weight* w, uint16_t* y_bf16,
                    void* workspace, size_t ws_bytes, void* stream) {
  int rc = check_weight(w);
  if (rc) return rc;
  if (!x_bf16 || !y_bf16 || M <= 0 || M > SGD_MAX_M) return SGD_EINVAL;
  if (!al16(x_bf16) || !al16(y_bf16)) return SGD_EALIGN;
  if (!workspace) return SGD_EWORKSPACE;
  if (!al16(workspace)) return SGD_EALIGN;
  const size_t need = stream_workspace_bytes(w->fmt, M, w->K, 0, w->N, w->K, false);
  if (need == 0) return SGD_EDIM;
  if (ws_bytes < need) return SGD_EWORKSPACE;
  Problem p{};
  p.fmt = w->fmt;
  p.M = M;
  p.x = x_bf16;
  p.K1 = w->K;
  p.w2 = w;
  p.y = y_bf16;
  p.ws = workspace;
  return launch_stream(p, as_stream(stream));
}

int sgd_scaled_gemm_f32(const uint16_t* x_bf16, int M, const sgd_weight* w, float* y_f32, void* workspace,
                        size_t ws_bytes, void* stream) {
  int rc = check_weight(w);
  if (rc) return rc;
  if (!x_bf16 || !y_f32 || M <= 0 || M > SGD_MAX_M) return SGD_EINVAL;
  if (!al16(x_bf16) || !al16(y_f32)) return SGD_EALIGN;
  if (!workspace) return SGD_EWORKSPACE;
  if (!al16(workspace)) return SGD_EALIGN;
  const size_t need = stream_workspace_bytes(w->fmt, M, w->K, 0, w->N, w->K, false);
  if (need == 0) return SGD_EDIM;
  if (ws_bytes < need) return SGD_EWORKSPACE;
  Problem p{};
  p.fmt = w->fmt;
  p.M = M;
  p.x = x_bf16;
  p.K1 = w->K;
  p.w2 = w;
  p.y32 = y_f32;
  p.ws = workspace;
  return launch_stream(p, as_stream(stream));
}

size_t sgd_act_scales_bytes(int fmt, int M, int K) {
  if (!fmt_ok(fmt) || M <= 0 || M > SGD_MAX_M || K <= 0 || K > MAX_DIM || (K % 128)) return 0;
  return fmt == SGD_FMT_BLOCK128 ? (size_t)(K / 128) * (size_t)act_mtile_pad(M) * 4 : (size_t)M * (size_t)(K / 32);
}

int sgd_swiglu_quantize(int fmt, const float* gu, int M, int ffn, uint8_t* aq, void* as, void* stream) {
  if (!fmt_ok(fmt)) return SGD_EFMT;
  if (!gu || !aq || !as || M <= 0 || M > SGD_MAX_M || ffn <= 0 || ffn > MAX_DIM) return SGD_EINVAL;
  if (ffn % 128) return SGD_EDIM;
  if (!al16(gu) || !al16(aq) || !al4(as)) return SGD_EALIGN;
  return launch_swiglu_quantize(fmt, gu, M, ffn, aq, as, as_stream(stream));
}

int sgd_scaled_gemm_q(const uint8_t* xq, const void* xs, int M, const sgd_weight* w, uint16_t* y_bf16,
                      void* workspace, size_t ws_bytes, void* stream) {
  int rc = check_weight(w);
  if (rc) return rc;
  if (!xq || !xs || !y_bf16 || M <= 0 || M > SGD_MAX_M) return SGD_EINVAL;
  if (!al16(xq) || !al4(xs) || !al16(y_bf16)) return SGD_EALIGN;
  if (!workspace) return SGD_EWORKSPACE;
  if (!al16(workspace)) return SGD_EALIGN;
  const size_t need = stream_workspace_bytes(w->fmt, M, w->K, 0, w->N, w->K, false);
  if (need == 0) return SGD_EDIM;
  if (ws_bytes < need) return SGD_EWORKSPACE;
  Problem p{};
  p.fmt = w->fmt;
  p.M = M;
  p.x = nullptr;
  p.K1 = w->K;
  p.w2 = w;
  p.y = y_bf16;
  p.ws = workspace;
  p.xq_in = xq;
  p.xs_in = xs;
  return launch_stream(p, as_stream(stream));
}

int sgd_fused_swiglu_mlp(const uint16_t* x_bf16, int M, const sgd_weight* gate, const sgd_weight* up,
                         const sgd_weight* down, uint16_t* y_bf16, void* workspace, size_t ws_bytes,
                         void* stream) {
  int rc = sgd::check_mlp_args(x_bf16, M, gate, up, down, y_bf16);
  if (rc) return rc;
  const int d = gate->K, F = gate->N;
  if (!workspace) return SGD_EWORKSPACE;
  if (!al16(workspace)) return SGD_EALIGN;
  const size_t need = stream_workspace_bytes(gate->fmt, M, d, F, d, F, true);
  if (need == 0) return SGD_EDIM;
  if (ws_bytes < need) return SGD_EWORKSPACE;
  Problem p{};
  p.fmt = gate->fmt;
  p.M = M;
  p.x = x_bf16;
  p.K1 = d;
  p.gate = gate;
  p.up = up;
  p.w2 = down;
  p.y = y_bf16;
  p.ws = workspace;
  return launch_stream(p, as_stream(stream));
}

int sgd_fused_swiglu_block(const float* h_in, int M, const sgd_weight* gate, const sgd_weight* up,
                           const sgd_weight* down, float eps, float* h_out, void* workspace, size_t ws_bytes,
                           void* stream) {
  // (the MLP's checks, with h_in and h_out standing in for x and y)
  int rc = sgd::check_mlp_args(reinterpret_cast<const uint16_t*>(h_in), M, gate, up, down,
                               reinterpret_cast<const uint16_t*>(h_out));
  if (rc) return rc;
  if (!(eps >= 0.0f) || eps > 1.0f) return SGD_EINVAL;
  const int d = gate->K, F = gate->N;
  const size_t bytes = (size_t)M * (size_t)d * sizeof(float);
  const uintptr_t i0 = reinterpret_cast<uintptr_t>(h_in), o0 = reinterpret_cast<uintptr_t>(h_out);
  if (i0 < o0 + bytes && o0 < i0 + bytes) return SGD_EINVAL;  // the output must not overlap the input
  if (!workspace) return SGD_EWORKSPACE;
  if (!al16(workspace)) return SGD_EALIGN;
  const size_t need = stream_workspace_bytes(gate->fmt, M, d, F, d, F, true);
  if (need == 0) return SGD_EDIM;
  if (ws_bytes < need) return SGD_EWORKSPACE;
  Problem p{};
  p.fmt = gate->fmt;
  p.M = M;
  p.x = nullptr;
  p.K1 = d;
  p.gate = gate;
  p.up = up;
  p.w2 = down;
  p.y = nullptr;
  p.ws = workspace;
  p.h_in = h_in;
  p.h_out = h_out;
  p.eps = eps;
  return launch_stream(p, as_stream(stream));
}

// ---- large-M (prefill) path ----
namespace {
inline size_t a256(size_t v) { return (v + 255) & ~size_t(255); }
// Rows past which the 32-bit offsets of the tiled kernels would overflow.
bool large_shape_ok(int M, int K) {
  const size_t Mpad = (size_t)((M + 15) / 16) * 16;
  return Mpad * (size_t)K < ((size_t)1 << 31);
}
}  // namespace

size_t sgd_gemm_large_workspace_bytes(int fmt, int M, int N, int K) {
  if (!fmt_ok(fmt) || M <= 0 || M > SGD_MAX_M_LARGE || N <= 0 || K <= 0 || N > MAX_DIM || K > MAX_DIM) return 0;
  if ((N % 128) || (K % 128) || !large_shape_ok(M, K)) return 0;
  return CONTROL_BLOCK_BYTES + a256(act_tiles_codes_bytes(M, K)) + a256(act_tiles_scales_bytes(fmt, M, K));
}

int sgd_scaled_gemm_large(const uint16_t* x_bf16, int M, const sgd_weight* w, uint16_t* y_bf16, void* workspace,
                          size_t ws_bytes, void* stream) {
  int rc = check_weight(w);
  if (rc) return rc;
  if (!x_bf16 || !y_bf16 || M <= 0 || M > SGD_MAX_M_LARGE) return SGD_EINVAL;
  if (!al16(x_bf16) || !al16(y_bf16)) return SGD_EALIGN;
  if (!workspace) return SGD_EWORKSPACE;
  if (!al16(workspace)) return SGD_EALIGN;
  const size_t need = sgd_gemm_large_workspace_bytes(w->fmt, M, w->N, w->K);
  if (need == 0) return SGD_EDIM;
  if (ws_bytes < need) return SGD_EWORKSPACE;
  // (the first CONTROL_BLOCK_BYTES are left alone: a workspace may be shared
  // with the persistent entry points, whose control block lives there)
  uint8_t* ws = static_cast<uint8_t*>(workspace) + CONTROL_BLOCK_BYTES;
  uint8_t* codes = ws;
  void* scales = ws + a256(act_tiles_codes_bytes(M, w->K));
  hipStream_t s = as_stream(stream);
  rc = launch_act_tiles(w->fmt, x_bf16, M, w->K, codes, scales, s);
  if (rc) return rc;
  return launch_tile_gemm(w->fmt, codes, scales, M, w->K, w, y_bf16, false, s);
}

size_t sgd_mlp_prefill_workspace_bytes(int fmt, int M, int d, int ffn) {
  if (!fmt_ok(fmt) || M <= 0 || M > SGD_MAX_M_LARGE || d <= 0 || ffn <= 0 || d > MAX_DIM || ffn > 32768) return 0;
  if ((d % 128) || (ffn % 128) || !large_shape_ok(M, d) || !large_shape_ok(M, 2 * ffn)) return 0;
  const size_t Mpad = (size_t)((M + 15) / 16) * 16;
  return CONTROL_BLOCK_BYTES + a256(act_tiles_codes_bytes(M, d)) + a256(act_tiles_scales_bytes(fmt, M, d)) +
         a256(Mpad * 2 * ffn * 4) + a256(act_tiles_codes_bytes(M, ffn)) + a256(act_tiles_scales_bytes(fmt, M, ffn));
}

int sgd_swiglu_mlp_prefill(const uint16_t* x_bf16, int M, const sgd_weight* gate_up, const sgd_weight* down,
                           uint16_t* y_bf16, void* workspace, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_weight(gate_up)) || (rc = check_weight(down))) return rc;
  if (gate_up->fmt != down->fmt) return SGD_EFMT;
  const int fmt = down->fmt, d = down->N, F = down->K;
  if (gate_up->N != 2 * F || gate_up->K != d) return SGD_EDIM;
  if (!x_bf16 || !y_bf16 || M <= 0 || M > SGD_MAX_M_LARGE) return SGD_EINVAL;
  if (!al16(x_bf16) || !al16(y_bf16)) return SGD_EALIGN;
  if (!workspace) return SGD_EWORKSPACE;
  if (!al16(workspace)) return SGD_EALIGN;
  const size_t need = sgd_mlp_prefill_workspace_bytes(fmt, M, d, F);
  if (need == 0) return SGD_EDIM;
  if (ws_bytes < need) return SGD_EWORKSPACE;
  const int Mpad = (M + 15) / 16 * 16;
  uint8_t* p = static_cast<uint8_t*>(workspace) + CONTROL_BLOCK_BYTES;  // (control block untouched)
  uint8_t* xq = p;
  p += a256(act_tiles_codes_bytes(M, d));
  void* xs = p;
  p += a256(act_tiles_scales_bytes(fmt, M, d));
  float* gu = reinterpret_cast<float*>(p);
  p += a256((size_t)Mpad * 2 * F * 4);
  uint8_t* aq = p;
  p += a256(act_tiles_codes_bytes(M, F));
  void* as = p;
  hipStream_t s = as_stream(stream);
  // Q(x); [g | u] = Q(x) [Wg; Wu]^T in fp32 for all Mpad rows (padded rows
  // are zero); Q(silu(g) * u); y = Q(a) Wd^T for the M rows
  if ((rc = launch_act_tiles(fmt, x_bf16, M, d, xq, xs, s))) return rc;
  if ((rc = launch_tile_gemm(fmt, xq, xs, Mpad, d, gate_up, gu, true, s))) return rc;
  if ((rc = launch_swiglu_quantize_tiles(fmt, gu, Mpad, F, aq, as, s))) return rc;
  // (the second GEMM may split K, its partial sums in the gate/up buffer,
  // which is no longer read)
  return launch_tile_gemm(fmt, aq, as, M, F, down, y_bf16, false, s, gu, (size_t)Mpad * 2 * F * 4);
}

// ---- paged decode attention ----
namespace {
constexpr int ATTN_HD = 128, ATTN_PAGE_BYTES = 2112;
bool attn_dims_ok(int B, int Hq, int Hkv, int n_pages, int max_pages) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || n_pages <= 0 || max_pages <= 0) return false;
  if (B > 65536 || Hq > 1024 || max_pages > (1 << 20)) return false;
  if (Hq % Hkv || Hq / Hkv > 16) return false;
  return (size_t)n_pages * (size_t)Hkv * ATTN_PAGE_BYTES < ((size_t)1 << 31);
}
}  // namespace

size_t sgd_kv_cache_bytes(int n_pages, int Hkv) {
  if (n_pages <= 0 || Hkv <= 0 || (size_t)n_pages * (size_t)Hkv * ATTN_PAGE_BYTES >= ((size_t)1 << 31)) return 0;
  return (size_t)n_pages * (size_t)Hkv * ATTN_PAGE_BYTES;
}

int sgd_kv_cache_write(int kind, const uint16_t* x_bf16, const int32_t* slots, int n, int Hkv, int head_dim,
                       uint8_t* cache, int n_pages, void* stream) {
  if (kind != 0 && kind != 1) return SGD_EINVAL;
  if (!x_bf16 || !slots || !cache || n <= 0 || n > (1 << 24) || Hkv <= 0 || Hkv > 1024) return SGD_EINVAL;
  if (head_dim != ATTN_HD) return SGD_EDIM;
  if (sgd_kv_cache_bytes(n_pages, Hkv) == 0) return SGD_EINVAL;
  if (!al16(x_bf16) || !al16(cache) || !al4(slots)) return SGD_EALIGN;
  return launch_kv_write(kind, x_bf16, slots, n, Hkv, cache, n_pages, as_stream(stream));
}

size_t sgd_paged_attention_workspace_bytes(int B, int Hq, int Hkv, int max_pages) {
  if (!attn_dims_ok(B, Hq, Hkv, 1, max_pages)) return 0;
  return attn_workspace_bytes(B, Hq, Hkv, max_pages);
}

int sgd_paged_decode_attention(const uint16_t* q_bf16, const uint8_t* k_cache, const uint8_t* v_cache, int n_pages,
                               const int32_t* block_table, int max_pages, const int32_t* seq_lens, int B, int Hq,
                               int Hkv, int head_dim, float sm_scale, uint16_t* out_bf16, void* workspace,
                               size_t ws_bytes, void* stream) {
  if (!q_bf16 || !k_cache || !v_cache || !block_table || !seq_lens || !out_bf16) return SGD_EINVAL;
  if (head_dim != ATTN_HD) return SGD_EDIM;
  if (!attn_dims_ok(B, Hq, Hkv, n_pages, max_pages)) return SGD_EINVAL;
  if (!(sm_scale > 0.0f) || sm_scale > 1e6f) return SGD_EINVAL;
  if (!al16(q_bf16) || !al16(k_cache) || !al16(v_cache) || !al16(out_bf16) || !al4(block_table) || !al4(seq_lens))
    return SGD_EALIGN;
  if (!workspace) return SGD_EWORKSPACE;
  if (!al16(workspace)) return SGD_EALIGN;
  if (ws_bytes < attn_workspace_bytes(B, Hq, Hkv, max_pages)) return SGD_EWORKSPACE;
  return launch_paged_decode(q_bf16, k_cache, v_cache, n_pages, block_table, max_pages, seq_lens, B, Hq, Hkv, sm_scale,
                             out_bf16, workspace, as_stream(stream));
}

int sgd_bf16_to_f32(const uint16_t* x_bf16, int M, int d, float* h, void* stream) {
  if (!x_bf16 || !h || M <= 0 || d <= 0 || M > 65536 || d > MAX_DIM) return SGD_EINVAL;
  if (d % 128) return SGD_EDIM;
  if (!al16(x_bf16) || !al16(h)) return SGD_EALIGN;
  return launch_bf16_to_f32(x_bf16, M, d, h, as_stream(stream));
}

int sgd_rmsnorm_bf16(const float* h, int M, int d, float eps, uint16_t* x_bf16, void* stream) {
  if (!x_bf16 || !h || M <= 0 || d <= 0 || M > 65536 || d > MAX_DIM || !(eps >= 0.0f)) return SGD_EINVAL;
  if (d % 128) return SGD_EDIM;
  if (!al16(x_bf16) || !al16(h)) return SGD_EALIGN;
  return launch_rmsnorm(h, M, d, eps, x_bf16, as_stream(stream));
}

int sgd_residual_add(float* h, const uint16_t* y_bf16, int M, int d, void* stream) {
  if (!y_bf16 || !h || M <= 0 || d <= 0 || M > 65536 || d > MAX_DIM) return SGD_EINVAL;
  if (d % 128) return SGD_EDIM;
  if (!al16(y_bf16) || !al16(h)) return SGD_EALIGN;
  return launch_residual_add(h, y_bf16, M, d, as_stream(stream));
}

int sgd_residual_rmsnorm_bf16(float* h, const uint16_t* y_bf16, int M, int d, float eps, uint16_t* x_bf16,
                              void* stream) {
  if (!h || !y_bf16 || !x_bf16 || M <= 0 || d <= 0 || M > 65536 || d > MAX_DIM || !(eps >= 0.0f))
    return SGD_EINVAL;
  if (d % 128) return SGD_EDIM;
  if (!al16(h) || !al16(y_bf16) || !al16(x_bf16)) return SGD_EALIGN;
  return launch_residual_rmsnorm(h, y_bf16, M, d, eps, x_bf16, as_stream(stream));
}

int sgd_head_logits(const float* h, int M, int K, const uint16_t* w_bf16, int N, float* logits,
                    void* stream) {
  if (!h || !w_bf16 || !logits || M <= 0 || M > SGD_MAX_M) return SGD_EINVAL;
  int rc = check_nk(N, K);
  if (rc) return rc;
  if (!al16(h) || !al16(w_bf16) || !al16(logits)) return SGD_EALIGN;
  return launch_head(h, M, K, w_bf16, N, logits, as_stream(stream));
}

int sgd_argmax_rows(const float* logits, int M, int N, int32_t* out, void* stream) {
  if (!logits || !out || M <= 0 || N <= 0 || M > 65536 || N > (1 << 24)) return SGD_EINVAL;
  if (!al4(logits) || !al4(out)) return SGD_EALIGN;
  return launch_argmax(logits, M, N, out, as_stream(stream));
}

}  // extern "C"

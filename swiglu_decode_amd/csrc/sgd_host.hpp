// Host-side declarations shared by the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "swiglu_decode.h"

namespace sgd {

// Kernel launchers (arguments already validated).  Return SGD_OK/SGD_EHIP.
int launch_pack_weight(int fmt, const uint16_t* w, int N, int K, void* codes, void* scales,
                       hipStream_t s);
int launch_unpack_weight(int fmt, const uint8_t* codes, const void* scales, int N, int K,
                         uint8_t* out_codes, void* out_scales, hipStream_t s);
int launch_quantize_act(int fmt, const uint16_t* x, int M, int K, uint8_t* codes, void* scales,
                        hipStream_t s);
int launch_fill_zero(void* p, size_t bytes, hipStream_t s);
int launch_read_stream(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s);

// Streaming GEMM / fused MLP.  `gate`/`up` are null for the plain GEMM.
struct Problem {
  int fmt;
  int M;
  const uint16_t* x;   // [M, K1]
  int K1;              // d (MLP) or K (GEMM)
  const sgd_weight* gate;
  const sgd_weight* up;
  const sgd_weight* w2;  // down [d, F] (MLP) or W [N, K] (GEMM)
  uint16_t* y;         // [M, w2->N] bf16
  void* ws;
  float* y32 = nullptr;               // fp32 output instead of y
  const uint8_t* xq_in = nullptr;     // x already quantized (workspace layout), x unused
  const void* xs_in = nullptr;
  // decode block: x = bf16(RMSNorm(h_in)) formed in the kernel (x unused),
  // output h_out = fl32(h_in + bf16(y)) (y unused)
  const float* h_in = nullptr;
  float* h_out = nullptr;
  float eps = 0.0f;
};
size_t stream_workspace_bytes(int fmt, int M, int K1, int F, int N, int K2, bool mlp);
// Byte offsets of the fused MLP's workspace regions: Q(x) codes, Q(x)
// scales, a (fp32), Q(a) codes, Q(a) scales.
int stream_workspace_layout(int fmt, int M, int K1, int F, size_t (&off)[5]);
// Rows of the activation scale layout (block format): M rounded up to 16,
// 32, 64 or 128.
int act_mtile_pad(int M);
// a = silu(g) * u from gu [M, 2F] fp32, quantized into the workspace layout.
int launch_swiglu_quantize(int fmt, const float* gu, int M, int F, uint8_t* aq, void* as, hipStream_t s);
int launch_swiglu_quantize_tiles(int fmt, const float* gu, int Mrows, int F, uint8_t* aq, void* as, hipStream_t s);
// Large-M path: Q(x) of bf16 x [M, K] in the full-tile activation layout
// (Mpad = 16*ceil(M/16) rows), and C = Q(A) W^T from that layout.
size_t act_tiles_codes_bytes(int M, int K);
size_t act_tiles_scales_bytes(int fmt, int M, int K);
int launch_act_tiles(int fmt, const uint16_t* x, int M, int K, uint8_t* codes, void* scales, hipStream_t s);
int launch_tile_gemm(int fmt, const uint8_t* a, const void* as, int M, int K, const sgd_weight* w, void* c,
                     bool out_f32, hipStream_t s, float* part = nullptr, size_t part_bytes = 0);
// Paged decode attention over an MXFP8 K/V cache (head_dim 128, 16-slot pages).
size_t attn_workspace_bytes(int B, int Hq, int Hkv, int max_pages);
int launch_kv_write(int kind, const uint16_t* x, const int32_t* slots, int n, int Hkv, uint8_t* cache, int n_pages,
                    hipStream_t s);
int launch_paged_decode(const uint16_t* q, const uint8_t* kc, const uint8_t* vc, int n_pages, const int32_t* bt,
                        int max_pages, const int32_t* lens, int B, int Hq, int Hkv, float sm_scale, uint16_t* out,
                        void* ws, hipStream_t s);
int launch_stream(const Problem& p, hipStream_t s);

// Host-side validation of a fused-MLP call's arguments other than its
// workspace: SGD_OK or the status the C ABI returns.
int check_mlp_args(const uint16_t* x_bf16, int M, const sgd_weight* gate, const sgd_weight* up,
                   const sgd_weight* down, const uint16_t* y_bf16);

// Decode-stack glue.
int launch_bf16_to_f32(const uint16_t* x, int M, int d, float* h, hipStream_t s);
int launch_rmsnorm(const float* h, int M, int d, float eps, uint16_t* x, hipStream_t s);
int launch_residual_add(float* h, const uint16_t* y, int M, int d, hipStream_t s);
int launch_residual_rmsnorm(float* h, const uint16_t* y, int M, int d, float eps, uint16_t* x, hipStream_t s);
int launch_head(const float* h, int M, int K, const uint16_t* w, int N, float* out, hipStream_t s);
int launch_argmax(const float* logits, int M, int N, int32_t* out, hipStream_t s);

// The workspace's leading control block (zeroed once; left ready by every
// completed call).
constexpr size_t CONTROL_BLOCK_BYTES = size_t(256) << 10;

// Word of the workspace control block that counts waits that gave up
// (sticky until the workspace is cleared).
constexpr int CTRL_ERR_WORD = 65;

// Longest a cross-workgroup wait of the persistent kernels may spin before
// the launch gives up (sgd_set_wait_budget_us), in ticks of the device's
// 100 MHz real-time counter.
uint64_t wait_budget_ticks();
// Whether fused calls also store a = silu(g)*u where their path does not
// need it (sgd_set_keep_intermediates).
bool keep_intermediates();

inline int hip_status(hipError_t e) { return e == hipSuccess ? SGD_OK : SGD_EHIP; }

}  // namespace sgd

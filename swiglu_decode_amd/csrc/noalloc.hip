// The fused SwiGLU MLP for callers that cannot allocate device memory (code
// under graph capture that must not call hipMalloc, tight serving loops,
// harnesses that forbid allocation): the same kernel as
// sgd_fused_swiglu_mlp, with its workspace in a fixed device array of this
// library instead of a buffer the caller brings.
#include "sgd_host.hpp"

#include <mutex>

using namespace sgd;

namespace {

constexpr size_t SCRATCH_BYTES = SGD_NOALLOC_SCRATCH_BYTES;
constexpr int MAX_DEVICES = 64;

// One copy per GPU the library runs on, held until the process ends.  In host
// code this name is only a stand-in for the symbol: its device address comes
// from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[SCRATCH_BYTES];

struct ScratchTable {
  std::mutex mu;
  void* ptr[MAX_DEVICES] = {};
};
ScratchTable g_scratch;

// The current device's copy of `scratch`, looked up with hipGetSymbolAddress
// on the first call on that device (with it current).  That first call also
// zero-fills the control block at the start of the array with a fill kernel
// on the caller's stream (no memset node): the kernels need it zeroed once,
// and every call that completes leaves it ready for the next.
int scratch_for_current_device(hipStream_t stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return SGD_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch.mu);
  if (!g_scratch.ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SGD_EHIP;
    const int rc = launch_fill_zero(p, CONTROL_BLOCK_BYTES, stream);
    if (rc != SGD_OK) return rc;
    g_scratch.ptr[dev] = p;
  }
  *out = g_scratch.ptr[dev];
  return SGD_OK;
}

}  // namespace

extern "C" {

int sgd_fused_swiglu_mlp_noalloc(const uint16_t* x_bf16, int M, const sgd_weight* gate, const sgd_weight* up,
                                 const sgd_weight* down, uint16_t* y_bf16, void* stream) {
  // the same checks as the workspace entry point, first: nothing is looked
  // up or launched for an invalid call
  int rc = check_mlp_args(x_bf16, M, gate, up, down, y_bf16);
  if (rc) return rc;
  const size_t need = sgd_mlp_workspace_bytes(gate->fmt, M, gate->K, gate->N);
  if (need == 0) return SGD_EDIM;
  if (need > SCRATCH_BYTES) return SGD_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  rc = scratch_for_current_device(s, &ws);
  if (rc != SGD_OK) return rc;
  return sgd_fused_swiglu_mlp(x_bf16, M, gate, up, down, y_bf16, ws, SCRATCH_BYTES, stream);
}

}  // extern "C"

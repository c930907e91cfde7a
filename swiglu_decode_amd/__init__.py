"""MI355X (gfx950) decode-shape FP8 SwiGLU MLP: Python binding.

Thin wrappers over the C ABI in include/swiglu_decode.h.  PyTorch only
supplies device memory and the current stream; every step of the path runs
in the library's HIP kernels.  Arguments are checked (dtype, exact shape,
contiguity, device) and never coerced: a wrong tensor raises instead of being
converted.
"""

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import FMT_BLOCK128, FMT_MX32, MAX_M, SgdError, SgdWeight

__all__ = [
    "FMT_BLOCK128", "FMT_MX32", "MAX_M", "SgdError", "PackedWeight", "Workspace",
    "fmt_code", "quantize_pack_weight", "unpack_weight", "quantize_act", "scaled_gemm",
    "fused_swiglu_mlp", "bf16_to_f32", "rmsnorm_bf16", "residual_add", "head_logits",
    "argmax_rows", "gemm_workspace_bytes", "mlp_workspace_bytes", "lib",
    "workspace_status", "set_wait_budget_us", "set_keep_intermediates", "mlp_workspace_layout", "fused_swiglu_mlp_noalloc",
    "scaled_gemm_f32", "swiglu_quantize", "scaled_gemm_q", "stack_packed", "unfused_swiglu_mlp",
]

_FMTS = {"block": FMT_BLOCK128, "mx": FMT_MX32, FMT_BLOCK128: FMT_BLOCK128, FMT_MX32: FMT_MX32}


def lib():
    return _lib.load()


def fmt_code(fmt):
    if fmt not in _FMTS:
        raise ValueError(f"unknown format {fmt!r} (use 'block' or 'mx')")
    return _FMTS[fmt]


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


@dataclass
class PackedWeight:
    """A weight [N, K] quantized and packed by quantize_pack_weight."""
    fmt: int
    N: int
    K: int
    codes: torch.Tensor   # uint8 [packed_codes_bytes]
    scales: torch.Tensor  # uint8 [packed_scales_bytes] (fp32 for block format)

    def c_struct(self):
        return SgdWeight(self.fmt, self.N, self.K, 0, self.codes.data_ptr(), self.scales.data_ptr())

    @property
    def device(self):
        return self.codes.device


def quantize_pack_weight(w, fmt):
    """bf16 weight [N, K] on the GPU -> PackedWeight (one launch)."""
    f = fmt_code(fmt)
    if w.dim() != 2:
        raise ValueError("weight must be 2-D [N, K]")
    _need(w, "w", torch.bfloat16)
    N, K = w.shape
    L = lib()
    nc = L.sgd_packed_codes_bytes(f, N, K)
    ns = L.sgd_packed_scales_bytes(f, N, K)
    if nc == 0 or ns == 0:
        raise ValueError(f"invalid weight shape {N}x{K} for the packed layout (multiples of 128)")
    codes = torch.empty(nc, dtype=torch.uint8, device=w.device)
    scales = torch.empty(ns, dtype=torch.uint8, device=w.device)
    _lib.check("sgd_quantize_pack_weight",
               L.sgd_quantize_pack_weight(f, _ptr(w), N, K, _ptr(codes), _ptr(scales), _stream(w)))
    return PackedWeight(f, N, K, codes, scales)


def unpack_weight(pw):
    """PackedWeight -> (codes uint8 [N, K], scales logical: fp32 [N/128, K/128] or uint8 [N, K/32])."""
    codes = torch.empty((pw.N, pw.K), dtype=torch.uint8, device=pw.device)
    if pw.fmt == FMT_BLOCK128:
        scales = torch.empty((pw.N // 128, pw.K // 128), dtype=torch.float32, device=pw.device)
    else:
        scales = torch.empty((pw.N, pw.K // 32), dtype=torch.uint8, device=pw.device)
    st = pw.c_struct()
    _lib.check("sgd_unpack_weight",
               lib().sgd_unpack_weight(ctypes.byref(st), _ptr(codes), _ptr(scales), _stream(codes)))
    return codes, scales


def quantize_act(x, fmt):
    """bf16 x [M, K] -> (codes uint8 [M, K], scales fp32 [M, K/128] | uint8 [M, K/32])."""
    f = fmt_code(fmt)
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    _need(x, "x", torch.bfloat16)
    M, K = x.shape
    codes = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if f == FMT_BLOCK128:
        scales = torch.empty((M, K // 128), dtype=torch.float32, device=x.device)
    else:
        scales = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device)
    _lib.check("sgd_quantize_act",
               lib().sgd_quantize_act(f, _ptr(x), M, K, _ptr(codes), _ptr(scales), _stream(x)))
    return codes, scales


def gemm_workspace_bytes(fmt, M, N, K):
    return lib().sgd_gemm_workspace_bytes(fmt_code(fmt), M, N, K)


def mlp_workspace_bytes(fmt, M, d, ffn):
    return lib().sgd_mlp_workspace_bytes(fmt_code(fmt), M, d, ffn)


class Workspace:
    """A zero-initialised device workspace that grows on demand.  The kernels
    leave its control block ready for the next call (counters zero, flags
    holding the number of the launch that raised them).  Calls that share a
    workspace must not overlap; the binding orders them (see
    _serialise_persistent), whatever stream each is issued on."""

    def __init__(self, device, nbytes=0):
        self.device = torch.device(device)
        self.tensor = None
        if nbytes:
            self.ensure(nbytes)

    def ensure(self, nbytes):
        nbytes = (int(nbytes) + 255) // 256 * 256
        if self.tensor is None or self.tensor.numel() < nbytes:
            self.tensor = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            _lib.check("sgd_workspace_clear",
                       lib().sgd_workspace_clear(_ptr(self.tensor), nbytes, _stream(self.tensor)))
        return self.tensor


    def clear(self):
        """Zero the whole workspace again (after SGD_ETIMEOUT or a fault)."""
        if self.tensor is not None:
            _lib.check("sgd_workspace_clear", lib().sgd_workspace_clear(
                _ptr(self.tensor), self.tensor.numel(), _stream(self.tensor)))

    def status(self):
        """SGD_OK (0) or SGD_ETIMEOUT (-7): whether a launch on this workspace
        gave up a wait since it was last cleared.  Synchronises the stream."""
        if self.tensor is None:
            return 0
        st = lib().sgd_workspace_status(_ptr(self.tensor), _stream(self.tensor))
        if st not in (0, _lib.SGD_ETIMEOUT):
            _lib.check("sgd_workspace_status", st)
        return st


# One default workspace per device (not per stream): persistent launches on
# one device must not overlap, whichever stream they are issued on.
_DEFAULT_WS = {}
# Per device: (stream handle, event) of the last persistent launch issued
# through this binding.
_LAST_LAUNCH = {}


def _workspace(device, nbytes, ws):
    if ws is None:
        ws = _DEFAULT_WS.get(device.index)
        if ws is None:
            ws = _DEFAULT_WS[device.index] = Workspace(device)
    t = ws.ensure(nbytes)
    return t


def _serialise_persistent(device, launch):
    """Run `launch()` (one persistent-kernel call, with the sizing of its
    workspace) so that it cannot overlap the previous persistent call on the
    same device: when that one was issued on another stream, the current
    stream first waits for it.  All workgroups of a persistent kernel must be
    resident at once, so two of them running side by side could each hold
    compute units the other waits for; and a workspace that grows must not be
    freed under a call still running on another stream.  (Inside a graph
    capture the captured stream's own order applies.)"""
    stream = torch.cuda.current_stream(device)
    capturing = torch.cuda.is_current_stream_capturing()
    last = _LAST_LAUNCH.get(device.index)
    if last is not None and not capturing and last[0] != stream.cuda_stream:
        stream.wait_event(last[1])
    out = launch()
    if not capturing:
        ev = torch.cuda.Event()
        ev.record(stream)
        _LAST_LAUNCH[device.index] = (stream.cuda_stream, ev)
    return out


def workspace_status(ws):
    """Status of a Workspace (see Workspace.status)."""
    return ws.status()


def set_wait_budget_us(us):
    """Set the persistent kernels' wait budget in microseconds (0: default
    1 s); returns the previous value.  Process-wide."""
    return int(lib().sgd_set_wait_budget_us(int(us)))


def set_keep_intermediates(keep):
    """Also store a = silu(g)*u in the workspace on the path that does not
    need it (M > 32), for inspection; returns the previous setting.
    Process-wide."""
    return int(lib().sgd_set_keep_intermediates(1 if keep else 0))


def mlp_workspace_layout(fmt, M, d, ffn):
    """Byte offsets of the fused MLP's intermediates in its workspace:
    dict(xq, xs, a, aq, as_) (layouts in swiglu_decode.h, for inspection)."""
    off = (ctypes.c_size_t * 5)()
    _lib.check("sgd_mlp_workspace_layout",
               lib().sgd_mlp_workspace_layout(fmt_code(fmt), M, d, ffn, off))
    return dict(zip(("xq", "xs", "a", "aq", "as_"), (int(v) for v in off)))


def scaled_gemm(x, w, out=None, workspace=None):
    """y [M, N] bf16 = Q(x) W^T for bf16 x [M, K] and a PackedWeight [N, K]."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    _need(x, "x", torch.bfloat16, device=w.device)
    M, K = x.shape
    if K != w.K:
        raise ValueError(f"x has K={K}, weight has K={w.K}")
    if out is None:
        out = torch.empty((M, w.N), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, (M, w.N), x.device)
    need = lib().sgd_gemm_workspace_bytes(w.fmt, M, w.N, w.K)
    if need == 0:
        raise ValueError(f"unsupported GEMM shape M={M} N={w.N} K={w.K}")
    st = w.c_struct()

    def launch():
        ws = _workspace(x.device, need, workspace)
        _lib.check("sgd_scaled_gemm", lib().sgd_scaled_gemm(
            _ptr(x), M, ctypes.byref(st), _ptr(out), _ptr(ws), ws.numel(), _stream(x)))
    _serialise_persistent(x.device, launch)
    return out


def fused_swiglu_mlp(x, gate, up, down, out=None, workspace=None):
    """y [M, d] bf16 = SwiGLU MLP of bf16 x [M, d] (one launch)."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, d]")
    _need(x, "x", torch.bfloat16, device=gate.device)
    M, d = x.shape
    if gate.K != d:
        raise ValueError(f"x has d={d}, gate weight has K={gate.K}")
    if out is None:
        out = torch.empty((M, d), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, (M, d), x.device)
    need = lib().sgd_mlp_workspace_bytes(gate.fmt, M, d, gate.N)
    if need == 0:
        raise ValueError(f"unsupported MLP shape M={M} d={d} ffn={gate.N}")
    g, u, dn = gate.c_struct(), up.c_struct(), down.c_struct()

    def launch():
        ws = _workspace(x.device, need, workspace)
        _lib.check("sgd_fused_swiglu_mlp", lib().sgd_fused_swiglu_mlp(
            _ptr(x), M, ctypes.byref(g), ctypes.byref(u), ctypes.byref(dn), _ptr(out),
            _ptr(ws), ws.numel(), _stream(x)))
    _serialise_persistent(x.device, launch)
    return out


def fused_swiglu_block(h, gate, up, down, eps=1e-6, out=None, workspace=None):
    """One pre-RMSNorm residual decode block in one launch:
    h_out [M, d] fp32 = h + bf16(MLP(bf16(RMSNorm(h)))), h [M, d] fp32.
    `out` must not overlap `h`."""
    if h.dim() != 2:
        raise ValueError("h must be 2-D [M, d]")
    _need(h, "h", torch.float32, device=gate.device)
    M, d = h.shape
    if gate.K != d:
        raise ValueError(f"h has d={d}, gate weight has K={gate.K}")
    if out is None:
        out = torch.empty((M, d), dtype=torch.float32, device=h.device)
    _need(out, "out", torch.float32, (M, d), h.device)
    need = lib().sgd_mlp_workspace_bytes(gate.fmt, M, d, gate.N)
    if need == 0:
        raise ValueError(f"unsupported MLP shape M={M} d={d} ffn={gate.N}")
    g, u, dn = gate.c_struct(), up.c_struct(), down.c_struct()

    def launch():
        ws = _workspace(h.device, need, workspace)
        _lib.check("sgd_fused_swiglu_block", lib().sgd_fused_swiglu_block(
            _ptr(h), M, ctypes.byref(g), ctypes.byref(u), ctypes.byref(dn), float(eps), _ptr(out),
            _ptr(ws), ws.numel(), _stream(h)))
    _serialise_persistent(h.device, launch)
    return out


def scaled_gemm_f32(x, w, out=None, workspace=None):
    """y [M, N] fp32 = Q(x) W^T (scaled_gemm with an fp32 output)."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    _need(x, "x", torch.bfloat16, device=w.device)
    M, K = x.shape
    if K != w.K:
        raise ValueError(f"x has K={K}, weight has K={w.K}")
    if out is None:
        out = torch.empty((M, w.N), dtype=torch.float32, device=x.device)
    _need(out, "out", torch.float32, (M, w.N), x.device)
    need = lib().sgd_gemm_workspace_bytes(w.fmt, M, w.N, w.K)
    if need == 0:
        raise ValueError(f"unsupported GEMM shape M={M} N={w.N} K={w.K}")
    st = w.c_struct()

    def launch():
        ws = _workspace(x.device, need, workspace)
        _lib.check("sgd_scaled_gemm_f32", lib().sgd_scaled_gemm_f32(
            _ptr(x), M, ctypes.byref(st), _ptr(out), _ptr(ws), ws.numel(), _stream(x)))
    _serialise_persistent(x.device, launch)
    return out


def swiglu_quantize(gu, fmt, out=None):
    """From gu [M, 2*ffn] fp32 (gate columns first, then up): Q(silu(g) * u)
    as (codes uint8 [M*ffn], scales uint8 [sgd_act_scales_bytes]) in the
    workspace layout (see swiglu_decode.h)."""
    f = fmt_code(fmt)
    if gu.dim() != 2 or gu.shape[1] % 2:
        raise ValueError("gu must be [M, 2*ffn]")
    _need(gu, "gu", torch.float32)
    M, F = gu.shape[0], gu.shape[1] // 2
    nsc = lib().sgd_act_scales_bytes(f, M, F)
    if nsc == 0:
        raise ValueError(f"unsupported shape M={M} ffn={F}")
    if out is None:
        out = (torch.empty(M * F, dtype=torch.uint8, device=gu.device),
               torch.empty(nsc, dtype=torch.uint8, device=gu.device))
    aq, sc = out
    _need(aq, "codes", torch.uint8, (M * F,), gu.device)
    _need(sc, "scales", torch.uint8, (nsc,), gu.device)
    _lib.check("sgd_swiglu_quantize",
               lib().sgd_swiglu_quantize(f, _ptr(gu), M, F, _ptr(aq), _ptr(sc), _stream(gu)))
    return aq, sc


def scaled_gemm_q(xq, xs, M, w, out=None, workspace=None):
    """y [M, N] bf16 = Q(x) W^T from activations already quantized in the
    workspace layout (codes xq uint8 [M*K], scales xs uint8)."""
    _need(xq, "xq", torch.uint8, (M * w.K,), w.device)
    _need(xs, "xs", torch.uint8, (lib().sgd_act_scales_bytes(w.fmt, M, w.K),), w.device)
    if out is None:
        out = torch.empty((M, w.N), dtype=torch.bfloat16, device=xq.device)
    _need(out, "out", torch.bfloat16, (M, w.N), xq.device)
    need = lib().sgd_gemm_workspace_bytes(w.fmt, M, w.N, w.K)
    if need == 0:
        raise ValueError(f"unsupported GEMM shape M={M} N={w.N} K={w.K}")
    st = w.c_struct()

    def launch():
        ws = _workspace(xq.device, need, workspace)
        _lib.check("sgd_scaled_gemm_q", lib().sgd_scaled_gemm_q(
            _ptr(xq), _ptr(xs), M, ctypes.byref(st), _ptr(out), _ptr(ws), ws.numel(), _stream(xq)))
    _serialise_persistent(xq.device, launch)
    return out


def stack_packed(a, b):
    """The packed weight of the row-stacked matrix [A; B] from packed A and B
    of one format and width (both packed layouts run band by band, so this is
    a concatenation of their codes and of their scales)."""
    if a.fmt != b.fmt or a.K != b.K or a.device != b.device:
        raise ValueError("weights to stack must share format, K and device")
    return PackedWeight(a.fmt, a.N + b.N, a.K, torch.cat([a.codes, b.codes]), torch.cat([a.scales, b.scales]))


def unfused_swiglu_mlp(x, gate_up, down, out=None, workspace=None, buffers=None):
    """The SwiGLU MLP in three launches with HBM intermediates: the gate/up
    GEMM into fp32 gu [M, 2*ffn] (gate_up = stack_packed(gate, up)), the
    standalone SwiGLU + re-quantization, the down GEMM from Q(a).  `buffers`
    (gu, aq, as) may be passed to reuse them (e.g. under graph capture)."""
    M = x.shape[0]
    F = gate_up.N // 2
    if buffers is None:
        buffers = (torch.empty((M, 2 * F), dtype=torch.float32, device=x.device),
                   torch.empty(M * F, dtype=torch.uint8, device=x.device),
                   torch.empty(lib().sgd_act_scales_bytes(gate_up.fmt, M, F), dtype=torch.uint8, device=x.device))
    gu, aq, sc = buffers
    scaled_gemm_f32(x, gate_up, out=gu, workspace=workspace)
    swiglu_quantize(gu, gate_up.fmt, out=(aq, sc))
    return scaled_gemm_q(aq, sc, M, down, out=out, workspace=workspace)


def scaled_gemm_large(x, w, out=None, workspace=None):
    """y [M, N] bf16 = Q(x) W^T for any 1 <= M <= 65536 (the large-M tiled
    path: quantize x, then the LDS-tiled fp8 GEMM)."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    _need(x, "x", torch.bfloat16, device=w.device)
    M, K = x.shape
    if K != w.K:
        raise ValueError(f"x has K={K}, weight has K={w.K}")
    if out is None:
        out = torch.empty((M, w.N), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, (M, w.N), x.device)
    need = lib().sgd_gemm_large_workspace_bytes(w.fmt, M, w.N, w.K)
    if need == 0:
        raise ValueError(f"unsupported large GEMM shape M={M} N={w.N} K={w.K}")
    st = w.c_struct()

    def launch():
        ws = _workspace(x.device, need, workspace)
        _lib.check("sgd_scaled_gemm_large", lib().sgd_scaled_gemm_large(
            _ptr(x), M, ctypes.byref(st), _ptr(out), _ptr(ws), ws.numel(), _stream(x)))
    _serialise_persistent(x.device, launch)
    return out


def swiglu_mlp_prefill(x, gate_up, down, out=None, workspace=None):
    """y [M, d] bf16 = SwiGLU MLP for large M (quantize x, tiled gate/up GEMM
    into fp32, SwiGLU + re-quantization, tiled down GEMM); gate_up =
    stack_packed(gate, up)."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, d]")
    _need(x, "x", torch.bfloat16, device=down.device)
    M, d = x.shape
    if gate_up.K != d or down.N != d or gate_up.N != 2 * down.K:
        raise ValueError("weights do not chain with x")
    if out is None:
        out = torch.empty((M, d), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, (M, d), x.device)
    need = lib().sgd_mlp_prefill_workspace_bytes(down.fmt, M, d, down.K)
    if need == 0:
        raise ValueError(f"unsupported prefill MLP shape M={M} d={d} ffn={down.K}")
    gu, dn = gate_up.c_struct(), down.c_struct()

    def launch():
        ws = _workspace(x.device, need, workspace)
        _lib.check("sgd_swiglu_mlp_prefill", lib().sgd_swiglu_mlp_prefill(
            _ptr(x), M, ctypes.byref(gu), ctypes.byref(dn), _ptr(out), _ptr(ws), ws.numel(), _stream(x)))
    _serialise_persistent(x.device, launch)
    return out


HEAD_DIM = 128
PAGE_SLOTS = 16
_CTRL_BYTES = 256 * 1024


def kv_cache_alloc(n_pages, Hkv, device):
    """A zeroed paged K or V cache: [n_pages * Hkv * 2112] uint8."""
    nbytes = lib().sgd_kv_cache_bytes(n_pages, Hkv)
    if nbytes == 0:
        raise ValueError(f"unsupported cache size n_pages={n_pages} Hkv={Hkv}")
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def kv_cache_write(kind, x, slots, cache, n_pages):
    """Quantize x [n, Hkv, 128] bf16 and write it into `cache` (kind "k" or
    "v") at int32 slots [n] (page * 16 + offset)."""
    if x.dim() != 3 or x.shape[2] != HEAD_DIM:
        raise ValueError("x must be [n, Hkv, 128]")
    _need(x, "x", torch.bfloat16)
    _need(slots, "slots", torch.int32, (x.shape[0],), x.device)
    _need(cache, "cache", torch.uint8, device=x.device)
    n, Hkv, _ = x.shape
    if cache.numel() < lib().sgd_kv_cache_bytes(n_pages, Hkv):
        raise ValueError("cache too small for n_pages")
    _lib.check("sgd_kv_cache_write", lib().sgd_kv_cache_write(
        {"k": 0, "v": 1}[kind], _ptr(x), _ptr(slots), n, Hkv, HEAD_DIM, _ptr(cache), n_pages, _stream(x)))
    return cache


def paged_decode_attention(q, k_cache, v_cache, n_pages, block_table, seq_lens, Hkv, sm_scale=None, out=None,
                           workspace=None):
    """out [B, Hq, 128] bf16: decode attention of q [B, Hq, 128] bf16 over the
    paged MXFP8 caches (block_table [B, max_pages] int32, seq_lens [B]
    int32), query head h reading KV head h // (Hq // Hkv)."""
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [B, Hq, 128]")
    _need(q, "q", torch.bfloat16)
    B, Hq, _ = q.shape
    _need(block_table, "block_table", torch.int32, device=q.device)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages]")
    max_pages = block_table.shape[1]
    _need(seq_lens, "seq_lens", torch.int32, (B,), q.device)
    _need(k_cache, "k_cache", torch.uint8, device=q.device)
    _need(v_cache, "v_cache", torch.uint8, device=q.device)
    if sm_scale is None:
        sm_scale = HEAD_DIM ** -0.5
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (B, Hq, HEAD_DIM), q.device)
    need = lib().sgd_paged_attention_workspace_bytes(B, Hq, Hkv, max_pages)
    if need == 0:
        raise ValueError(f"unsupported attention sizes B={B} Hq={Hq} Hkv={Hkv} max_pages={max_pages}")

    def launch():
        # (past the first 256 KB: a shared workspace keeps the persistent
        # kernels' control block there)
        ws = _workspace(q.device, need + _CTRL_BYTES, workspace)
        _lib.check("sgd_paged_decode_attention", lib().sgd_paged_decode_attention(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), n_pages, _ptr(block_table), max_pages, _ptr(seq_lens), B, Hq,
            Hkv, HEAD_DIM, float(sm_scale), _ptr(out), ctypes.c_void_p(ws.data_ptr() + _CTRL_BYTES),
            ws.numel() - _CTRL_BYTES, _stream(q)))
    _serialise_persistent(q.device, launch)
    return out


def fused_swiglu_mlp_noalloc(x, gate, up, down, out):
    """The fused MLP through the entry point that allocates nothing (its
    workspace is the library's fixed per-device array): y [M, d] bf16 into
    the caller's `out`."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, d]")
    _need(x, "x", torch.bfloat16, device=gate.device)
    M, d = x.shape
    _need(out, "out", torch.bfloat16, (M, d), x.device)
    g, u, dn = gate.c_struct(), up.c_struct(), down.c_struct()
    _serialise_persistent(x.device, lambda: _lib.check(
        "sgd_fused_swiglu_mlp_noalloc", lib().sgd_fused_swiglu_mlp_noalloc(
            _ptr(x), M, ctypes.byref(g), ctypes.byref(u), ctypes.byref(dn), _ptr(out), _stream(x))))
    return out


def bf16_to_f32(x, out=None):
    _need(x, "x", torch.bfloat16)
    M, d = x.shape
    if out is None:
        out = torch.empty((M, d), dtype=torch.float32, device=x.device)
    _need(out, "out", torch.float32, (M, d), x.device)
    _lib.check("sgd_bf16_to_f32", lib().sgd_bf16_to_f32(_ptr(x), M, d, _ptr(out), _stream(x)))
    return out


def rmsnorm_bf16(h, eps=1e-6, out=None):
    _need(h, "h", torch.float32)
    M, d = h.shape
    if out is None:
        out = torch.empty((M, d), dtype=torch.bfloat16, device=h.device)
    _need(out, "out", torch.bfloat16, (M, d), h.device)
    _lib.check("sgd_rmsnorm_bf16", lib().sgd_rmsnorm_bf16(_ptr(h), M, d, float(eps), _ptr(out), _stream(h)))
    return out


def residual_add(h, y):
    _need(h, "h", torch.float32)
    _need(y, "y", torch.bfloat16, tuple(h.shape), h.device)
    M, d = h.shape
    _lib.check("sgd_residual_add", lib().sgd_residual_add(_ptr(h), _ptr(y), M, d, _stream(h)))
    return h


def residual_rmsnorm_bf16(h, y, eps=1e-6, out=None):
    """h += y, then the next block's input x = bf16(RMSNorm(h)), in one
    launch (bit-identical to residual_add followed by rmsnorm_bf16)."""
    _need(h, "h", torch.float32)
    M, d = h.shape
    _need(y, "y", torch.bfloat16, (M, d), h.device)
    if out is None:
        out = torch.empty((M, d), dtype=torch.bfloat16, device=h.device)
    _need(out, "out", torch.bfloat16, (M, d), h.device)
    _lib.check("sgd_residual_rmsnorm_bf16",
               lib().sgd_residual_rmsnorm_bf16(_ptr(h), _ptr(y), M, d, float(eps), _ptr(out), _stream(h)))
    return out


def head_logits(h, w, out=None):
    _need(h, "h", torch.float32)
    M, K = h.shape
    _need(w, "w", torch.bfloat16, device=h.device)
    N = w.shape[0]
    if tuple(w.shape) != (N, K):
        raise ValueError(f"head weight must be [N, {K}], got {tuple(w.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=h.device)
    _need(out, "out", torch.float32, (M, N), h.device)
    _lib.check("sgd_head_logits", lib().sgd_head_logits(_ptr(h), M, K, _ptr(w), N, _ptr(out), _stream(h)))
    return out


def argmax_rows(logits, out=None):
    _need(logits, "logits", torch.float32)
    M, N = logits.shape
    if out is None:
        out = torch.empty((M,), dtype=torch.int32, device=logits.device)
    _need(out, "out", torch.int32, (M,), logits.device)
    _lib.check("sgd_argmax_rows", lib().sgd_argmax_rows(_ptr(logits), M, N, _ptr(out), _stream(logits)))
    return out


def read_stream(buf, sink=None):
    """One plain streaming read of the bytes of `buf` (a contiguous CUDA
    tensor whose size is a multiple of 16 bytes): a measurement aid for the
    attainable HBM read rate.  `sink` is a one-element int32 tensor the
    kernel may write (allocated here when not given)."""
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise TypeError("buf must be a contiguous CUDA tensor")
    if sink is None:
        sink = torch.empty((1,), dtype=torch.int32, device=buf.device)
    _need(sink, "sink", torch.int32, (1,), buf.device)
    nbytes = buf.numel() * buf.element_size()
    _lib.check("sgd_read_stream", lib().sgd_read_stream(_ptr(buf), nbytes, _ptr(sink), _stream(buf)))
    return sink

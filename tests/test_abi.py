"""CPU tests of the C-ABI library: it loads without a GPU, exports every
function the header declares, and rejects invalid arguments on the host
(these calls return before touching the HIP runtime)."""

import ctypes
import subprocess

import pytest

from swiglu_decode_amd import _lib
from swiglu_decode_amd._lib import SgdWeight

E = dict(OK=0, EINVAL=-1, EALIGN=-2, EDIM=-3, EWORKSPACE=-4, EFMT=-5, EHIP=-6, ETIMEOUT=-7)
BLK, MX = 1, 2


@pytest.fixture(scope="module")
def L():
    return _lib.load()


def test_every_header_function_is_exported(L):
    names = _lib.header_symbols()
    assert len(names) >= 17
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(L, n)
    assert set(_lib.SIGNATURES) == set(names)


def test_status_strings_and_version(L):
    for code in E.values():
        assert L.sgd_status_str(code)
    assert b"unknown" in L.sgd_status_str(12345)
    assert L.sgd_abi_version() == 2


def test_packed_sizes(L):
    assert L.sgd_packed_codes_bytes(BLK, 256, 512) == 256 * 512
    assert L.sgd_packed_scales_bytes(BLK, 256, 512) == 2 * 4 * 4
    assert L.sgd_packed_scales_bytes(MX, 256, 512) == 256 * 512 // 32
    # K = 256: two k-tiles padded to a group of four
    assert L.sgd_packed_scales_bytes(MX, 256, 256) == (256 // 16) * 256
    assert L.sgd_packed_codes_bytes(3, 256, 256) == 0
    assert L.sgd_packed_codes_bytes(BLK, 200, 256) == 0
    assert L.sgd_packed_codes_bytes(BLK, 0, 256) == 0
    # a weight holds fewer than 2^31 codes (32-bit offsets in the streaming
    # kernels), each dimension at most 2^20
    assert L.sgd_packed_codes_bytes(BLK, 1 << 16, (1 << 15) - 128) == (1 << 16) * ((1 << 15) - 128)
    assert L.sgd_packed_codes_bytes(BLK, 1 << 16, 1 << 15) == 0
    assert L.sgd_packed_scales_bytes(MX, 1 << 20, 1 << 11) == 0
    assert L.sgd_packed_codes_bytes(BLK, (1 << 20) + 128, 128) == 0


def test_workspace_sizes(L):
    a = L.sgd_mlp_workspace_bytes(MX, 1, 4096, 12288)
    b = L.sgd_mlp_workspace_bytes(MX, 128, 4096, 12288)
    assert 0 < a < b
    assert L.sgd_mlp_workspace_bytes(MX, 129, 4096, 12288) == 0
    assert L.sgd_mlp_workspace_bytes(MX, 0, 4096, 12288) == 0
    assert L.sgd_mlp_workspace_bytes(MX, 1, 4000, 12288) == 0
    assert L.sgd_gemm_workspace_bytes(BLK, 16, 6144, 2048) > 0
    assert L.sgd_gemm_workspace_bytes(BLK, 16, 6144, 2000) == 0


def _w(fmt=BLK, N=256, K=256, codes=0x1000, scales=0x2000, reserved=0):
    return SgdWeight(fmt, N, K, reserved, codes, scales)


P = ctypes.c_void_p


def test_argument_errors_launch_nothing(L):
    # pack
    assert L.sgd_quantize_pack_weight(7, P(0x1000), 256, 256, P(0x1000), P(0x1000), None) == E["EFMT"]
    assert L.sgd_quantize_pack_weight(BLK, P(0x1000), 200, 256, P(0x1000), P(0x1000), None) == E["EDIM"]
    assert L.sgd_quantize_pack_weight(BLK, None, 256, 256, P(0x1000), P(0x1000), None) == E["EINVAL"]
    assert L.sgd_quantize_pack_weight(BLK, P(0x1001), 256, 256, P(0x1000), P(0x1000), None) == E["EALIGN"]
    assert L.sgd_quantize_pack_weight(BLK, P(0x1000), -128, 256, P(0x1000), P(0x1000), None) == E["EINVAL"]
    # act quant
    assert L.sgd_quantize_act(MX, P(0x1000), 0, 256, P(0x1000), P(0x1000), None) == E["EINVAL"]
    assert L.sgd_quantize_act(MX, P(0x1000), 4, 100, P(0x1000), P(0x1000), None) == E["EDIM"]
    assert L.sgd_quantize_act(MX, P(0x1000), 4, 256, P(0x1008), P(0x1000), None) == E["EALIGN"]
    # unpack
    w = _w(reserved=1)
    assert L.sgd_unpack_weight(ctypes.byref(w), P(0x1000), P(0x1000), None) == E["EINVAL"]
    w = _w(codes=0x1004)
    assert L.sgd_unpack_weight(ctypes.byref(w), P(0x1000), P(0x1000), None) == E["EALIGN"]
    # gemm
    w = _w()
    ws_need = L.sgd_gemm_workspace_bytes(BLK, 4, 256, 256)
    assert L.sgd_scaled_gemm(P(0x1000), 0, ctypes.byref(w), P(0x1000), P(0x1000), ws_need, None) == E["EINVAL"]
    assert L.sgd_scaled_gemm(P(0x1000), 129, ctypes.byref(w), P(0x1000), P(0x1000), ws_need, None) == E["EINVAL"]
    assert L.sgd_scaled_gemm(P(0x1000), 4, None, P(0x1000), P(0x1000), ws_need, None) == E["EINVAL"]
    assert L.sgd_scaled_gemm(P(0x1000), 4, ctypes.byref(w), P(0x1000), None, ws_need, None) == E["EWORKSPACE"]
    assert L.sgd_scaled_gemm(P(0x1000), 4, ctypes.byref(w), P(0x1000), P(0x1000), ws_need - 1, None) == E["EWORKSPACE"]
    assert L.sgd_scaled_gemm(P(0x1002), 4, ctypes.byref(w), P(0x1000), P(0x1000), ws_need, None) == E["EALIGN"]
    bad = _w(fmt=9)
    assert L.sgd_scaled_gemm(P(0x1000), 4, ctypes.byref(bad), P(0x1000), P(0x1000), ws_need, None) == E["EFMT"]
    big = _w(N=1 << 16, K=1 << 15)  # 2^31 codes: past the 32-bit offsets
    assert L.sgd_scaled_gemm(P(0x1000), 4, ctypes.byref(big), P(0x1000), P(0x1000), 1 << 40, None) == E["EDIM"]
    assert L.sgd_quantize_pack_weight(BLK, P(0x1000), 1 << 16, 1 << 15, P(0x1000), P(0x1000), None) == E["EDIM"]
    # fused mlp: shapes must chain, formats must agree
    g, u, d = _w(N=512, K=256), _w(N=512, K=256), _w(N=256, K=512)
    need = L.sgd_mlp_workspace_bytes(BLK, 4, 256, 512)
    args = lambda g_, u_, d_, ws=need: L.sgd_fused_swiglu_mlp(
        P(0x1000), 4, ctypes.byref(g_), ctypes.byref(u_), ctypes.byref(d_), P(0x1000), P(0x1000), ws, None)
    assert args(g, u, _w(N=256, K=384)) == E["EDIM"]
    assert args(g, _w(fmt=MX, N=512, K=256), d) == E["EFMT"]
    assert args(g, u, d, need - 16) == E["EWORKSPACE"]
    gb, ub, db = _w(N=1 << 15, K=1 << 16), _w(N=1 << 15, K=1 << 16), _w(N=1 << 16, K=1 << 15)
    assert args(gb, ub, db, 1 << 40) == E["EDIM"]
    # the entry point without a workspace: same argument checks, and shapes
    # whose workspace exceeds its fixed array are refused before any launch
    na = lambda g_, u_, d_, M=4, x=0x1000: L.sgd_fused_swiglu_mlp_noalloc(
        P(x), M, ctypes.byref(g_), ctypes.byref(u_), ctypes.byref(d_), P(0x1000), None)
    assert na(g, u, _w(N=256, K=384)) == E["EDIM"]
    assert na(g, u, d, M=0) == E["EINVAL"]
    assert na(g, u, d, x=0x1002) == E["EALIGN"]
    assert na(g, _w(fmt=MX, N=512, K=256), d) == E["EFMT"]
    wide_g, wide_u, wide_d = _w(N=128, K=262144), _w(N=128, K=262144), _w(N=262144, K=128)
    assert L.sgd_mlp_workspace_bytes(BLK, 128, 262144, 128) > (64 << 20)
    assert na(wide_g, wide_u, wide_d, M=128) == E["EWORKSPACE"]
    # decode block: the MLP's checks, plus eps and an output that must not
    # overlap the input (h is 4 x 256 fp32 = 4 KB)
    blk = lambda g_, u_, d_, hi=0x10000, ho=0x20000, eps=1e-6, ws=need, M=4: L.sgd_fused_swiglu_block(
        P(hi), M, ctypes.byref(g_), ctypes.byref(u_), ctypes.byref(d_), ctypes.c_float(eps), P(ho), P(0x1000), ws,
        None)
    assert blk(g, u, _w(N=256, K=384)) == E["EDIM"]
    assert blk(g, _w(fmt=MX, N=512, K=256), d) == E["EFMT"]
    assert blk(g, u, d, M=0) == E["EINVAL"]
    assert blk(g, u, d, hi=0) == E["EINVAL"]
    assert blk(g, u, d, ho=0x10008) == E["EALIGN"]
    assert blk(g, u, d, ho=0x10000) == E["EINVAL"]
    assert blk(g, u, d, ho=0x10000 + 4096 - 16) == E["EINVAL"]
    assert blk(g, u, d, hi=0x20000 + 4096 - 16) == E["EINVAL"]
    assert blk(g, u, d, eps=-1.0) == E["EINVAL"]
    assert blk(g, u, d, eps=float("nan")) == E["EINVAL"]
    assert blk(g, u, d, ws=need - 16) == E["EWORKSPACE"]
    # paged decode attention and its cache writer: argument errors only
    assert L.sgd_kv_cache_bytes(10, 8) == 10 * 8 * 2112
    assert L.sgd_kv_cache_bytes(1 << 20, 1024) == 0
    kw = lambda kind=0, x=0x1000, sl=0x2000, n=4, Hkv=2, hd=128, c=0x3000, npg=8: L.sgd_kv_cache_write(
        kind, P(x), P(sl), n, Hkv, hd, P(c), npg, None)
    assert kw(kind=2) == E["EINVAL"]
    assert kw(hd=64) == E["EDIM"]
    assert kw(n=0) == E["EINVAL"]
    assert kw(x=0) == E["EINVAL"]
    assert kw(x=0x1008) == E["EALIGN"]
    assert kw(sl=0x2002) == E["EALIGN"]
    assert L.sgd_paged_attention_workspace_bytes(4, 32, 8, 100) > 0
    assert L.sgd_paged_attention_workspace_bytes(4, 30, 8, 100) == 0  # Hq not a multiple of Hkv
    assert L.sgd_paged_attention_workspace_bytes(4, 64, 2, 100) == 0  # 32 query heads per KV head
    wsa = L.sgd_paged_attention_workspace_bytes(4, 32, 8, 100)
    pa = lambda q=0x1000, B=4, Hq=32, Hkv=8, hd=128, sc=0.088, ws=wsa, bt=0x4000: L.sgd_paged_decode_attention(
        P(q), P(0x2000), P(0x3000), 50, P(bt), 100, P(0x5000), B, Hq, Hkv, hd, ctypes.c_float(sc), P(0x6000),
        P(0x7000), ws, None)
    assert pa(hd=64) == E["EDIM"]
    assert pa(Hq=30) == E["EINVAL"]
    assert pa(B=0) == E["EINVAL"]
    assert pa(sc=0.0) == E["EINVAL"]
    assert pa(sc=float("nan")) == E["EINVAL"]
    assert pa(q=0x1008) == E["EALIGN"]
    assert pa(bt=0x4002) == E["EALIGN"]
    assert pa(ws=wsa - 4) == E["EWORKSPACE"]
    # large-M path: rows up to SGD_MAX_M_LARGE, offsets within 32 bits
    w = _w(N=256, K=512)
    lneed = L.sgd_gemm_large_workspace_bytes(BLK, 1000, 256, 512)
    assert lneed > 256 * 1024
    assert L.sgd_gemm_large_workspace_bytes(BLK, 65537, 256, 512) == 0
    assert L.sgd_gemm_large_workspace_bytes(BLK, 65536, 256, 1 << 15) == 0  # 2^31 codes of Q(x)
    assert L.sgd_gemm_large_workspace_bytes(3, 16, 256, 512) == 0
    lg = lambda x=0x1000, M=1000, w_=w, y=0x2000, ws=0x10000, n=lneed: L.sgd_scaled_gemm_large(
        P(x), M, ctypes.byref(w_), P(y), P(ws), n, None)
    assert lg(M=0) == E["EINVAL"]
    assert lg(M=65537) == E["EINVAL"]
    assert lg(x=0) == E["EINVAL"]
    assert lg(y=0x2008) == E["EALIGN"]
    assert lg(ws=0) == E["EWORKSPACE"]
    assert lg(ws=0x10008) == E["EALIGN"]
    assert lg(n=lneed - 16) == E["EWORKSPACE"]
    assert lg(w_=_w(fmt=9, N=256, K=512)) == E["EFMT"]
    gu2, dn2 = _w(N=1024, K=256), _w(N=256, K=512)
    pneed = L.sgd_mlp_prefill_workspace_bytes(BLK, 300, 256, 512)
    assert pneed > lneed // 4
    assert L.sgd_mlp_prefill_workspace_bytes(BLK, 300, 256, 40000) == 0
    pf = lambda gu_=gu2, dn_=dn2, M=300, n=pneed: L.sgd_swiglu_mlp_prefill(
        P(0x1000), M, ctypes.byref(gu_), ctypes.byref(dn_), P(0x2000), P(0x10000), n, None)
    assert pf(dn_=_w(N=256, K=384)) == E["EDIM"]  # gate/up rows must be 2 ffn
    assert pf(gu_=_w(fmt=MX, N=1024, K=256)) == E["EFMT"]
    assert pf(M=0) == E["EINVAL"]
    assert pf(n=pneed - 256) == E["EWORKSPACE"]
    # workspace status query: argument errors only (no GPU here)
    assert L.sgd_workspace_status(None, None) == E["EINVAL"]
    assert L.sgd_workspace_status(P(0x1004), None) == E["EALIGN"]
    # glue
    assert L.sgd_rmsnorm_bf16(P(0x1000), 4, 100, ctypes.c_float(1e-6), P(0x1000), None) == E["EDIM"]
    assert L.sgd_rmsnorm_bf16(P(0x1000), 4, 128, ctypes.c_float(-1.0), P(0x1000), None) == E["EINVAL"]
    assert L.sgd_residual_rmsnorm_bf16(P(0x1000), P(0x2000), 4, 100, ctypes.c_float(1e-6), P(0x3000), None) == E["EDIM"]
    assert L.sgd_residual_rmsnorm_bf16(P(0x1000), P(0x2000), 4, 128, ctypes.c_float(-1.0), P(0x3000), None) == E["EINVAL"]
    assert L.sgd_residual_rmsnorm_bf16(None, P(0x2000), 4, 128, ctypes.c_float(1e-6), P(0x3000), None) == E["EINVAL"]
    assert L.sgd_residual_rmsnorm_bf16(P(0x1000), P(0x2008), 4, 128, ctypes.c_float(1e-6), P(0x3000), None) == E["EALIGN"]
    assert L.sgd_head_logits(P(0x1000), 200, 256, P(0x1000), 256, P(0x1000), None) == E["EINVAL"]
    assert L.sgd_argmax_rows(P(0x1000), 0, 10, P(0x1000), None) == E["EINVAL"]
    assert L.sgd_workspace_clear(P(0x1000), 24, None) == E["EALIGN"]
    # measurement aid
    assert L.sgd_read_stream(None, 1024, P(0x1000), None) == E["EINVAL"]
    assert L.sgd_read_stream(P(0x1000), 1024, None, None) == E["EINVAL"]
    assert L.sgd_read_stream(P(0x1000), 1000, P(0x1000), None) == E["EALIGN"]
    assert L.sgd_read_stream(P(0x1008), 1024, P(0x1000), None) == E["EALIGN"]
    assert L.sgd_read_stream(P(0x1000), 1024, P(0x1002), None) == E["EALIGN"]


def test_wait_budget_setting(L):
    # process-wide; 0 restores the default (1 s); returns the previous value
    prev = L.sgd_set_wait_budget_us(250)
    assert L.sgd_set_wait_budget_us(0) == 250
    assert L.sgd_set_wait_budget_us(prev) == 1000000
    L.sgd_set_wait_budget_us(0)


def test_keep_intermediates_setting(L):
    # process-wide, off by default; any nonzero value reads back as 1
    prev = L.sgd_set_keep_intermediates(7)
    assert prev == 0
    assert L.sgd_set_keep_intermediates(0) == 1
    assert L.sgd_set_keep_intermediates(0) == 0


def test_binding_refuses_wrong_dtypes_without_gpu():
    import torch
    import swiglu_decode_amd as sgd
    x = torch.zeros(4, 256, dtype=torch.float32)
    with pytest.raises(TypeError):
        sgd.quantize_act(x, "block")
    with pytest.raises(ValueError):
        sgd.fmt_code("fp4")

"""The host-side validation layer of the C ABI (capi.hip, noalloc.hip) built
with AddressSanitizer and UndefinedBehaviorSanitizer on the host code only
(device code is unchanged), linked with the library's other objects, and
driven on the CPU: the ABI tests, plus every size and layout query over
extreme and invalid integers (signed overflow in a size computation is
undefined behaviour, which UBSan turns into a failure here).  No GPU is
touched: every call returns before launching anything."""

import os
import subprocess
import sys
import textwrap

import pytest

from swiglu_decode_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SANITIZED = ("capi.hip", "noalloc.hip")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_runtime():
    clang = os.path.join(os.path.dirname(os.path.realpath(B._hipcc())), "..", "lib", "llvm", "bin", "clang")
    for c in (clang, "/opt/rocm/lib/llvm/bin/clang"):
        if os.path.exists(c):
            r = subprocess.run([c, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
            p = r.stdout.strip()
            if r.returncode == 0 and os.path.isabs(p) and os.path.exists(p):
                return p
    return None


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this toolchain")
    others = [f for f in B.sources() if os.path.basename(f) not in SANITIZED]
    objs = [os.path.join(B.BUILD, os.path.basename(f)[:-4] + ".o") for f in others]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    out = tmp_path_factory.mktemp("san")
    flags = [f for f in B.HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"]
    san_objs = []
    for name in SANITIZED:
        o = str(out / (name[:-4] + ".o"))
        r = subprocess.run([B._hipcc(), *flags, *SAN_FLAGS, "-c", os.path.join(B.CSRC, name), "-o", o],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        san_objs.append(o)
    lib = str(out / "libswiglu_decode_san.so")
    r = subprocess.run([B._hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", *san_objs, *objs, "-o", lib],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return lib, rt


def _run(lib, rt, code):
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    prog = f"import sys; sys.path.insert(0, {ROOT!r})\nimport swiglu_decode_amd._lib as L\nL.LIB_PATH = {lib!r}\n" + code
    r = subprocess.run([sys.executable, "-c", prog], capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    text = r.stdout + r.stderr
    assert "AddressSanitizer" not in text and "runtime error" not in text, text[-4000:]
    assert r.returncode == 0, text[-4000:]
    return r.stdout


def test_abi_tests_under_sanitizers(sanitized_lib):
    lib, rt = sanitized_lib
    out = _run(lib, rt, textwrap.dedent("""
        import pytest
        rc = pytest.main(["-q", "-p", "no:cacheprovider", "tests/test_abi.py"])
        print("maps:", any("libswiglu_decode_san" in l for l in open("/proc/self/maps")))
        sys.exit(rc)
    """))
    assert "maps: True" in out


def test_size_and_layout_queries_over_extreme_integers(sanitized_lib):
    lib, rt = sanitized_lib
    out = _run(lib, rt, textwrap.dedent("""
        import ctypes, itertools
        lib = L.load()
        vals = [-(1 << 31), -1, 0, 1, 16, 127, 128, 129, 4096, 12288, 65536, 65537, (1 << 20), (1 << 20) + 128,
                (1 << 30), (1 << 31) - 1]
        fmts = [-1, 0, 1, 2, 3]
        n = 0
        for f in fmts:
            for a, b in itertools.product(vals, repeat=2):
                lib.sgd_packed_codes_bytes(f, a, b)
                lib.sgd_packed_scales_bytes(f, a, b)
                n += 2
            for m, a, b in itertools.product(vals, repeat=3):
                lib.sgd_gemm_workspace_bytes(f, m, a, b)
                lib.sgd_mlp_workspace_bytes(f, m, a, b)
                lib.sgd_gemm_large_workspace_bytes(f, m, a, b)
                lib.sgd_mlp_prefill_workspace_bytes(f, m, a, b)
                offs = (ctypes.c_size_t * 5)()
                lib.sgd_mlp_workspace_layout(f, m, a, b, offs)
                lib.sgd_mlp_workspace_layout(f, m, a, b, None)
                n += 6
            for m, k in itertools.product(vals, repeat=2):
                lib.sgd_act_scales_bytes(f, m, k)
                n += 1
        for a, b in itertools.product(vals, repeat=2):
            lib.sgd_kv_cache_bytes(a, b)
            n += 1
        for a, b, c, d in itertools.product(vals[::2], repeat=4):
            lib.sgd_paged_attention_workspace_bytes(a, b, c, d)
            n += 1
        for s in vals + [-7, -6, 12345]:
            lib.sgd_status_str(s)
        print("calls", n)
    """))
    assert "calls" in out

"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

* The oracle (oracle.c) is built with -fsanitize=address,undefined and the pin
  suite runs against that build in a fresh process.
* The C ABI's host layer (q4_api.cpp: every argument check before a launch)
  is built the same way with host-only stand-ins for the launchers
  (tests/sanitize/q4_launch_stub.cpp), and the boundary suite plus checks
  that valid calls reach the right launcher run against it.
* Two planted mistakes in copies of the oracle (a write one element past an
  output row, a shift wider than an int) must be reported by the sanitizers:
  this shows the instrumentation is live.  The real sources are never
  modified, and nothing here touches a GPU.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "oracle.c")
CSRC = os.path.join(ROOT, "bit_weight_gemv_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _clang_asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def _build_oracle(src, out):
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-fast-math",
           "-ffp-contract=off", "-I", os.path.dirname(ORACLE_SRC), src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True)
    return out


def _run_pins(lib, tests=("tests/test_oracle_pins.py",)):
    """The pin suite in a fresh process against `lib`, with the gcc sanitizer
    runtimes preloaded (they must come first in the process)."""
    pre = [p for p in (_gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")) if p]
    env = dict(os.environ, Q4_ORACLE_LIB=lib, LD_PRELOAD=":".join(pre), **SAN_ENV)
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider", *tests],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


needs_gcc_san = pytest.mark.skipif(_gcc_runtime("libasan.so") is None, reason="gcc's AddressSanitizer runtime is absent")


@needs_gcc_san
def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = _build_oracle(ORACLE_SRC, str(tmp_path / "liboracle_san.so"))
    r = _run_pins(lib, ("tests/test_oracle_pins.py", "tests/test_golden.py", "tests/test_workloads.py"))
    out = r.stdout + r.stderr
    assert "Sanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]


# Planted mistakes: (anchor, replacement, what the report must name).
PLANTED = {
    "dequant_writes_past_row": (
        "    for (int64_t m = 0; m < M; ++m)\n        for (int64_t k = 0; k < K; ++k) {\n"
        "            double s = oracle_f16_to_f64(scales[m * (K / 64) + k / 64]);\n            What",
        "    for (int64_t m = 0; m < M; ++m)\n        for (int64_t k = 0; k <= K; ++k) {\n"
        "            double s = oracle_f16_to_f64(scales[m * (K / 64) + k / 64]);\n            What",
        "AddressSanitizer"),
    "nibble_shift_wider_than_int": (
        "return (k % 2 == 0) ? (byte & 0xf) : (byte >> 4);",
        "return (k % 2 == 0) ? (byte & 0xf) : ((byte >> 4) & (0xf << (k & 63)) >> (k & 63));",
        "runtime error: left shift"),
}


@needs_gcc_san
@pytest.mark.parametrize("name", sorted(PLANTED))
def test_sanitizers_report_planted_mistake(name, tmp_path):
    old, new, report = PLANTED[name]
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, f"anchor for {name} not found exactly once"
    mpath = tmp_path / "oracle_planted.c"
    mpath.write_text(src.replace(old, new))
    lib = _build_oracle(str(mpath), str(tmp_path / "liboracle_planted.so"))
    r = _run_pins(lib)
    out = r.stdout + r.stderr
    assert r.returncode != 0, f"planted {name} ran clean:\n{out[-2000:]}"
    assert report in out, f"planted {name}: no sanitizer report:\n{out[-3000:]}"


needs_host_san = pytest.mark.skipif(_clang_asan_runtime() is None or not os.path.exists(HIPCC),
                                    reason="hipcc or clang's AddressSanitizer runtime is absent")

# Run inside the sanitized process: the boundary suite, then valid calls that
# must reach the launcher stand-ins with their shapes.
_ABI_DRIVER = r"""
import ctypes, sys
sys.path.insert(0, {root!r})
import bit_weight_gemv_amd as q4
q4.LIB_PATH = {lib!r}
import pytest
rc = pytest.main(["-q", "-x", "-s", "-p", "no:cacheprovider", {boundary!r}])
if rc != 0:
    sys.exit(rc)
L = q4.lib()
L.q4stub_calls.restype = ctypes.c_int
L.q4stub_last.restype = ctypes.c_char_p
buf = ctypes.create_string_buffer(1 << 22)
base = (ctypes.addressof(buf) + 255) & ~255
A, B, C, D, E = (base + i * (1 << 19) for i in range(5))
def last():
    return L.q4stub_last().decode()
n0 = L.q4stub_calls()
assert L.q4_gemv(A, B, 100, 2048, C, D, None) == 0 and last() == "gemv M=100 K=2048", last()
assert L.q4_gemm_smalln(A, B, 100, 2048, C, 17, D, None) == 0 and last() == "gemm_smalln M=100 K=2048 N=17", last()
assert L.q4_gemm_smalln(A, B, 100, 2048, C, 0, D, None) == 0 and last() == "gemm_smalln M=100 K=2048 N=17", last()
L.q4_gemm_smalln_ws.argtypes = [ctypes.c_void_p] * 2 + [ctypes.c_int64] * 2 + [ctypes.c_void_p, ctypes.c_int64] + [ctypes.c_void_p] * 2 + [ctypes.c_size_t, ctypes.c_void_p]
L.q4_gemm_smalln_ws_bytes.restype = ctypes.c_size_t
L.q4_gemm_smalln_ws_bytes.argtypes = [ctypes.c_int64] * 3
need = L.q4_gemm_smalln_ws_bytes(100, 11008, 9)
assert need == 6 * 9 * 100 * 4, need
assert L.q4_gemm_smalln_ws(A, B, 100, 11008, C, 9, D, E, need, None) == 0 and last() == "gemm_smalln_ws M=100 K=11008 N=9", last()
assert L.q4_gemm_smalln_ws(A, B, 100, 11008, C, 9, D, E, need - 1, None) == 6
L.q4_gemm_smalln_noalloc.argtypes = [ctypes.c_void_p] * 2 + [ctypes.c_int64] * 2 + [ctypes.c_void_p, ctypes.c_int64] + [ctypes.c_void_p] * 2
assert L.q4_gemm_smalln_noalloc(A, B, 100, 11008, C, 9, D, None) == 0 and last() == "gemm_smalln_noalloc M=100 K=11008 N=9", last()
assert L.q4_gemm_smalln_noalloc(1 << 32, 2 << 32, 100000, 4096, 3 << 32, 32, 4 << 32, None) == 6  # never dereferenced
assert L.q4_pack(A, 8, 128, B, C, D, None) == 0 and last() == "pack M=8 K=128", last()
assert L.q4_gemv_affine(A, B, C, 9, 192, D, E, None) == 0 and last() == "gemv_affine M=9 K=192", last()
assert L.q4_gemv_nvfp4(A, B, C, 9, 192, D, E, None) == 0 and last() == "gemv_nvfp4 M=9 K=192", last()
assert L.q4_quantize_x8(A, 2048, 2, B, C, D, None) == 0 and last() == "quantize_x8 K=2048 words=2", last()
assert L.q4_gather_rows(A, B, 16, 128, C, 4, 1, D, E, None) == 0 and last() == "gather_rows_bf16 M=16 K=128 n=4", last()
ops = (q4.Operand * 2)(q4.Operand(A, B, 64, None), q4.Operand(C, D, 64, None))
ys = (ctypes.c_void_p * 1)(E)
assert L.q4_gemv_fused(ops, 2, 2048, base + 6 * (1 << 19), 1, ys, None, None) == 0, last()
assert last() == "gemv_fused swiglu count=2 K=2048 rows=128", last()
aops = (q4.OperandAffine * 1)(q4.OperandAffine(A, B, C, 64, None))
assert L.q4_gemv_fused_affine(aops, 1, 2048, base + 6 * (1 << 19), 0, ys, None, None) == 0, last()
assert last() == "gemv_fused_affine count=1 K=2048 rows=64", last()
nops = (q4.OperandNvfp4 * 2)(q4.OperandNvfp4(A, B, C, 64, None), q4.OperandNvfp4(D, base + 7 * (1 << 19), C, 64, None))
assert L.q4_gemv_fused_nvfp4(nops, 2, 2048, base + 6 * (1 << 19), 1, ys, None, None) == 0, last()
assert last() == "gemv_fused_nvfp4 swiglu count=2 K=2048 rows=128", last()
assert L.q4stub_calls() == n0 + 12, L.q4stub_calls() - n0
print("launch stand-ins reached:", L.q4stub_calls() - n0)
"""


@needs_host_san
def test_c_abi_host_layer_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "libq4_host_san.so")
    # Host-side sanitizers only (-Xarch_host before each -fsanitize): no
    # device code is built from these sources.
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared", "-g", "-O1",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "q4_api.cpp"), os.path.join(ROOT, "tests", "sanitize", "q4_launch_stub.cpp"),
           "-o", lib]
    subprocess.run(cmd, check=True, capture_output=True)
    driver = tmp_path / "abi_driver.py"
    driver.write_text(_ABI_DRIVER.format(root=ROOT, lib=lib,
                                         boundary=os.path.join(ROOT, "tests", "test_boundary.py")))
    env = dict(os.environ, LD_PRELOAD=_clang_asan_runtime(), **SAN_ENV)
    r = subprocess.run([sys.executable, str(driver)], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert "Sanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "launch stand-ins reached: 12" in out, out[-2000:]

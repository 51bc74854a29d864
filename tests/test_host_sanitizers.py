"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

1. The oracle (oracle/aria_oracle.c) built with gcc -fsanitize=address,undefined
   runs every oracle pin; any out-of-bounds access, use after free or undefined
   operation aborts the run.
2. The C-ABI's host code (api.hip: argument validation, overlap checks,
   workspace layout) built with clang's sanitizers on the host side only (the
   GPU code is compiled as usual) runs the ABI validation tests; no GPU is
   touched, every call there fails validation before any launch.

Each runs in a child process with the sanitizer runtime preloaded (the Python
interpreter is not instrumented); leak checking is off (the interpreter's own
allocations would be reported)."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "quantized_diffusion_transformer_qlinear_amd")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:verify_asan_link_order=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}
PINS = ["tests/test_oracle_codec.py", "tests/test_oracle_quant.py", "tests/test_oracle_pack.py",
        "tests/test_oracle_gemm.py", "tests/test_oracle_epilogue.py", "tests/test_oracle_block.py",
        "tests/test_oracle_chain.py"]


def _pytest(files, env):
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           "-W", "ignore::RuntimeWarning", "-m", "not gpu", *files],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


def _instrumented(lib):
    out = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    return "__asan_report_load" in out and "__ubsan_handle" in out


def test_sanitizer_catches_a_planted_overflow(tmp_path):
    """Positive control, host only: a one-element heap overflow in a tiny C
    library, called the way the oracle is, must be reported and abort."""
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = tmp_path / "oob.c"
    src.write_text("#include <stdlib.h>\nint oob(void) { int* a = malloc(4 * sizeof(int)); int v = a[4]; free(a); return v; }\n")
    so = str(tmp_path / "liboob.so")
    subprocess.run([gcc, "-O1", "-g", "-fsanitize=address,undefined", "-fPIC", "-shared", str(src), "-o", so], check=True)
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(os.environ, **SAN_ENV, LD_PRELOAD=asan)
    r = subprocess.run([sys.executable, "-c", f"import ctypes; ctypes.CDLL({so!r}).oob()"], env=env,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and ("heap-buffer-overflow" in r.stderr or "runtime error:" in r.stderr), r.stderr[-2000:]


def test_oracle_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    import oracle
    so = str(tmp_path / "liboracle_san.so")
    flags = [f for f in oracle._CFLAGS if f != "-O2"]
    subprocess.run([gcc, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", *flags, oracle._SRC, "-o", so, "-lm"], check=True)
    assert _instrumented(so)
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(os.environ, **SAN_ENV, LD_PRELOAD=asan, ARIA_ORACLE_LIB=so, OMP_NUM_THREADS="4")
    r = _pytest(PINS, env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr


def test_abi_host_code_under_asan_ubsan(tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objs = sorted(glob.glob(os.path.join(PKG, "_build", "*.o")))
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not os.path.exists(hipcc) or not rt or not any(o.endswith("api.o") for o in objs):
        pytest.skip("hipcc, the clang sanitizer runtime or the library's objects are missing")
    sys.path.insert(0, PKG)
    try:
        import build as hipbuild
    finally:
        sys.path.pop(0)
    api_o = str(tmp_path / "api_san.o")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
    subprocess.run([hipcc, *hipbuild.FLAGS, *san, "-g", "-c", os.path.join(PKG, "csrc", "api.hip"), "-o", api_o],
                   check=True, capture_output=True, text=True)
    lib = str(tmp_path / "libaria_qlinear_san.so")
    others = [o for o in objs if not o.endswith("api.o")]
    subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libasan", *san, api_o, *others,
                    "-o", lib], check=True, capture_output=True, text=True)
    assert _instrumented(lib)
    env = dict(os.environ, **SAN_ENV, LD_PRELOAD=rt[-1], ARIA_QLINEAR_LIB=lib)
    r = _pytest(["tests/test_abi.py"], env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr

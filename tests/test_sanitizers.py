"""AddressSanitizer + UndefinedBehaviorSanitizer runs of the host code (CPU only).

* The fp64 oracle is rebuilt with gcc -fsanitize=address,undefined (every
  report fatal) and the whole oracle pin suite runs against that build.
* The C ABI's host side (argument validation and dispatch in ttt_api.hip) is
  rebuilt with host-only sanitizers (GPU code is not instrumented), linked with
  the library's kernel objects, and tests/test_abi.py (every entry point,
  every rejected-argument case) runs against it.

Both run in a subprocess with the sanitizer runtime preloaded, since the
Python interpreter itself is not instrumented.  Leak checking is off: the
interpreter's own allocations are not this code's.
"""
import glob
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ENV_SAN = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _run(code, preload, *args):
    env = dict(os.environ, LD_PRELOAD=preload, **ENV_SAN)
    r = subprocess.run([sys.executable, "-c", code, *args], env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    return out


def test_oracle_pins_under_asan_ubsan():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("gcc's AddressSanitizer runtime not found")
    from oracle import oracle
    with tempfile.TemporaryDirectory() as tmp:
        lib = os.path.join(tmp, "liboracle_san.so")
        oracle.build(os.path.join(ROOT, "oracle", "ttt_oracle.c"), lib,
                     extra_flags=("-g", "-O1", "-fno-omit-frame-pointer",
                                  "-fsanitize=address,undefined", "-fno-sanitize-recover=all"))
        code = (
            "import sys; sys.path[:0] = [sys.argv[1], sys.argv[1] + '/tests']\n"
            "import test_oracle_pins as T\n"
            "from oracle import oracle\n"
            "lib = oracle.load(sys.argv[2])\n"
            "for p in T.PINS:\n"
            "    p(lib)\n"
            "print('pins', len(T.PINS))\n")
        out = _run(code, asan, ROOT, lib)
        assert "pins" in out


def test_abi_host_validation_under_asan_ubsan():
    from test_rnn_layers_head_amd import build
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rt or not os.path.exists(build.hipcc()):
        pytest.skip("hipcc or clang's AddressSanitizer runtime not found")
    build.build()  # the kernel objects under _build/
    objs = [o for o in glob.glob(os.path.join(build.BUILD, "*.o"))
            if not os.path.basename(o).startswith("ttt_api")]
    with tempfile.TemporaryDirectory() as tmp:
        api_o = os.path.join(tmp, "ttt_api_san.o")
        lib = os.path.join(tmp, "libttt_san.so")
        # sanitizers apply to the host compilation only (each flag after -Xarch_host)
        san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
        subprocess.run([build.hipcc(), *build.HIPCC_FLAGS, "-g", *san, "-c",
                        os.path.join(build.CSRC, "ttt_api.hip"), "-o", api_o],
                       check=True, capture_output=True, text=True)
        subprocess.run([build.hipcc(), f"--offload-arch={build.ARCH}", "-shared", "-fPIC",
                        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                        api_o, *objs, "-o", lib], check=True, capture_output=True, text=True)
        code = (
            "import sys; sys.path[:0] = [sys.argv[1], sys.argv[1] + '/tests']\n"
            "from test_rnn_layers_head_amd import _lib\n"
            "_lib.LIB_PATH = sys.argv[2]\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-p', 'no:xdist',\n"
            "                      sys.argv[1] + '/tests/test_abi.py']))\n")
        out = _run(code, rt[0], ROOT, lib)
        assert " passed" in out

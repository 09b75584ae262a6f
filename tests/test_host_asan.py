"""Host-side memory checking of the C ABI: the library's host code (argument validation, size
queries, the host cu_seqlens check, workspace layouts) built with AddressSanitizer and driven by
the ABI and binding tests, which never reach a kernel launch. A planted over-read (a host
cu_seqlens one entry short) shows the sanitizer is live.

CPU only. Needs the objects of a previous build (`__graft_entry__.build()` or
`python -m causal_flashattention_amd.build`); the device code is not instrumented."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build")
OUT = os.path.join(BUILD, "asan")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
RUNTIME = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
KERNEL_OBJECTS = sorted(o for o in glob.glob(os.path.join(BUILD, "*.o")) if not o.endswith("cfa_api.cpp.o"))
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and RUNTIME and len(KERNEL_OBJECTS) >= 7),
                                reason="needs hipcc, the clang ASan runtime and the objects of a previous build")


@pytest.fixture(scope="module")
def asan_lib():
    os.makedirs(OUT, exist_ok=True)
    obj = os.path.join(OUT, "cfa_api.cpp.o")
    lib = os.path.join(OUT, "libcfa_asan.so")
    src = os.path.join(ROOT, "causal_flashattention_amd", "csrc", "cfa_api.cpp")
    common = ["--offload-arch=gfx950", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
              "-I", os.path.join(ROOT, "causal_flashattention_amd", "csrc")]
    r = subprocess.run([HIPCC, *common, "-O1", "-g", *SANITIZE, "-x", "hip", "-c", src, "-o", obj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SANITIZE[:2], "-shared-libasan",
                        "-o", lib, obj, *KERNEL_OBJECTS], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return lib


def _run(lib, code):
    env = dict(os.environ, LD_PRELOAD=RUNTIME[-1], ASAN_OPTIONS="detect_leaks=0")
    prog = ("import sys; sys.path.insert(0, %r)\n" % ROOT +
            "import causal_flashattention_amd._lib as L\n" +
            "L.LIB_PATH = %r\n" % lib + code)
    return subprocess.run([sys.executable, "-c", prog], capture_output=True, text=True, env=env, cwd=ROOT,
                          timeout=600)


def test_abi_and_binding_checks_run_clean_under_asan(asan_lib):
    r = _run(asan_lib, "import pytest\nsys.exit(pytest.main(['-q', '-x', '-m', 'not gpu', '-p', "
                       "'no:cacheprovider', 'tests/test_abi.py', 'tests/test_binding_checks.py']))\n")
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "ERROR: AddressSanitizer" not in r.stderr


def test_asan_reports_a_planted_host_overread(asan_lib):
    # n_docs = 3 but the host mirror holds only 3 entries: validating it reads one past its end
    r = _run(asan_lib, "import ctypes, numpy as np\n"
                       "lib = L.lib()\n"
                       "buf = np.array([0, 40, 100], dtype=np.int32)\n"
                       "p = ctypes.c_void_p(16 << 20)\n"
                       "lib.attn_fwd(p, p, p, p, p, p, buf.ctypes.data, 3, 100, 0, 4, 2, 128, 0.088, 1, 1, None, p,"
                       " 1 << 30, None)\n")
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]

"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

libs3r.so is rebuilt with the sanitizers on its host code only (each -fsanitize= behind -Xarch_host; the
gfx950 code is built as usual), loaded by a child Python with the ASan runtime preloaded, and driven through
every host-logic test of test_library_cpu.py: the argument checks, workspace sizes, exports and the no-GPU
error path.  Any sanitizer report fails the test.
"""
import os
import subprocess
import sys

from stochastic_rounding_quantization_amd import build

ROOT = build.ROOT

RUNNER = r"""
import inspect, sys
sys.path.insert(0, {root!r})
from stochastic_rounding_quantization_amd import s3r
s3r.LIB_PATH = {lib!r}
import tests.test_library_cpu as t
L = s3r.lib()
skip = ("test_gemm_m0_written_only_by_its_dma_assembly", "test_product_path_does_not_import_oracle")
for n in sorted(x for x in dir(t) if x.startswith("test_") and x not in skip):
    f = getattr(t, n)
    f(L) if "L" in inspect.signature(f).parameters else f()
    print("ok", n, flush=True)
"""


def test_c_abi_host_code_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "libs3r_sanitized.so")
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-O3", "-Wall", "-Wno-unused-function")]
    san = ["-O1", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-shared-libsan"]
    srcs = [os.path.join(build.CSRC, s) for s in build.SOURCES]
    res = subprocess.run([build.hipcc(), *flags, *san, "-I", os.path.join(ROOT, "include"), *srcs, "-o", lib],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    clang = os.path.join(os.path.dirname(build.hipcc()), "..", "llvm", "bin", "clang")
    rt = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    assert os.path.exists(rt), rt
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([sys.executable, "-c", RUNNER.format(root=ROOT, lib=lib)], capture_output=True, text=True,
                         env=env, cwd=str(tmp_path), timeout=600)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert out.count("ok test_") >= 8, out[-2000:]

"""The host-side checks of tests/test_abi_host.py against a build of the
library whose host code is instrumented with AddressSanitizer.

Every source is compiled with ``-Xarch_host -fsanitize=address`` (host code
only: the argument validation, workspace carving, launch planning and error
reporting of the C ABI; the GPU kernels are built as usual), linked against
the shared ASan runtime, and loaded into a fresh Python process with that
runtime preloaded.  The host tests then run there: an out-of-bounds access or
use-after-free in the host layer aborts the process.  CPU only (no HIP call
is made: every case fails validation first); skipped when hipcc or the ASan
runtime is not installed.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "head_latent_attention_fwd_amd")

RUNNER = r"""
import importlib.util, sys
sys.path.insert(0, sys.argv[1])
import head_latent_attention_fwd_amd as mla
assert mla.__file__.startswith(sys.argv[1]), mla.__file__
spec = importlib.util.spec_from_file_location("host_tests", sys.argv[2])
t = importlib.util.module_from_spec(spec)
spec.loader.exec_module(t)
n = 0
for name in sorted(dir(t)):
    if name.startswith("test_"):
        getattr(t, name)()
        n += 1
print("ran", n, "host tests")
"""


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_host_layer_under_address_sanitizer(tmp_path):
    sys.path.insert(0, ROOT)
    from head_latent_attention_fwd_amd import build as b
    rt = _asan_runtime()
    if shutil.which(b.HIPCC) is None and not os.path.exists(b.HIPCC) or rt is None:
        pytest.skip("hipcc or the ASan runtime is not installed")
    flags = [f for f in b.FLAGS if f != "-O3"] + ["-O1", "-g", "-Xarch_host", "-fsanitize=address",
                                                  "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([b.HIPCC, *flags, "-I", b.CSRC, "-I", os.path.join(ROOT, "include"), "-c", src,
                            "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, f"hipcc failed for {src}:\n{r.stderr[-3000:]}"
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, b.sources()))
    pkg = tmp_path / "pkg" / "head_latent_attention_fwd_amd"
    pkg.mkdir(parents=True)
    for f in glob.glob(os.path.join(PKG, "*.py")):
        shutil.copy(f, pkg)
    lib = str(pkg / "libmla.so")
    # host link with the compiler driver (the objects carry their device code)
    clang = os.path.join(os.path.dirname(os.path.realpath(b.HIPCC)), "..", "lib", "llvm", "bin", "clang++")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang++"
    r = subprocess.run([clang, "-shared", "-fPIC", "-fsanitize=address", "-shared-libasan", "-o", lib, *objs,
                        "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_" in nm, "the library is not instrumented"
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([sys.executable, "-c", RUNNER, str(tmp_path / "pkg"),
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, f"host tests under ASan failed:\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
    assert "ran" in r.stdout and "host tests" in r.stdout, r.stdout

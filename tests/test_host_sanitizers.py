"""Host AddressSanitizer + UndefinedBehaviorSanitizer over the C ABI and the
oracle (CPU only; skipped where a GPU is visible).

The HIP library is rebuilt from its own sources with its host code
instrumented (the sanitizer flags apply to the host pass only; device code is
built as usual and never runs here), the C oracle is rebuilt with the same
clang sanitizer runtime, and the host tests of the boundary (every validation
and error path, with fake device addresses), the binding's checks, the golden
fixture and the oracle pins run against them in a child process that preloads
that runtime. Any sanitizer report fails the test.
"""
import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from rmsnorm_train_fwd_amd import build as libbuild  # noqa: E402

LLVM = "/opt/rocm/llvm"
HIPCC = libbuild.HIPCC
RUNTIME = sorted(glob.glob(f"{LLVM}/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
TESTS = ["tests/test_abi_host.py", "tests/test_abi_fuzz.py", "tests/test_binding_checks.py",
         "tests/test_golden.py", "tests/test_oracle_pins.py"]


def _gpu_visible() -> bool:
    import torch
    return torch.cuda.device_count() > 0


pytestmark = pytest.mark.skipif(
    not RUNTIME or not os.path.exists(HIPCC) or _gpu_visible(),
    reason="needs hipcc and clang's ASan runtime, and runs on a host without a GPU only")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    if r.returncode != 0:
        raise AssertionError(f"{' '.join(cmd[:3])} ... failed:\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}")
    return r


def _build_library(out_dir: str) -> str:
    flags = [f for f in libbuild.FLAGS if f != "-O3"] + ["-O1", "-g"] + HOST_SAN

    def compile_one(src):
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *flags]
        if src.endswith(".cpp"):
            cmd += ["-x", "hip"]
        _run(cmd + ["-c", os.path.join(libbuild.CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(len(libbuild.SOURCES)) as ex:
        objs = list(ex.map(compile_one, libbuild.SOURCES))
    pkg = os.path.join(out_dir, "pkg", "rmsnorm_train_fwd_amd")
    os.makedirs(pkg)
    shutil.copy(os.path.join(libbuild.PKG, "__init__.py"), pkg)
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libasan", *HOST_SAN,
          "-o", os.path.join(pkg, "librmsnorm_train.so"), *objs])
    return os.path.dirname(pkg)


def _build_oracle(out_dir: str) -> str:
    lib = os.path.join(out_dir, "liboracle_san.so")
    src = os.path.join(ROOT, "oracle", "rmsn_oracle.c")
    _run([f"{LLVM}/bin/clang", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-frounding-math", "-fsanitize=address", "-fsanitize=undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-shared-libasan",
          "-o", lib, src, "-lm"])
    return lib


def test_boundary_and_oracle_under_asan_and_ubsan(tmp_path):
    out = str(tmp_path)
    with ThreadPoolExecutor(2) as ex:
        f_lib, f_orc = ex.submit(_build_library, out), ex.submit(_build_oracle, out)
        pkg_root, oracle_lib = f_lib.result(), f_orc.result()
    logs = os.path.join(out, "san")
    env = dict(os.environ,
               LD_PRELOAD=RUNTIME[-1],
               ASAN_OPTIONS=f"detect_leaks=0:abort_on_error=0:log_path={logs}",
               UBSAN_OPTIONS=f"print_stacktrace=1:log_path={logs}",
               RMSN_ORACLE_LIB=oracle_lib)
    # The instrumented package is imported first, so the tests' own
    # `import rmsnorm_train_fwd_amd` finds it already loaded.
    code = (f"import sys; sys.path.insert(0, {pkg_root!r}); import rmsnorm_train_fwd_amd as R; "
            f"assert R.LIB_PATH.startswith({pkg_root!r}), R.LIB_PATH; import pytest; "
            f"sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', *{TESTS!r}]))")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    reports = sorted(glob.glob(logs + "*"))
    text = "".join(open(p).read()[:4000] for p in reports)
    assert not reports, f"sanitizer reports:\n{text}"
    assert r.returncode == 0, f"tests failed under the sanitizers:\n{r.stdout[-4000:]}{r.stderr[-2000:]}"
    assert " passed" in r.stdout

"""CPU-only sanitizer build of libprhs.so and a run of the host-side ABI tests
against it.

The host code of every source (argument validation, workspace layout, launch
set-up) is compiled with AddressSanitizer and UndefinedBehaviorSanitizer; the
gfx950 device code is compiled as usual (the sanitizers apply to the host pass
only). The library goes to _build/asan/libprhs.so and is loaded, with the
sanitizer runtime preloaded, by a separate Python process that runs
tests/test_abi_host.py, which exercises every error path without a GPU.

Usage: python -m sparse_top_kv_head_amd.sanitize   (exit status of the tests)
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

from sparse_top_kv_head_amd import build as B

OUT = os.path.join(B.BUILD, "asan")
LIB = os.path.join(OUT, "libprhs.so")
# each sanitizer flag applies to the host pass only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def runtime() -> str:
    """The AddressSanitizer runtime of the compiler that built the library (it
    carries the UndefinedBehaviorSanitizer handlers too)."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return hits[-1]


def _compile(src):
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    cmd = [B.hipcc(), *B.HIPCC_FLAGS, *HOST_SAN, "-c", os.path.join(B.CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitizer compile failed: {src}\n{r.stderr}")
    return obj


def build_sanitized(jobs: int | None = None) -> str:
    os.makedirs(OUT, exist_ok=True)
    jobs = jobs or min(len(B.SOURCES), os.cpu_count() or 1)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, B.SOURCES))
    cmd = [B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-o", LIB, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitizer link failed\n{r.stderr}")
    return LIB


def _env():
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": runtime(),
        "PRHS_LIB": LIB,
        # Python and the libraries it loads are not instrumented: only report
        # errors found in the instrumented code, and no leaks at exit
        "ASAN_OPTIONS": "detect_leaks=0:alloc_dealloc_mismatch=0:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    return env


def loaded_objects(timeout: int = 300) -> list:
    """The shared objects a child process with the sanitizer environment maps
    once it has loaded the library (to check which build it runs)."""
    code = ("from sparse_top_kv_head_amd import prhs as P; P.lib(); "
            "print('\\n'.join(sorted({l.split()[-1] for l in open('/proc/self/maps') "
            "if l.rstrip().endswith('.so')})))")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=_env(),
                       cwd=B.ROOT, timeout=timeout)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized load failed\n{r.stderr[-4000:]}")
    return r.stdout.split()


def run_host_tests(timeout: int = 600) -> subprocess.CompletedProcess:
    """tests/test_abi_host.py in a child process on the sanitized library."""
    env = _env()
    cmd = [sys.executable, "-m", "pytest", os.path.join(B.ROOT, "tests", "test_abi_host.py"), "-q",
           "-p", "no:cacheprovider"]
    return subprocess.run(cmd, capture_output=True, text=True, env=env, cwd=B.ROOT, timeout=timeout)


if __name__ == "__main__":
    print(build_sanitized(), flush=True)
    res = run_host_tests()
    print(res.stdout[-4000:])
    print(res.stderr[-4000:], file=sys.stderr)
    sys.exit(res.returncode)

"""Build libprhs.so (HIP kernels for gfx950 + the C ABI) in the package directory.

Usage: python -m sparse_top_kv_head_amd.build [--jobs N] [--verbose] [--checked]
       python -m sparse_top_kv_head_amd.build --resources OUT.md
       python -m sparse_top_kv_head_amd.build --sanitize
Cross-compiles without a GPU; always rebuilds. --checked builds
libprhs_checked.so, whose kernels check input contracts and invariants and
whose calls report a broken one as an error. --resources writes the
compiler's per-kernel register, LDS and occupancy report instead. --sanitize
builds the host code with address and undefined-behaviour checks into
_build/asan and runs the host-side ABI tests on it (sanitize.py).
"""

from __future__ import annotations

import argparse
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libprhs.so")

SOURCES = ["score.hip", "select.hip", "cis.hip", "decode.hip", "dense.hip", "append.hip", "probe.hip",
           "prhs_abi.cpp"]
# The checked build: kernels record broken input contracts and invariants in
# device check words that every call reads back (an error, never a trap).
CHECKED_LIB = os.path.join(PKG, "libprhs_checked.so")
CHECKED_FLAGS = ["-DPRHS_DEVICE_CHECKS"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Wno-unused-result", "-Wno-unknown-pragmas",
    # keep the compiler from emitting packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; ROCm is required to build libprhs.so")
    return exe


def _compile(src, verbose, out_dir=BUILD, extra=()):
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
    if r.stderr.strip() and verbose:
        print(r.stderr, file=sys.stderr)
    return obj


def build(jobs: int | None = None, verbose: bool = False, checked: bool = False) -> str:
    """libprhs.so, or with `checked` the device-checked libprhs_checked.so."""
    out_dir = os.path.join(BUILD, "checked") if checked else BUILD
    lib = CHECKED_LIB if checked else LIB
    extra = CHECKED_FLAGS if checked else ()
    os.makedirs(out_dir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, out_dir, extra), SOURCES))
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


def _demangle_short(name):
    """prhs::(anonymous namespace)::kernel<args> from an Itanium-mangled name."""
    exe = shutil.which("llvm-cxxfilt") or shutil.which("c++filt")
    if exe is None:
        return name
    out = subprocess.run([exe, name], capture_output=True, text=True).stdout.strip() or name
    out = out.replace("prhs::(anonymous namespace)::", "").replace("void ", "")
    return out.split("(")[0]


def resources(out_md: str) -> None:
    """Compile every kernel source with the compiler's resource report and
    tabulate, per kernel, VGPRs, AGPRs, SGPRs, scratch, LDS and the occupancy
    limit (waves per SIMD) the compiler derives from them."""
    import re
    rows = []
    for src in SOURCES:
        if not src.endswith(".hip"):
            continue
        cmd = [hipcc(), *HIPCC_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c",
               os.path.join(CSRC, src), "-o", os.devnull]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {src}\n{r.stderr}")
        cur = None
        for line in r.stderr.splitlines():
            f = re.search(r"remark: Function Name: (\S+)", line)
            if f:
                cur = {"kernel": _demangle_short(f.group(1)), "src": src}
                rows.append(cur)
                continue
            m = re.search(r"remark:\s+(.*?): (.*?) \[-Rpass-analysis", line)
            if m and cur is not None:
                cur[m.group(1).strip()] = m.group(2).strip()
    cols = [("VGPRs", "VGPRs"), ("AGPRs", "AGPRs"), ("TotalSGPRs", "SGPRs"),
            ("ScratchSize [bytes/lane]", "scratch B/lane"), ("LDS Size [bytes/block]", "LDS B/WG"),
            ("Occupancy [waves/SIMD]", "waves/SIMD")]
    lines = ["# Kernel resources and occupancy limits (gfx950)\n",
             "Command (repository root, no GPU needed):\n", "```",
             "python -m sparse_top_kv_head_amd.build --resources profiles/kernel_resources.md", "```\n",
             "From the compiler's kernel-resource-usage report for the flags the library is built "
             "with. waves/SIMD is the occupancy limit those resources allow (registers, LDS, "
             "workgroup size); the achieved occupancy of the benchmarked kernels is in the SQ "
             "counter profiles.\n",
             "| kernel | source | " + " | ".join(c[1] for c in cols) + " |",
             "|---|---|" + "---|" * len(cols)]
    for r in rows:
        if not r["kernel"] or "kernel" not in r["kernel"]:
            continue
        lines.append(f"| `{r['kernel'][:70]}` | {r['src']} | " +
                     " | ".join(r.get(c[0], "") for c in cols) + " |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resources", metavar="OUT_MD", default=None,
                    help="write the per-kernel resource and occupancy table instead of building")
    ap.add_argument("--checked", action="store_true",
                    help="build the device-checked library libprhs_checked.so")
    ap.add_argument("--sanitize", action="store_true",
                    help="sanitizer build of the host code, then the host-side ABI tests on it")
    a = ap.parse_args()
    if a.sanitize:
        from sparse_top_kv_head_amd import sanitize
        print(sanitize.build_sanitized(a.jobs), flush=True)
        res = sanitize.run_host_tests()
        print(res.stdout[-4000:], res.stderr[-4000:])
        sys.exit(res.returncode)
    if a.resources:
        resources(a.resources)
    else:
        print(build(a.jobs, a.verbose, a.checked))

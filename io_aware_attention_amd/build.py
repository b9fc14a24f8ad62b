"""Build libfa355.so (gfx950) in-tree with hipcc.

    python -m io_aware_attention_amd.build [--jobs N] [--verbose] [--lds-poison]

Each shard of kernel variants compiles to its own object in parallel; the host
C-ABI file links with them into io_aware_attention_amd/libfa355.so.  With
--lds-poison the same sources build, with FA355_LDS_POISON=1, into
libfa355_lds_poison.so: a debug library whose kernels fill every LDS stage with
NaN bytes before refilling it and do not overlap staging with compute (its output
must equal the normal library's bit for bit).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libfa355.so")
LDS_POISON_LIB_PATH = os.path.join(PKG, "libfa355_lds_poison.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed fp32 VALU ops are turned off: the kernels are written as scalar fp32 and
# must not be lowered to v_pk_{add,mul,fma}_f32.
COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Wno-unused-command-line-argument",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC]


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def _compile(src: str, verbose: bool, out_dir: str, defines: list[str]) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *defines, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    t0 = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{msgs}")
    if verbose:
        print(f"  {os.path.basename(src)}: {time.time() - t0:.1f}s", flush=True)
        if msgs.strip():
            print(msgs, flush=True)
    return obj


def build(jobs: int | None = None, verbose: bool = False, lds_poison: bool = False) -> str:
    """Compile every kernel shard and the host library; returns the .so path."""
    out_dir = os.path.join(BUILD_DIR, "lds_poison") if lds_poison else BUILD_DIR
    lib_path = LDS_POISON_LIB_PATH if lds_poison else LIB_PATH
    defines = ["-DFA355_LDS_POISON=1"] if lds_poison else []
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), os.cpu_count() or 1)
    t0 = time.time()
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, out_dir, defines), srcs))
    tmp = lib_path + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs,
           "-Wl,--no-undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path} in {time.time() - t0:.1f}s", flush=True)
    return lib_path


EXAMPLE_SRC = os.path.join(PKG, "example", "fa355_example.c")
EXAMPLE_BIN = os.path.join(PKG, "fa355_example")


def build_example(verbose: bool = False) -> str:
    """Compile the C client of the library (HIP runtime + C ABI, no Python) next to
    libfa355.so, which it finds through an $ORIGIN run path."""
    clang = os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "bin", "clang")
    rocm = os.path.dirname(os.path.dirname(HIPCC))
    cmd = [clang, "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
           "-I", INCLUDE, EXAMPLE_SRC, "-o", EXAMPLE_BIN + ".tmp", "-L", PKG, "-lfa355",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm", "-Wl,-rpath,$ORIGIN"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("example build failed:\n" + r.stdout + r.stderr)
    os.replace(EXAMPLE_BIN + ".tmp", EXAMPLE_BIN)
    if verbose:
        print(f"built {EXAMPLE_BIN}", flush=True)
    return EXAMPLE_BIN


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--lds-poison", action="store_true")
    a = ap.parse_args(argv)
    build(a.jobs, a.verbose, a.lds_poison)
    if not a.lds_poison:
        build_example(a.verbose)
    return 0


if __name__ == "__main__":
    sys.exit(main())

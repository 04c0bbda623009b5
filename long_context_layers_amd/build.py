"""Build liblightning_attn.so (gfx950) in-tree with hipcc.

    python -m long_context_layers_amd.build

Each HIP source is compiled to an object (in parallel), then linked into
``long_context_layers_amd/lib/liblightning_attn.so``; the benchmark's
ceiling probes go into ``lib/liblapeak.so``, and the plain-C test program
``tests/c/la_c_program.c`` (gcc, C99, HIP runtime C API) into
``tests/c/la_c_program``.  Always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIB_DIR, "liblightning_attn.so")

SOURCES = ["la_api.hip", "prefill_bf16.hip", "prefill_f32.hip", "decode.hip", "layer_ops.hip",
           "cp.hip"]
PEAK_SOURCES = ["peak_probe.hip"]
PEAK_LIB = os.path.join(LIB_DIR, "liblapeak.so")
C_PROGRAM_SRC = os.path.join(ROOT, "tests", "c", "la_c_program.c")
C_PROGRAM = os.path.join(ROOT, "tests", "c", "la_c_program")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMPILE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # packed fp32 vector ops stay off in device code (see the design notes)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMPILE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(ln for ln in r.stderr.splitlines()
                     if "packed-fp32-ops" not in ln and ln.strip())
    if warn:
        print(f"[build] {src}: {warn}", file=sys.stderr)
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"[build] {lib}")


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    srcs = SOURCES + PEAK_SOURCES
    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB, verbose)
    _link(objs[len(SOURCES):], PEAK_LIB, verbose)
    _build_c_program(verbose)
    return LIB


def _build_c_program(verbose: bool) -> None:
    """The C ABI from a plain C99 program (gcc, HIP runtime C API)."""
    gcc = shutil.which("gcc")
    if gcc is None:
        raise RuntimeError("gcc not found: needed for tests/c/la_c_program")
    tmp = C_PROGRAM + ".tmp%d" % os.getpid()
    cmd = [gcc, "-std=c99", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", INCLUDE, C_PROGRAM_SRC, "-o", tmp,
           "-L", LIB_DIR, "-llightning_attn", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../long_context_layers_amd/lib",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C program build failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, C_PROGRAM)
    if verbose:
        print(f"[build] {C_PROGRAM}")


if __name__ == "__main__":
    build()

"""Build ``libsgemm_rm.so`` in-tree with hipcc for gfx950.

Every HIP source is compiled with ``-Xclang -target-feature -Xclang
-packed-fp32-ops`` so that the compiler never emits packed FP32 VALU
instructions, and without fast-math so that FP32 rounding is IEEE.

A second library, ``libsgemm_rm_poison.so``, is the same sources with
``-DSGEMM_RM_POISON_LDS=1``: every kernel fills its LDS with NaN before
use, so that the GPU tests that load it catch a read of unwritten LDS.
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsgemm_rm.so")
POISON_BUILD_DIR = os.path.join(HERE, "_build_poison")
POISON_LIB = os.path.join(HERE, "libsgemm_rm_poison.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["sgemm_rm.hip", "k_naive.hip", "k_lds_tiled.hip", "k_regblock.hip", "k_mfma_nn.hip", "k_mfma_nt.hip",
           "k_mfma_tn.hip", "k_mfma_tt.hip"]
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(job) -> str:
    src, out_dir, extra = job
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *HIP_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{proc.stdout}\n{proc.stderr}")
    return obj


PROBE_DIR = os.path.join(ROOT, "tests", "probes")
PROBES = ["mfma_layout_probe.hip", "lds_bank_probe.hip"]


def build_probes() -> list:
    """Compile the hardware probes the tests run (tests/probes/*.hip -> tests/probes/bin/)."""
    out_dir = os.path.join(PROBE_DIR, "bin")
    os.makedirs(out_dir, exist_ok=True)
    built = []
    for src in PROBES:
        exe = os.path.join(out_dir, os.path.splitext(src)[0])
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", os.path.join(PROBE_DIR, src), "-o", exe]
        proc = subprocess.run(cmd, capture_output=True, text=True)
        if proc.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{proc.stdout}\n{proc.stderr}")
        built.append(exe)
    built.append(build_c_client(out_dir))
    return built


def build_c_client(out_dir: str) -> str:
    """Compile the plain C client of the library (tests/c_client/sgemm_client.c) with gcc,
    linked against the in-tree libsgemm_rm.so (found through a relative rpath)."""
    src = os.path.join(ROOT, "tests", "c_client", "sgemm_client.c")
    exe = os.path.join(out_dir, "sgemm_client")
    rel = os.path.relpath(HERE, out_dir)
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           f"-I{INCLUDE}", src, "-o", exe, f"-L{HERE}", "-l:libsgemm_rm.so", "-L/opt/rocm/lib", "-lamdhip64",
           f"-Wl,-rpath,$ORIGIN/{rel}", "-Wl,-rpath,/opt/rocm/lib"]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"gcc failed on {src}:\n{proc.stdout}\n{proc.stderr}")
    return exe


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    # -Bsymbolic: the library's calls between its own entry points stay inside it, also
    # when the production and the poisoned library are loaded in one process
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-Bsymbolic", "-o", tmp, *objs]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"link failed:\n{proc.stdout}\n{proc.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False, poison: bool = True) -> str:
    """Compile every kernel source and link the shared library (and, with `poison`, the
    LDS-poisoning debug library beside it); returns the production library's path."""
    jobs = [(src, BUILD_DIR, []) for src in SOURCES]
    os.makedirs(BUILD_DIR, exist_ok=True)
    if poison:
        os.makedirs(POISON_BUILD_DIR, exist_ok=True)
        jobs += [(src, POISON_BUILD_DIR, ["-DSGEMM_RM_POISON_LDS=1"]) for src in SOURCES]
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(_compile, jobs))
    _link(objs[:len(SOURCES)], LIB)
    if poison:
        _link(objs[len(SOURCES):], POISON_LIB)
    if verbose:
        print(f"built {LIB}" + (f" and {POISON_LIB}" if poison else ""))
    return LIB


if __name__ == "__main__":
    build(verbose=True)

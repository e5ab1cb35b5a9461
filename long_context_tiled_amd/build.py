"""Build libskipattn.so in-tree with hipcc for gfx950.

    python -m long_context_tiled_amd.build        # or build() from Python

Every HIP source under csrc/ is compiled for gfx950 only and linked into
long_context_tiled_amd/libskipattn.so. The prefill kernel's hand-scheduled
tile steps (csrc/prefill_steps.inc) are rewritten from
csrc/gen_prefill_steps.py first.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libskipattn.so")
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.hip", "prefill.hip", "decode.hip", "kvq4.hip", "kvq2.hip", "kvq_quant.hip", "fp8.hip"]
HEADERS = ["common.hpp", "launch.hpp", "kvq_common.hpp", "lane_max.hpp", "sas.hpp",
           "prefill_steps.inc"]

# Packed fp32 VALU ops are disabled: hipcc otherwise forms them from plain
# float code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(HERE, "..", "include")]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def generate() -> None:
    """Rewrite csrc/prefill_steps.inc from its generator."""
    r = subprocess.run([sys.executable, os.path.join(CSRC, "gen_prefill_steps.py")],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gen_prefill_steps.py failed:\n{r.stdout}\n{r.stderr}")


def build(verbose: bool = False) -> str:
    generate()
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

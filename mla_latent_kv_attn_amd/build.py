"""Build the HIP library (gfx950) in-tree: mla_latent_kv_attn_amd/libmla_amd.so.

    python -m mla_latent_kv_attn_amd.build [--jobs N] [--save-temps]

Every source under csrc/ is compiled with hipcc for gfx950 and linked into one shared library
exporting the C ABI of include/mla.h.  Packed fp32 instructions are disabled for all device code
(-Xclang -target-feature -Xclang -packed-fp32-ops).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmla_amd.so")
ARCH = "gfx950"

SOURCES = ["mla_abi.hip", "decode_generic.hip", "absorb_uv_mfma.hip", "decode_partial_mfma.hip", "decode_step.hip",
           "decode_partial_small.hip", "cache_append.hip",
           "mha_decode.hip", "proj.hip"]

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-lambda-capture",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Per-source extra flags.  The small-batch partial kernel keeps its output accumulator in VGPRs
# (it needs about 220 registers in all): with AGPR accumulators the compiler copies the whole
# accumulator between register classes on every tile around the conditional rescale.
EXTRA_FLAGS = {"decode_partial_small.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the MLA library needs ROCm's hipcc to build")


# Kernels whose DMA pipeline counts outstanding vector-memory operations (s_waitcnt vmcnt): a
# spill to scratch memory inside them would add scratch loads/stores to that count, so they must
# use no scratch (SGPR spills into VGPR lanes are fine).
NO_SCRATCH_KERNELS = ("k_partial_mfma", "k_partial_small", "k_step_b1")


def _check_spills(src: str, remarks: str) -> None:
    """Parse -Rpass-analysis=kernel-resource-usage remarks; fail if a guarded kernel uses scratch."""
    current = None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            current = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and current and any(k in current for k in NO_SCRATCH_KERNELS) and int(m.group(1)) > 0:
            raise RuntimeError(f"{src}: kernel {current} uses {m.group(1)} bytes/lane of scratch; "
                               "the tile pipeline requires a register allocation without spills to memory")


def _compile(src: str, save_temps: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *CFLAGS, *EXTRA_FLAGS.get(src, []), "-Rpass-analysis=kernel-resource-usage", "-c",
           os.path.join(CSRC, src), "-o", obj]
    if save_temps:
        cmd += ["-save-temps=obj"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    text = r.stdout + r.stderr
    out = "\n".join(l for l in text.splitlines()
                    if "packed-fp32-ops" not in l and "kernel-resource-usage" not in l and "remark:" not in l
                    and l.strip() and not l.lstrip().startswith(("|", "^")))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    _check_spills(src, text)
    return obj


def build(jobs: int = 0, save_temps: bool = False) -> str:
    """Compile every source and link libmla_amd.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, save_temps), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--save-temps", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.save_temps))


if __name__ == "__main__":
    main()

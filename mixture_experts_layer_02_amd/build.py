"""Build libmoe.so (all HIP sources under csrc/) for gfx950 with hipcc.

Usage: python -m mixture_experts_layer_02_amd.build [-q] [--no-light-dma]
       (or __graft_entry__.build())
Objects go to _build/ at the repository root; the library is written next to
this file so that it travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmoe.so")
OBJ = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# packed-fp32-ops off: the v_pk_*_f32 forms are not trusted on these parts.
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
SOURCES = ["api.hip", "route.hip", "permute.hip", "ffn.hip", "hold.hip", "fp8.hip"]
# ffn.hip: the GEMMs' dynamic tile claims are one lane's atomic whose result is
# used a k-tile later; LLVM's atomic optimizer would rewrite them into a form
# that waits for the result at once (and for every load in flight before it).
EXTRA = {"ffn.hip": ["-Xarch_device", "-mllvm=-amdgpu-atomic-optimizer-strategy=None"]}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + out)
    return out


# Sources holding the LDS-DMA GEMM kernels: their device assembly is checked
# for the SGPR wait-state hazard of the inline-asm DMA (hazard_check.py).
CHECKED = ["ffn.hip", "fp8.hip"]


def _compile(light: bool, verbose: bool):
    """Objects of every source and device assembly of the checked ones."""
    defs = [] if light else ["-DMOE_LIGHT_DMA=0"]
    objs, asms, cmds = [], [], []
    for src in SOURCES:
        obj = os.path.join(OBJ, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, *defs, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    for src in CHECKED:
        asm = os.path.join(OBJ, src.replace(".hip", ".gfx950.s"))
        asms.append(asm)
        cmds.append([HIPCC, *FLAGS, *defs, *EXTRA.get(src, []), "--cuda-device-only", "-S",
                     os.path.join(CSRC, src), "-o", asm])
    with cf.ThreadPoolExecutor(min(len(cmds), max(1, os.cpu_count() or 1))) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    return objs, asms


def _check(asms):
    """(LDS DMAs, hazards, report) over the given device assembly files."""
    sys.path.insert(0, HERE)
    try:
        import hazard_check
    finally:
        sys.path.pop(0)
    import io
    report = io.StringIO()
    n_dma = n_bad = 0
    for asm in asms:
        t, b = hazard_check.check(asm, report)
        n_dma += t
        n_bad += b
    return n_dma, n_bad, report.getvalue()


def build(verbose: bool = False, light: bool = True) -> str:
    """Compile and link libmoe.so. The steady-loop DMAs carry one wait state
    (light) unless the generated code has a VALU write of a DMA's SGPR within
    five wait states; then everything is compiled again with five everywhere."""
    os.makedirs(OBJ, exist_ok=True)
    objs, asms = _compile(light, verbose)
    n_dma, n_bad, report = _check(asms)
    if n_bad and light:
        print(f"warning: {n_bad} of {n_dma} LDS DMAs have a VALU write of an SGPR operand within five wait "
              "states; compiling again with five wait states before every DMA (slower steady loop)\n" + report,
              file=sys.stderr)
        light = False
        objs, asms = _compile(light, verbose)
        n_dma, n_bad, report = _check(asms)
    if n_bad:
        raise RuntimeError(f"LDS-DMA wait-state hazards in the generated code ({n_bad} of {n_dma}):\n" + report)
    if verbose:
        print(f"hazard check: {n_dma} LDS-DMA instructions, none within 5 wait states of a VALU write of its SGPRs"
              + ("" if light else " (five wait states before every DMA)"))
    tmp = OUT + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv, light="--no-light-dma" not in sys.argv)

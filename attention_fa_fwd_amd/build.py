"""Compile the HIP sources of this package into libfa.so for gfx950 (in-tree).

Usage: python -m attention_fa_fwd_amd.build   (or call build()).
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libfa.so")
# the trace build: the same sources with per-tile visit counters (include/fa_trace.h)
TRACE_LIB = os.path.join(PKG, "libfa_trace.so")
TRACE_DEFINES = ("FA_TRACE_VISITS",)
SOURCES = ["fa_api.hip", "fa_fwd.hip", "fa_bwd.hip", "fa_bwd_kv.hip", "fa_bwd_kv_atomic.hip", "fa_decode.hip",
           "fa_layout.hip", "fa_large.hip"]
# sources whose MFMA results are kept in VGPRs (see common_flags)
VGPR_FORM_SOURCES = {s for s in os.environ.get("FA_VGPR_FORM", "fa_fwd.hip,fa_bwd.hip,fa_bwd_kv_atomic.hip,fa_decode.hip").split(",") if s}
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def common_flags(src: str = ""):
    flags = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"),
             # no packed-fp32 instructions in any generated code
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-result"]
    if src in VGPR_FORM_SOURCES:
        # MFMA results in VGPRs: these kernels read their accumulators with VALU
        # code, and the default placement shuttled them through AGPRs
        flags += ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]
    return flags


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln]
    return r.returncode, "\n".join(lines)


def check_no_spill_with_dma(asm_path: str) -> None:
    """Fail the build if a kernel that issues global_load_lds also uses scratch
    memory (register spills): in-flight LDS DMA and scratch reloads together give
    wrong values.  SGPR spills into VGPR lanes use no memory and are allowed."""
    text = open(asm_path).read()
    bodies = {}
    for m in re.finditer(r"^(_Z\w+):[^\n]*\n(.*?)^\s*s_endpgm", text, re.M | re.S):
        bodies[m.group(1)] = "global_load_lds" in m.group(2)
    bad = []
    meta = text[text.find("amdhsa.kernels:"):]
    for entry in re.split(r"\n  - \.", meta)[1:]:
        name = re.search(r"\.name:\s+(\S+)", entry)
        scratch = re.search(r"\.private_segment_fixed_size:\s+(\d+)", entry)
        if name and scratch and int(scratch.group(1)) > 0 and bodies.get(name.group(1), True):
            bad.append(f"{name.group(1)} ({scratch.group(1)} bytes of scratch per lane)")
    if bad:
        raise RuntimeError("kernels with LDS DMA must not use scratch: " + ", ".join(bad))


def build(verbose: bool = False, target: str = LIB, defines=()) -> str:
    """Compile every source and link libfa.so (or `target`); returns the library path."""
    build_dir = (os.path.join(PKG, "_build") if target == LIB
                 else os.path.join(os.path.dirname(target), "_build_" + os.path.basename(target)))
    os.makedirs(build_dir, exist_ok=True)
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc()] + common_flags(src) + [f"-D{d}" for d in defines] +
                    ["-c", os.path.join(CSRC, src), "-o", obj])
    asm_cmds = [[hipcc()] + common_flags(src) + [f"-D{d}" for d in defines] +
                ["--cuda-device-only", "-S", os.path.join(CSRC, src), "-o",
                 os.path.join(build_dir, src.replace(".hip", ".s"))] for src in SOURCES]
    with ThreadPoolExecutor(max_workers=2 * len(cmds)) as ex:
        results = list(ex.map(_run, cmds + asm_cmds))[:len(cmds)]
    for cmd, (rc, out) in zip(cmds, results):
        if verbose and out.strip():
            print(out)
        if rc != 0:
            raise RuntimeError(f"hipcc failed ({rc}) for {cmd[-3]}:\n{out}")
    for src in SOURCES:
        check_no_spill_with_dma(os.path.join(build_dir, src.replace(".hip", ".s")))
    tmp = target + ".tmp"
    rc, out = _run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs)
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{out}")
    os.replace(tmp, target)
    return target


def build_all(verbose: bool = False):
    """The product library and its trace build."""
    return build(verbose), build(verbose, TRACE_LIB, TRACE_DEFINES)


if __name__ == "__main__":
    print(build_all(verbose="-v" in sys.argv))

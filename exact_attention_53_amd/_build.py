"""Builds the HIP library libattn53.so in-tree with hipcc for gfx950.

Usage: python -m exact_attention_53_amd._build   (or __graft_entry__.build())
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libattn53.so")
BUILD_DIR = os.path.join(ROOT, "_build")

# Each backward launcher configuration (kernel, element type, head dims, mask) is one
# compilation of attn_bwd_inst.hip, so that they compile in parallel.
# Masks: 0 none, 1 causal, 2 causal + sliding window, 3 causal + ALiBi, 4 block-sparse map,
# 5 block-sparse map + causal, 6 key bias, 7 key bias + causal, 8 dropout, 9 dropout + causal
# (4-9 bf16 only).
INSTANCES = [(kind, elem, dqk, dv, mask) for kind in ("kv", "dq") for elem in ("bf16", "f16")
             for dqk, dv in ((64, 64), (128, 128), (192, 128)) for mask in range(10)
             if mask < 4 or elem == "bf16"]
# the key/value and dQ work of d = 64 in one launch (plain and causal masks)
INSTANCES += [("kvdq", elem, 64, 64, mask) for elem in ("bf16", "f16") for mask in (0, 1)]
INST_KIND = {"kv": 0, "dq": 1, "kvdq": 2}
MASK_NAMES = ("full", "causal", "window", "alibi", "bsp", "bsp_causal", "kbias", "kbias_causal", "drop", "drop_causal")
SOURCES = ["attn_fwd.hip", "attn_fwd_fp8.hip", "attn_bwd.hip", "attn_plan.hip", "attn_blocksparse.hip", "attn_bias.hip",
           "attn_dropout.hip", "attn_api.cpp"]

# -packed-fp32-ops: keep hipcc from forming packed fp32 VALU instructions.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I" + INCLUDE, "-I" + CSRC,
]


# MFMA results in VGPRs (the key/value kernel at d_qk <= 128, the dQ kernel at
# d_qk >= 128): the MFMAs of S and dP write VGPRs, which the softmax VALU work reads,
# instead of accumulation registers that each need a v_accvgpr_read first (64 per 64-key
# step per 32-row tile at d = 128); long-lived operands (the dK / dV accumulators, the dQ
# kernel's Q and dO fragments) then sit in the accumulation registers.  Measured per
# kernel: the d_qk = 192 key/value kernel is 10 % slower in this form (and two of its
# mask modes do not compile in it), so it keeps the default; at d = 64 both kernels fit
# in VGPRs without it.
KV_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
DQ_FLAGS = KV_FLAGS


def _extra_flags(kind: str, dqk: int, mask: int) -> list:
    if kind == "kv":
        return KV_FLAGS if dqk <= 128 else []
    return DQ_FLAGS if dqk >= 128 else []


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # The host pass warns that it does not know the packed-fp32 feature; that is harmless.
    out = "\n".join(l for l in r.stdout.splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + out)
    return out


def _includes(src: str, seen=None) -> set:
    """src and every local header it includes (quoted #include, searched next to the
    including file, then in include/), recursively."""
    import re
    seen = set() if seen is None else seen
    if src in seen or not os.path.exists(src):
        return seen
    seen.add(src)
    with open(src) as f:
        for name in re.findall(r'^\s*#\s*include\s+"([^"]+)"', f.read(), flags=re.M):
            for base in (os.path.dirname(src), INCLUDE, CSRC):
                cand = os.path.normpath(os.path.join(base, name))
                if os.path.exists(cand):
                    _includes(cand, seen)
                    break
    return seen


def _stale(obj: str, src: str) -> bool:
    """True unless obj is newer than its source, the headers it includes and this script."""
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(d) >= t for d in _includes(src) | {os.path.abspath(__file__)})


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compiles every source and links libattn53.so; returns its path.  incremental:
    skip objects newer than every source (a developer convenience; the default always
    compiles everything)."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        objs.append(obj)
        lang = [] if src.endswith(".hip") else ["-x", "hip"]
        cmds.append([hipcc, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
    for kind, elem, dqk, dv, mask in INSTANCES:
        obj = os.path.join(BUILD_DIR, f"attn_bwd_{kind}_{elem}_{dqk}_{dv}_{MASK_NAMES[mask]}.o")
        objs.append(obj)
        defs = [f"-DATTN_INST_DQ={INST_KIND[kind]}", f"-DATTN_INST_ELEM={elem}", f"-DATTN_INST_DQK={dqk}",
                f"-DATTN_INST_DV={dv}", f"-DATTN_INST_MASK={mask}"]
        extra = _extra_flags(kind, dqk, mask)
        cmds.append([hipcc, *FLAGS, *extra, *defs, "-c", os.path.join(CSRC, "attn_bwd_inst.hip"), "-o", obj])
    if incremental:
        cmds = [c for c in cmds if _stale(c[-1], c[-3])]
    cmds.sort(key=lambda c: "attn_bwd_inst.hip" not in c[-3])  # longest compilations first
    with cf.ThreadPoolExecutor(max_workers=max(1, min(len(cmds), os.cpu_count() or 8))) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = OUT + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    _check_kernel_stubs(tmp)
    os.replace(tmp, OUT)
    return OUT


def _check_kernel_stubs(path: str) -> None:
    """Every kernel launched from host code must have its host-side stub defined; a
    silently dropped instantiation would otherwise only fail when the library loads."""
    nm = shutil.which("nm") or "/usr/bin/nm"
    r = subprocess.run([nm, "-C", path], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    missing = [l.strip() for l in r.stdout.splitlines() if "__device_stub__" in l and l.strip().startswith("U ")]
    if missing:
        raise RuntimeError("build produced undefined kernel stubs:\n" + "\n".join(missing))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, incremental="--incremental" in sys.argv))

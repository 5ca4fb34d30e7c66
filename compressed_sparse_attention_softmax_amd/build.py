"""Builds libcsa.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m compressed_sparse_attention_softmax_amd.build

hipcc cross-compiles for gfx950 on a machine without a GPU.  Packed fp32
VALU ops are disabled (-packed-fp32-ops) for every HIP translation unit.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcsa.so")

SOURCES = ["compress.hip", "index_topk.hip", "attn.hip", "indexer_loss.hip", "dsa_gqa.hip", "abi.cpp", "timing.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
         "-Wno-unused-variable"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stderr or "").splitlines()
            if ln.strip() and "packed-fp32-ops" not in ln and "unknown target feature" not in ln]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    return obj


# Sources whose kernels issue MFMAs from inline asm (accumulators pinned to
# AGPRs); the compiler's hazard recognizer does not look inside those blocks.
ASM_MFMA_SOURCES = ["attn.hip"]
MFMA_LEAD_WAITS = 2        # VALU / v_accvgpr write of a source -> MFMA read
MFMA_TAIL_WAITS = 10       # MFMA result -> any read or write (4-pass XDL op on gfx950: 8)


def asm_mfma_blocks(text: str):
    """The instructions of every inline-asm block (between ;;#ASMSTART and
    ;;#ASMEND) of an assembly listing that holds an MFMA."""
    blocks, cur = [], None
    for ln in text.splitlines():
        t = ln.strip()
        if t.startswith(";;#ASMSTART"):
            cur = []
        elif t.startswith(";;#ASMEND"):
            if cur is not None and any(i.startswith("v_mfma") for i in cur):
                blocks.append(cur)
            cur = None
        elif cur is not None and t and not t.startswith(";"):
            cur.append(t)
    return blocks


def asm_mfma_block_ok(block) -> bool:
    """True when the block holds only MFMAs and s_nops, with at least
    MFMA_LEAD_WAITS wait states before its first MFMA and MFMA_TAIL_WAITS
    after its last (s_nop n gives n + 1 wait states)."""
    def waits(ins):
        return sum(int(i.split()[1], 0) + 1 for i in ins if i.startswith("s_nop"))
    if any(not (i.startswith("v_mfma") or i.startswith("s_nop")) for i in block):
        return False
    first = next(k for k, i in enumerate(block) if i.startswith("v_mfma"))
    last = max(k for k, i in enumerate(block) if i.startswith("v_mfma"))
    return waits(block[:first]) >= MFMA_LEAD_WAITS and waits(block[last + 1:]) >= MFMA_TAIL_WAITS


def check_asm_mfma(src: str) -> int:
    """Compiles `src` to gfx950 assembly and checks that every inline-asm
    block holding an MFMA is self-contained: at least MFMA_LEAD_WAITS wait
    states before its first MFMA and at least MFMA_TAIL_WAITS after its last
    one, inside the block.  Then no instruction the compiler places around
    the block (a copy, a spill, a loop-exit move of an accumulator) can touch
    its registers inside an MFMA's write latency.  Returns the number of
    blocks checked; raises on a violation."""
    asm_path = os.path.join(BUILD, os.path.splitext(src)[0] + ".s")
    cmd = [HIPCC] + FLAGS + ["-S", "--offload-device-only", os.path.join(CSRC, src), "-o", asm_path]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{res.stderr[-2000:]}")
    blocks = asm_mfma_blocks(open(asm_path).read())
    bad = [b for b in blocks if not asm_mfma_block_ok(b)]
    if bad:
        raise RuntimeError(f"{src}: inline-asm MFMA block without its own wait states:\n" + "\n".join(bad[0]))
    return len(blocks)


def build(verbose: bool = False, jobs: int = 4) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
        checked = list(ex.map(check_asm_mfma, ASM_MFMA_SOURCES))
    if verbose:
        print(f"inline-asm MFMA blocks checked: {dict(zip(ASM_MFMA_SOURCES, checked))}", file=sys.stderr)
    tmp = LIB + f".tmp{os.getpid()}"
    subprocess.check_call([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Builds libmoeffn.so (all HIP kernels and the C ABI) for gfx950 with hipcc.

Objects go to _build/ at the repository root; the library lands next to this file,
where the binding loads it. Usage: python -m expert_offloaded_ffn_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmoeffn.so")
SOURCES = ["capi.cpp", "profile.cpp", "pack.cpp", "slot_cache.cpp", "slot_cache_device.hip", "route.hip", "permute.hip", "grouped_ffn.hip", "combine.hip"]
ARCH = os.environ.get("MOEFFN_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed-fp32 instructions are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the fp8 block-scale promotion reads every partial product
    # with VALU instructions, which would otherwise copy each one out of the AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


# Sources whose kernels load global memory straight into LDS with inline assembly that sets
# M0 itself (lds_dma.h dma16_asm, gemm_fp8.h dma4_asm). The compiler reserves M0 and does
# not honour it as a clobber, so the build checks the device code instead: every instruction
# that names M0 must be one of those sequences.
M0_CHECKED = ["grouped_ffn.hip", "route.hip"]


def _llvm_tool(name: str) -> str:
    p = os.path.join("/opt/rocm/llvm/bin", name)
    return p if os.path.exists(p) else name


def device_asm(obj: str) -> str:
    """AMD GPU disassembly of the gfx950 code object embedded in a hipcc object file."""
    import tempfile
    with tempfile.TemporaryDirectory() as td:
        fat, co = os.path.join(td, "fat.bin"), os.path.join(td, "dev.co")
        subprocess.run([_llvm_tool("llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", obj, os.path.join(td, "x.o")],
                       check=True, capture_output=True)
        subprocess.run([_llvm_tool("clang-offload-bundler"), "--unbundle", "--type=o", f"--input={fat}",
                        f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}", f"--output={co}"], check=True, capture_output=True)
        return subprocess.run([_llvm_tool("llvm-objdump"), "-d", co], check=True, capture_output=True,
                              text=True).stdout


def check_m0(asm: str) -> int:
    """Raises unless every instruction naming M0 is `s_mov_b32 m0, sN` directly followed by
    `s_nop 0` and a global_load_lds instruction. Returns the number of such sequences."""
    lines = [l.split("//")[0].strip() for l in asm.splitlines()]
    ins = [l for l in lines if l and not l.endswith(":") and not l.startswith("Disassembly")]
    n = 0
    for i, l in enumerate(ins):
        ops = l.replace(",", " ").split()
        if "m0" not in ops:
            continue
        ok = (len(ops) == 3 and ops[0] == "s_mov_b32" and ops[1] == "m0"
              and (ops[2].startswith("s") or ops[2] in ("vcc_lo", "vcc_hi"))
              and i + 2 < len(ins) and ins[i + 1] == "s_nop 0" and ins[i + 2].startswith("global_load_lds_"))
        if not ok:
            ctx = "\n".join(ins[max(0, i - 2):i + 3])
            raise RuntimeError(f"M0 is used outside the LDS DMA sequences:\n{ctx}")
        n += 1
    return n


def build(verbose: bool = True) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    for src, obj in zip(SOURCES, objs):
        if src in M0_CHECKED:
            n = check_m0(device_asm(obj))
            if verbose:
                print(f"{src}: {n} LDS DMA sequences own M0; no other M0 use")
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()

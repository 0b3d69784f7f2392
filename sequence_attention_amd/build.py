"""Build the HIP library in-tree: sequence_attention_amd/libxs_attn.so (gfx950 only).

    python -m sequence_attention_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libxs_attn.so")
DEMO = os.path.join(PKG, "c_api_demo")  # host program using the C ABI alone
OBJDIR = os.path.join(PKG, "_build")
SOURCES = ["xs_attn_api.cpp", "attn_fwd_bf16.hip", "attn_fwd_fp8.hip", "attn_combine.hip",
           "burst_gap.hip", "ceiling.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from emitting packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Per-source extra flags.  The attention kernels' half-height instantiations
# (4 waves per workgroup) can hold only one wave per SIMD at D = 128, because
# the LDS ring already fills the compute unit; given that register budget the
# compiler would switch every MFMA to the accumulation-register form and copy
# the scores out for the softmax.  The vector-register form keeps them at the
# 8-wave kernels' layout (no AGPRs, no spills); the 8-wave instantiations
# compile to the same code either way.
SOURCE_FLAGS = {"attn_fwd_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "attn_fwd_fp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o",
           obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    # the C-ABI demo links the library by name and finds it next to itself
    cmd = [HIPCC, "-O2", "-std=c++17", f"-I{INCLUDE}", os.path.join(CSRC, "c_api_demo.cpp"),
           f"-L{PKG}", "-lxs_attn", "-Wl,-rpath,$ORIGIN", "-o", DEMO + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"c_api_demo build failed:\n{r.stderr}")
    os.replace(DEMO + ".tmp", DEMO)
    if verbose:
        print(f"built {LIB} and {DEMO}")
    return LIB


def resource_usage() -> str:
    """Markdown table of every kernel's register, LDS and spill usage, from the
    compiler's kernel-resource-usage remarks (same flags as the build)."""
    import re

    rows = []
    for src in SOURCES:
        if not src.endswith(".hip"):
            continue
        cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), "-Rpass-analysis=kernel-resource-usage",
               "-c", os.path.join(CSRC, src),
               "-o", os.devnull]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        cur = None
        for line in r.stderr.splitlines():
            m = re.search(r"remark: (?:\s*)([A-Za-z][^:\[]*?)(?: \[[^\]]*\])?: (.*?) \[-Rpass", line)
            if not m:
                continue
            key, val = m.group(1).strip(), m.group(2).strip()
            if key == "Function Name":
                cur = {"kernel": val, "source": src}
                rows.append(cur)
            elif cur is not None:
                cur[key] = val
    demangle = subprocess.run(["c++filt"], input="\n".join(r["kernel"] for r in rows),
                              capture_output=True, text=True).stdout.splitlines()
    cols = [("VGPRs", "VGPRs"), ("AGPRs", "AGPRs"), ("TotalSGPRs", "SGPRs"),
            ("VGPRs Spill", "VGPR spills"), ("SGPRs Spill", "SGPR spills"),
            ("ScratchSize", "scratch B/lane"),
            ("LDS Size", "LDS B/block"), ("Occupancy", "waves/SIMD")]
    out = ["| kernel | " + " | ".join(c[1] for c in cols) + " |",
           "|---|" + "---|" * len(cols)]
    for r, name in zip(rows, demangle):
        out.append(f"| `{name}` | " + " | ".join(r.get(c[0], "") for c in cols) + " |")
    return "\n".join(out)


if __name__ == "__main__":
    if "--resources" in sys.argv:
        print(resource_usage())
    else:
        build(verbose=True)
    sys.exit(0)

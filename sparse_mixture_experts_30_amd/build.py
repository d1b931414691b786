"""Builds libmoe.so (HIP, gfx950) in-tree with hipcc.

    python -m sparse_mixture_experts_30_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmoe.so")
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["gate.hip", "permute.hip", "ffn_sched.hip", "ffn_bf16.hip", "ffn_bf16_packed.hip",
           "ffn_fp8.hip", "ffn_fp8_packed.hip", "ffn_fp8_mx.hip",
           "ffn_f32.hip", "combine.hip", "bias.hip", "ffn_backward.hip", "ffn_backward_fp8.hip", "decode.hip", "decode_layer.hip",
           "layer_backward.hip", "moe_api.cpp",
           "timer.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         # no packed-fp32 instructions anywhere in device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]

# Per-file flags.  The fp8 GEMM adds each 128-k partial product (an MFMA
# result) to the fp32 accumulator with vector FMAs; with the MFMA results
# kept in VGPRs the compiler no longer copies every partial out of the
# accumulation registers first (about half of that kernel's vector
# instructions, 5-7% of its time).
FILE_FLAGS = {"ffn_fp8_packed.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"


def _scratch_kernels(stderr: str):
    """(kernel, bytes/lane) for every kernel the compiler gave private
    scratch memory (register spills or arrays it could not keep in VGPRs)."""
    out, name = [], None
    for line in stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) and name:
            out.append((name, int(m.group(1))))
    return out


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, src + ".o")
    flags = (FLAGS + FILE_FLAGS.get(src, []) + list(extra) +
             ([RESOURCE_REMARKS] if src.endswith(".hip") else []))
    cmd = [HIPCC] + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC] + flags + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode == 0:
        # Device kernels must not use scratch: it turns register traffic into
        # memory traffic on every access.
        bad = _scratch_kernels(r.stderr or "")
        if bad:
            raise RuntimeError(f"{src}: kernels with scratch memory: {bad}")
    lines, skip = [], False
    for l in (r.stderr or "").splitlines():
        if "remark:" in l:          # a remark and the source excerpt under it
            skip = True
            continue
        if skip and re.match(r"^\s*(\d+\s*)?\|", l):
            continue
        skip = False
        if "packed-fp32-ops" not in l:
            lines.append(l)
    err = "\n".join(lines)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(out: str = OUT, build_dir: str = BUILD, extra=()) -> str:
    """Compile every source and link `out`; `extra` adds compiler flags."""
    os.makedirs(build_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda f: _compile(f, build_dir, extra), SOURCES))
    tmp = out + ".tmp"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())

"""Builds libpkv.so (HIP, gfx950) in-tree with hipcc.

Each source is compiled to an object under ``<repo>/_build/`` in parallel and
linked into ``paged_kv_cache_fill_amd/libpkv.so``.  Packed-FP32 instruction
selection is switched off for device code (``-packed-fp32-ops``).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpkv.so")
SOURCES = ["abi.cpp", "tq.cpp", "slots.hip", "cache_write_v.hip", "cache_write_k.hip", "decode_attn.hip",
           "prefill_attn.hip", "mla_cache.hip"]

# Per-source flags: the prefill kernel keeps its MFMA accumulators in VGPRs
# (the accumulator-register form made the compiler copy them back and forth
# around every online-softmax rescale).
EXTRA = {"prefill_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC, *CFLAGS, *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # the host pass does not know the device-only target feature: harmless
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append((src, text))
        elif verbose and text.strip():
            print(text)
    if failed:
        for src, text in failed:
            print(f"--- {src}\n{text}", file=sys.stderr)
        raise RuntimeError("hipcc failed for: " + ", ".join(s for s, _ in failed))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

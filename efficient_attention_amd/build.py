"""Build liblinattn.so (the HIP library behind include/linattn.h) in-tree for gfx950.

    python -m efficient_attention_amd.build [--resource-usage]

Every source is compiled by hipcc for gfx950 only, with packed-fp32 VALU instructions
disabled, and linked into efficient_attention_amd/liblinattn.so.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblinattn.so")
SOURCES = ["la_api.hip", "la_noncausal.hip", "la_causal.hip", "la_decode.hip", "la_favor.hip", "la_ceiling.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]


def _compile(src: str, resource_usage: bool) -> tuple[str, str]:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if resource_usage:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
    msgs = [ln for ln in r.stderr.splitlines()
            if "not a recognized feature" not in ln and ln.strip()]
    return obj, "\n".join(msgs)


def build(resource_usage: bool = False, quiet: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        results = list(ex.map(lambda s: _compile(s, resource_usage), SOURCES))
    if not quiet:
        for _, msg in results:
            if msg:
                print(msg)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(resource_usage="--resource-usage" in sys.argv)
    print("built", LIB)

"""Build libpaged_attn.so in-tree with hipcc for gfx950.

    python -m paged_gqa_attention_amd.build [--verbose]

Each source compiles to an object under ``_build/`` (in parallel), then one
shared library is linked next to this file.  HIP code is compiled with packed
FP32 instructions disabled.  The compiler's per-kernel resource report
(registers, spills, scratch, occupancy, LDS) is kept in
``_build/kernel_resources.json`` for the resource checks of the test suite.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import json
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpaged_attn.so")
SOURCES = ["api.cpp", "decode.hip", "prefill.hip", "prefill_wide.hip", "probe.hip", "append.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return p


def common_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    ]


RESOURCES = os.path.join(BUILD, "kernel_resources.json")
REMARK = "-Rpass-analysis=kernel-resource-usage"


def parse_resources(text: str) -> dict:
    """{mangled kernel name: {field: value}} from the compiler's resource remarks."""
    out, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][^:\[]*?)(?: \[[^\]]*\])?: (\S+) \[-Rpass", line)
        if m and cur is not None:
            v = m.group(2)
            cur[m.group(1).strip()] = int(v) if v.lstrip("-").isdigit() else v
    return out


def sources_hash() -> str:
    """Hash of every source and header the library is built from."""
    h = hashlib.sha256()
    for d in (CSRC, os.path.join(ROOT, "include")):
        for n in sorted(os.listdir(d)):
            if n.endswith((".hip", ".cpp", ".h")):
                with open(os.path.join(d, n), "rb") as f:
                    h.update(n.encode() + f.read())
    return h.hexdigest()[:16]


def _compile(src: str, verbose: bool):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + common_flags()
    if src.endswith(".hip"):
        cmd.append(REMARK)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops" not in l and "kernel-resource-usage" not in l
                    and l.strip() and not l.lstrip()[:1].isdigit() and l.strip() != "|"
                    and not l.strip().startswith("| "))
    if err and verbose:
        print(err, file=sys.stderr)
    return obj, parse_resources(r.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    h = sources_hash()
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        res = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    objs = [o for o, _ in res]
    kernels = {}
    for _, r in res:
        kernels.update(r)
    with open(RESOURCES, "w") as f:
        json.dump({"sources_hash": h, "kernels": kernels}, f, indent=0)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))

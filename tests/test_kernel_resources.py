"""Resource guards on every compiled kernel (no GPU needed).

The build keeps the compiler's per-kernel resource report; when it is missing
or older than the sources, the kernels are compiled here for the device only.
Every instantiation must run without private scratch memory, VGPR spills or
a dynamic stack; SGPR spills (to VGPR lanes, no memory traffic) are allowed
only where listed.  The headline decode and prefill kernels keep the register
and LDS budgets that give their measured occupancy."""
import concurrent.futures as cf
import json
import os
import re
import subprocess

import pytest

from paged_gqa_attention_amd import build as B

HEADLINE = {
    # decode_valu<bf16, bf16, d 128, 4 rows, no per-vector scales>: 3 waves per SIMD
    "_ZN2pa11decode_valuILi2ELi2ELi128ELi4ELb0EEEvNS_10DecodeArgsE": dict(max_vgprs=168, occupancy=3),
    # prefill_mfma<bf16, bf16, d 64, 2 heads, dense, no per-vector scales>: 4 waves per
    # SIMD, two 8-wave workgroups per CU by LDS
    "_ZN2pa12prefill_mfmaILi2ELi2ELi64ELi2ELb0ELb0EEEvNS_11PrefillArgsE":
        dict(max_vgprs=128, occupancy=4, max_lds=80 * 1024),
    "_ZN2pa12decode_mergeILi128EEEvNS_10DecodeArgsE": dict(max_vgprs=64),
    # the 8-bit prefill variants of the headline shape (e4m3fn K/V, bf16 Q; with
    # and without per-vector scales) keep four waves per SIMD as well
    "_ZN2pa12prefill_mfmaILi3ELi2ELi64ELi2ELb0ELb0EEEvNS_11PrefillArgsE":
        dict(max_vgprs=128, occupancy=4, max_lds=80 * 1024),
    "_ZN2pa12prefill_mfmaILi3ELi2ELi64ELi2ELb0ELb1EEEvNS_11PrefillArgsE":
        dict(max_vgprs=128, occupancy=4, max_lds=80 * 1024),
}


def _resources():
    path = B.RESOURCES
    if os.path.exists(path):
        with open(path) as f:
            d = json.load(f)
        if d.get("sources_hash") == B.sources_hash():
            return d["kernels"]
    # compile the kernels for the device only, with the resource report

    def one(src):
        cmd = [B.hipcc(), "-x", "hip", "-c", os.path.join(B.CSRC, src), "-o", os.devnull,
               "--offload-device-only", B.REMARK] + B.common_flags()
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return B.parse_resources(r.stderr)

    srcs = [s for s in B.SOURCES if s.endswith(".hip")]
    out = {}
    with cf.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        for r in ex.map(one, srcs):
            out.update(r)
    return out


@pytest.fixture(scope="module")
def kernels():
    k = _resources()
    assert len(k) > 100, "the resource report lists too few kernels"
    return k


def test_no_scratch_no_vgpr_spills_no_dynamic_stack(kernels):
    bad = {n: r for n, r in kernels.items()
           if r.get("ScratchSize") != 0 or r.get("VGPRs Spill") != 0
           or r.get("Dynamic Stack") != "False"}
    assert not bad, "kernels using private memory: " + ", ".join(sorted(bad))


def _block_mask_variant(name):
    # prefill_mfma<KV, Q, D, HPW, MASK = true, VS> and attn_wide<KV, Q, MASK = true, VS, DEC>
    return bool(re.search(r"prefill_mfmaILi\d+ELi\d+ELi\d+ELi\d+ELb1E", name) or
                re.search(r"attn_wideILi\d+ELi\d+ELb1E", name))


def test_no_sgpr_spills(kernels):
    """No kernel spills SGPRs, except the block-mask prefill variants: they keep
    the epilogue's kernel arguments (output and sink pointers, strides) in VGPR
    lanes across the tile loop; the spill and reload code sits in the prologue,
    the tile-list builder and the epilogue, outside the MFMA loop, and is bounded."""
    bad = sorted(n for n, r in kernels.items()
                 if r.get("SGPRs Spill", 0) != 0 and not _block_mask_variant(n))
    assert not bad, f"{len(bad)} kernels spill SGPRs: " + ", ".join(bad[:8])
    masked = {n: r.get("SGPRs Spill", 0) for n, r in kernels.items() if _block_mask_variant(n)}
    assert masked and max(masked.values()) <= 32, masked


@pytest.mark.parametrize("name", sorted(HEADLINE))
def test_headline_kernel_budgets(kernels, name):
    r = kernels[name]
    lim = HEADLINE[name]
    print(name, r)
    assert r["VGPRs"] + r.get("AGPRs", 0) <= lim["max_vgprs"]
    if "occupancy" in lim:
        assert r["Occupancy"] >= lim["occupancy"]
    if "max_lds" in lim:
        assert r["LDS Size"] <= lim["max_lds"]

"""Every kernel of libmk.so fits its registers: no spill to scratch.

The compiler's resource report for the library as built (saved by
transformer_megakernel_persistent_amd.build beside libmk.so) must list every
instantiation of the decode kernel with 0 bytes of scratch per lane and at
most 256 VGPRs (two waves per SIMD: one loader and one consumer wave).  A
spill turns register traffic into memory round trips inside the hot loop,
the first failure the page cloud.baidu.com/article/9434380 section 八
(question one) tells to look for when a fused kernel is slow.  No GPU needed.
"""
import json
import os

import pytest

from transformer_megakernel_persistent_amd import build as mkbuild

GROUPS = (1, 2, 4, 8)
LANES = (8, 16)


@pytest.fixture(scope="module")
def resources():
    need = not os.path.exists(mkbuild.RESOURCES) or not os.path.exists(mkbuild.LIB)
    if not need:
        with open(mkbuild.RESOURCES) as f:
            need = json.load(f).get("sources_hash") != mkbuild.sources_hash()
    if need:  # stale or missing: rebuild (about a minute)
        mkbuild.build()
    with open(mkbuild.RESOURCES) as f:
        rec = json.load(f)
    assert rec["sources_hash"] == mkbuild.sources_hash()
    return rec["kernels"]


def test_every_decode_instantiation_is_reported(resources):
    # <dtype, group, lanes per cache row, LOGITS, position-major attention>;
    # the position-major mapping exists for groups of four query heads only
    names = {k["name"] for k in resources}
    for dt in (0, 1, 2):  # float32, bfloat16, weight-only INT8
        for gq in GROUPS:
            for lpp in LANES:
                for logits in ("b0", "b1"):
                    for pm in (("b0", "b1") if gq == 4 else ("b0",)):
                        n = f"_Z16mk_decode_kernelILi{dt}ELi{gq}ELi{lpp}EL{logits}EL{pm}EEv8MkParams"
                        assert n in names, n


def test_no_kernel_spills_to_scratch(resources):
    spilled = [(k["name"], k.get("scratch")) for k in resources if k.get("scratch", 0) != 0]
    assert not spilled, spilled


def test_decode_kernels_fit_two_waves_per_simd(resources):
    for k in resources:
        if "mk_decode_kernel" in k["name"]:
            assert k["vgprs"] + k.get("agprs", 0) <= 256, k
            assert k["occupancy"] >= 2, k

"""Static checks of the generated retrieval-kernel code (no GPU needed).

The retrieval loop's copies and counter waits are inline asm, so wait states
and register lifetimes around them are checked on the compiler's output:
first the checker itself on planted mistakes, then the real kernels."""
from __future__ import annotations

import shutil

import pytest

from cross_model_sparse_amd import isa_check

PLANTED = """
_Zk_retrieve_mfma_demo:
\tv_readfirstlane_b32 s8, v10
\tv_readfirstlane_b32 s9, v11
\tglobal_load_dwordx2 v[20:21], v30, s[8:9]
\ts_mov_b32 m0, s12
\tglobal_load_lds_dwordx4 v31, s[8:9]
\tv_add_u32_e32 v40, v20, v41
\ts_waitcnt vmcnt(0)
\ts_endpgm
.Lfunc_end0:
\t.amdhsa_kernel x
    .name:           _Zk_retrieve_mfma_demo
    .private_segment_fixed_size: 16
    .vgpr_count:     64
"""

CLEAN = """
_Zk_retrieve_mfma_demo:
\tv_readfirstlane_b32 s8, v10
\tv_readfirstlane_b32 s9, v11
\ts_nop 4
\tglobal_load_dwordx2 v[20:21], v30, s[8:9]
\ts_mov_b32 m0, s12
\ts_nop 0
\tglobal_load_lds_dwordx4 v31, s[8:9]
\ts_waitcnt vmcnt(1)
\tv_add_u32_e32 v40, v20, v41
\ts_waitcnt vmcnt(0)
\ts_endpgm
.Lfunc_end0:
\t.amdhsa_kernel x
    .name:           _Zk_retrieve_mfma_demo
    .private_segment_fixed_size: 0
    .vgpr_count:     64
"""


def _check_text(tmp_path, text):
    p = tmp_path / "k.s"
    p.write_text(text)
    res = isa_check.check_asm(str(p), pattern="k_retrieve_mfma")
    assert list(res) == ["_Zk_retrieve_mfma_demo"]
    return res["_Zk_retrieve_mfma_demo"]


def test_checker_flags_planted_mistakes(tmp_path):
    r = _check_text(tmp_path, PLANTED)
    assert r["scratch"] == 16
    # both loads read s[8:9] within 5 wait states of each of its two VALU writes
    assert len(r["valu_sgpr"]) == 4
    assert len(r["m0_dma"]) == 1
    assert [s for _, s in r["inflight"]] == ["v_add_u32_e32 v40, v20, v41"]


M0_LIVE = """
_Zk_retrieve_mfma_demo:
\ts_mov_b32 m0, s12
\ts_mov_b32 m0, s13
\ts_nop 0
\tglobal_load_lds_dwordx4 v31, s[8:9]
\tv_movrel_b32_e32 v1, v2
\ts_mov_b32 m0, -1
\tv_movrel_b32_e32 v3, v4
\ts_waitcnt vmcnt(0)
\ts_endpgm
.Lfunc_end0:
\t.amdhsa_kernel x
    .name:           _Zk_retrieve_mfma_demo
    .private_segment_fixed_size: 0
    .vgpr_count:     64
"""


def test_checker_flags_m0_live_across_a_copy(tmp_path):
    r = _check_text(tmp_path, M0_LIVE)
    # the first v_movrel reads the copy's M0; the second follows a fresh write
    assert [s for _, s in r["m0_live"]] == ["v_movrel_b32_e32 v1, v2"]


def test_checker_flags_vmem_after_any_valu_sgpr_write(tmp_path):
    # a compare mask and a carry out are VALU writes of SGPRs too
    text = PLANTED.replace("\tv_readfirstlane_b32 s8, v10\n\tv_readfirstlane_b32 s9, v11\n",
                           "\tv_cmp_gt_i32_e64 s[8:9], v10, v11\n")
    r = _check_text(tmp_path, text)
    assert [s for _, s in r["valu_sgpr"]] == ["global_load_dwordx2 v[20:21], v30, s[8:9]",
                                              "global_load_lds_dwordx4 v31, s[8:9]"]
    text = PLANTED.replace("\tv_readfirstlane_b32 s8, v10\n\tv_readfirstlane_b32 s9, v11\n",
                           "\tv_mad_u64_u32 v[2:3], s[8:9], s10, v4, 0\n")
    r = _check_text(tmp_path, text)
    assert len(r["valu_sgpr"]) == 2
    # a VALU write of another SGPR, or a scalar write, is not a hazard
    text = PLANTED.replace("\tv_readfirstlane_b32 s8, v10\n\tv_readfirstlane_b32 s9, v11\n",
                           "\tv_cmp_gt_i32_e64 s[20:21], v10, v11\n\ts_add_u32 s8, s8, 64\n")
    r = _check_text(tmp_path, text)
    assert not r["valu_sgpr"]


TWO_PATHS = """
_Zk_retrieve_mfma_demo:
\ts_cbranch_scc1 .LBB0_2
\tglobal_load_dwordx2 v[20:21], v30, s[8:9]
.LBB0_2:
\tv_add_u32_e32 v40, v22, v41
\ts_waitcnt vmcnt(0)
\ts_endpgm
"""


def test_checker_reports_a_walk_it_cannot_finish():
    # two paths meet with different loads in flight: two states at the join.
    # With room for one, the walk cannot finish and says so instead of
    # passing the kernel; with room for two it finishes and finds nothing.
    lines = TWO_PATHS.strip("\n").split("\n")
    body = isa_check._functions(lines)["_Zk_retrieve_mfma_demo"]
    r = isa_check._inflight(body, max_states=1)
    assert r and all("walk incomplete" in s for _, s in r)
    assert isa_check._inflight(body, max_states=2) == []


def test_checker_counts_copies_into_lds_toward_waits(tmp_path):
    # a register load, then two copies into LDS: vmcnt(2) retires the load,
    # vmcnt(3) does not
    text = CLEAN.replace("\ts_waitcnt vmcnt(1)\n",
                         "\tglobal_load_lds_dwordx4 v31, s[8:9]\n\ts_waitcnt vmcnt(3)\n")
    r = _check_text(tmp_path, text)
    assert [s for _, s in r["inflight"]] == ["v_add_u32_e32 v40, v20, v41"]
    text = CLEAN.replace("\ts_waitcnt vmcnt(1)\n",
                         "\tglobal_load_lds_dwordx4 v31, s[8:9]\n\ts_waitcnt vmcnt(2)\n")
    r = _check_text(tmp_path, text)
    assert not r["inflight"]


def test_checker_accepts_the_fixed_forms(tmp_path):
    r = _check_text(tmp_path, CLEAN)
    assert r["scratch"] == 0 and not r["valu_sgpr"] and not r["m0_dma"] and not r["inflight"]
    assert not r["m0_live"]


# one instantiation per code shape: bf16/fp16, 1 or 2 receiver pairs, 2 or 3
# tile buffers, the four head-mix plans (full groups, remainder 1, 2, 3), each
# for one sequence (Lb0E) and for a packed batch (Lb1E)
KERNELS = [k + v for k in ("ILb1ELi5ELi2E", "ILb1ELi6ELi2E", "ILb1ELi3ELi1E", "ILb0ELi4ELi2E",
                           "ILb0ELi6ELi1E", "ILb1ELi1ELi1E") for v in ("Lb0E", "Lb1E")]


@pytest.fixture(scope="module")
def retrieve_asm(tmp_path_factory):
    if shutil.which("hipcc") is None and not isa_check.Path("/opt/rocm/bin/hipcc").exists():
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "k_retrieve.s"
    isa_check.compile_to_asm(isa_check.HERE / "csrc" / "k_retrieve.hip", out)
    return str(out)


@pytest.fixture(scope="module")
def retrieve_findings(retrieve_asm):
    return isa_check.check_asm(retrieve_asm, pattern="k_")


# pair-stage kernels (B >= 32, up to 40 sender heads): bf16/fp16, 1 or 2
# receiver pairs, the head-mix plans; one sequence, a packed batch, or one
# sequence with long rows split into parts
PAIR_KERNELS = [k + v for k in ("ILb1ELi5ELi2E", "ILb1ELi3ELi1E", "ILb1ELi4ELi2E", "ILb0ELi4ELi2E",
                                "ILb0ELi5ELi1E", "ILb1ELi1ELi1E", "ILb1ELi2ELi2E")
                for v in ("Lb0ELb0E", "Lb1ELb0E", "Lb0ELb1E")]


@pytest.mark.parametrize("tag", ["k_retrieve_mfma" + t for t in KERNELS] +
                         ["k_retrieve_pair" + t for t in PAIR_KERNELS])
def test_retrieve_kernels_have_no_hazards(retrieve_findings, tag):
    res = {n: r for n, r in retrieve_findings.items() if tag in n}
    assert len(res) == 1, tag
    (name, r), = res.items()
    assert r["scratch"] == 0, name
    assert not r["valu_sgpr"], r["valu_sgpr"][:3]
    assert not r["m0_dma"], r["m0_dma"][:3]
    assert not r["inflight"], r["inflight"][:3]
    assert not r["m0_live"], r["m0_live"][:3]


def test_every_retrieval_kernel_is_clean(retrieve_findings):
    res = retrieve_findings
    assert len(res) > 100
    bad = {n: r for n, r in res.items()
           if r["scratch"] or r["inflight"] or r["valu_sgpr"] or r["m0_dma"] or r["m0_live"]}
    assert not bad, sorted(bad)[:3]

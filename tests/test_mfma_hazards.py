"""CPU check of the generated gfx950 code: no path from a matrix instruction
to a read of its result is shorter than the wait states the compiler itself
requires for that instruction (see mfma_hazards.py), in every kernel of every
source of the library.  Uses the assembly the build keeps beside its objects,
or compiles it when that is missing or older than the sources."""

import os

import pytest

import mfma_hazards as M
from linear_attention_gdn_amd import build as B

HEADERS = [os.path.join(B.CSRC, n) for n in ("gdn_common.h", "tree_common.h")]


def _asm(src):
    path = B.device_asm_path(src)
    newest = max([os.path.getmtime(src)] + [os.path.getmtime(p) for p in HEADERS])
    if os.path.exists(path) and os.path.getmtime(path) >= newest:
        with open(path) as f:
            return f.read()
    flags = [f for f in B.HIPCC_FLAGS if f != "-save-temps=obj"]
    return M.device_asm(src, flags, B.hipcc())


@pytest.fixture(scope="module")
def probed(tmp_path_factory):
    flags = [f for f in B.HIPCC_FLAGS if f not in ("-save-temps=obj", "-fPIC")]
    req = M.probed_requirements(flags, B.hipcc(), str(tmp_path_factory.mktemp("probe")))
    assert set(req) == set(M.PROBES), req  # every probe read its result in straight line
    return req


def test_probed_requirements_are_positive(probed):
    assert all(w >= 1 for w in probed.values()), probed


@pytest.mark.parametrize("src", B.sources(), ids=lambda p: os.path.basename(p))
def test_no_mfma_result_read_too_early(src, probed):
    asm = _asm(src)
    used = {ins.op for k in M.parse_kernels(asm) for ins in k.instrs if ins.op.startswith("v_mfma")}
    assert used <= set(probed), f"no probe for {sorted(used - set(probed))}"
    bad, req = M.check(asm, probed)
    detail = "\n".join(f"{k[:70]}: {mf} -> {rd} after {w} < {need} wait states"
                       for k, mf, w, rd, need in bad[:10])
    assert not bad, f"{len(bad)} early reads of MFMA results:\n{detail}"


def test_checker_finds_a_planted_early_read():
    """A read one instruction after an MFMA, reached through a branch, is
    reported; the same read after the compiler's padding is not."""
    asm = "\n".join([
        "_Zkernel:",
        "  v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], 0",
        "  s_nop 7",
        "  v_accvgpr_read_b32 v8, a0",          # straight line: 8 wait states
        "  v_mfma_f32_16x16x32_bf16 a[4:7], v[0:3], v[4:7], 0",
        "  s_cbranch_vccnz .LBB0_2",
        "  s_nop 7",
        ".LBB0_2:",
        "  v_accvgpr_read_b32 v9, a7",          # 1 wait state on the taken branch
        "  s_endpgm",
        ".Lfunc_end0:",
    ])
    bad, req = M.check(asm)
    assert req == {"v_mfma_f32_16x16x32_bf16": 8}
    assert len(bad) == 1 and bad[0][2] == 1 and "a7" in bad[0][3]

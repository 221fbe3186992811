"""Every path from an MFMA to a use of its result leaves enough wait states.

The library's kernels are compiled to gfx950 assembly here (no GPU needed)
and scanned with tests/isa_hazards.py; the checker itself is first tried on
short hand-written instruction streams with known answers.
"""

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

import isa_hazards as hz
from transformer_exact_attention_flashattention_amd import build


def _fn(body: str) -> str:
    return "_Zkernel:\n" + body + "\n\ts_endpgm\n.Lfunc_end0:\n"


MFMA32 = "\tv_mfma_f32_32x32x2_f32 v[0:15], v20, v21, v[0:15]\n"
MFMA16 = "\tv_mfma_f32_32x32x16_bf16 v[32:47], v[60:63], v[64:67], v[32:47]\n"


def test_straight_path_counts():
    ok = _fn(MFMA16 + "\ts_nop 7\n\ts_nop 3\n\tv_add_f32_e32 v1, v32, v2")  # 8 + 4 = 12
    short = _fn(MFMA16 + "\ts_nop 7\n\ts_nop 2\n\tv_add_f32_e32 v1, v32, v2")  # 11
    assert hz.short_paths(ok) == []
    found = hz.short_paths(short)
    assert [(f[2], f[3]) for f in found] == [(11, 12)]
    # independent instructions count one each; a register the MFMA does not
    # write is no use of it
    indep = _fn(MFMA32 + "\tv_add_f32_e32 v30, v31, v31\n" * 17 + "\tv_mov_b32_e32 v40, v0")
    assert [(f[2], f[3]) for f in hz.short_paths(indep)] == [(17, 18)]
    other = _fn(MFMA32 + "\tv_mov_b32_e32 v40, v16")
    assert hz.short_paths(other) == []


def test_taken_branch_path_is_checked():
    # The fall-through path has 6 + 2 + 10 = 18 wait states, the taken
    # branch 1 + 1 + 10 = 12: the read must be reported with 12.
    body = (MFMA32 + "\ts_cbranch_vccnz .LBB0_2\n" + "\ts_add_i32 s4, s4, 1\n" * 6 + ".LBB0_2:\n"
            "\ts_andn2_b64 vcc, exec, s[4:5]\n\ts_nop 9\n\tv_fma_f32 v1, v0, v2, -v3")
    found = hz.short_paths(_fn(body))
    assert [(f[1], f[2], f[3]) for f in found] == [("v_fma_f32 v1, v0, v2, -v3", 12, 18)]
    # with the wait stated before the branch every path is long enough
    guarded = body.replace("\ts_cbranch_vccnz", "\ts_nop 7\n\ts_nop 7\n\ts_nop 5\n\ts_cbranch_vccnz")
    assert hz.short_paths(_fn(guarded)) == []


def test_loop_back_edge_and_older_writer():
    # A use at the loop head is reached from the latch too.
    loop = ("\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n.LBB0_1:\n\tv_mov_b32_e32 v40, v5\n" + MFMA32 +
            "\ts_nop 4\n\ts_cbranch_scc1 .LBB0_1")
    assert [(f[2], f[3]) for f in hz.short_paths(_fn(loop))] == [(6, 18)]
    # v0 (written by the older 16-pass product) is read along with v32 (the
    # younger 8-pass one, itself one wait state): the older writer decides.
    both = _fn(MFMA32 + MFMA16 + "\ts_nop 7\n\ts_nop 5\n\tv_add_f32_e32 v1, v32, v0")
    assert [(f[2], f[3]) for f in hz.short_paths(both)] == [(15, 18)]


def test_stores_and_mfma_operands_are_uses():
    store = _fn(MFMA16 + "\tds_write_b64 v9, v[46:47]")
    assert [(f[2], f[3]) for f in hz.short_paths(store)] == [(0, 12)]
    chained = _fn(MFMA16 + MFMA16)  # same accumulator: resolved by the hardware
    assert hz.short_paths(chained) == []
    operand = _fn(MFMA16 + "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[32:35], v[64:67], v[0:15]")
    assert [(f[2], f[3]) for f in hz.short_paths(operand)] == [(0, 12)]


def _have_hipcc() -> bool:
    try:
        build.hipcc()
        return True
    except RuntimeError:
        return False


@pytest.mark.skipif(not _have_hipcc(), reason="hipcc not available")
def test_library_kernels(tmp_path):
    """Both sources, as libfa.so and libfa_sync.so compile them."""
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-shared", "-fPIC", "-Wall")]
    jobs = []
    for src in build.SOURCES:
        for extra in ([], ["-DFA_SYNC_CHECK"]):
            out = tmp_path / (os.path.basename(src) + ("_sync" if extra else "") + ".s")
            jobs.append([build.hipcc(), *flags, *extra, "-I", os.path.join(build.ROOT, "include"),
                         "--cuda-device-only", "-S", "-o", str(out), src])

    def run(cmd):
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return cmd[-2]

    with ThreadPoolExecutor(len(jobs)) as ex:
        outs = list(ex.map(run, jobs))
    kernels = 0
    for path in outs:
        asm = open(path).read()
        kernels += len(hz.functions(asm))
        short = hz.short_paths(asm)
        assert short == [], f"{os.path.basename(path)}: " + "; ".join(
            f"{f[0][:60]}: '{f[1]}' after {f[2]} wait states, needs {f[3]}" for f in short[:8])
    assert kernels >= 40

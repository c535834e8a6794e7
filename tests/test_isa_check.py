"""The build-time ISA checks on synthetic gfx950 assembly: each rule fires on the pattern it guards
against and stays quiet on the same code made safe."""
import os
import sys

sys.path.insert(0, os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "prefix_shared_branch_amd"))
import isa_check  # noqa: E402


def test_store_data_overwrite_is_flagged():
    asm = "\n".join([
        "_Zk:",
        "  buffer_store_dwordx4 v[0:3], v8, s[4:7], s9 offen",
        "  v_mov_b32_e32 v2, 0",
        "  s_endpgm",
    ])
    assert isa_check.scan(asm)


def test_store_data_overwrite_after_wait_states_is_clean():
    asm = "\n".join([
        "_Zk:",
        "  buffer_store_dwordx4 v[0:3], v8, s[4:7], s9 offen",
        "  s_nop 1",
        "  v_mov_b32_e32 v2, 0",
        "  v_mov_b32_e32 v9, 0",
        "  s_endpgm",
    ])
    assert isa_check.scan(asm) == []


def _kernel(name, body):
    return "\n".join([f"{name}:", *body, "  s_endpgm"])


LOOP_WITH_SCRATCH = [
    "  s_mov_b32 s0, 4",
    ".LBB0_1:",
    "  v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]",
    "  scratch_load_dwordx4 v[24:27], off, off offset:16",
    "  s_sub_u32 s0, s0, 1",
    "  s_cmp_eq_u32 s0, 0",
    "  s_cbranch_scc0 .LBB0_1",
]
LOOP_SCRATCH_OUTSIDE = [
    "  scratch_store_dwordx4 off, v[24:27], off offset:16",
    ".LBB0_1:",
    "  v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]",
    "  s_sub_u32 s0, s0, 1",
    "  s_cbranch_scc0 .LBB0_1",
    "  scratch_load_dwordx4 v[24:27], off, off offset:16",
]


def test_scratch_in_a_loop_of_a_guarded_kernel_is_flagged():
    asm = _kernel("_ZN3lsr12_GLOBAL__N_119replay_bwd_dkdv_w64ENS_7BwdArgsE", LOOP_WITH_SCRATCH)
    bad = isa_check.loop_scratch(asm)
    assert len(bad) == 1 and "scratch_load_dwordx4" in bad[0]


def test_scratch_outside_loops_or_in_other_kernels_is_allowed():
    guarded = _kernel("_ZN3lsr12_GLOBAL__N_119replay_bwd_dkdv_w64ENS_7BwdArgsE", LOOP_SCRATCH_OUTSIDE)
    other = _kernel("_ZN3lsr12_GLOBAL__N_113grpo_rows_vecE", LOOP_WITH_SCRATCH)
    assert isa_check.loop_scratch(guarded) == []
    assert isa_check.loop_scratch(other) == []

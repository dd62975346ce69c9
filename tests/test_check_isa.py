"""The structural check of the interpreter's compiled code (check_isa.py)
accepts well-formed slot code and reports each kind of hazard, on small
synthetic assembly listings in the compiler's output format."""
from persistent_megakernel_decode_cu_amd import check_isa

CLEAN = """\
.LBB0_1:                                ; =>This Inner Loop Header: Depth=1
\ts_nop 4
\tbuffer_load_dwordx4 v[168:171], v1, s[8:11], 0 offen nt ; slot_load
\tv_add_f32_e32 v2, v3, v4
\ts_waitcnt vmcnt(12) ; slot_wait
\tv_mov_b64 v[10:11], v[168:169] ; slot_take
\tv_fma_f32 v5, v10, v11, v5
\ts_cbranch_scc1 .LBB0_1
"""


def lines(txt):
    return txt.split("\n")


def test_clean_listing_has_no_problems():
    problems, n_load, n_take, max_compiler, top = check_isa.check_kernel(lines(CLEAN))
    assert problems == [] and n_load == 1 and n_take == 1
    assert max_compiler < check_isa.SLOT_VGPR0 and top == 171
    assert check_isa.slice_loop_waits(lines(CLEAN))[2] == []


def test_compiler_instruction_naming_a_slot_register_is_reported():
    bad = CLEAN.replace("v_add_f32_e32 v2, v3, v4", "v_add_f32_e32 v2, v170, v4")
    problems = check_isa.check_kernel(lines(bad))[0]
    assert any("names a slot register" in p for p in problems)


def test_slot_copy_without_a_wait_in_its_block_is_reported():
    bad = CLEAN.replace("\ts_waitcnt vmcnt(12) ; slot_wait\n", "")
    problems = check_isa.check_kernel(lines(bad))[0]
    assert any("without a preceding slot_wait" in p for p in problems)
    # a wait in an earlier block does not cover a copy after a label
    bad2 = CLEAN.replace("\tv_mov_b64 v[10:11], v[168:169] ; slot_take",
                         ".LBB0_2:                                ;   in Loop: Header=BB0_1 Depth=1\n"
                         "\tv_mov_b64 v[10:11], v[168:169] ; slot_take")
    assert any("without a preceding slot_wait" in p for p in check_isa.check_kernel(lines(bad2))[0])


def test_malformed_slot_load_is_reported():
    bad = CLEAN.replace("buffer_load_dwordx4 v[168:171]", "buffer_load_dwordx4 v[40:43]")
    problems = check_isa.check_kernel(lines(bad))[0]
    assert any("malformed slot load" in p for p in problems)


def test_compiler_wait_inside_the_slice_loop_is_counted():
    bad = CLEAN.replace("\tv_fma_f32 v5, v10, v11, v5", "\ts_waitcnt vmcnt(0)\n\tv_fma_f32 v5, v10, v11, v5")
    hdrs, n, waits = check_isa.slice_loop_waits(lines(bad))
    assert hdrs == ["BB0_1"] and len(waits) == 1

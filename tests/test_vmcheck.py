"""The build's check of registers named while their loads are in flight
(weight_only_int4_02_amd/vmcheck.py), on hand-written gfx9 assembly: each
case is a hazard the check must report or a correct wait it must accept."""
from weight_only_int4_02_amd import vmcheck


def found(body: str):
    asm = "_Zkern:\n" + body.strip("\n") + "\n.Lfunc_end0:\n"
    return vmcheck.check_asm(asm).get("_Zkern", [])


def test_read_before_wait_is_reported():
    f = found("""
    buffer_load_dwordx4 v[4:7], v1, s[8:11], 0 offen
    v_accvgpr_write_b32 a3, v5
    s_waitcnt vmcnt(0)
    s_endpgm
""")
    assert len(f) == 1 and "v_accvgpr_write_b32" in f[0][1] and ("v", 5) in f[0][2]


def test_read_after_wait_is_accepted():
    assert found("""
    buffer_load_dwordx4 v[4:7], v1, s[8:11], 0 offen
    s_waitcnt vmcnt(0)
    v_accvgpr_write_b32 a3, v5
    s_endpgm
""") == []


def test_partial_wait_completes_the_older_loads_only():
    body = """
    buffer_load_dword v4, v1, s[8:11], 0 offen
    buffer_load_dword v5, v1, s[8:11], 0 offen offset:64
    s_waitcnt vmcnt(1)
    v_add_u32_e32 v6, v4, v4
    {}
    s_waitcnt vmcnt(0)
    s_endpgm
"""
    assert found(body.format("")) == []
    f = found(body.format("v_add_u32_e32 v7, v5, v5"))
    assert len(f) == 1 and ("v", 5) in f[0][2]


def test_buffer_to_lds_copies_count_in_the_counter():
    # the copy is issued after the load: vmcnt(1) leaves the copy pending and
    # completes the load; vmcnt(2) would not
    body = """
    buffer_load_dword v4, v1, s[8:11], 0 offen
    buffer_load_dword v2, s[8:11], 0 offen lds
    s_waitcnt vmcnt({})
    v_add_u32_e32 v6, v4, v4
    s_endpgm
"""
    assert found(body.format(1)) == []
    assert len(found(body.format(2))) == 1


def test_a_second_load_into_a_pending_register_is_reported():
    f = found("""
    buffer_load_dword v4, v1, s[8:11], 0 offen
    buffer_load_dword v4, v1, s[8:11], 0 offen offset:64
    s_waitcnt vmcnt(0)
    s_endpgm
""")
    assert len(f) == 1 and f[0][1].startswith("buffer_load_dword v4")


def test_pending_on_every_path_into_a_block():
    # both branches leave the load pending: the read after the merge counts
    f = found("""
    buffer_load_dword v4, v1, s[8:11], 0 offen
    s_cbranch_scc0 .LBB0_2
    v_mov_b32_e32 v9, 0
    s_branch .LBB0_3
.LBB0_2:
    v_mov_b32_e32 v9, 1
.LBB0_3:
    v_add_u32_e32 v6, v4, v9
    s_waitcnt vmcnt(0)
    s_endpgm
""")
    assert len(f) == 1 and ("v", 4) in f[0][2]


def test_pending_on_one_path_only_is_not_reported():
    # one branch waits: what is pending on every path is checked
    assert found("""
    buffer_load_dword v4, v1, s[8:11], 0 offen
    s_cbranch_scc0 .LBB0_2
    s_waitcnt vmcnt(0)
.LBB0_2:
    v_add_u32_e32 v6, v8, v9
    s_waitcnt vmcnt(0)
    v_add_u32_e32 v6, v4, v9
    s_endpgm
""") == []


def test_a_load_issued_at_the_end_of_a_loop_reaches_its_top():
    # a ring: the first load before the loop, the next one at the end of
    # each iteration; the iteration reads the register before its wait
    f = found("""
    buffer_load_dword v4, v1, s[8:11], 0 offen
.LBB0_1:
    v_add_u32_e32 v6, v4, v6
    buffer_load_dword v4, v1, s[8:11], 0 offen offset:64
    s_cbranch_scc1 .LBB0_1
    s_waitcnt vmcnt(0)
    s_endpgm
""")
    assert [x for x in f if x[1].startswith("v_add_u32")]


def test_the_loop_with_its_wait_is_accepted():
    assert found("""
    buffer_load_dword v4, v1, s[8:11], 0 offen
.LBB0_1:
    s_waitcnt vmcnt(0)
    v_add_u32_e32 v6, v4, v6
    buffer_load_dword v4, v1, s[8:11], 0 offen offset:64
    s_cbranch_scc1 .LBB0_1
    s_waitcnt vmcnt(0)
    s_endpgm
""") == []

"""The in-flight-load checker (isa_hazards) on small hand-written gfx950
assembly: each case has a known answer, so a model error in the checker (wrong
retirement order, a lost path) fails here rather than passing kernels."""
import isa_hazards as H


def fn(body):
    return "k:\n" + "\n".join("\t" + l if not l.endswith(":") else l for l in body.strip().split("\n")) + \
        "\n\ts_endpgm\n.Lfunc_end0:\n"


def lines(body):
    return [h[2].split()[0] for h in H.hazards(fn(body))]


def test_use_before_wait_is_reported():
    assert lines("ds_read_b64 v[0:1], v8\nv_mov_b32 v2, v0\ns_waitcnt lgkmcnt(0)") == ["v_mov_b32"]


def test_use_after_wait_is_not():
    assert lines("ds_read_b64 v[0:1], v8\ns_waitcnt lgkmcnt(0)\nv_mov_b32 v2, v0") == []


def test_overwrite_of_a_register_in_flight_is_reported():
    assert lines("ds_read_b64 v[0:1], v8\nv_mov_b32 v1, 0\ns_waitcnt lgkmcnt(0)") == ["v_mov_b32"]


def test_lds_reads_retire_in_order():
    body = "ds_read_b32 v0, v8\nds_read_b32 v1, v9\ns_waitcnt lgkmcnt(1)\nv_add_f32 v2, v0, v0\nv_add_f32 v3, v1, v1"
    assert lines(body) == ["v_add_f32"]
    assert H.hazards(fn(body))[0][2].split()[1] == "v3,"


def test_scalar_loads_retire_only_at_zero():
    body = "s_load_dword s4, s[0:1], 0x0\nds_read_b32 v1, v9\ns_waitcnt lgkmcnt(1)\ns_add_i32 s5, s4, 1"
    assert lines(body) == ["s_add_i32"]
    body = "s_load_dword s4, s[0:1], 0x0\ns_waitcnt lgkmcnt(0)\ns_add_i32 s5, s4, 1"
    assert lines(body) == []


def test_vector_memory_counts_stores_and_lds_copies():
    body = ("global_load_dwordx4 v[2:5], v[10:11], off\nglobal_store_dwordx4 v[12:13], v[6:9], off\n"
            "buffer_load_dword v1, s[4:7], 0 offen lds\ns_waitcnt vmcnt(2)\nv_mov_b32 v20, v2")
    assert lines(body) == []
    body = "global_load_dwordx4 v[2:5], v[10:11], off\ns_waitcnt vmcnt(1)\nv_mov_b32 v20, v2"
    assert lines(body) == ["v_mov_b32"]


def test_younger_load_into_the_same_registers_is_allowed():
    assert lines("ds_read_b32 v0, v8\nds_read_b32 v0, v9\ns_waitcnt lgkmcnt(0)") == []
    # but a load whose address is a register still being loaded is not
    assert lines("ds_read_b32 v0, v8\nds_read_b32 v1, v0\ns_waitcnt lgkmcnt(0)") == ["ds_read_b32"]


def test_paths_join():
    # the read is waited on the taken path only: the fall-through path reuses
    # its register before any wait
    body = """ds_read_b32 v0, v8
s_cbranch_scc1 .LBB0_2
v_mov_b32 v0, 1
s_branch .LBB0_3
.LBB0_2:
s_waitcnt lgkmcnt(0)
v_mov_b32 v0, 2
.LBB0_3:
s_nop 0"""
    hz = H.hazards(fn(body))
    assert [h[2] for h in hz] == ["v_mov_b32 v0, 1"]


def test_loop_back_edge_carries_loads():
    # a read issued at the end of the loop body is in flight at the top of the
    # next trip, where its register is read before the wait
    body = """.LBB0_1:
v_add_f32 v2, v0, v0
s_waitcnt lgkmcnt(0)
ds_read_b32 v0, v8
s_cbranch_scc1 .LBB0_1
s_waitcnt lgkmcnt(0)"""
    assert lines(body) == ["v_add_f32"]

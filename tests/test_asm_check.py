"""The inline-asm load check (sparse_state_linear_product_amd/asm_check.py) on
small assembly listings with a known answer, and on the library's kernels."""
import pytest

from sparse_state_linear_product_amd import asm_check


def _kernel(body):
    lines = ["_Z1kv:"] + [("\t" + l) if not l.endswith(":") else l for l in body.strip().splitlines()]
    return lines + ["\ts_endpgm"]


LOAD = ";;#ASMSTART\nglobal_load_dwordx4 v[4:7], v[0:1], off\n;;#ASMEND"
WAIT = ";;#ASMSTART\ns_waitcnt vmcnt(0)\n;;#ASMEND"


def _check(body):
    return asm_check.check_kernel(_kernel(body))


def test_use_after_the_wait_is_clean():
    assert _check(f"{LOAD}\nv_add_u32 v8, v9, v10\n{WAIT}\nv_mov_b32 v11, v5") == []


def test_use_before_the_wait_is_reported():
    rep = _check(f"{LOAD}\nv_mov_b32 v12, v6\n{WAIT}")
    assert rep and ("v", 6) in rep[0][1]


def test_overwrite_before_the_wait_is_reported():
    rep = _check(f"{LOAD}\nv_mov_b32 v[4:5], 0\n{WAIT}")
    assert rep and ("v", 4) in rep[0][1]


def test_compiler_wait_for_zero_also_completes_the_load():
    assert _check(f"{LOAD}\ns_waitcnt vmcnt(0)\nv_mov_b32 v12, v6") == []
    assert _check(f"{LOAD}\ns_waitcnt vmcnt(1)\nv_mov_b32 v12, v6") != []


def test_load_at_the_loop_end_reaches_the_exit_path():
    # the prefetch issued at the end of an iteration is waited for at the top
    # of the next one, but the loop exit skips that wait: a use there is reported
    body = f"""
.LBB0_1:
{WAIT}
v_mov_b32 v20, v4
{LOAD}
s_cbranch_scc1 .LBB0_1
v_mov_b32 v21, v7
"""
    rep = _check(body)
    assert len(rep) == 1 and ("v", 7) in rep[0][1]
    assert _check(body.replace("v_mov_b32 v21, v7", f"{WAIT}\nv_mov_b32 v21, v7")) == []


def test_fallthrough_blocks_labelled_by_comments_are_separate():
    # the compiler labels a block that no branch targets only in a comment; the
    # branch around it must not carry its load into the branch target
    body = f"""
s_cbranch_scc1 .LBB0_2
; %bb.1:
{LOAD}
s_branch .LBB0_3
.LBB0_2:
v_mov_b32 v4, 0
.LBB0_3:
{WAIT}
v_mov_b32 v9, v4
"""
    assert _check(body) == []
    # falling through from the load block into a use is still reported
    rep = _check(body.replace("s_branch .LBB0_3\n", "v_mov_b32 v10, v5\n"))
    assert rep and ("v", 5) in rep[0][1]


def test_lds_reads_are_tracked_by_lgkmcnt():
    rd = ";;#ASMSTART\nds_read_b64 v[2:3], v1 offset:16\n;;#ASMEND"
    assert _check(f"{rd}\ns_waitcnt vmcnt(0)\nv_mov_b32 v9, v2") != []
    assert _check(f"{rd}\n;;#ASMSTART\ns_waitcnt lgkmcnt(0)\n;;#ASMEND\nv_mov_b32 v9, v2") == []


def test_library_kernels_pass():
    import shutil
    if shutil.which("/opt/rocm/bin/hipcc") is None:
        pytest.skip("hipcc not available")
    counts = asm_check.run()
    assert counts["gdn_chunk.hip"] > 0 and counts["sdm_chunk.hip"] > 0

"""Compiled-code properties of the HIP kernels (gfx950 assembly from hipcc,
no GPU needed): no barrier inside a loop that part of a wave can keep
running, and GEMM k loops whose only vector-memory waits are the ring's.
See tests/isa_check.py for why each matters."""
import os

import pytest

from tests import isa_check as ic

pytestmark = pytest.mark.skipif(not os.path.exists(ic.HIPCC), reason="hipcc not installed")

SOURCES = ["fused.hip", "experts.hip", "router.hip", "permute.hip"]


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    d = tmp_path_factory.mktemp("isa")
    return {src: ic.compile_asm(src, str(d / (src + ".s"))) for src in SOURCES}


@pytest.mark.parametrize("src", SOURCES)
def test_no_barrier_in_divergent_loop(asm, src):
    ks = ic.kernels(asm[src])
    assert ks, f"no kernels found in {src}"
    bad = {k[:80]: ic.barrier_loops_with_exec_exits(v) for k, v in ks.items()}
    bad = {k: v for k, v in bad.items() if v}
    assert not bad, f"loops with barriers and exec-masked exits: {bad}"


@pytest.mark.parametrize("src", ["fused.hip", "experts.hip"])
def test_gemm_k_loops_wait_only_for_the_ring(asm, src):
    ks = ic.kernels(asm[src])
    found = 0
    for name, body in ks.items():
        waits = ic.gemm_loop_vm_waits(body)
        found += len(waits)
        heavy = {h: n for h, n in waits.items() if n > 2}
        assert not heavy, f"{name[:80]}: k loops with more than the ring's waits: {heavy}"
    assert found, f"no GEMM k loops found in {src}"


def test_checker_flags_a_divergent_barrier_loop():
    """The barrier check on a hand-written fragment in the compiler's
    comment format: a loop with a barrier whose latch masks exec."""
    body = """_Zfake:
.LBB0_1:                                ; =>This Loop Header: Depth=1
	s_barrier
	v_cmp_eq_u32_e32 vcc, 0, v0
	s_or_b64 s[4:5], vcc, s[4:5]
	s_andn2_b64 exec, exec, s[4:5]
	s_cbranch_execnz .LBB0_1
	s_endpgm""".split("\n")
    assert ic.barrier_loops_with_exec_exits(body) == ["BB0_1"]
    uniform = [l.replace("s_andn2_b64 exec, exec, s[4:5]", "s_and_b64 vcc, exec, s[4:5]")
                .replace("s_cbranch_execnz", "s_cbranch_vccnz") for l in body]
    assert ic.barrier_loops_with_exec_exits(uniform) == []

"""Launch-plan self-checks of the HIP library, without a GPU.

In moe_forward the bf16 router gate reads a copy of the router weights --
the split copy (three bf16 parts per fp32 weight) or the blocked fp32 copy
-- through per-wavefront indices that depend on the launch plan.
moe_check_gate_split_reach walks that plan on the host with the kernel's own
index arithmetic; here it must stay inside the copy for every shape class:
expert counts that leave the last workgroup row partly empty (E = 129 .. 160
over blocks of 4 expert blocks), hidden sizes that split K unevenly, and the
token counts where the forward switches either copy on."""
import ctypes

import pytest

from expert_token_routing_fp32_amd import _lib


@pytest.fixture(scope="module")
def reach():
    lib = _lib.load()
    fn = lib.moe_check_gate_split_reach
    fn.restype = ctypes.c_int32
    fn.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                   ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]

    def call(B, d, E):
        r, c = ctypes.c_int64(), ctypes.c_int64()
        used = fn(B, d, E, ctypes.byref(r), ctypes.byref(c))
        return used, r.value, c.value
    return call


def test_bad_arguments(reach):
    assert reach(0, 64, 8)[0] == -1
    assert reach(64, 12, 8)[0] == -1
    assert reach(64, 64, 1025)[0] == -1


def test_reported_case_e160(reach):
    # five expert blocks over workgroups of four: the second workgroup row
    # has three blocks past the last one
    used, end, size = reach(8192, 512, 160)
    assert used == 1
    assert 0 < end <= size


def test_split_reads_stay_in_the_copy(reach):
    Es = sorted(set(list(range(1, 257)) + list(range(257, 1025, 7)) + [1024]))
    ds = [8, 16, 56, 64, 120, 128, 264, 320, 328, 512, 1000, 1024, 2048, 4096, 7168]
    Bs = [8192, 16384, 32768, 65536]
    n_used = {0: 0, 1: 0, 2: 0}
    for E in Es:
        for d in ds:
            for B in Bs:
                used, end, size = reach(B, d, E)
                assert used in (0, 1, 2)
                assert end <= size, (B, d, E, end, size)
                n_used[used] += 1
    # each copy is switched on for many of these shapes
    assert n_used[1] > 100 and n_used[2] > 100, n_used

"""The C ABI, checked without a GPU: the library loads, exports every function
include/moe.h declares, the ctypes struct matches the C layout, and the
host-only helpers agree with the oracle's capacity and reject bad problems."""
import ctypes
import os
import re
import shutil
import subprocess

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    from expert_token_routing_fp32_amd import _lib
    return _lib


@pytest.fixture(scope="module")
def lib(L):
    return L.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert "moe_forward" in names and "moe_dispatch" in names and len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n


def test_probe_library_exports_its_header():
    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "moe_probe.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))
    assert names == ["moe_probe_hbm", "moe_probe_mfma", "moe_probe_mfma_flop"]
    probe = ctypes.CDLL(os.path.join(ROOT, "expert_token_routing_fp32_amd", "libmoe_probe.so"))
    for n in names:
        assert hasattr(probe, n), n
    probe.moe_probe_mfma_flop.restype = ctypes.c_double
    probe.moe_probe_mfma_flop.argtypes = [ctypes.c_int, ctypes.c_int]
    assert probe.moe_probe_mfma_flop(256, 10) == 256 * 4 * 10 * 64 * 32768.0
    # invalid arguments are rejected on the host, before any launch
    probe.moe_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p]
    assert probe.moe_probe_mfma(None, 256, 10, 1, None) == 1
    probe.moe_probe_hbm.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                    ctypes.c_void_p]
    assert probe.moe_probe_hbm(3, None, None, 16, None, 1, None) == 1
    assert probe.moe_probe_hbm(0, None, None, 16, None, 1, None) == 1
    assert probe.moe_probe_hbm(1, None, ctypes.c_void_p(16), 15, None, 1, None) == 1


def test_ctypes_layout_matches_c(L, tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    fields = [f for f, _ in L.Problem._fields_]
    ofields = [f for f, _ in L.ForwardOut._fields_]
    sfields = [f for f, _ in L.RoutingStats._fields_]
    efields = [f for f, _ in L.ExpertChoiceOut._fields_]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "moe.h"', "int main(void){",
             'printf("%zu\\n", sizeof(moe_problem_t));']
    lines += [f'printf("%zu\\n", offsetof(moe_problem_t, {f}));' for f in fields]
    lines += ['printf("%zu\\n", sizeof(moe_forward_out_t));']
    lines += [f'printf("%zu\\n", offsetof(moe_forward_out_t, {f}));' for f in ofields]
    lines += ['printf("%zu\\n", sizeof(moe_routing_stats_t));']
    lines += [f'printf("%zu\\n", offsetof(moe_routing_stats_t, {f}));' for f in sfields]
    lines += ['printf("%zu\\n", sizeof(moe_expert_choice_out_t));']
    lines += [f'printf("%zu\\n", offsetof(moe_expert_choice_out_t, {f}));' for f in efields]
    lines += ["return 0;}"]
    c = tmp_path / "layout.c"
    c.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    r = subprocess.run([gcc, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                        "-I", "/opt/rocm/include", str(c), "-o", str(exe)],
                       capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("cannot compile against the HIP headers: " + r.stderr[-300:])
    vals = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()]
    want = [ctypes.sizeof(L.Problem)] + [getattr(L.Problem, f).offset for f in fields]
    want += [ctypes.sizeof(L.ForwardOut)] + [getattr(L.ForwardOut, f).offset for f in ofields]
    want += [ctypes.sizeof(L.RoutingStats)] + [getattr(L.RoutingStats, f).offset for f in sfields]
    want += [ctypes.sizeof(L.ExpertChoiceOut)] + [getattr(L.ExpertChoiceOut, f).offset
                                                  for f in efields]
    assert vals == want


@settings(max_examples=300, deadline=None)
@given(st.integers(0, 1 << 20), st.integers(1, 16), st.integers(1, 1024),
       st.sampled_from([0.5, 1.0, 1.1, 1.25, 1.5, 2.0, 0.3, 3.7]))
def test_capacity_matches_oracle(B, k, E, c):
    from expert_token_routing_fp32_amd import _lib
    lib = _lib.load()
    assert lib.moe_capacity(B, k, E, c) == oracle.capacity(B, k, E, c)


def _prob(L, **kw):
    base = dict(B=64, d=32, E=8, k=2, c=1.25, C=-1, n_ranks=2, e_begin=0, e_end=8, f=48,
                act=L.MOE_GELU, x_dtype=L.MOE_BF16, tau=1.0, add_residual=0)
    base.update(kw)
    return L.Problem(**base)


@pytest.mark.parametrize("change,code", [
    ({}, 0),
    ({"B": 0}, 0),
    ({"B": -1}, 1), ({"d": 12}, 1), ({"d": 0}, 1), ({"E": 0}, 1), ({"k": 0}, 1), ({"k": 9}, 1),
    ({"c": 0.0}, 1), ({"c": 0.0, "C": 5}, 0), ({"n_ranks": 3}, 1), ({"n_ranks": 0}, 1),
    ({"e_begin": 3, "e_end": 2}, 1), ({"e_end": 9}, 1), ({"f": 4}, 1), ({"act": 7}, 1),
    ({"x_dtype": 5}, 1), ({"tau": 0.0}, 1), ({"add_residual": 2}, 1),
    ({"E": 2048, "e_end": 2048, "n_ranks": 1}, 2), ({"k": 17, "E": 32, "e_end": 32}, 2),
    ({"B": 1 << 30, "k": 4}, 2), ({"B": (1 << 25) + 1, "k": 1}, 2), ({"B": 1 << 25, "k": 1}, 0),
])
def test_validate_codes(L, lib, change, code):
    p = _prob(L, **change)
    assert lib.moe_validate(ctypes.byref(p)) == code
    if code:
        assert lib.moe_workspace_bytes(ctypes.byref(p), L.MOE_OP_FORWARD) == ctypes.c_size_t(-1).value
        assert lib.moe_max_kept(ctypes.byref(p)) == -1


def test_max_kept_and_workspace(L, lib):
    p = _prob(L)
    C = oracle.capacity(64, 2, 8, 1.25)
    assert lib.moe_problem_capacity(ctypes.byref(p)) == C
    assert lib.moe_max_kept(ctypes.byref(p)) == min(64 * 2, 8 * min(C, 64))
    p2 = _prob(L, C=3)
    assert lib.moe_max_kept(ctypes.byref(p2)) == 8 * 3
    for op in (L.MOE_OP_DISPATCH, L.MOE_OP_FFN, L.MOE_OP_FORWARD, L.MOE_OP_ROUTING_STATS):
        assert 0 < lib.moe_workspace_bytes(ctypes.byref(p), op) < 1 << 30
    # routing statistics: one fp32 row of E + 1 partial sums per block
    assert lib.moe_workspace_bytes(ctypes.byref(p), L.MOE_OP_ROUTING_STATS) % (4 * 9) == 0
    assert lib.moe_workspace_bytes(ctypes.byref(_prob(L, B=0)), L.MOE_OP_ROUTING_STATS) == 0


def test_status_strings(lib):
    for code in range(5):
        assert lib.moe_status_str(code)


def test_calls_reject_before_launch(L, lib):
    """Invalid problems and missing buffers are refused on the host; no GPU
    is touched (this runs without one)."""
    bad = _prob(L, E=0)
    nul = None
    assert lib.moe_route(ctypes.byref(bad), nul, nul, nul, nul) == L.MOE_ERR_INVALID
    p = _prob(L)
    assert lib.moe_route(ctypes.byref(p), nul, nul, nul, nul) == L.MOE_ERR_INVALID
    assert lib.moe_gate(ctypes.byref(p), nul, nul, nul, nul, nul) == L.MOE_ERR_INVALID
    assert lib.moe_combine(ctypes.byref(p), nul, nul, nul, nul, nul, nul) == L.MOE_ERR_INVALID
    assert lib.moe_unpack(ctypes.byref(p), nul, nul, nul, nul) == L.MOE_ERR_INVALID
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: the workspace check fails first
    r = lib.moe_dispatch(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                         fake, fake, None, 0, None)
    assert r == L.MOE_ERR_WORKSPACE
    r = lib.moe_forward(ctypes.byref(p), fake, fake, None, fake, fake, None, None, 0, None)
    assert r == L.MOE_ERR_WORKSPACE
    unaligned = ctypes.c_void_p((1 << 20) + 2)
    r = lib.moe_gate(ctypes.byref(p), unaligned, fake, None, fake, None)
    assert r == L.MOE_ERR_INVALID
    assert lib.moe_routing_stats(ctypes.byref(p), fake, fake, fake, None, None, 0,
                                 None) == L.MOE_ERR_INVALID
    out = L.RoutingStats(prob_mean=1 << 20, token_frac=1 << 20, utilization=1 << 20,
                         dropped=1 << 20, summary=1 << 20)
    assert lib.moe_routing_stats(ctypes.byref(p), fake, fake, fake, ctypes.byref(out), None, 0,
                                 None) == L.MOE_ERR_WORKSPACE
    out.summary = (1 << 20) + 4  # doubles need 8-byte alignment
    assert lib.moe_routing_stats(ctypes.byref(p), fake, fake, fake, ctypes.byref(out), fake,
                                 1 << 30, None) == L.MOE_ERR_INVALID


def test_shared_expert_host_checks(L, lib):
    """The shared expert's problem must be a single always-chosen expert on
    bf16 activations; its workspace holds H [B][f] (checked without a GPU)."""
    ps = _prob(L, E=1, k=1, c=1.0, n_ranks=1, e_begin=0, e_end=1, f=48)
    n = lib.moe_workspace_bytes(ctypes.byref(ps), L.MOE_OP_SHARED_FFN)
    assert n >= 64 * 48 * 2
    p = _prob(L)
    m = lib.moe_forward_shared_workspace_bytes(ctypes.byref(p), ctypes.byref(ps))
    assert m >= lib.moe_workspace_bytes(ctypes.byref(p), L.MOE_OP_FORWARD) + n + 64 * 32 * 2
    fake = ctypes.c_void_p(1 << 20)
    assert lib.moe_shared_ffn(ctypes.byref(p), fake, fake, fake, fake, 1 << 30,
                              None) == L.MOE_ERR_INVALID            # E != 1
    f32 = _prob(L, E=1, k=1, c=1.0, n_ranks=1, e_begin=0, e_end=1, x_dtype=L.MOE_F32)
    assert lib.moe_shared_ffn(ctypes.byref(f32), fake, fake, fake, fake, 1 << 30,
                              None) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_shared_ffn(ctypes.byref(ps), fake, fake, fake, None, 0,
                              None) == L.MOE_ERR_WORKSPACE
    assert lib.moe_forward_shared_workspace_bytes(ctypes.byref(p), ctypes.byref(p)) == \
        ctypes.c_size_t(-1).value
    bad_b = _prob(L, B=65, E=1, k=1, c=1.0, n_ranks=1, e_begin=0, e_end=1)
    assert lib.moe_forward_shared(ctypes.byref(p), ctypes.byref(bad_b), fake, fake, None, fake,
                                  fake, fake, None, fake, 1 << 30, None) == L.MOE_ERR_INVALID
    assert lib.moe_combine_shared(ctypes.byref(p), fake, fake, fake, None, None, fake,
                                  None) == L.MOE_ERR_INVALID


def test_expert_choice_host_checks(L, lib):
    """Rows E * min(C, B); all experts must be local; workspace carving."""
    p = _prob(L, n_ranks=1)          # B 64, E 8, k 2, c 1.25 -> C 20
    assert lib.moe_expert_choice_rows(ctypes.byref(p)) == 8 * 20
    big = _prob(L, n_ranks=1, C=1000)
    assert lib.moe_expert_choice_rows(ctypes.byref(big)) == 8 * 64
    assert lib.moe_workspace_bytes(ctypes.byref(p), L.MOE_OP_FORWARD_EXPERT_CHOICE) > \
        8 * 20 * (32 + 48) * 2
    part = _prob(L, n_ranks=2, e_begin=0, e_end=4)
    fake = ctypes.c_void_p(1 << 20)
    assert lib.moe_expert_choice(ctypes.byref(part), fake, fake, fake, fake, fake,
                                 None) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_forward_expert_choice(ctypes.byref(p), fake, fake, None, fake, fake, None,
                                         None, 0, None) == L.MOE_ERR_WORKSPACE


def test_overflow_policy_checks(L, lib):
    """overflow: 0 drop, 1 redirect (forward only; the router ranks
    min(2k, E) <= 16 experts)."""
    assert lib.moe_validate(ctypes.byref(_prob(L, overflow=1))) == 0
    assert lib.moe_validate(ctypes.byref(_prob(L, overflow=2))) == L.MOE_ERR_INVALID
    wide = _prob(L, E=64, k=9, e_end=64, overflow=1)    # 18 ranked choices
    assert lib.moe_validate(ctypes.byref(wide)) == L.MOE_ERR_UNSUPPORTED
    p = _prob(L, overflow=1)
    fake = ctypes.c_void_p(1 << 20)
    r = lib.moe_dispatch(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                         fake, fake, fake, 1 << 30, None)
    assert r == L.MOE_ERR_UNSUPPORTED
    # the redirect's extra buffers live in the forward workspace
    assert lib.moe_workspace_bytes(ctypes.byref(p), L.MOE_OP_FORWARD) > \
        lib.moe_workspace_bytes(ctypes.byref(_prob(L)), L.MOE_OP_FORWARD)


def test_stage_event_count_and_pairs_match_the_header(L):
    """The header's MOE_STAGE_EVENTS, the binding's constant and the stage /
    gap pairs agree: each pair is ordered, the stages (the expert FFN as its
    two GEMMs) and the gaps together walk the events 0 .. MOE_STAGE_EVENTS - 1
    in order (dispatch runs from the route's end to the pack's end, so it
    shares event 3 with the route), and the FFN's pair spans its GEMMs'."""
    import expert_token_routing_fp32_amd as moe
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    n = int(re.search(r"#define MOE_STAGE_EVENTS (\d+)", text).group(1))
    assert n == L.MOE_STAGE_EVENTS == moe.N_STAGE_EVENTS == len(L.ForwardOut().events)
    stages = {k: v for k, v in moe.STAGE_EVENTS.items() if k != "expert_ffn"}
    g1, g2 = moe.FFN_GEMM_EVENTS["gemm1"], moe.FFN_GEMM_EVENTS["gemm2"]
    assert moe.STAGE_EVENTS["expert_ffn"] == (g1[0], g2[1])
    pairs = sorted(list(stages.values()) + [g1, g2] + list(moe.LAUNCH_GAPS.values()))
    assert all(a < b for a, b in pairs)
    assert pairs[0][0] == 0 and pairs[-1][1] == n - 1
    assert all(p[1] == q[0] for p, q in zip(pairs, pairs[1:]))


def test_check_header_symbols_are_exported(lib):
    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "moe_check.h")).read(),
                 flags=re.S)
    names = sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))
    assert names == ["moe_check_gate_split_reach"]
    for n in names:
        assert hasattr(lib, n), n


def test_pack_weights_checks_full_shapes(L, lib):
    """Weights are [in, out] per expert (W1, W3 [n_local, d, f], W2
    [n_local, f, d]); the same tensors transposed have the same size and must
    be refused by their shape, before anything is allocated or launched."""
    import torch
    import expert_token_routing_fp32_amd as moe
    p = moe.make_problem(B=64, d=32, E=4, k=2, c=1.0, f=48, act="swiglu")
    W1 = torch.zeros(4, 32, 48, dtype=torch.bfloat16)
    W2 = torch.zeros(4, 48, 32, dtype=torch.bfloat16)
    for args, what in [((W1.transpose(1, 2), W1, W2), "W1"), ((W1, W1, W2.transpose(1, 2)), "W2"),
                       ((W1, W1.transpose(1, 2), W2), "W3"), ((W1[:2], W1, W2), "W1")]:
        with pytest.raises(ValueError, match=f"{what}: shape"):
            moe.pack_weights(p, *args)


def test_dispatch_noalloc_host_checks(L, lib):
    """Refusals that happen on the host, before the table's device address is
    looked up or anything is launched: a table past the fixed size, a bad
    problem, the overflow redirect (a forward-only policy)."""
    import expert_token_routing_fp32_amd as moe
    big = moe.make_problem(B=1 << 21, d=64, E=1024, k=8, c=1.0, f=16)
    assert moe.workspace_bytes(big, "dispatch") > L.MOE_DISPATCH_NOALLOC_SCRATCH_BYTES
    v = ctypes.c_void_p(16)
    args = (v,) * 11 + (None,)
    assert lib.moe_dispatch_noalloc(ctypes.byref(big), *args) == L.MOE_ERR_UNSUPPORTED
    bad = moe.make_problem(B=64, d=12, E=8, k=2)
    assert lib.moe_dispatch_noalloc(ctypes.byref(bad), *args) == L.MOE_ERR_INVALID
    nxt = moe.make_problem(B=64, d=16, E=8, k=2, overflow="next")
    assert lib.moe_dispatch_noalloc(ctypes.byref(nxt), *args) == L.MOE_ERR_UNSUPPORTED
    src = open(HEADER).read()
    assert "#define MOE_DISPATCH_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)" in src
    assert L.MOE_DISPATCH_NOALLOC_SCRATCH_BYTES == 16 << 20

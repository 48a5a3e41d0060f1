"""moe_dispatch_noalloc (no workspace argument; the library's own
device-resident table) against moe_dispatch with a caller workspace, through
the C ABI: every output bit for bit, on two calls in a row on one stream, the
second on a smaller problem (the table keeps the first call's contents, which
must not leak into the second), and a problem whose table exceeds the fixed
size is refused before any launch."""
import ctypes

import numpy as np
import pytest

from _helpers import say, to_np

pytestmark = pytest.mark.gpu

KEYS = ("pos", "keep", "dest", "expert_load", "expert_count", "expert_offset", "rank_offset",
        "pack_src", "packed")


def _inputs(B, d, E, k, seed):
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    x = torch.randn(B, d, device="cuda", generator=g).to(torch.bfloat16)
    # skewed choices (distinct per token) so that some experts overflow
    scores = torch.rand(B, E, device="cuda", generator=g) + \
        torch.linspace(1.0, 0.0, E, device="cuda")[None, :]
    idx = torch.topk(scores, k, dim=1).indices.to(torch.int32).contiguous()
    return x, idx


def _run(B, d, E, k, c, n_ranks, seed):
    import torch
    import expert_token_routing_fp32_amd as moe
    p = moe.make_problem(B=B, d=d, E=E, k=k, c=c, f=16, act="gelu", x_dtype="bf16",
                         n_ranks=n_ranks)
    x, idx = _inputs(B, d, E, k, seed)
    ref = moe.dispatch(p, x, idx)
    # the no-allocation call writes into buffers made here, pre-filled with
    # junk so that anything it leaves unwritten shows
    out = {key: torch.full_like(t, -7 if t.dtype != torch.uint8 else 200)
           for key, t in ref.items()}
    got = moe.dispatch_noalloc(p, x, idx, out=out)
    torch.cuda.synchronize()
    K = int(ref["expert_offset"][-1])
    for key in KEYS:
        a, b = to_np(got[key]), to_np(ref[key])
        if key in ("pack_src", "packed"):
            a, b = a[:K], b[:K]
        np.testing.assert_array_equal(a, b, err_msg=key)
    dropped = int((~ref["keep"].bool()).sum())
    say(f"  B={B} E={E} k={k}: K={K} dropped={dropped}, table "
        f"{moe.workspace_bytes(p, 'dispatch')} bytes: bit-exact")
    return dropped


def test_noalloc_matches_dispatch_two_calls():
    # first call: a large table (157 tiles x 256 experts); second: smaller
    d1 = _run(B=20000, d=256, E=256, k=8, c=1.0, n_ranks=8, seed=1)
    d2 = _run(B=3000, d=128, E=64, k=2, c=0.9, n_ranks=4, seed=2)
    assert d1 > 0 and d2 > 0


def test_noalloc_refuses_a_table_past_the_limit():
    import expert_token_routing_fp32_amd as moe
    from expert_token_routing_fp32_amd import _lib as L
    # 2^21 tokens x 8 choices over 1024 experts: 8192 tiles x 1024 x 4 bytes = 32 MiB
    p = moe.make_problem(B=1 << 21, d=64, E=1024, k=8, c=1.0, f=16)
    assert moe.workspace_bytes(p, "dispatch") > L.MOE_DISPATCH_NOALLOC_SCRATCH_BYTES
    v = ctypes.c_void_p(16)  # never dereferenced: refused before any launch
    st = moe.lib().moe_dispatch_noalloc(ctypes.byref(p), v, v, v, v, v, v, v, v, v, v, v, None)
    assert st == L.MOE_ERR_UNSUPPORTED

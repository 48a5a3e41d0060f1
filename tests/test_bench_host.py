"""Host-side checks of bench.py (no GPU): the one-GPU scope of --gpus and the
algorithmic byte / FLOP counts its roofline divides by.

The counts follow the work the layer must do per forward ("Expert
Parallelism", narrativegoldmine.com, "Formal Algorithm": the expert compute
is proportional to the tokens each expert receives times the cost of its
FFN); each case below is worked out by hand from the arrays it passes in.
"""
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _w(**kw):
    base = dict(B=4, d=8, E=4, k=2, f=16, x_dtype="f32", act="gelu", e_begin=0, e_end=4)
    base.update(kw)
    return SimpleNamespace(**base)


def test_algorithmic_all_local_fp32_tokens():
    # 4 tokens, 4 experts, top-2; expert rows: e0 = 2, e1 = 1, e2 = 0, e3 = 2
    # (5 kept), token 3 has both choices dropped
    keep = np.array([[1, 1], [1, 0], [1, 1], [0, 0]], dtype=bool)
    eo = np.array([0, 2, 3, 3, 5])
    dest = np.array([[0, 3], [1, -1], [2, 4], [-1, -1]])
    a = bench.algorithmic(_w(), keep, eo, dest)
    d, f = 8, 16
    assert a["K"] == 5 and a["Kloc"] == 5 and a["t_act"] == 3 and a["active_local"] == 3
    assert a["ffn_flop"] == 2 * d * f * 2 * 5                 # two matrices per kept row
    assert a["ffn_bytes"] == 3 * 2 * d * f * 2 + 4 * d * 5    # active experts' bf16 weights
    assert a["pack_bytes"] == 3 * d * 4 + 2 * d * 5            # fp32 rows read, bf16 rows out
    assert a["combine_bytes"] == 2 * d * 5 + 4 * d * 4 + 8 * 2 * 4
    assert a["route_bytes"] == 4 * (4 * 4 + 8 * 2)
    assert a["gate_flop"] == 2 * 4 * d * 4


def test_algorithmic_rank_share_bf16_tokens_gathers_local_rows():
    # experts 2..3 local (rows 3..5), SwiGLU; bf16 tokens: the first GEMM
    # gathers the local rows from x, so the pack moves only the remote ones
    keep = np.array([[1, 1], [1, 0], [1, 1], [0, 0]], dtype=bool)
    eo = np.array([0, 2, 3, 3, 5])
    dest = np.array([[0, 3], [1, -1], [2, 4], [-1, -1]])
    a = bench.algorithmic(_w(x_dtype="bf16", act="swiglu", e_begin=2, e_end=4), keep, eo, dest)
    d, f = 8, 16
    assert a["Kloc"] == 2 and a["active_local"] == 1
    assert a["ffn_flop"] == 2 * d * f * 3 * 2
    assert a["ffn_bytes"] == 1 * 2 * d * f * 3 + 4 * d * 2
    # remote rows 0, 1, 2 of tokens 0, 1, 2: each token read once, each row written
    assert a["pack_bytes"] == 3 * d * 2 + 2 * d * 3


def test_algorithmic_ep_share_flop():
    # one GPU's share of the 256-expert layer: 32 local SwiGLU experts,
    # d = 7168, f = 2048; 32976 kept local rows give 2.9045 TFLOP per forward
    Kloc = 32976
    eo = np.zeros(257, dtype=np.int64)
    eo[1:33] = np.cumsum(np.full(32, Kloc // 32))
    eo[1:33][-1] += Kloc - eo[32]
    eo[33:] = eo[32]
    w = _w(B=1, d=7168, E=256, k=8, f=2048, x_dtype="bf16", act="swiglu", e_begin=0, e_end=32)
    a = bench.algorithmic(w, np.zeros((1, 8), dtype=bool), eo, np.full((1, 8), -1))
    assert a["Kloc"] == Kloc
    assert a["ffn_flop"] == 2904538742784.0

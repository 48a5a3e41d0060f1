"""Pins for the oracle's backward pass ("Expert Parallelism",
narrativegoldmine.com, "About": training by backpropagation with an
auxiliary load-balancing loss; "Formal Algorithm": the auxiliary loss joins
the training loss).

Each backward step is checked against something other than itself:
* central finite differences of the forward oracle's own steps (with the
  routing decisions held fixed, or on perturbations too small to move them);
* torch float64 autograd of an independent dense formulation of the layer
  (no slots, no packed buffer: every kept (token, choice) pair multiplies its
  expert's MLP output by its softmax probability);
* the adjoint identity of the pack (a gather) and its transpose;
* special cases: dropped assignments get zero gradient; with capacity 0 only
  the residual and the auxiliary loss carry gradient."""
import numpy as np
import pytest
import torch

import oracle
from moe_synth import f32_to_bf16_bits


def _layer(rng, B=10, d=8, f=12, E=6, act="swiglu", bf16=False, nl=None):
    nl = E if nl is None else nl
    x = rng.standard_normal((B, d)).astype(np.float32)
    Wg = (rng.standard_normal((d, E)) * 0.7).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.3).astype(np.float32)
    W1 = (rng.standard_normal((nl, d, f)) / 3).astype(np.float32)
    W3 = (rng.standard_normal((nl, d, f)) / 3).astype(np.float32) if act == "swiglu" else None
    W2 = (rng.standard_normal((nl, f, d)) / 3).astype(np.float32)
    if bf16:
        x = f32_to_bf16_bits(x)
        W1 = f32_to_bf16_bits(W1)
        W2 = f32_to_bf16_bits(W2)
        W3 = None if W3 is None else f32_to_bf16_bits(W3)
    return x, Wg, bias, W1, W3, W2


def _vals(a):
    return oracle.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


# ---------------------------------------------------------------- combine
def test_combine_backward_finite_differences():
    rng = np.random.default_rng(1)
    B, k, K, d = 7, 3, 15, 5
    ret = rng.standard_normal((K, d))
    dest = np.full((B, k), -1, dtype=np.int32)
    perm = rng.permutation(K)
    flat = [(t, j) for t in range(B) for j in range(k)]
    keep_ids = rng.choice(len(flat), size=K, replace=False)
    for n, q in enumerate(keep_ids):
        t, j = flat[q]
        dest[t, j] = perm[n]
    w = rng.random((B, k)).astype(np.float32).astype(np.float64)
    dy = rng.standard_normal((B, d))
    dret, dw = oracle.combine_backward(dy, ret, dest, w)

    def L(ret_, w_):
        return float((dy * oracle.combine(ret_, dest, w_)).sum())
    h = 1e-6
    for _ in range(6):
        r, c = rng.integers(K), rng.integers(d)
        e = np.zeros_like(ret)
        e[r, c] = h
        fd = (L(ret + e, w) - L(ret - e, w)) / (2 * h)
        assert abs(fd - dret[r, c]) < 1e-8
    # w enters combine at float32 precision, so perturb by float32-exact steps
    h = 2.0 ** -12
    for t in range(B):
        for j in range(k):
            e = np.zeros_like(w)
            e[t, j] = h
            fd = (L(ret, w + e) - L(ret, w - e)) / (2 * h)
            assert abs(fd - dw[t, j]) < 1e-9
            if dest[t, j] < 0:
                assert dw[t, j] == 0.0


def test_combine_backward_rows_subset():
    rng = np.random.default_rng(2)
    B, k, K, d = 9, 2, 12, 4
    ret = rng.standard_normal((K, d))
    dest = np.full((B, k), -1, dtype=np.int32)
    slots = rng.permutation(B * k)[:K]
    dest.reshape(-1)[slots] = np.arange(K)
    w = rng.random((B, k))
    dy = rng.standard_normal((B, d))
    full_r, full_w = oracle.combine_backward(dy, ret, dest, w)
    rows = np.array([0, 3, 4, 11])
    sub_r, sub_w = oracle.combine_backward(dy, ret[rows], dest, w, rows=rows)
    np.testing.assert_array_equal(sub_r, full_r[rows])
    listed = np.isin(dest, rows)
    np.testing.assert_array_equal(sub_w[listed], full_w[listed])
    assert np.isnan(sub_w[(dest >= 0) & ~listed]).all()


# ---------------------------------------------------------------- route
@pytest.mark.parametrize("tau,aux", [(1.0, 0.0), (0.7, 0.0), (1.3, 0.05)])
def test_route_backward_finite_differences(tau, aux):
    rng = np.random.default_rng(3)
    B, E, k = 6, 7, 3
    l = (rng.standard_normal((B, E)) * 2).astype(np.float32)
    idx, _ = oracle.route(l, k, tau)
    dw = rng.standard_normal((B, k))
    n = np.bincount(idx.reshape(-1), minlength=E)
    dl = oracle.route_backward(l, idx, dw, tau, aux, n)

    def L(lv):
        p = oracle.softmax(lv, tau)
        w = np.take_along_axis(p, idx.astype(np.int64), axis=1)
        return float((dw * w).sum() + aux * ((n / B) * p.mean(axis=0)).sum())
    h = 2.0 ** -12  # float32-exact perturbations (softmax reads float32 logits)
    for t in range(B):
        for e in range(E):
            d_ = np.zeros_like(l)
            d_[t, e] = h
            fd = (L(l + d_) - L(l - d_)) / (2 * h)
            assert abs(fd - dl[t, e]) < 2e-6 * max(1.0, abs(dl[t, e]))


def test_route_backward_against_torch():
    rng = np.random.default_rng(4)
    B, E, k, tau, aux = 20, 9, 2, 0.9, 0.3
    l = (rng.standard_normal((B, E)) * 2).astype(np.float32)
    idx, _ = oracle.route(l, k, tau)
    dw = rng.standard_normal((B, k))
    n = np.bincount(idx.reshape(-1), minlength=E)
    dl = oracle.route_backward(l, idx, dw, tau, aux, n)
    tl = torch.tensor(l.astype(np.float64), requires_grad=True)
    p = torch.softmax(tl / tau, dim=1)
    w = p.gather(1, torch.from_numpy(idx.astype(np.int64)))
    L = (torch.from_numpy(dw) * w).sum() + aux * (torch.from_numpy(n / B) * p.mean(0)).sum()
    L.backward()
    np.testing.assert_allclose(dl, tl.grad.numpy(), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- expert MLP
@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_expert_mlp_backward_against_torch(act):
    rng = np.random.default_rng(5)
    n, d, f = 7, 6, 10
    xr = rng.standard_normal((n, d))
    W1 = f32_to_bf16_bits((rng.standard_normal((d, f)) / 2).astype(np.float32))
    W3 = f32_to_bf16_bits((rng.standard_normal((d, f)) / 2).astype(np.float32))
    W2 = f32_to_bf16_bits((rng.standard_normal((f, d)) / 3).astype(np.float32))
    dout = rng.standard_normal((n, d))
    dxr, dW1, dW2, dW3 = oracle.expert_mlp_backward(xr, W1, W2, W3 if act == "swiglu" else None,
                                                    act, dout)
    tx = torch.tensor(xr, requires_grad=True)
    tw = [torch.tensor(_vals(W), requires_grad=True) for W in (W1, W3, W2)]
    z1 = tx @ tw[0]
    h = torch.nn.functional.gelu(z1) if act == "gelu" else \
        torch.nn.functional.silu(z1) * (tx @ tw[1])
    (torch.from_numpy(dout) * (h @ tw[2])).sum().backward()
    np.testing.assert_allclose(dxr, tx.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dW1, tw[0].grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dW2, tw[2].grad.numpy(), rtol=1e-12, atol=1e-12)
    if act == "swiglu":
        np.testing.assert_allclose(dW3, tw[1].grad.numpy(), rtol=1e-12, atol=1e-12)
    else:
        assert dW3 is None


def test_expert_mlp_backward_finite_differences():
    rng = np.random.default_rng(6)
    n, d, f = 4, 5, 6
    xr = rng.standard_normal((n, d))
    # weights enter the oracle at float32 precision: float32 weights and
    # float32-exact steps
    W1 = (rng.standard_normal((d, f)) / 2).astype(np.float32)
    W3 = (rng.standard_normal((d, f)) / 2).astype(np.float32)
    W2 = (rng.standard_normal((f, d)) / 3).astype(np.float32)
    dout = rng.standard_normal((n, d))
    for act in ("gelu", "swiglu"):
        g = oracle.expert_mlp_backward(xr, W1, W2, W3, act, dout)

        def L(xv, a, b, c):
            return float((dout * oracle.expert_mlp(xv, a, c, b, act)).sum())
        for which, arr in ((0, xr), (1, W1), (2, W2), (3, W3)):
            h = 1e-5 if which == 0 else 2.0 ** -12
            if act == "gelu" and which == 3:
                continue
            for _ in range(3):
                pos = tuple(rng.integers(s) for s in arr.shape)
                e = np.zeros_like(arr)
                e[pos] = h
                args_p = [xr, W1, W3, W2]
                args_m = [xr, W1, W3, W2]
                slot = {0: 0, 1: 1, 2: 3, 3: 2}[which]
                args_p[slot] = arr + e
                args_m[slot] = arr - e
                fd = (L(*args_p) - L(*args_m)) / (2 * h)
                assert abs(fd - g[which][pos]) < 1e-6 * max(1.0, abs(fd))


# ---------------------------------------------------------------- pack / gate
def test_dispatch_backward_is_the_adjoint_of_the_pack():
    rng = np.random.default_rng(7)
    B, k, d, E = 12, 3, 5, 6
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(B)]).astype(np.int32)
    pos, keep, load, count = oracle.assign_slots(idx, E, 4)
    eo, ro, dest, ps = oracle.layout(idx, pos, keep, E, 1, 4)
    x = rng.standard_normal((B, d))
    v = rng.standard_normal((len(ps), d))
    lhs = float((x[ps] * v).sum())
    rhs = float((x * oracle.dispatch_backward(v, dest)).sum())
    assert abs(lhs - rhs) < 1e-12


def test_gate_backward_finite_differences():
    rng = np.random.default_rng(8)
    B, d, E = 5, 4, 3
    x = rng.standard_normal((B, d)).astype(np.float32)
    Wg = rng.standard_normal((d, E)).astype(np.float32)
    dl = rng.standard_normal((B, E))
    dx, dWg, db = oracle.gate_backward(x, Wg, dl)
    xv, wv = x.astype(np.float64), Wg.astype(np.float64)
    np.testing.assert_allclose(dx, dl @ wv.T, rtol=1e-14)
    # linear map: the directional derivative is exact
    for _ in range(4):
        V = rng.standard_normal((d, E))
        assert abs(float((dl * (xv @ V)).sum()) - float((dWg * V).sum())) < 1e-12
    assert np.allclose(db, dl.sum(axis=0))


# ---------------------------------------------------------------- whole layer
def _torch_layer_grads(x, Wg, bias, W1, W3, W2, fwd, dy, act, tau, aux, e_begin, e_end,
                       add_residual):
    """Independent dense formulation: y[t] = sum over kept (t, j) of
    p[t, e] * out_e(x_t) with e = idx[t, j] (out_e the MLP for a local
    expert, the bf16 copy of x_t for a remote one), plus the residual.  The
    logits take the oracle's float32 values but their gradient flows into x,
    Wg and bias (straight through the rounding)."""
    tx = torch.tensor(_vals(x), requires_grad=True)
    tWg = torch.tensor(Wg.astype(np.float64), requires_grad=True)
    tb = torch.tensor(bias.astype(np.float64), requires_grad=True)
    tW = [None if W is None else torch.tensor(_vals(W), requires_grad=True) for W in (W1, W3, W2)]
    lin = tx @ tWg + tb
    l = torch.from_numpy(fwd["logits"].astype(np.float64)) + (lin - lin.detach())
    p = torch.softmax(l / tau, dim=1)
    B, k = fwd["idx"].shape
    xb = torch.from_numpy(oracle.bf16_bits_to_f64(oracle.pack(x, np.arange(B))))
    y = torch.zeros_like(tx)
    for t in range(B):
        for j in range(k):
            if not fwd["keep"][t, j]:
                continue
            e = int(fwd["idx"][t, j])
            if e_begin <= e < e_end:
                i = e - e_begin
                z1 = tx[t] @ tW[0][i]
                h = torch.nn.functional.gelu(z1) if act == "gelu" else \
                    torch.nn.functional.silu(z1) * (tx[t] @ tW[1][i])
                out = h @ tW[2][i]
            else:
                # remote expert: the identity return (value: the bf16 copy)
                out = xb[t] + (tx[t] - tx[t].detach())
            # the combine takes the weight at float32 precision: straight through
            w = p[t, e]
            w32 = float(np.float32(w.item()))
            y[t] = y[t] + (w32 + (w - w.detach())) * out
    if add_residual:
        y = y + tx
    n = torch.from_numpy(fwd["expert_load"].astype(np.float64))
    L = (torch.from_numpy(np.asarray(dy, np.float64)) * y).sum() + aux * ((n / B) * p.mean(0)).sum()
    L.backward()
    g = dict(dx=tx.grad.numpy(), dWg=tWg.grad.numpy(), dbias=tb.grad.numpy(),
             dW1=tW[0].grad.numpy(), dW2=tW[2].grad.numpy())
    if tW[1] is not None:
        g["dW3"] = tW[1].grad.numpy()
    return g


@pytest.mark.parametrize("case", ["swiglu_drops", "gelu_residual_aux", "remote_rows_bf16"])
def test_layer_backward_against_torch_autograd(case):
    rng = np.random.default_rng({"swiglu_drops": 11, "gelu_residual_aux": 12,
                                 "remote_rows_bf16": 13}[case])
    act = "gelu" if case == "gelu_residual_aux" else "swiglu"
    bf16 = case == "remote_rows_bf16"
    E = 6
    e_begin, e_end = (0, 3) if case == "remote_rows_bf16" else (0, E)
    x, Wg, bias, W1, W3, W2 = _layer(rng, B=12, E=E, act=act, bf16=bf16, nl=e_end - e_begin)
    k, c = 2, (0.6 if case == "swiglu_drops" else 2.0)
    tau, aux, res = (1.0, 0.0, False) if case != "gelu_residual_aux" else (0.8, 0.1, True)
    fwd = oracle.forward(x, Wg, bias, W1, W3, W2, k=k, c=c, act=act, tau=tau,
                         n_ranks=2 if case == "remote_rows_bf16" else 1, e_begin=e_begin,
                         e_end=e_end, add_residual=res)
    if case == "swiglu_drops":
        assert (~fwd["keep"]).any()
    dy = rng.standard_normal(fwd["y"].shape)
    g = oracle.backward(x, Wg, bias, W1, W3, W2, fwd, dy, act=act, e_begin=e_begin, e_end=e_end,
                        tau=tau, aux_coef=aux, add_residual=res)
    ref = _torch_layer_grads(x, Wg, bias, W1, W3, W2, fwd, dy, act, tau, aux, e_begin, e_end, res)
    for key, r in ref.items():
        np.testing.assert_allclose(g[key], r, rtol=1e-10, atol=1e-12, err_msg=key)
    assert (g["dw"][~fwd["keep"]] == 0).all()


def test_layer_backward_finite_differences_on_expert_weights():
    """Perturbing an expert weight moves no routing decision, so the forward
    oracle's loss is smooth in it; central differences match dW."""
    rng = np.random.default_rng(14)
    x, Wg, bias, W1, W3, W2 = _layer(rng, B=9, E=4, act="swiglu")
    kw = dict(k=2, c=0.8, act="swiglu")
    fwd = oracle.forward(x, Wg, bias, W1, W3, W2, **kw)
    dy = rng.standard_normal(fwd["y"].shape)
    g = oracle.backward(x, Wg, bias, W1, W3, W2, fwd, dy, act="swiglu")

    def L(a, b, c_):
        return float((dy * oracle.forward(x, Wg, bias, a, b, c_, **kw)["y"]).sum())
    h = 2.0 ** -12  # float32-exact steps on float32 weights
    for name, arr in (("dW1", W1), ("dW3", W3), ("dW2", W2)):
        for _ in range(4):
            pos = tuple(rng.integers(s) for s in arr.shape)
            e = np.zeros_like(arr)
            e[pos] = h
            args = {"dW1": (0, W1), "dW3": (1, W3), "dW2": (2, W2)}[name]
            p_, m_ = [W1, W3, W2], [W1, W3, W2]
            p_[args[0]] = arr + e
            m_[args[0]] = arr - e
            fd = (L(*p_) - L(*m_)) / (2 * h)
            assert abs(fd - g[name][pos]) < 1e-5 * max(1.0, abs(fd)), (name, pos)


def test_zero_capacity_leaves_only_residual_and_aux():
    rng = np.random.default_rng(15)
    x, Wg, bias, W1, W3, W2 = _layer(rng, B=8, E=5, act="gelu")
    fwd = oracle.forward(x, Wg, bias, W1, None, W2, k=2, c=1.0, act="gelu", C=0,
                         add_residual=True)
    dy = rng.standard_normal(fwd["y"].shape)
    g = oracle.backward(x, Wg, bias, W1, None, W2, fwd, dy, act="gelu", aux_coef=0.0,
                        add_residual=True)
    np.testing.assert_array_equal(g["dx"], dy)
    assert (g["dW1"] == 0).all() and (g["dW2"] == 0).all() and (g["dlogits"] == 0).all()
    g2 = oracle.backward(x, Wg, bias, W1, None, W2, fwd, dy, act="gelu", aux_coef=0.5,
                         add_residual=True)
    assert np.abs(g2["dlogits"]).max() > 0 and (g2["dW1"] == 0).all()

"""Pins of the residual-MoE oracle (oracle/residual_moe.py, reading R16):
its special cases against the plain layer and dense FFNs computed
separately with torch.nn.functional, and its backward against float64
central differences of its own forward and against torch.autograd through
a separately written per-token formulation."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import moe_oracle as O
from oracle import residual_moe as R


def _case(seed, T=7, d=6, E=3, h=5, k=2):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(T, d))
    lg = rng.normal(size=(T, E)) * 2
    w1, b1 = rng.normal(size=(E, h, d)) * 0.4, rng.normal(size=(E, h)) * 0.1
    w2, b2 = rng.normal(size=(E, d, h)) * 0.4, rng.normal(size=(E, d)) * 0.1
    mlp = (rng.normal(size=(h, d)) * 0.4, rng.normal(size=h) * 0.1, rng.normal(size=(d, h)) * 0.4,
           rng.normal(size=d) * 0.1)
    cw, cb = rng.normal(size=(2, d)) * 0.5, rng.normal(size=2) * 0.2
    return x, lg, (w1, b1, w2, b2), mlp, cw, cb


def _torch_ffn(x, w1, b1, w2, b2):
    t = lambda v: torch.as_tensor(v, dtype=torch.float64)
    return F.linear(F.gelu(F.linear(t(x), t(w1), t(b1))), t(w2), t(b2)).numpy()


def test_forward_is_the_mix_of_the_layer_and_a_dense_ffn():
    x, lg, (w1, b1, w2, b2), mlp, cw, cb = _case(0)
    kw = dict(k=2, capacity_factor=10.0, min_capacity=1, drop_tokens=True, act=O.ACT_GELU, dtype="f64")
    r = R.forward(x, lg, w1, b1, w2, b2, mlp, cw, cb, **kw)
    plain = O.layer_forward(x, lg, w1, b1, w2, b2, **kw)
    dense = _torch_ffn(x, *mlp)
    c = torch.softmax(torch.as_tensor(x @ cw.T + cb), dim=1).numpy()
    np.testing.assert_allclose(r["out"], c[:, :1] * plain["out"] + c[:, 1:] * dense, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["coef"].sum(axis=1), 1.0, rtol=1e-14)
    # without coefficient weights: the plain residual sum
    r0 = R.forward(x, lg, w1, b1, w2, b2, mlp, **kw)
    np.testing.assert_allclose(r0["out"], plain["out"] + dense, rtol=1e-12, atol=1e-12)
    # routing, counts and the loss are the layer's
    for key in ("expert_idx", "slot", "expert_count", "gate_loss"):
        assert np.array_equal(r[key], plain[key]), key


def test_single_expert_mix_reduces_to_two_dense_ffns():
    """E = 1, k = 1, no drops: every token's weight is 1, so the layer is
    c0 * FFN_expert(x) + c1 * FFN_mlp(x)."""
    x, _, (w1, b1, w2, b2), mlp, cw, cb = _case(1, E=1, k=1)
    lg = np.zeros((x.shape[0], 1))
    r = R.forward(x, lg, w1, b1, w2, b2, mlp, cw, cb, k=1, capacity_factor=1.0, min_capacity=1,
                  drop_tokens=False, act=O.ACT_GELU, dtype="f64")
    c = R.coefficients(x, cw, cb)
    want = c[:, :1] * _torch_ffn(x, w1[0], b1[0], w2[0], b2[0]) + c[:, 1:] * _torch_ffn(x, *mlp)
    np.testing.assert_allclose(r["out"], want, rtol=1e-12, atol=1e-12)


def test_bf16_rounding_points():
    x, lg, (w1, b1, w2, b2), mlp, cw, cb = _case(2)
    x = O.round_bf16(x)
    r = R.forward(x, lg, w1, b1, w2, b2, mlp, cw, cb, k=2, capacity_factor=10.0, min_capacity=1, drop_tokens=True,
                  act=O.ACT_GELU, dtype="bf16")
    assert np.array_equal(r["mlp_y"], O.round_bf16(r["mlp_y"]))
    assert np.array_equal(r["out"], O.round_bf16(r["coef"][:, :1] * r["moe"] + r["coef"][:, 1:] * r["mlp_y"]))


@pytest.mark.parametrize("coef", [True, False])
def test_backward_against_central_differences(coef):
    x, lg, (w1, b1, w2, b2), mlp, cw, cb = _case(3)
    rng = np.random.default_rng(9)
    wr = rng.normal(size=(3, x.shape[1])) * 0.5
    dout = rng.normal(size=x.shape)
    dloss = 0.4
    kw = dict(k=2, capacity_factor=10.0, min_capacity=1, drop_tokens=True, act=O.ACT_GELU, dtype="f64")

    def objective(xx=x, ww=wr, m=mlp, c_w=cw, c_b=cb):
        r = R.forward(xx, O.router_logits(xx, ww), w1, b1, w2, b2, m, c_w if coef else None,
                      c_b if coef else None, **kw)
        return float((dout * r["out"]).sum() + dloss * r["gate_loss"]), r

    _, r = objective()
    g = R.backward(x, wr, r, w1, w2, mlp, cw if coef else None, dout, dloss, act=O.ACT_GELU, dtype="f64")
    eps = 1e-6

    def fd(f, arr, idx):
        p, m = arr.copy(), arr.copy()
        p[idx] += eps
        m[idx] -= eps
        return (f(p)[0] - f(m)[0]) / (2 * eps)

    for idx in [(0, 0), (3, 2), (6, 5)]:
        assert abs(g["dx"][idx] - fd(lambda a: objective(xx=a), x, idx)) < 1e-6
    for idx in [(0, 1), (2, 4)]:
        assert abs(g["dw_router"][idx] - fd(lambda a: objective(ww=a), wr, idx)) < 1e-6
    names = ("mlp_dw1", "mlp_db1", "mlp_dw2", "mlp_db2")
    for i, name in enumerate(names):
        arr = mlp[i]
        for idx in ([(0, 0), (2, 3)] if arr.ndim == 2 else [(0,), (3,)]):
            def f(a, i=i):
                m = list(mlp)
                m[i] = a
                return objective(m=tuple(m))
            assert abs(g[name][idx] - fd(f, arr, idx)) < 1e-6, name
    if coef:
        for idx in [(0, 0), (1, 5)]:
            assert abs(g["dcoef_w"][idx] - fd(lambda a: objective(c_w=a), cw, idx)) < 1e-6
        for idx in [(0,), (1,)]:
            assert abs(g["dcoef_b"][idx] - fd(lambda a: objective(c_b=a), cb, idx)) < 1e-6
    # an expert weight, through the MoE branch scaled by c0
    def fe(a):
        return (float((dout * R.forward(x, O.router_logits(x, wr), a, b1, w2, b2, mlp, cw if coef else None,
                                        cb if coef else None, **kw)["out"]).sum()
                      + dloss * R.forward(x, O.router_logits(x, wr), a, b1, w2, b2, mlp, None, None,
                                          **kw)["gate_loss"]),)
    assert abs(g["dw1"][1, 2, 3] - fd(fe, w1, (1, 2, 3))) < 1e-6


def test_backward_against_autograd_per_token():
    """A per-token formulation of the residual layer (no capacity), written
    here with torch ops, differentiated by torch.autograd."""
    x, lg0, (w1, b1, w2, b2), mlp, cw, cb = _case(4)
    rng = np.random.default_rng(5)
    wr = rng.normal(size=(3, x.shape[1])) * 0.5
    dout = rng.normal(size=x.shape)
    kw = dict(k=2, capacity_factor=1.0, min_capacity=1, drop_tokens=False, act=O.ACT_GELU, dtype="f64")
    r = R.forward(x, O.router_logits(x, wr), w1, b1, w2, b2, mlp, cw, cb, **kw)
    g = R.backward(x, wr, r, w1, w2, mlp, cw, dout, 0.0, act=O.ACT_GELU, dtype="f64")
    t = lambda v: torch.tensor(v, dtype=torch.float64, requires_grad=True)
    X, WR, CW, CB = t(x), t(wr), t(cw), t(cb)
    M = [t(v) for v in mlp]
    idx = r["expert_idx"]
    p = torch.softmax(X @ WR.T, dim=1)
    outs = []
    for i in range(x.shape[0]):
        moe = 0
        for j in range(2):
            e = int(idx[i, j])
            ffn = F.linear(F.gelu(F.linear(X[i], torch.as_tensor(w1[e]), torch.as_tensor(b1[e]))),
                           torch.as_tensor(w2[e]), torch.as_tensor(b2[e]))
            moe = moe + p[i, e] * ffn
        dense = F.linear(F.gelu(F.linear(X[i], M[0], M[1])), M[2], M[3])
        c = torch.softmax(X[i] @ CW.T + CB, dim=0)
        outs.append(c[0] * moe + c[1] * dense)
    (torch.stack(outs) * torch.as_tensor(dout)).sum().backward()
    np.testing.assert_allclose(g["dx"], X.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(g["dw_router"], WR.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(g["dcoef_w"], CW.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(g["dcoef_b"], CB.grad.numpy(), rtol=1e-9, atol=1e-11)
    for i, name in enumerate(("mlp_dw1", "mlp_db1", "mlp_dw2", "mlp_db2")):
        np.testing.assert_allclose(g[name], M[i].grad.numpy(), rtol=1e-9, atol=1e-11)


def test_pyramid_of_layers():
    """The pyramid ([ds.moe] §2.3, §4.2: num_experts = [4, 8, 16]) is three
    layers with their own expert counts; each is the residual layer with its
    E, applied in turn."""
    rng = np.random.default_rng(6)
    T, d, h = 9, 6, 5
    x = rng.normal(size=(T, d))
    for E in (4, 8, 16):
        w1, b1 = rng.normal(size=(E, h, d)) * 0.3, rng.normal(size=(E, h)) * 0.1
        w2, b2 = rng.normal(size=(E, d, h)) * 0.3, rng.normal(size=(E, d)) * 0.1
        mlp = (rng.normal(size=(h, d)) * 0.3, rng.normal(size=h) * 0.1, rng.normal(size=(d, h)) * 0.3,
               rng.normal(size=d) * 0.1)
        wr = rng.normal(size=(E, d))
        r = R.forward(x, O.router_logits(x, wr), w1, b1, w2, b2, mlp, k=1, capacity_factor=2.0, min_capacity=1,
                      drop_tokens=True, act=O.ACT_GELU, dtype="f64")
        assert r["expert_count"].shape == (E,) and r["out"].shape == (T, d)
        x = r["out"]
    assert np.isfinite(x).all()

"""Pins of the oracle's full-layer backward (``layer_backward``).

Independent checks, none of which reuses the backward's own formulas:
  * central finite differences of the oracle's forward (router Linear ->
    ``layer_forward``) for every input and parameter, in float64 with no
    storage rounding, on small problems whose routing does not move under the
    perturbation (drops included);
  * torch.autograd through a separately written per-token formulation of the
    same layer (torch ops, float64), as in the pages' pseudocode
    ([DS-MoE-traps] ch.1 moe_forward);
  * the sparsity the pages state for the top-k router ([DS-MoE-traps] §3.1
    TopKRouter: gradient only at the chosen positions): with weights
    renormalised over the top k and a loss that depends on counts only, the
    logit gradient is exactly zero outside the top k; and experts that get no
    token get zero weight gradients ([DS-MoE-traps] §2.1 gradient mask).
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O


def _problem(seed, T=9, d=6, E=4, h=5, k=2):
    rng = np.random.default_rng(seed)
    return dict(x=rng.normal(size=(T, d)), wr=rng.normal(size=(E, d)), br=rng.normal(size=E) * 0.3,
                w1=rng.normal(size=(E, h, d)) * 0.5, b1=rng.normal(size=(E, h)) * 0.2,
                w2=rng.normal(size=(E, d, h)) * 0.5, b2=rng.normal(size=(E, d)) * 0.2,
                dout=rng.normal(size=(T, d)), k=k)


def _forward(P, cfg):
    logits = O.router_logits(P["x"], P["wr"], P["br"])
    r = O.layer_forward(P["x"], logits, P["w1"], P["b1"], P["w2"], P["b2"], k=P["k"],
                        capacity_factor=cfg["cf"], min_capacity=cfg["min_cap"], drop_tokens=cfg["drop"],
                        act=cfg["act"], dtype="f64", normalize_topk=cfg["norm"], loss_kind=cfg["loss"])
    return r


def _objective(P, cfg, dloss):
    r = _forward(P, cfg)
    return float(np.sum(P["dout"] * r["out"]) + dloss * r["gate_loss"]), r


CFGS = [
    dict(cf=1.0, min_cap=1, drop=True, act=O.ACT_GELU, norm=False, loss=O.LOSS_BALANCE),
    dict(cf=0.6, min_cap=1, drop=True, act=O.ACT_RELU, norm=True, loss=O.LOSS_BALANCE),
    dict(cf=1.0, min_cap=1, drop=False, act=O.ACT_NONE, norm=False, loss=O.LOSS_USAGE_STD),
    dict(cf=0.8, min_cap=2, drop=True, act=O.ACT_GELU, norm=True, loss=O.LOSS_USAGE_STD),
]


@pytest.mark.parametrize("ci", range(len(CFGS)))
def test_layer_backward_matches_finite_differences(ci):
    cfg = CFGS[ci]
    P = _problem(100 + ci)
    dloss = 0.7
    base, r = _objective(P, cfg, dloss)
    g = O.layer_backward(P["x"], P["wr"], r, P["w1"], P["w2"], P["dout"], dloss, act=cfg["act"], dtype="f64",
                         normalize_topk=cfg["norm"], loss_kind=cfg["loss"])
    # the biases of the expert Linears and of the router
    grads = dict(x=g["dx"], wr=g["dw_router"], br=g["db_router"], w1=g["dw1"], b1=g["db1"], w2=g["dw2"],
                 b2=g["db2"])
    eps = 1e-6
    for name, want in grads.items():
        p = P[name]
        fd = np.zeros_like(p)
        for i in np.ndindex(p.shape):
            old = p[i]
            p[i] = old + eps
            up, ru = _objective(P, cfg, dloss)
            p[i] = old - eps
            dn, rd = _objective(P, cfg, dloss)
            p[i] = old
            # the routing must not move under the perturbation
            assert np.array_equal(ru["expert_idx"], r["expert_idx"]) and np.array_equal(ru["slot"], r["slot"])
            assert np.array_equal(rd["expert_idx"], r["expert_idx"]) and np.array_equal(rd["slot"], r["slot"])
            fd[i] = (up - dn) / (2 * eps)
        np.testing.assert_allclose(want, fd, rtol=1e-5, atol=1e-7, err_msg=name)
    if cfg["drop"]:
        assert (r["slot"] < 0).any(), "the case should drop some claims"


def _torch_layer(x, wr, br, w1, b1, w2, b2, idx, slot, cfg):
    """Per-token formulation: out[t] = sum_j kept(t,j) * w[t,j] * FFN_e(x[t])
    with w from the softmax over all experts (or renormalised over the k),
    plus the gate loss from the probabilities (routing held fixed)."""
    logits = x @ wr.T + br
    p = torch.softmax(logits, dim=1)
    T, k = idx.shape
    E = wr.shape[0]
    outs = []
    for t in range(T):
        pk = torch.stack([p[t, int(idx[t, j])] for j in range(k)])
        wk = pk / pk.sum() if cfg["norm"] else pk
        o = torch.zeros_like(x[t])
        for j in range(k):
            if slot[t, j] < 0:
                continue
            e = int(idx[t, j])
            a = w1[e] @ x[t] + b1[e]
            if cfg["act"] == O.ACT_GELU:
                hh = torch.nn.functional.gelu(a)
            elif cfg["act"] == O.ACT_RELU:
                hh = torch.relu(a)
            else:
                hh = a
            o = o + wk[j] * (w2[e] @ hh + b2[e])
        outs.append(o)
    out = torch.stack(outs)
    if cfg["loss"] == O.LOSS_BALANCE:
        ce = torch.tensor(np.bincount(idx[:, 0], minlength=E) / T, dtype=torch.float64)
        loss = E * torch.sum(p.mean(dim=0) * ce)
    else:
        loss = torch.zeros((), dtype=torch.float64)
    return out, loss


@pytest.mark.parametrize("ci", range(len(CFGS)))
def test_layer_backward_matches_autograd(ci):
    cfg = CFGS[ci]
    P = _problem(200 + ci, T=11, d=8, E=5, h=6)
    dloss = -1.3
    _, r = _objective(P, cfg, dloss)
    g = O.layer_backward(P["x"], P["wr"], r, P["w1"], P["w2"], P["dout"], dloss, act=cfg["act"], dtype="f64",
                         normalize_topk=cfg["norm"], loss_kind=cfg["loss"])
    tens = {n: torch.tensor(P[n], dtype=torch.float64, requires_grad=True)
            for n in ("x", "wr", "br", "w1", "b1", "w2", "b2")}
    out, loss = _torch_layer(tens["x"], tens["wr"], tens["br"], tens["w1"], tens["b1"], tens["w2"], tens["b2"],
                             r["expert_idx"], r["slot"], cfg)
    obj = (torch.tensor(P["dout"]) * out).sum() + dloss * loss
    obj.backward()
    pairs = dict(x="dx", wr="dw_router", br="db_router", w1="dw1", b1="db1", w2="dw2", b2="db2")
    for n, key in pairs.items():
        np.testing.assert_allclose(g[key], tens[n].grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=n)


def test_renormalised_topk_gradient_is_sparse_and_idle_experts_get_nothing():
    P = _problem(7, T=16, d=6, E=8, h=4)
    P["br"][5] = -100.0   # expert 5 never wins a token
    cfg = dict(cf=1.0, min_cap=1, drop=True, act=O.ACT_GELU, norm=True, loss=O.LOSS_USAGE_STD)
    _, r = _objective(P, cfg, 0.0)
    g = O.layer_backward(P["x"], P["wr"], r, P["w1"], P["w2"], P["dout"], 0.5, act=cfg["act"], dtype="f64",
                         normalize_topk=True, loss_kind=O.LOSS_USAGE_STD)
    dl = g["dlogits"]
    chosen = np.zeros_like(dl, dtype=bool)
    np.put_along_axis(chosen, r["expert_idx"], True, axis=1)
    assert np.abs(dl[~chosen]).max() < 1e-12
    assert np.abs(dl[chosen]).max() > 1e-4
    idle = np.where(r["expert_count"] == 0)[0]
    assert idle.size, "the case should leave an expert without tokens"
    for e in idle:
        assert not g["dw1"][e].any() and not g["dw2"][e].any() and not g["db1"][e].any()


def test_given_logits_returns_logit_gradient():
    """Without a router (logits are inputs) the gradient stops at the logits;
    it matches finite differences of the layer in the logits."""
    P = _problem(9, T=6, d=4, E=3, h=3, k=1)
    cfg = dict(cf=1.0, min_cap=1, drop=True, act=O.ACT_RELU, norm=False, loss=O.LOSS_BALANCE)
    logits = O.router_logits(P["x"], P["wr"], P["br"])

    def obj(L):
        r = O.layer_forward(P["x"], L, P["w1"], P["b1"], P["w2"], P["b2"], k=1, capacity_factor=1.0,
                            min_capacity=1, drop_tokens=True, act=cfg["act"], dtype="f64")
        return float(np.sum(P["dout"] * r["out"]) + 0.4 * r["gate_loss"]), r

    _, r = obj(logits)
    g = O.layer_backward(P["x"], None, r, P["w1"], P["w2"], P["dout"], 0.4, act=cfg["act"], dtype="f64")
    assert g["dw_router"] is None
    fd = np.zeros_like(logits)
    for i in np.ndindex(logits.shape):
        L = logits.copy()
        L[i] += 1e-6
        up, _ = obj(L)
        L[i] -= 2e-6
        dn, _ = obj(L)
        fd[i] = (up - dn) / 2e-6
    np.testing.assert_allclose(g["dlogits"], fd, rtol=1e-5, atol=1e-7)

"""Pins of the oracle's storage rounding, activations, dispatch, expert FFNs,
combine and FFN backward (CPU only).

Pins: torch's own float32->bfloat16 conversion (a library routine), the erf
closed form of GELU from ``math.erf``, the single-expert reduction to a dense
FFN computed with ``torch.nn.functional`` in float64, the per-token
formulation of the layer, central finite differences and ``torch.autograd`` on
tiny shapes.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import moe_oracle as O


# ----------------------------------------------------------------- bf16 rounding
def test_round_bf16_matches_torch_cast():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.normal(size=20000).astype(np.float32),
                        (rng.normal(size=2000) * 1e-38).astype(np.float32),
                        (rng.normal(size=2000) * 1e30).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.4e38, 1e-45], np.float32)])
    # exact ties: 1 + 2^-8 (half an ulp of bf16 at 1) rounds to even (1.0);
    # 1 + 3*2^-8 rounds up to 1 + 2^-6
    v = np.concatenate([v, np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], np.float32)])
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(v.astype(np.float64))
    np.testing.assert_array_equal(got, want)
    assert O.round_bf16(1 + 2 ** -8) == 1.0
    assert O.round_bf16(1 + 3 * 2 ** -8) == 1 + 2 ** -6


# ----------------------------------------------------------------- activations
def test_gelu_closed_form_points():
    xs = np.array([-5.0, -1.5, -0.1, 0.0, 0.3, 1.0, 2.5, 8.0])
    want = np.array([0.5 * x * (1 + math.erf(x / math.sqrt(2))) for x in xs])
    np.testing.assert_allclose(O.gelu(xs), want, rtol=1e-14, atol=1e-300)
    assert O.gelu(np.array([0.0]))[0] == 0.0
    # GELU(x) - GELU(-x) = x  (since erf is odd)
    np.testing.assert_allclose(O.gelu(xs) - O.gelu(-xs), xs, atol=1e-14)


def test_gelu_grad_finite_difference():
    xs = np.linspace(-6, 6, 241)
    hstep = 1e-6
    fd = (O.gelu(xs + hstep) - O.gelu(xs - hstep)) / (2 * hstep)
    np.testing.assert_allclose(O.gelu_grad(xs), fd, atol=1e-8)


# ----------------------------------------------------------------- helpers
def _rand_layer(rng, T, d, E, h, scale=0.3):
    x = rng.normal(size=(T, d))
    L = rng.normal(size=(T, E))
    w1 = rng.normal(size=(E, h if h else d, d)) * scale
    b1 = rng.normal(size=(E, h if h else d)) * scale
    w2 = rng.normal(size=(E, d, h)) * scale if h else None
    b2 = rng.normal(size=(E, d)) * scale if h else None
    return x, L, w1, b1, w2, b2


# ----------------------------------------------------------------- dense reduction
@pytest.mark.parametrize("act,torch_act", [(O.ACT_GELU, F.gelu), (O.ACT_RELU, F.relu),
                                           (O.ACT_NONE, lambda z: z)])
def test_single_expert_is_dense_ffn(act, torch_act):
    rng = np.random.default_rng(2)
    x, L, w1, b1, w2, b2 = _rand_layer(rng, 13, 6, 1, 10)
    r = O.layer_forward(x, L, w1, b1, w2, b2, k=1, capacity_factor=1.0, min_capacity=0,
                        drop_tokens=False, act=act, dtype="f64")
    xt = torch.from_numpy(x)
    dense = F.linear(torch_act(F.linear(xt, torch.from_numpy(w1[0]), torch.from_numpy(b1[0]))),
                     torch.from_numpy(w2[0]), torch.from_numpy(b2[0])).numpy()
    # one expert: p = 1 for every token, nothing dropped
    np.testing.assert_allclose(r["out"], dense, rtol=1e-13, atol=1e-13)
    assert r["gate_loss"] == 1.0


def test_single_linear_expert_is_dense_linear():
    rng = np.random.default_rng(3)
    x, L, w1, b1, _, _ = _rand_layer(rng, 9, 5, 1, 0)
    r = O.layer_forward(x, L, w1, b1, None, None, k=1, capacity_factor=1.0, min_capacity=0,
                        drop_tokens=False, act=O.ACT_NONE, dtype="f64")
    want = F.linear(torch.from_numpy(x), torch.from_numpy(w1[0]), torch.from_numpy(b1[0])).numpy()
    np.testing.assert_allclose(r["out"], want, rtol=1e-13, atol=1e-13)


# ----------------------------------------------------------------- two formulations
@pytest.mark.parametrize("k,normalize", [(1, False), (2, False), (2, True)])
def test_dispatch_form_equals_per_token_form_without_drops(k, normalize):
    rng = np.random.default_rng(4 + k)
    x, L, w1, b1, w2, b2 = _rand_layer(rng, 21, 7, 5, 11)
    r = O.layer_forward(x, L, w1, b1, w2, b2, k=k, capacity_factor=1.0, min_capacity=0,
                        drop_tokens=False, act=O.ACT_GELU, dtype="f64", normalize_topk=normalize)
    direct = O.direct_forward(x, L, w1, b1, w2, b2, k=k, act=O.ACT_GELU, dtype="f64",
                              normalize_topk=normalize)
    np.testing.assert_allclose(r["out"], direct, rtol=1e-12, atol=1e-12)


def test_top1_output_is_pmax_times_expert():
    rng = np.random.default_rng(7)
    x, L, w1, b1, w2, b2 = _rand_layer(rng, 8, 4, 3, 6)
    r = O.layer_forward(x, L, w1, b1, w2, b2, k=1, capacity_factor=1.0, min_capacity=0,
                        drop_tokens=False, act=O.ACT_RELU, dtype="f64")
    for t in range(8):
        e = int(np.argmax(L[t]))
        p = math.exp(L[t, e]) / sum(math.exp(v) for v in L[t])
        y = np.maximum(x[t] @ w1[e].T + b1[e], 0) @ w2[e].T + b2[e]
        np.testing.assert_allclose(r["out"][t], p * y, rtol=1e-12, atol=1e-12)


def test_dropped_token_gives_zero_row_and_dispatch_is_permutation():
    rng = np.random.default_rng(8)
    x, L, w1, b1, w2, b2 = _rand_layer(rng, 12, 4, 2, 5)
    L[:, 0] += 10.0   # everyone prefers expert 0
    r = O.layer_forward(x, L, w1, b1, w2, b2, k=1, capacity_factor=1.0, min_capacity=0,
                        drop_tokens=True, act=O.ACT_GELU, dtype="f64")
    C = r["capacity"]
    assert C == 6
    dropped = np.where(r["slot"][:, 0] < 0)[0]
    assert dropped.tolist() == list(range(6, 12))
    np.testing.assert_array_equal(r["out"][dropped], 0.0)
    # the dispatched rows are exactly the kept tokens, in slot order
    kept = np.where(r["slot"][:, 0] >= 0)[0]
    np.testing.assert_array_equal(r["x_disp"], x[kept])


# ----------------------------------------------------------------- backward
def _ffn_backward_inputs(rng, rows_per_expert, d, h, dtype):
    E = len(rows_per_expert)
    off = np.concatenate([[0], np.cumsum(rows_per_expert)])
    n = int(off[-1])
    x = rng.normal(size=(n, d))
    w1 = rng.normal(size=(E, h, d)) * 0.4
    b1 = rng.normal(size=(E, h)) * 0.4
    w2 = rng.normal(size=(E, d, h)) * 0.4
    b2 = rng.normal(size=(E, d)) * 0.4
    dy = rng.normal(size=(n, d))
    a, hh, y = O.expert_ffn(x, off, w1, b1, w2, b2, O.ACT_GELU, dtype)
    return off, x, w1, b1, w2, b2, dy, a, hh, y


def test_ffn_backward_matches_autograd():
    rng = np.random.default_rng(9)
    off, x, w1, b1, w2, b2, dy, a, hh, y = _ffn_backward_inputs(rng, [3, 0, 5, 2], 4, 6, "f64")
    dx, dw1, db1, dw2, db2 = O.expert_ffn_backward(x, off, w1, w2, a, hh, dy, O.ACT_GELU, "f64")
    xt = torch.from_numpy(x).requires_grad_()
    W1 = torch.from_numpy(w1).requires_grad_()
    B1 = torch.from_numpy(b1).requires_grad_()
    W2 = torch.from_numpy(w2).requires_grad_()
    B2 = torch.from_numpy(b2).requires_grad_()
    outs = []
    for e in range(4):
        r0, r1 = int(off[e]), int(off[e + 1])
        outs.append(F.linear(F.gelu(F.linear(xt[r0:r1], W1[e], B1[e])), W2[e], B2[e]))
    Y = torch.cat(outs)
    np.testing.assert_allclose(Y.detach().numpy(), y, rtol=1e-12, atol=1e-12)
    Y.backward(torch.from_numpy(dy))
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dw1, W1.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dw2, W2.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(db1, B1.grad.numpy().astype(np.float32), rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(db2, B2.grad.numpy().astype(np.float32), rtol=1e-6, atol=1e-6)


def test_ffn_backward_finite_differences():
    rng = np.random.default_rng(10)
    off, x, w1, b1, w2, b2, dy, a, hh, y = _ffn_backward_inputs(rng, [2, 3], 3, 4, "f64")
    dx, dw1, _, dw2, _ = O.expert_ffn_backward(x, off, w1, w2, a, hh, dy, O.ACT_GELU, "f64")

    def objective(x_, w1_, w2_):
        _, _, yy = O.expert_ffn(x_, off, w1_, b1, w2_, b2, O.ACT_GELU, "f64")
        return float(np.sum(yy * dy))

    eps = 1e-6
    for arr, grad in ((x, dx), (w1, dw1), (w2, dw2)):
        flat = arr.reshape(-1)
        for i in range(0, flat.size, max(1, flat.size // 17)):
            old = flat[i]
            flat[i] = old + eps
            fp = objective(x, w1, w2)
            flat[i] = old - eps
            fm = objective(x, w1, w2)
            flat[i] = old
            assert abs((fp - fm) / (2 * eps) - grad.reshape(-1)[i]) < 1e-6


def test_ffn_backward_zero_upstream():
    rng = np.random.default_rng(11)
    off, x, w1, b1, w2, b2, dy, a, hh, y = _ffn_backward_inputs(rng, [4, 1], 3, 5, "bf16")
    dx, dw1, db1, dw2, db2 = O.expert_ffn_backward(x, off, w1, w2, a, hh, np.zeros_like(dy),
                                                   O.ACT_GELU, "bf16")
    for g in (dx, dw1, db1, dw2, db2):
        assert not np.any(g)

"""GPU parity of the residual MoE layer (PR-MoE's use_residual; reading R16)
against oracle/residual_moe.py.

Routing takes drawn logits (given to both sides) so that indices, slots,
counts and offsets compare bit-exact; the coefficients within the fp32
dot-product bound of their logits (the softmax over two entries moves by at
most half the logits' error); bf16 outputs and gradients within
|g - o| <= 2e-2*|o| + 2e-2*rms(o)."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_39_amd import binding as B
from oracle import moe_oracle as O
from oracle import residual_moe as R
from tests.gpu_util import close, experts, f64, i64, workspace

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _draw(g, shape, std, dtype=torch.bfloat16):
    return (torch.randn(*shape, generator=g, device=DEV, dtype=torch.float32) * std).to(dtype)


def _inputs(T, d, E, h, seed, coef=True):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    hid = h if h else d
    inp = dict(x=_draw(g, (T, d), 1.0), logits=_draw(g, (T, E), 1.0, torch.float32),
               w_router=_draw(g, (E, d), 0.02), w1=_draw(g, (E, hid, d), 0.03), b1=_draw(g, (E, hid), 0.02),
               m_w1=_draw(g, (hid, d), 0.03), m_b1=_draw(g, (hid,), 0.02))
    inp["w2"] = _draw(g, (E, d, h), 0.03) if h else None
    inp["b2"] = _draw(g, (E, d), 0.02) if h else None
    inp["m_w2"] = _draw(g, (d, h), 0.03) if h else None
    inp["m_b2"] = _draw(g, (d,), 0.02) if h else None
    inp["c_w"] = _draw(g, (2, d), 0.05) if coef else None
    inp["c_b"] = _draw(g, (2,), 0.5, torch.float32) if coef else None
    return inp


def _mlp(inp):
    return tuple(None if inp[k] is None else f64(inp[k]) for k in ("m_w1", "m_b1", "m_w2", "m_b2"))


def _forward(cfg, inp, given=True, ws=None):
    T, d, E, k = cfg.num_tokens, cfg.hidden_size, cfg.num_experts, cfg.k
    ws = workspace(cfg, DEV) if ws is None else ws
    out = torch.full((T, d), 3.0, dtype=torch.bfloat16, device=DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    o = dict(loss=torch.empty(1, **f32), count=torch.empty(E, dtype=torch.int32, device=DEV),
             coef=torch.full((T, 2), -1.0, **f32), logits=torch.empty(T, E, **f32),
             idx=torch.empty(T, k, dtype=torch.int32, device=DEV), slot=torch.empty(T, k, dtype=torch.int32, device=DEV),
             weight=torch.empty(T, k, **f32))
    B.moe_residual_layer_forward(cfg, inp["x"], None if given else inp["w_router"], None,
                                 inp["logits"] if given else None, inp["w1"], inp["b1"], inp["w2"], inp["b2"],
                                 inp["m_w1"], inp["m_b1"], inp["m_w2"], inp["m_b2"], inp["c_w"], inp["c_b"], out,
                                 o["loss"], o["count"], coef_out=o["coef"], logits_out=o["logits"],
                                 expert_idx=o["idx"], slot=o["slot"], weight=o["weight"], ws=ws)
    torch.cuda.synchronize()
    return out, o, ws


def _coef_bound(x, cw):
    u = 2.0 ** -24
    d = x.shape[1]
    return d * u / (1 - d * u) * (np.abs(x) @ np.abs(cw).T) + 1e-6


CASES = [  # T, d, E, k, h, act, cf, drop, coef
    (300, 256, 8, 2, 512, O.ACT_GELU, 1.25, True, True),
    (1000, 512, 16, 1, 256, O.ACT_RELU, 1.0, True, False),
    (777, 256, 4, 2, 0, O.ACT_NONE, 1.0, True, True),
    (2048, 1024, 64, 2, 768, O.ACT_GELU, 1.0, False, True),
    (33, 128, 3, 1, 128, O.ACT_GELU, 0.5, True, True),
]


@pytest.mark.parametrize("T,d,E,k,h,act,cf,drop,coef", CASES, ids=lambda v: str(v))
def test_residual_forward(T, d, E, k, h, act, cf, drop, coef):
    inp = _inputs(T, d, E, h, seed=T + d + E, coef=coef)
    cfg = B.make_config(T, d, E, k, cf, 1, drop, h, act, B.MOE_BF16, use_residual=True)
    out, o, ws = _forward(cfg, inp)
    x, L = f64(inp["x"]), f64(inp["logits"])
    r = R.forward(x, L, experts(inp["w1"]), experts(inp["b1"]), experts(inp["w2"]), experts(inp["b2"]), _mlp(inp),
                  None if not coef else f64(inp["c_w"]), None if not coef else f64(inp["c_b"]), k=k,
                  capacity_factor=cf, min_capacity=1, drop_tokens=drop, act=act, dtype="bf16")
    np.testing.assert_array_equal(i64(o["idx"]), r["expert_idx"])
    np.testing.assert_array_equal(i64(o["slot"]), r["slot"])
    np.testing.assert_array_equal(i64(o["count"]), r["expert_count"])
    assert abs(float(o["loss"][0]) - r["gate_loss"]) <= 1e-5 * max(r["gate_loss"], 1e-6)
    if coef:
        bound = _coef_bound(x, f64(inp["c_w"]))
        assert (np.abs(f64(o["coef"]) - r["coef"]) <= bound.max(axis=1, keepdims=True)).all()
    else:
        assert (f64(o["coef"]) == 1.0).all()
    close(f64(out), r["out"], 2e-2)
    # the mix is not the plain layer's output
    plain = O.store(r["moe"], "bf16")
    assert np.abs(r["out"] - plain).max() > 0.1 * np.abs(plain).max()


def test_residual_router_path_and_determinism():
    T, d, E, h = 513, 512, 16, 384
    inp = _inputs(T, d, E, h, seed=77)
    cfg = B.make_config(T, d, E, 2, 1.25, 4, True, h, B.MOE_ACT_GELU, B.MOE_BF16, use_residual=True)
    out, o, ws = _forward(cfg, inp, given=False)
    x, w = f64(inp["x"]), f64(inp["w_router"])
    u = 2.0 ** -24
    assert (np.abs(f64(o["logits"]) - O.router_logits(x, w)) <= d * u / (1 - d * u) * (np.abs(x) @ np.abs(w).T)).all()
    out1 = out.clone()
    out2, o2, _ = _forward(cfg, inp, given=False, ws=ws)
    assert torch.equal(out1, out2) and torch.equal(o["coef"], o2["coef"])
    inp2 = dict(inp, logits=o["logits"].clone())
    out3, _, _ = _forward(cfg, inp2, given=True)
    assert torch.equal(out3, out1)


@pytest.mark.parametrize("T,d,E,k,h,coef,router", [(300, 256, 8, 2, 512, True, True), (640, 512, 16, 1, 256, False, True),
                                                    (129, 256, 4, 2, 128, True, False)])
def test_residual_backward(T, d, E, k, h, coef, router):
    inp = _inputs(T, d, E, h, seed=5 * T + E, coef=coef)
    cfg = B.make_config(T, d, E, k, 1.25, 1, True, h, B.MOE_ACT_GELU, B.MOE_BF16, use_residual=True,
                        save_preact=True)
    out, o, ws = _forward(cfg, inp)
    g0 = torch.Generator(device=DEV)
    g0.manual_seed(T)
    dout = _draw(g0, (T, d), 1.0)
    f32 = dict(dtype=torch.float32, device=DEV)
    gr = dict(dx=torch.full((T, d), 5.0, dtype=torch.bfloat16, device=DEV), dlogits=torch.empty(T, E, **f32),
              dw1=torch.empty_like(inp["w1"]), dw2=torch.empty_like(inp["w2"]), db1=torch.empty(E, h, **f32),
              db2=torch.empty(E, d, **f32), mlp_dw1=torch.empty_like(inp["m_w1"]),
              mlp_dw2=torch.empty_like(inp["m_w2"]), mlp_db1=torch.empty(h, **f32), mlp_db2=torch.empty(d, **f32))
    if router:
        gr.update(dw_router=torch.empty(E, d, **f32), db_router=torch.empty(E, **f32))
    if coef:
        gr.update(dcoef_w=torch.empty(2, d, **f32), dcoef_b=torch.empty(2, **f32))
    dloss = torch.tensor([0.7], **f32)
    B.moe_residual_layer_backward(cfg, inp["x"], inp["w_router"] if router else None, inp["w1"], inp["w2"],
                                  inp["m_w1"], inp["m_w2"], inp["c_w"], dout, dloss, gr["dx"], gr["dw1"], gr["dw2"],
                                  gr["mlp_dw1"], gr["mlp_dw2"], logits=o["logits"], expert_idx=o["idx"],
                                  slot=o["slot"], weight=o["weight"], dlogits=gr["dlogits"],
                                  dw_router=gr.get("dw_router"), db_router=gr.get("db_router"), db1=gr["db1"],
                                  db2=gr["db2"], mlp_db1=gr["mlp_db1"], mlp_db2=gr["mlp_db2"],
                                  dcoef_w=gr.get("dcoef_w"), dcoef_b=gr.get("dcoef_b"), ws=ws)
    torch.cuda.synchronize()
    x, L = f64(inp["x"]), f64(inp["logits"])
    W1, B1, W2, B2 = experts(inp["w1"]), experts(inp["b1"]), experts(inp["w2"]), experts(inp["b2"])
    cw = f64(inp["c_w"]) if coef else None
    r = R.forward(x, L, W1, B1, W2, B2, _mlp(inp), cw, f64(inp["c_b"]) if coef else None, k=k, capacity_factor=1.25,
                  min_capacity=1, drop_tokens=True, act=O.ACT_GELU, dtype="bf16")
    # the backward uses the GPU's coefficients (their rounding is not the point here)
    r["coef"] = f64(o["coef"])
    want = R.backward(x, f64(inp["w_router"]) if router else None, r, W1, W2, _mlp(inp), cw, f64(dout), 0.7,
                      act=O.ACT_GELU, dtype="bf16")
    keys = {"dx": "dx", "dlogits": "dlogits", "dw1": "dw1", "dw2": "dw2", "db1": "db1", "db2": "db2",
            "mlp_dw1": "mlp_dw1", "mlp_dw2": "mlp_dw2", "mlp_db1": "mlp_db1", "mlp_db2": "mlp_db2",
            "dw_router": "dw_router", "db_router": "db_router", "dcoef_w": "dcoef_w", "dcoef_b": "dcoef_b"}
    for name, key in keys.items():
        if name in gr:
            close(f64(gr[name]), want[key], 2e-2)


def test_pyramid_of_residual_layers():
    """[ds.moe] §2.3 / §4.2's pyramid num_experts = [4, 8, 16]: three residual
    layers with their own expert counts, each fed the previous GPU output and
    checked against the oracle on that same input."""
    T, d, h = 700, 256, 256
    x = torch.randn(T, d, generator=torch.Generator(device=DEV).manual_seed(1), device=DEV).to(torch.bfloat16)
    for i, E in enumerate((4, 8, 16)):
        inp = _inputs(T, d, E, h, seed=40 + i)
        inp["x"] = x
        cfg = B.make_config(T, d, E, 1, 1.0, 4, True, h, B.MOE_ACT_GELU, B.MOE_BF16, use_residual=True)
        out, o, _ = _forward(cfg, inp)
        r = R.forward(f64(x), f64(inp["logits"]), experts(inp["w1"]), experts(inp["b1"]), experts(inp["w2"]),
                      experts(inp["b2"]), _mlp(inp), f64(inp["c_w"]), f64(inp["c_b"]), k=1, capacity_factor=1.0,
                      min_capacity=4, drop_tokens=True, act=O.ACT_GELU, dtype="bf16")
        np.testing.assert_array_equal(i64(o["count"]), r["expert_count"])
        close(f64(out), r["out"], 2e-2)
        x = out


def test_residual_full_size_sampled():
    """residual_e64 as the bench runs it (T = 16384, d = 2048, E = 64, top-2,
    h = 5120, cf 1.25, router from x): routing, slots and counts for the
    whole batch from the oracle's gate on the GPU's logits; 48 sampled
    tokens' outputs computed one by one (their kept experts' FFNs, the dense
    MLP, the coefficients and the mix, with the layer's roundings)."""
    from mixture_experts_layer_39_amd.synthetic import make_inputs, spec
    sp = spec("residual_e64")
    inp = make_inputs(sp, DEV)
    T, d, E, k, h = sp["T"], sp["d"], sp["E"], sp["k"], sp["h"]
    cfg = B.make_config(T, d, E, k, sp["cf"], sp["min_cap"], True, h, sp["act"], B.MOE_BF16, use_residual=True)
    ws = workspace(cfg, DEV)
    out = torch.empty(T, d, dtype=torch.bfloat16, device=DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    loss, cnt = torch.empty(1, **f32), torch.empty(E, dtype=torch.int32, device=DEV)
    lg, coef = torch.empty(T, E, **f32), torch.empty(T, 2, **f32)
    idx_t = torch.empty(T, k, dtype=torch.int32, device=DEV)
    slot_t = torch.empty(T, k, dtype=torch.int32, device=DEV)
    wt_t = torch.empty(T, k, **f32)
    B.moe_residual_layer_forward(cfg, inp["x"], inp["w_router"], None, None, inp["w1"], inp["b1"], inp["w2"],
                                 inp["b2"], inp["mlp_w1"], inp["mlp_b1"], inp["mlp_w2"], inp["mlp_b2"],
                                 inp["coef_w"], inp["coef_b"], out, loss, cnt, coef_out=coef, logits_out=lg,
                                 expert_idx=idx_t, slot=slot_t, weight=wt_t, ws=ws)
    torch.cuda.synchronize()
    L = f64(lg)
    r = O.route(L, k, sp["cf"], sp["min_cap"], True)
    np.testing.assert_array_equal(i64(idx_t), r["expert_idx"])
    np.testing.assert_array_equal(i64(slot_t), r["slot"])
    np.testing.assert_array_equal(i64(cnt), r["expert_count"])
    rows = np.random.default_rng(11).choice(T, 48, replace=False)
    sel = torch.as_tensor(rows, device=DEV)
    X = f64(inp["x"][sel])
    W1, B1, W2, B2 = experts(inp["w1"]), experts(inp["b1"]), experts(inp["w2"]), experts(inp["b2"])
    mlp = tuple(f64(inp[n]) for n in ("mlp_w1", "mlp_b1", "mlp_w2", "mlp_b2"))
    _, _, ym = R.dense_mlp(X, mlp, sp["act"], "bf16")
    c = R.coefficients(X, f64(inp["coef_w"]), f64(inp["coef_b"]))
    bound = _coef_bound(X, f64(inp["coef_w"]))
    assert (np.abs(f64(coef[sel]) - c) <= bound.max(axis=1, keepdims=True)).all()
    want = np.zeros((len(rows), d))
    for i, t in enumerate(rows):
        moe = np.zeros(d)
        for j in range(k):
            if r["slot"][t, j] >= 0:
                _, _, y = O._ffn_rows(X[i:i + 1], int(r["expert_idx"][t, j]), W1, B1, W2, B2, sp["act"], "bf16")
                moe += r["weight"][t, j] * y[0]
        want[i] = c[i, 0] * moe + c[i, 1] * ym[i]
    close(f64(out[sel]), O.store(want, "bf16"), 2e-2)


def test_residual_no_tokens():
    """T = 0: the forward returns zero counts and loss; the backward zero
    weight, bias and coefficient gradients."""
    d, E, h = 256, 4, 128
    inp = _inputs(1, d, E, h, seed=9)
    cfg = B.make_config(0, d, E, 2, 1.0, 1, True, h, B.MOE_ACT_GELU, B.MOE_BF16, use_residual=True,
                        save_preact=True)
    ws = workspace(cfg, DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    loss, cnt = torch.full((1,), 5.0, **f32), torch.full((E,), 5, dtype=torch.int32, device=DEV)
    out = torch.empty(0, d, dtype=torch.bfloat16, device=DEV)
    B.moe_residual_layer_forward(cfg, None, inp["w_router"], None, None, inp["w1"], inp["b1"], inp["w2"], inp["b2"],
                                 inp["m_w1"], inp["m_b1"], inp["m_w2"], inp["m_b2"], inp["c_w"], inp["c_b"], out,
                                 loss, cnt, ws=ws)
    g = {n: torch.full(s, 7.0, dtype=dt, device=DEV) for n, s, dt in
         (("dw1", (E, h, d), torch.bfloat16), ("dw2", (E, d, h), torch.bfloat16), ("db1", (E, h), torch.float32),
          ("db2", (E, d), torch.float32), ("mdw1", (h, d), torch.bfloat16), ("mdw2", (d, h), torch.bfloat16),
          ("mdb1", (h,), torch.float32), ("mdb2", (d,), torch.float32), ("dwr", (E, d), torch.float32),
          ("dbr", (E,), torch.float32), ("dcw", (2, d), torch.float32), ("dcb", (2,), torch.float32))}
    B.moe_residual_layer_backward(cfg, None, inp["w_router"], inp["w1"], inp["w2"], inp["m_w1"], inp["m_w2"],
                                  inp["c_w"], None, None, None, g["dw1"], g["dw2"], g["mdw1"], g["mdw2"],
                                  dw_router=g["dwr"], db_router=g["dbr"], db1=g["db1"], db2=g["db2"],
                                  mlp_db1=g["mdb1"], mlp_db2=g["mdb2"], dcoef_w=g["dcw"], dcoef_b=g["dcb"], ws=ws)
    torch.cuda.synchronize()
    assert float(loss[0]) == 0.0 and int(cnt.abs().sum()) == 0
    for n, t in g.items():
        assert not t.float().abs().sum().item(), n

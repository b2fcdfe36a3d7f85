"""GPU parity of the seeded random gate options (noisy_gate_policy Jitter /
RSample, second-expert sampling, Random Token Selection; reading R15)
against oracle/stochastic_gate.py, on the same seed.

The Philox words, the uniforms and the jitter factors are exact integer or
once-rounded fp32 arithmetic on both sides, so the jittered router input is
compared bit-exact (a router weight of one-hot rows makes each logit one
element of it).  A Gumbel draw goes through log, whose last bit may differ
between the GPU and NumPy, so a noisy choice is checked as: the GPU's expert
is the oracle's, or ties it within 1e-6 of the key; everything downstream
(slots, drops, counts, offsets, the RTS selection) is then bit-exact against
the oracle run on the GPU's choices, weights within 1e-5, loss 1e-5
relative, bf16 outputs 2e-2."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_39_amd import binding as B
from oracle import moe_oracle as O
from oracle import stochastic_gate as S
from tests.gpu_util import alloc_gate, close, experts, f64, i64, workspace

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _gate(cfg, x=None, w_router=None, logits=None):
    g = alloc_gate(cfg, DEV)
    ws = workspace(cfg, DEV)
    B.moe_gate(cfg, x, w_router, None, logits, g["logits"], g["idx"], g["slot"], g["weight"], g["count"],
               g["offset"], g["loss"], ws)
    torch.cuda.synchronize()
    return g


def _check_choice(got, keys, exclude=None):
    """got[t] must be the largest key of row t (ties to the lower index), or
    within 1e-6 (relative to the key's size) of it."""
    k = np.asarray(keys, np.float64).copy()
    if exclude is not None:
        k[np.arange(len(k)), exclude] = -np.inf
    best = S._argbest(k)
    amb = 0
    for t in np.nonzero(got != best)[0]:
        top = k[t, best[t]]
        assert top - k[t, got[t]] <= 1e-6 * max(1.0, abs(top)), (t, got[t], best[t])
        amb += 1
    assert amb <= max(2, len(got) // 1000)


def _downstream(g, lg, k, cf, mc, drop, seed, rts, norm=False, loss=O.LOSS_BALANCE):
    """Slots, counts, offsets, weights and loss from the oracle on the GPU's
    choices (bit-exact / 1e-5)."""
    idx = i64(g["idx"])
    T, E = lg.shape
    p = O.softmax(lg)
    C = O.capacity(k, T, E, cf, mc, drop)
    if rts:
        slot, _ = S.rts_slots(idx, E, C, seed)
    else:
        slot, _ = O.assign_slots(idx, E, C)
    count, offset = O.expert_count_and_offset(idx, slot, E)
    np.testing.assert_array_equal(i64(g["slot"]), slot)
    np.testing.assert_array_equal(i64(g["count"]), count)
    np.testing.assert_array_equal(i64(g["offset"]), offset)
    assert np.abs(f64(g["weight"]) - O.gate_weights(p, idx, norm)).max() <= 1e-5
    want = O.gate_loss(p, idx, E, loss)
    assert abs(float(g["loss"][0]) - want) <= 1e-5 * max(want, 1e-6)
    return slot, offset


@pytest.mark.parametrize("T,E,seed", [(3000, 8, 1), (777, 64, 2), (4096, 256, 3), (5, 3, 4)])
def test_rsample_top1(T, E, seed):
    g0 = torch.Generator(device=DEV)
    g0.manual_seed(40 + seed)
    lg = torch.randn(T, E, generator=g0, device=DEV)
    cfg = B.make_config(T, 128, E, 1, 1.25, 4, True, 0, B.MOE_ACT_NONE, B.MOE_BF16,
                        noisy_gate_policy=B.MOE_NOISE_RSAMPLE, seed=seed)
    g = _gate(cfg, logits=lg)
    L = f64(lg)
    _check_choice(i64(g["idx"])[:, 0], S.noisy_keys(L, seed, S.STREAM_RSAMPLE))
    # the noise changed the choice somewhere (it is not the plain top-1)
    if T > 100:
        assert (i64(g["idx"])[:, 0] != O.top_k(L, 1)[:, 0]).mean() > 0.05
    _downstream(g, L, 1, 1.25, 4, True, seed, rts=False)


@pytest.mark.parametrize("T,E,seed,norm", [(3000, 8, 5, False), (1000, 64, 6, True), (2048, 200, 7, False)])
def test_second_expert_sampling(T, E, seed, norm):
    g0 = torch.Generator(device=DEV)
    g0.manual_seed(50 + seed)
    lg = torch.randn(T, E, generator=g0, device=DEV)
    cfg = B.make_config(T, 128, E, 2, 1.0, 4, True, 0, B.MOE_ACT_NONE, B.MOE_BF16, normalize_topk=norm,
                        second_expert_sampling=True, seed=seed)
    g = _gate(cfg, logits=lg)
    L = f64(lg)
    idx = i64(g["idx"])
    np.testing.assert_array_equal(idx[:, 0], O.top_k(L, 1)[:, 0])
    assert (idx[:, 1] != idx[:, 0]).all()
    _check_choice(idx[:, 1], S.noisy_keys(L, seed, S.STREAM_SECOND), exclude=idx[:, 0])
    assert (idx[:, 1] != O.top_k(L, 2)[:, 1]).mean() > 0.05
    _downstream(g, L, 2, 1.0, 4, True, seed, rts=False, norm=norm)


@pytest.mark.parametrize("T,E,cf,seed,rsample", [(4000, 8, 1.0, 8, False), (4000, 8, 1.0, 9, True),
                                                 (1500, 16, 0.5, 10, False), (70, 4, 1.0, 11, False),
                                                 (20000, 64, 1.0, 12, True)])
def test_random_token_selection(T, E, cf, seed, rsample):
    """Over-capacity experts keep the claims of largest priority; experts
    within capacity keep the first-come slots."""
    g0 = torch.Generator(device=DEV)
    g0.manual_seed(60 + seed)
    bias = torch.zeros(E, device=DEV)
    bias[0], bias[1] = 2.0, 1.0   # experts 0 and 1 overflow
    lg = torch.randn(T, E, generator=g0, device=DEV) + bias
    cfg = B.make_config(T, 128, E, 1, cf, 4, True, 0, B.MOE_ACT_NONE, B.MOE_BF16, use_rts=True, seed=seed,
                        noisy_gate_policy=B.MOE_NOISE_RSAMPLE if rsample else 0)
    g = _gate(cfg, logits=lg)
    L = f64(lg)
    idx = i64(g["idx"])
    if rsample:
        _check_choice(idx[:, 0], S.noisy_keys(L, seed, S.STREAM_RSAMPLE))
    else:
        np.testing.assert_array_equal(idx, O.top_k(L, 1))
    slot, _ = _downstream(g, L, 1, cf, 4, True, seed, rts=True)
    C = O.capacity(1, T, E, cf, 4, True)
    demand = np.bincount(idx[:, 0], minlength=E)
    assert demand.max() > C
    # RTS differs from first-come on the overflowing experts
    det, _ = O.assign_slots(idx, E, C)
    over = np.isin(idx[:, 0], np.nonzero(demand > C)[0])
    assert not np.array_equal(slot[over], det[over])
    assert np.array_equal(slot[~over], det[~over])


@pytest.mark.parametrize("T,seed", [(100, 21), (257, 22), (64, 23)])
def test_jitter_router_input_bit_exact(T, seed):
    """With one-hot router rows (expert e reads feature e) each logit is one
    jittered input element, so the GPU's jittered x is compared bit-exact."""
    d = E = 256
    g0 = torch.Generator(device=DEV)
    g0.manual_seed(70 + seed)
    x = torch.randn(T, d, generator=g0, device=DEV).to(torch.bfloat16)
    w = torch.eye(E, d, device=DEV).to(torch.bfloat16)
    cfg = B.make_config(T, d, E, 2, 1.0, 4, True, 0, B.MOE_ACT_NONE, B.MOE_BF16,
                        noisy_gate_policy=B.MOE_NOISE_JITTER, seed=seed)
    g = _gate(cfg, x=x, w_router=w)
    want = S.jittered_input(f64(x), seed)
    np.testing.assert_array_equal(f64(g["logits"]), want)
    assert not np.array_equal(want, f64(x))
    # without jitter the logits are x itself
    g2 = _gate(B.make_config(T, d, E, 2, 1.0, 4, True, 0, B.MOE_ACT_NONE, B.MOE_BF16), x=x, w_router=w)
    np.testing.assert_array_equal(f64(g2["logits"]), f64(x))


def test_jitter_router_logits_and_routing():
    """A dense router on jittered input: logits within the fp32 dot-product
    bound of the oracle's router on the oracle's jittered input; routing
    exact where the top-2 keys are clear of that bound."""
    T, d, E, seed = 2048, 2048, 64, 31
    g0 = torch.Generator(device=DEV)
    g0.manual_seed(99)
    x = torch.randn(T, d, generator=g0, device=DEV).to(torch.bfloat16)
    w = (torch.randn(E, d, generator=g0, device=DEV) * 0.02).to(torch.bfloat16)
    cfg = B.make_config(T, d, E, 2, 1.25, 4, True, 0, B.MOE_ACT_NONE, B.MOE_BF16,
                        noisy_gate_policy=B.MOE_NOISE_JITTER, seed=seed)
    g = _gate(cfg, x=x, w_router=w)
    xj = S.jittered_input(f64(x), seed)
    want = O.router_logits(xj, f64(w))
    u = 2.0 ** -24
    bound = d * u / (1 - d * u) * (np.abs(xj) @ np.abs(f64(w)).T)
    got = f64(g["logits"])
    assert (np.abs(got - want) <= bound).all()
    # the jitter moved the logits by more than the rounding bound somewhere
    plain = O.router_logits(f64(x), f64(w))
    assert (np.abs(plain - want) > bound).any()
    _downstream(g, got, 2, 1.25, 4, True, seed, rts=False)


def test_jitter_needs_the_router():
    cfg = B.make_config(64, 128, 4, 1, 1.0, 4, True, 0, B.MOE_ACT_NONE, B.MOE_BF16,
                        noisy_gate_policy=B.MOE_NOISE_JITTER, seed=1)
    lg = torch.zeros(64, 4, device=DEV)
    with pytest.raises(B.MoeError) as ei:
        _gate(cfg, logits=lg)
    assert ei.value.status == B.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("T,k,small", [(3000, 2, 0), (9, 2, 1), (3000, 1, 0), (16, 1, 1)])
def test_layer_forward_with_random_gate(T, k, small):
    """The whole forward with the options on (the small-batch kernel does not
    take them, so small T runs the multi-kernel path): the experts see the
    clean x, and out matches the oracle's layer on the GPU's routing."""
    d, E, h, seed = 256, 16, 512, 77
    g0 = torch.Generator(device=DEV)
    g0.manual_seed(123 + T)
    x = torch.randn(T, d, generator=g0, device=DEV).to(torch.bfloat16)
    wr = (torch.randn(E, d, generator=g0, device=DEV) * 0.1).to(torch.bfloat16)
    w1 = (torch.randn(E, h, d, generator=g0, device=DEV) * 0.05).to(torch.bfloat16)
    b1 = (torch.randn(E, h, generator=g0, device=DEV) * 0.05).to(torch.bfloat16)
    w2 = (torch.randn(E, d, h, generator=g0, device=DEV) * 0.05).to(torch.bfloat16)
    b2 = (torch.randn(E, d, generator=g0, device=DEV) * 0.05).to(torch.bfloat16)
    opts = dict(noisy_gate_policy=B.MOE_NOISE_JITTER, second_expert_sampling=True) if k == 2 else \
        dict(noisy_gate_policy=B.MOE_NOISE_RSAMPLE, use_rts=True)
    cf = 1.0
    cfg = B.make_config(T, d, E, k, cf, 2, True, h, B.MOE_ACT_GELU, B.MOE_BF16, seed=seed, small_batch=small,
                        **opts)
    g = alloc_gate(cfg, DEV)
    ws = workspace(cfg, DEV)
    out = torch.empty(T, d, dtype=torch.bfloat16, device=DEV)
    B.moe_layer_forward(cfg, x, wr, None, None, w1, b1, w2, b2, out, g["loss"], g["count"], logits_out=g["logits"],
                        expert_idx=g["idx"], slot=g["slot"], weight=g["weight"], ws=ws)
    torch.cuda.synchronize()
    L = f64(g["logits"])
    idx = i64(g["idx"])
    if k == 2:
        xj = S.jittered_input(f64(x), seed)
        want = O.router_logits(xj, f64(wr))
        u = 2.0 ** -24
        assert (np.abs(L - want) <= d * u / (1 - d * u) * (np.abs(xj) @ np.abs(f64(wr)).T)).all()
        np.testing.assert_array_equal(idx[:, 0], O.top_k(L, 1)[:, 0])
        _check_choice(idx[:, 1], S.noisy_keys(L, seed, S.STREAM_SECOND), exclude=idx[:, 0])
    else:
        _check_choice(idx[:, 0], S.noisy_keys(L, seed, S.STREAM_RSAMPLE))
    C = O.capacity(k, T, E, cf, 2, True)
    slot = S.rts_slots(idx, E, C, seed)[0] if k == 1 else O.assign_slots(idx, E, C)[0]
    np.testing.assert_array_equal(i64(g["slot"]), slot)
    count, offset = O.expert_count_and_offset(idx, slot, E)
    np.testing.assert_array_equal(i64(g["count"]), count)
    p = O.softmax(L)
    w = O.gate_weights(p, idx, False)
    x64 = f64(x)
    xd = O.dispatch(x64, idx, slot, offset)
    W1, B1, W2, B2 = experts(w1), experts(b1), experts(w2), experts(b2)
    _, hh, y = O.expert_ffn(xd, offset, W1, B1, W2, B2, B.MOE_ACT_GELU, "bf16")
    want_out = O.combine(y, idx, slot, w, offset, T, "bf16")
    close(f64(out), want_out, 2e-2)


def test_same_seed_same_bits_other_seed_other_routing():
    T, E = 4096, 32
    g0 = torch.Generator(device=DEV)
    g0.manual_seed(5)
    lg = torch.randn(T, E, generator=g0, device=DEV)
    res = []
    for seed in (1, 1, 2):
        cfg = B.make_config(T, 128, E, 2, 1.0, 4, True, 0, B.MOE_ACT_NONE, B.MOE_BF16, second_expert_sampling=True,
                            seed=seed)
        res.append(_gate(cfg, logits=lg))
    for key in ("idx", "slot", "weight", "count", "loss"):
        assert torch.equal(res[0][key], res[1][key]), key
    assert not torch.equal(res[0]["idx"], res[2]["idx"])


@pytest.mark.parametrize("T,d,E,k,h", [(300, 256, 8, 2, 256), (1000, 512, 16, 1, 384)])
def test_layer_backward_with_jitter(T, d, E, k, h):
    """Training with a jittered router: the forward routes on the jittered
    router's logits; the backward's router weight gradient contracts with
    the jittered input and its input gradient carries the factors (R15);
    everything against the oracle on the GPU's logits."""
    seed = 1234 + T
    g0 = torch.Generator(device=DEV)
    g0.manual_seed(T)
    x = torch.randn(T, d, generator=g0, device=DEV).to(torch.bfloat16)
    wr = (torch.randn(E, d, generator=g0, device=DEV) * 0.05).to(torch.bfloat16)
    w1 = (torch.randn(E, h, d, generator=g0, device=DEV) * 0.05).to(torch.bfloat16)
    b1 = (torch.randn(E, h, generator=g0, device=DEV) * 0.05).to(torch.bfloat16)
    w2 = (torch.randn(E, d, h, generator=g0, device=DEV) * 0.05).to(torch.bfloat16)
    b2 = (torch.randn(E, d, generator=g0, device=DEV) * 0.05).to(torch.bfloat16)
    dout = torch.randn(T, d, generator=g0, device=DEV).to(torch.bfloat16)
    cfg = B.make_config(T, d, E, k, 1.25, 1, True, h, B.MOE_ACT_GELU, B.MOE_BF16, save_preact=True,
                        noisy_gate_policy=B.MOE_NOISE_JITTER, seed=seed)
    ws = workspace(cfg, DEV)
    out = torch.empty(T, d, dtype=torch.bfloat16, device=DEV)
    loss = torch.empty(1, dtype=torch.float32, device=DEV)
    cnt = torch.empty(E, dtype=torch.int32, device=DEV)
    lg = torch.empty(T, E, dtype=torch.float32, device=DEV)
    B.moe_layer_forward(cfg, x, wr, None, None, w1, b1, w2, b2, out, loss, cnt, logits_out=lg, ws=ws)
    f32 = dict(dtype=torch.float32, device=DEV)
    dx = torch.empty(T, d, dtype=torch.bfloat16, device=DEV)
    dw1, dw2 = torch.empty_like(w1), torch.empty_like(w2)
    dlg, dwr, dbr = torch.empty(T, E, **f32), torch.empty(E, d, **f32), torch.empty(E, **f32)
    dloss = torch.tensor([0.6], **f32)
    B.moe_layer_backward(cfg, x, wr, w1, w2, dout, dloss, dx, dw1, dw2, logits=lg, dlogits=dlg, dw_router=dwr,
                         db_router=dbr, ws=ws)
    torch.cuda.synchronize()
    X, L = f64(x), f64(lg)
    W1, B1, W2, B2 = experts(w1), experts(b1), experts(w2), experts(b2)
    r = O.layer_forward(X, L, W1, B1, W2, B2, k=k, capacity_factor=1.25, min_capacity=1, drop_tokens=True,
                        act=O.ACT_GELU, dtype="bf16")
    np.testing.assert_array_equal(i64(cnt), r["expert_count"])
    close(f64(out), r["out"], 2e-2)
    want = S.layer_backward_jitter(X, f64(wr), r, W1, W2, f64(dout), 0.6, act=O.ACT_GELU, dtype="bf16", seed=seed)
    for key, got in (("dx", dx), ("dlogits", dlg), ("dw_router", dwr), ("db_router", dbr), ("dw1", dw1),
                     ("dw2", dw2)):
        close(f64(got), want[key], 2e-2)
    # the router weight gradient (fp32, near-fp32 accurate) is much closer to
    # the jittered-input gradient than to the plain one
    plain = O.layer_backward(X, f64(wr), r, W1, W2, f64(dout), 0.6, act=O.ACT_GELU, dtype="bf16")
    g_dwr = f64(dwr)
    assert np.linalg.norm(g_dwr - want["dw_router"]) < 0.1 * np.linalg.norm(g_dwr - plain["dw_router"])


def test_full_size_jitter_and_second_expert_sampling():
    """The top2_e64 gate (T = 16384, d = 2048, E = 64, cf 1.25) with jitter and
    second-expert sampling, as a training step would run it: sampled tokens'
    logits against the oracle's router on their jittered rows; the second
    choices against the oracle's noisy keys on the GPU's logits; slots,
    counts and loss on the GPU's choices for the whole batch."""
    from mixture_experts_layer_39_amd.synthetic import make_inputs, spec
    sp = spec("top2_e64")
    inp = make_inputs(sp, DEV)
    T, d, E, seed = sp["T"], sp["d"], sp["E"], 20240
    cfg = B.make_config(T, d, E, 2, sp["cf"], sp["min_cap"], True, 0, B.MOE_ACT_NONE, B.MOE_BF16,
                        noisy_gate_policy=B.MOE_NOISE_JITTER, second_expert_sampling=True, seed=seed)
    g = _gate(cfg, x=inp["x"], w_router=inp["w_router"])
    L = f64(g["logits"])
    rows = np.random.default_rng(3).choice(T, 64, replace=False)
    xj = S.jittered_input(f64(inp["x"][torch.as_tensor(rows, device=DEV)]), seed, rows=rows)
    w = f64(inp["w_router"])
    u = 2.0 ** -24
    bound = d * u / (1 - d * u) * (np.abs(xj) @ np.abs(w).T)
    assert (np.abs(L[rows] - O.router_logits(xj, w)) <= bound).all()
    idx = i64(g["idx"])
    np.testing.assert_array_equal(idx[:, 0], O.top_k(L, 1)[:, 0])
    _check_choice(idx[:, 1], S.noisy_keys(L, seed, S.STREAM_SECOND), exclude=idx[:, 0])
    _downstream(g, L, 2, sp["cf"], sp["min_cap"], True, seed, rts=False)


def test_random_gate_no_tokens_and_no_overflow():
    """T = 0 with every option on runs nothing and returns zeros; RTS with
    room for every claim keeps the first-come slots."""
    cfg = B.make_config(0, 128, 4, 1, 1.0, 4, True, 0, B.MOE_ACT_NONE, B.MOE_BF16, use_rts=True,
                        noisy_gate_policy=B.MOE_NOISE_RSAMPLE, seed=3)
    g = _gate(cfg, logits=torch.zeros(0, 4, device=DEV))
    assert int(g["count"].abs().sum()) == 0 and float(g["loss"][0]) == 0.0
    T, E = 500, 8
    lg = torch.randn(T, E, generator=torch.Generator(device=DEV).manual_seed(4), device=DEV)
    cfg = B.make_config(T, 128, E, 1, 8.0, 4, True, 0, B.MOE_ACT_NONE, B.MOE_BF16, use_rts=True, seed=3)
    g = _gate(cfg, logits=lg)
    L = f64(lg)
    r = O.route(L, 1, 8.0, 4, True)
    np.testing.assert_array_equal(i64(g["slot"]), r["slot"])

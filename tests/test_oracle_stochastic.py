"""Pins of the stochastic-gate oracle (oracle/stochastic_gate.py, reading
R15) against facts outside it: the Philox round against NumPy's Philox4x64
bit generator (a library routine with the same round structure) and against
the published Philox4x32-10 known-answer vectors of the Random123 library
(Salmon et al. 2011); the uniform and Gumbel draws against their
distributions; the Gumbel-max rule against the softmax it must reproduce;
Random Token Selection against its invariants and its keep probability;
the options switched off against the deterministic gate."""
import math

import numpy as np
import pytest

from oracle import moe_oracle as O
from oracle import stochastic_gate as S


def chi2_ok(counts, probs, crit):
    n = counts.sum()
    exp = n * np.asarray(probs)
    return float(((counts - exp) ** 2 / exp).sum()) < crit


@pytest.mark.parametrize("key,ctr", [((1, 2), (10, 0, 0, 0)), ((0, 0), (0, 0, 0, 0)),
                                     ((2 ** 64 - 1, 12345), (7, 99, 3, 1)), ((0xDEADBEEF, 1 << 40), (2 ** 64 - 1, 5, 0, 0))])
def test_philox_round_matches_numpy_philox4x64(key, ctr):
    """NumPy's Philox bit generator (4x64, 10 rounds) advances its counter,
    carrying across words, before each block; our round in 64-bit words must
    give its outputs."""
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(ctr, dtype=np.uint64))
    raw = [int(v) for v in bg.random_raw(8)]
    c = list(ctr)
    got = []
    for _ in range(2):
        i = 0
        while True:   # the counter increment with carry
            c[i] = (c[i] + 1) % 2 ** 64
            if c[i] or i == 3:
                break
            i += 1
        got += list(S.philox4(c, key, bits=64))
    assert got == raw


def test_philox4x32_known_answers():
    """Philox4x32-10 known-answer vectors published with Random123."""
    kat = [((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
           ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF), (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
           ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
            (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1))]
    for ctr, key, want in kat:
        assert S.philox4(ctr, key) == want
        got = S.philox4x32_np(*([v] for v in ctr), *key)
        assert tuple(int(w[0]) for w in got) == want


def test_vectorised_philox_matches_scalar():
    rng = np.random.default_rng(1)
    c = rng.integers(0, 2 ** 32, size=(4, 50), dtype=np.uint64)
    k = rng.integers(0, 2 ** 32, size=2)
    vec = S.philox4x32_np(c[0], c[1], c[2], c[3], k[0], k[1])
    for i in range(50):
        assert tuple(int(w[i]) for w in vec) == S.philox4([int(v) for v in c[:, i]], [int(v) for v in k])


def test_draw_layout():
    """Draw n of stream s is word n % 4 of the block at counter
    (n // 4 lo, n // 4 hi, s, 0), key (seed lo, seed hi)."""
    seed = 0x0123456789ABCDEF
    ns = np.array([0, 1, 2, 3, 4, 7, 1 << 33, (1 << 34) + 6, 123456789], np.int64)
    for s in range(4):
        d = S.draws(seed, s, ns)
        for n, w in zip(ns.tolist(), d.tolist()):
            blk = n // 4
            want = S.philox4((blk & 0xFFFFFFFF, blk >> 32, s, 0), (seed & 0xFFFFFFFF, seed >> 32))[n % 4]
            assert w == want
    # streams and seeds are different sequences
    n = np.arange(4096)
    assert not np.array_equal(S.draws(1, 0, n), S.draws(1, 1, n))
    assert not np.array_equal(S.draws(1, 0, n), S.draws(2, 0, n))


def test_uniform_draws():
    w = S.draws(7, 0, np.arange(1 << 20))
    u = S.uniform01(w)
    assert u.dtype == np.float32
    assert (u > 0).all() and (u < 1).all()
    # exactly (2m + 1) / 2^24: odd multiples of 2^-24, representable in fp32
    m = u.astype(np.float64) * 2.0 ** 24
    assert (m == np.round(m)).all() and (np.round(m) % 2 == 1).all()
    assert abs(float(u.mean()) - 0.5) < 5 * math.sqrt(1 / 12 / u.size)
    counts = np.bincount(np.minimum((u * 64).astype(np.int64), 63), minlength=64)
    assert chi2_ok(counts, np.full(64, 1 / 64), 120.0)   # 63 dof, p ~ 1e-5
    # the words themselves: every bit is a fair coin
    bits = np.unpackbits(w.view(np.uint8)).reshape(-1, 32).mean(axis=0)
    assert np.abs(bits - 0.5).max() < 5 * 0.5 / math.sqrt(w.size)


def test_gumbel_draws():
    g = S.gumbel(S.uniform01(S.draws(3, 1, np.arange(1 << 20))))
    euler_gamma = 0.5772156649015329
    assert abs(g.mean() - euler_gamma) < 5 * (math.pi / math.sqrt(6)) / math.sqrt(g.size)
    assert abs(g.var() - math.pi ** 2 / 6) < 0.02
    # CDF exp(-exp(-x)) at a few points
    for x in (-1.0, 0.0, 1.0, 3.0):
        assert abs((g <= x).mean() - math.exp(-math.exp(-x))) < 0.003


def test_rsample_selects_with_softmax_probabilities():
    """Gumbel-max: argmax(l + G) is drawn from softmax(l)."""
    l = np.array([1.0, 0.5, -0.25, 0.0, -2.0])
    T = 60000
    idx = S.select_experts(np.tile(l, (T, 1)), 1, seed=11, rsample=True)
    counts = np.bincount(idx[:, 0], minlength=5)
    assert chi2_ok(counts, O.softmax(l[None, :])[0], 23.5)   # 4 dof, p ~ 1e-4


def test_second_expert_sampling():
    """The first choice stays the deterministic top-1; the second is drawn
    from the softmax over the other experts and never repeats the first."""
    l = np.array([0.3, 1.2, -0.4, 0.9])
    T = 60000
    idx = S.select_experts(np.tile(l, (T, 1)), 2, seed=5, second_sampling=True)
    assert (idx[:, 0] == 1).all()
    assert (idx[:, 1] != 1).all()
    counts = np.bincount(idx[:, 1], minlength=4)[[0, 2, 3]]
    p = np.exp(l[[0, 2, 3]])
    assert chi2_ok(counts, p / p.sum(), 18.5)   # 2 dof, p ~ 1e-4
    # RSample is a k = 1 option; sampling the second expert a k = 2 option
    base = O.top_k(np.tile(l, (8, 1)), 2)
    assert np.array_equal(S.select_experts(np.tile(l, (8, 1)), 2, seed=5, rsample=True), base)


def test_options_off_reduce_to_the_deterministic_gate():
    rng = np.random.default_rng(0)
    for k in (1, 2):
        lg = rng.normal(size=(300, 9))
        a = S.route(lg, k, 1.0, 2, True, seed=99)
        b = O.route(lg, k, 1.0, 2, True)
        for key in ("expert_idx", "slot", "expert_count", "expert_offset"):
            assert np.array_equal(a[key], b[key]), key
        assert np.allclose(a["weight"], b["weight"]) and a["gate_loss"] == b["gate_loss"]


def test_rts_invariants_and_keep_probability():
    rng = np.random.default_rng(4)
    E, T = 5, 400
    lg = rng.normal(size=(T, E)) + np.array([2.0, 0.5, 0, 0, 0])   # expert 0 overflows
    C = O.capacity(1, T, E, 1.0, 4, True)
    for seed in (1, 2, 3):
        r = S.route(lg, 1, 1.0, 4, True, seed=seed, rts=True)
        d = O.route(lg, 1, 1.0, 4, True)
        # which token is routed where, counts, offsets and loss are unchanged
        for key in ("expert_idx", "expert_count", "expert_offset"):
            assert np.array_equal(r[key], d[key]), key
        assert r["gate_loss"] == d["gate_loss"]
        prio = S.draws(seed, S.STREAM_RTS, np.arange(T)).astype(np.int64)
        for e in range(E):
            toks = np.nonzero(r["expert_idx"][:, 0] == e)[0]
            s = r["slot"][toks, 0]
            kept = toks[s >= 0]
            assert len(kept) == min(len(toks), C)
            assert np.array_equal(s[s >= 0], np.arange(len(kept)))   # token order
            drop = toks[s < 0]
            if len(drop):
                worst_kept = min((prio[t], -t) for t in kept)
                assert all((prio[t], -t) < worst_kept for t in drop)
        # an expert within capacity keeps the first-come slots
        ok = [e for e in range(E) if d["demand"][0, e] <= C]
        m = np.isin(r["expert_idx"][:, 0], ok)
        assert np.array_equal(r["slot"][m], d["slot"][m])
    # each claimant of an overflowing expert is kept with probability C / D
    toks = np.nonzero(O.top_k(lg, 1)[:, 0] == 0)[0]
    D = len(toks)
    assert D > C
    kept = np.zeros(T)
    n = 300
    for seed in range(n):
        kept += S.rts_slots(O.top_k(lg, 1), E, C, seed)[0][:, 0] >= 0
    frac = kept[toks] / n
    assert abs(frac.mean() - C / D) < 1e-12   # exactly C kept every time
    assert np.abs(frac - C / D).max() < 5 * math.sqrt(C / D * (1 - C / D) / n)
    # the deterministic gate keeps the first C in token order instead
    assert (O.route(lg, 1, 1.0, 4, True)["slot"][toks[:C], 0] >= 0).all()


def test_rts_without_capacity_or_overflow_is_deterministic():
    lg = np.random.default_rng(8).normal(size=(50, 4))
    a = S.route(lg, 1, 1.0, 4, False, seed=3, rts=True)
    b = O.route(lg, 1, 1.0, 4, False)
    assert np.array_equal(a["slot"], b["slot"])
    a = S.route(lg, 1, 100.0, 4, True, seed=3, rts=True)
    b = O.route(lg, 1, 100.0, 4, True)
    assert np.array_equal(a["slot"], b["slot"])


def test_jitter_factors_and_input():
    T, d = 64, 256
    f = S.jitter_factors(17, T, d)
    assert f.dtype == np.float32
    lo, hi = np.float32(1 - S.JITTER_EPS), np.float32(1 + S.JITTER_EPS)
    assert (f >= lo).all() and (f <= hi).all()
    assert abs(float(f.mean()) - 1.0) < 5 * (S.JITTER_EPS / math.sqrt(3)) / math.sqrt(f.size)
    assert len(np.unique(f)) > 0.9 * f.size
    # eps = 0 leaves x as it is; x = 1 gives the factors rounded to bf16
    x = O.round_bf16(np.random.default_rng(2).normal(size=(T, d)))
    assert np.array_equal(S.jittered_input(x, 17, eps=0.0), x)
    assert np.array_equal(S.jittered_input(np.ones((T, d)), 17), O.round_bf16(f.astype(np.float64)))
    # the factor is (1 - eps) + (2 eps) * u with two fp32 roundings
    u = S.uniform01(S.draws(17, S.STREAM_JITTER, np.arange(T * d))).reshape(T, d)
    assert np.array_equal(f, (np.float32(0.99) + (np.float32(0.02) * u).astype(np.float32)).astype(np.float32))
    # selected rows give the same factors as the whole matrix
    rows = np.array([5, 0, 63, 17])
    assert np.array_equal(S.jitter_factors(17, T, d, rows=rows), f[rows])
    assert np.array_equal(S.jittered_input(x[rows], 17, rows=rows), S.jittered_input(x, 17)[rows])
    # jitter leaves |x_j / x - 1| <= eps plus the bf16 rounding
    xj = S.jittered_input(x, 17)
    nz = x != 0
    assert np.abs(xj[nz] / x[nz] - 1).max() <= S.JITTER_EPS + 2 ** -8


def test_seed_determinism():
    lg = np.random.default_rng(6).normal(size=(200, 8))
    a = S.route(lg, 2, 1.0, 4, True, seed=42, second_sampling=True)
    b = S.route(lg, 2, 1.0, 4, True, seed=42, second_sampling=True)
    c = S.route(lg, 2, 1.0, 4, True, seed=43, second_sampling=True)
    assert np.array_equal(a["expert_idx"], b["expert_idx"])
    assert not np.array_equal(a["expert_idx"], c["expert_idx"])


def test_jitter_backward_against_finite_differences():
    """The router gradients under jitter, checked by float64 central
    differences of <dOut, out> + dloss * loss through a router that reads
    x * factor (no bf16 rounding in the float64 mode, so the chain rule is
    exact), on a tiny layer with no ties."""
    rng = np.random.default_rng(12)
    T, d, E, h, k, seed = 6, 8, 3, 5, 2, 9
    x = rng.normal(size=(T, d))
    wr = rng.normal(size=(E, d)) * 0.5
    w1 = rng.normal(size=(E, h, d)) * 0.3
    b1 = rng.normal(size=(E, h)) * 0.1
    w2 = rng.normal(size=(E, d, h)) * 0.3
    b2 = rng.normal(size=(E, d)) * 0.1
    dout = rng.normal(size=(T, d))
    dloss = 0.7
    f = S.jitter_factors(seed, T, d).astype(np.float64)

    def objective(xx, ww):
        lg = O.router_logits(xx * f, ww)
        r = O.layer_forward(xx, lg, w1, b1, w2, b2, k=k, capacity_factor=10.0, min_capacity=1, drop_tokens=True,
                            act=O.ACT_GELU, dtype="f64")
        return float((dout * r["out"]).sum() + dloss * r["gate_loss"]), r

    _, r = objective(x, wr)
    g = O.layer_backward(x, wr, r, w1, w2, dout, dloss, act=O.ACT_GELU, dtype="f64", router_input=x * f,
                         router_input_scale=f)
    eps = 1e-6
    for (i, j) in [(0, 0), (2, 5), (5, 7), (3, 1)]:
        xp, xm = x.copy(), x.copy()
        xp[i, j] += eps
        xm[i, j] -= eps
        fd = (objective(xp, wr)[0] - objective(xm, wr)[0]) / (2 * eps)
        assert abs(g["dx"][i, j] - fd) <= 1e-6 * max(1.0, abs(fd))
    for (e, j) in [(0, 0), (1, 4), (2, 7)]:
        wp, wm = wr.copy(), wr.copy()
        wp[e, j] += eps
        wm[e, j] -= eps
        fd = (objective(x, wp)[0] - objective(x, wm)[0]) / (2 * eps)
        assert abs(g["dw_router"][e, j] - fd) <= 1e-6 * max(1.0, abs(fd))
    # without the scale the input gradient would be off by the factors
    g0 = O.layer_backward(x, wr, r, w1, w2, dout, dloss, act=O.ACT_GELU, dtype="f64")
    assert not np.allclose(g0["dx"], g["dx"], rtol=1e-4, atol=0)

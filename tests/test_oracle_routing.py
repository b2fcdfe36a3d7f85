"""Pins of the oracle's gate: softmax, top-k, capacity slots, drops, counts
and gate_loss (CPU only).

Pins used, none of which re-runs the oracle's own code:
  * a case worked by hand (T=4, E=3, k=2, C=2) with every index, slot, count,
    weight and loss written out below with its derivation;
  * brute force over every logit matrix in {-1,0,1}^(T x E) for tiny T, E,
    against a claim-list formulation written here from scratch (exhaustive
    search for the top-k, claims sorted by (choice, token) and handed out to
    each expert in order);
  * invariants on random inputs (hypothesis);
  * closed forms of the losses in special cases.
"""
import itertools
import math

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import moe_oracle as O


# ----------------------------------------------------------------- worked case
HAND_LOGITS = [[2, 1, 0], [1, 1, 0], [0, 3, 3], [5, 0, 0]]


def test_hand_worked_case():
    """T=4, E=3, k=2, capacity_factor 0.5, min_capacity 1.

    C = max(1, ceil(8/3 * 0.5)) = ceil(1.333) = 2.
    top-1/top-2 by (logit desc, index asc):
      t0 [2,1,0] -> 0,1   t1 [1,1,0] -> 0,1 (tie to 0)
      t2 [0,3,3] -> 1,2 (tie to 1)   t3 [5,0,0] -> 0,1 (tie for 2nd to 1)
    top-1 claims in token order: e0 gets t0->0, t1->1, t3->2 (>= C: dropped);
      e1 gets t2->0.  top-1 demand: e0 3, e1 1, e2 0.
    top-2 claims continue each expert's counter: e1 gets t0->1, t1->2 (drop),
      t3->3 (drop); e2 gets t2->0.
    """
    r = O.route(np.array(HAND_LOGITS, float), k=2, capacity_factor=0.5,
                min_capacity=1, drop_tokens=True)
    assert r["capacity"] == 2
    assert r["expert_idx"].tolist() == [[0, 1], [0, 1], [1, 2], [0, 1]]
    assert r["slot"].tolist() == [[0, 1], [1, -1], [0, 0], [-1, -1]]
    assert r["expert_count"].tolist() == [2, 2, 1]
    assert r["expert_offset"].tolist() == [0, 2, 4, 5]
    assert r["demand"].tolist() == [[3, 1, 0], [0, 3, 1]]
    e1, e2, e3, e5 = math.e, math.e ** 2, math.e ** 3, math.e ** 5
    # softmax probabilities written out per row
    p = [[e2 / (e2 + e1 + 1), e1 / (e2 + e1 + 1), 1 / (e2 + e1 + 1)],
         [e1 / (2 * e1 + 1), e1 / (2 * e1 + 1), 1 / (2 * e1 + 1)],
         [1 / (1 + 2 * e3), e3 / (1 + 2 * e3), e3 / (1 + 2 * e3)],
         [e5 / (e5 + 2), 1 / (e5 + 2), 1 / (e5 + 2)]]
    np.testing.assert_allclose(r["probs"], p, rtol=0, atol=1e-15)
    np.testing.assert_allclose(r["weight"], [[p[0][0], p[0][1]], [p[1][0], p[1][1]],
                                             [p[2][1], p[2][2]], [p[3][0], p[3][1]]],
                               rtol=0, atol=1e-15)
    # values computed by hand: me = column means of p = [0.52463799, 0.29038779,
    # 0.18497422]; ce = top-1 shares [3/4, 1/4, 0]; 3*(me.ce) = 1.398226313
    assert abs(r["gate_loss"] - 1.398226313) < 1e-9
    # usage over both choices = [3,4,1]/8; population std 0.155902391; +1e-6
    r2 = O.route(np.array(HAND_LOGITS, float), k=2, capacity_factor=0.5,
                 min_capacity=1, drop_tokens=True, loss_kind=O.LOSS_USAGE_STD)
    assert abs(r2["gate_loss"] - 0.155903391) < 1e-9
    # renormalised weights: t0 e^2/(e^2+e), t1 and t2 exactly 1/2, t3 e^5/(e^5+1)
    r3 = O.route(np.array(HAND_LOGITS, float), k=2, capacity_factor=0.5,
                 min_capacity=1, drop_tokens=True, normalize_topk=True)
    np.testing.assert_allclose(r3["weight"], [[e2 / (e2 + e1), e1 / (e2 + e1)], [0.5, 0.5],
                                              [0.5, 0.5], [e5 / (e5 + 1), 1 / (e5 + 1)]],
                               rtol=0, atol=1e-15)
    assert r3["slot"].tolist() == r["slot"].tolist()


# ----------------------------------------------------------------- brute force
def _claims_reference(L, k, cap):
    """Formulation written from scratch: exhaustive top-k, then a claim list."""
    T, E = len(L), len(L[0])
    idx = []
    for t in range(T):
        chosen = []
        for _ in range(k):
            best = None
            for e in range(E):
                if e in chosen:
                    continue
                if best is None or L[t][e] > L[t][best]:
                    best = e
            chosen.append(best)
        idx.append(chosen)
    claims = sorted((j, t) for t in range(T) for j in range(k))
    per_expert = {e: [] for e in range(E)}
    for (j, t) in claims:
        per_expert[idx[t][j]].append((t, j))
    slot = [[None] * k for _ in range(T)]
    for e, lst in per_expert.items():
        for pos, (t, j) in enumerate(lst):
            slot[t][j] = pos if (cap is None or pos < cap) else -1
    count = [sum(1 for pos in range(len(per_expert[e])) if cap is None or pos < cap) for e in range(E)]
    return idx, slot, count


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (2, 2, 1), (2, 2, 2), (3, 2, 2), (2, 3, 2),
                                   (3, 3, 1), (3, 3, 2), (4, 2, 2), (2, 4, 2)])
def test_bruteforce_all_tie_patterns(T, E, k):
    caps = [None] + sorted(set([0, 1, 2, k * T]))
    for vals in itertools.product((-1.0, 0.0, 1.0), repeat=T * E):
        L = [list(vals[t * E:(t + 1) * E]) for t in range(T)]
        for cap in caps:
            idx_r, slot_r, count_r = _claims_reference(L, k, cap)
            idx = O.top_k(np.array(L), k)
            slot, _ = O.assign_slots(idx, E, cap)
            cnt, off = O.expert_count_and_offset(idx, slot, E)
            assert idx.tolist() == idx_r, (L, cap)
            assert slot.tolist() == slot_r, (L, cap)
            assert cnt.tolist() == count_r, (L, cap)
            assert off.tolist() == [sum(count_r[:i]) for i in range(E + 1)]


def test_negative_zero_ties_positive_zero():
    L = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]])
    assert O.top_k(L, 2).tolist() == [[0, 1], [0, 1]]


# ----------------------------------------------------------------- invariants
@settings(max_examples=150, deadline=None)
@given(T=st.integers(0, 40), E=st.integers(1, 9), k=st.integers(1, 2),
       cf=st.sampled_from([0.25, 0.5, 1.0, 1.25, 2.0]), min_cap=st.integers(0, 5),
       drop=st.booleans(), seed=st.integers(0, 2 ** 31 - 1), ints=st.booleans())
def test_routing_invariants(T, E, k, cf, min_cap, drop, seed, ints):
    if k > E:
        k = E
    rng = np.random.default_rng(seed)
    L = rng.integers(-2, 3, size=(T, E)).astype(float) if ints else rng.normal(size=(T, E))
    r = O.route(L, k, cf, min_cap, drop)
    idx, slot, cnt, C = r["expert_idx"], r["slot"], r["expert_count"], r["capacity"]
    dropped = int((slot < 0).sum())
    assert cnt.sum() == k * T - dropped
    if C is not None:
        assert (cnt <= C).all()
    else:
        assert dropped == 0
    for t in range(T):
        assert len(set(idx[t].tolist())) == k
    for e in range(E):
        kept = sorted(int(s) for s, i in zip(slot.reshape(-1), idx.reshape(-1)) if i == e and s >= 0)
        assert kept == list(range(cnt[e]))
        if k == 2:
            s1 = slot[:, 0][(idx[:, 0] == e) & (slot[:, 0] >= 0)]
            s2 = slot[:, 1][(idx[:, 1] == e) & (slot[:, 1] >= 0)]
            if len(s1) and len(s2):
                assert s1.max() < s2.min()
    if T:
        np.testing.assert_allclose(r["probs"].sum(axis=1), 1.0, atol=1e-12)
        # the chosen experts carry the k largest probabilities
        for t in range(T):
            chosen = r["probs"][t, idx[t]]
            others = np.delete(r["probs"][t], idx[t])
            if others.size:
                assert chosen.min() >= others.max()
    # a large enough capacity is the same as no capacity
    r_big = O.route(L, k, 1.0, k * T, True)
    r_none = O.route(L, k, 1.0, 0, False)
    assert (r_big["slot"] == r_none["slot"]).all()


def test_single_expert_reduces_to_token_order():
    L = np.random.default_rng(0).normal(size=(10, 1))
    # C = max(6, ceil(10/1 * 0.5)) = 6
    r = O.route(L, 1, 0.5, 6, True)
    np.testing.assert_array_equal(r["probs"], 1.0)
    assert r["slot"][:, 0].tolist() == [0, 1, 2, 3, 4, 5, -1, -1, -1, -1]
    assert r["expert_count"].tolist() == [6]


def test_round_robin_gives_equal_counts():
    T, E = 24, 4
    L = np.zeros((T, E))
    for t in range(T):
        L[t, t % E] = 1.0
        L[t, (t + 1) % E] = 0.5
    r = O.route(L, 2, 1.0, 0, True)
    assert r["capacity"] == 12
    assert r["expert_count"].tolist() == [12, 12, 12, 12]
    assert (r["slot"] >= 0).all()
    r1 = O.route(L, 1, 1.0, 0, True)
    # k=1: the slot is the token's rank among tokens of the same expert
    assert r1["slot"][:, 0].tolist() == [t // E for t in range(T)]


def test_empty_batch():
    r = O.route(np.zeros((0, 5)), 2, 1.0, 4, True)
    assert r["slot"].shape == (0, 2)
    assert r["expert_count"].tolist() == [0] * 5
    assert r["gate_loss"] == 0.0


# ----------------------------------------------------------------- loss closed forms
def test_balance_loss_is_one_when_probs_uniform():
    # all logits equal: p = 1/E everywhere, every top-1 goes to expert 0 by the
    # tie rule, and E * sum_e (1/E) * ce_e = sum_e ce_e = 1 whatever ce is.
    for E in (1, 2, 5, 64):
        r = O.route(np.zeros((37, E)), 1 if E == 1 else 2, 1.0, 4, True)
        assert abs(r["gate_loss"] - 1.0) < 1e-12
        assert r["expert_idx"][:, 0].tolist() == [0] * 37


def test_balance_loss_collapse_tends_to_E():
    E = 8
    L = np.zeros((50, E))
    L[:, 3] = 60.0
    r = O.route(L, 2, 1.0, 4, True)
    assert abs(r["gate_loss"] - E) < 1e-12 * E + E * 7 * math.exp(-60)


def test_usage_std_closed_forms():
    T, E = 32, 4
    L = np.zeros((T, E))
    for t in range(T):
        L[t, t % E] = 1.0
    r = O.route(L, 1, 1.0, 4, True, loss_kind=O.LOSS_USAGE_STD)
    assert abs(r["gate_loss"] - 1e-6) < 1e-15
    # every token to expert 0, k = 1: sqrt((1/E)(1 - 1/E)) + 1e-6
    L0 = np.zeros((T, E))
    L0[:, 0] = 1.0
    r0 = O.route(L0, 1, 1.0, 4, True, loss_kind=O.LOSS_USAGE_STD)
    assert abs(r0["gate_loss"] - (math.sqrt((1 / E) * (1 - 1 / E)) + 1e-6)) < 1e-14


def test_loss_uses_demand_not_kept():
    # capacity 1 drops most claims but both losses count choices before capacity
    L = np.zeros((8, 2))
    L[:, 0] = 1.0
    a = O.route(L, 1, 0.125, 1, True)   # C = max(1, ceil(8/2 * 0.125)) = 1
    b = O.route(L, 1, 1.0, 0, False)
    assert a["gate_loss"] == b["gate_loss"]
    assert a["expert_count"].tolist() == [1, 0]

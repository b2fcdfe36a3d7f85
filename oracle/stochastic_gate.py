"""CPU oracle for the seeded stochastic gate options of the MoE layer.

TEST INFRASTRUCTURE ONLY, like ``moe_oracle``: only the test suite, the smoke
check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may use
it.  It shares no code, constant or helper with the HIP library.

The "deepspeed.moe 模块" overview ([ds.moe] §2.1, the MoE arguments; §3.1
step 1; §4, load-imbalance remedies) names three random options of the gate
and gives no formula for any of them:
  noisy_gate_policy  "Jitter" or "RSample": gate noise against expert
                     selection bias;
  use_rts            Random Token Selection, for convergence;
  top2_2nd_expert_sampling  sample the second expert of a top-2 gate.
Reading R15 (the pages name the options of DeepSpeed's MoE layer, the library
they document, so its published gate is the plainest reading; parity of
these definitions is unpinned against any number on the pages and is pinned
by their distributions and invariants instead):
  Jitter   the router's input x is multiplied elementwise by factors drawn
           uniformly from [1 - eps, 1 + eps], eps = 0.01; the experts see the
           clean x.  Both k.  Stored as bf16 before the router product (R8).
  RSample  k = 1: the expert is the argmax of logit + Gumbel(0, 1) noise (the
           Gumbel-max rule, so it is drawn with the softmax probabilities);
           the weight stays the clean softmax probability.
  2nd-expert sampling  k = 2: the second expert is the argmax, over the
           experts other than the first, of logit + Gumbel(0, 1) noise; the
           first stays the deterministic top-1.
  RTS      k = 1 with a capacity: an expert whose demand exceeds C keeps the
           C claims with the largest random priorities (ties to the lower
           token) instead of the first C in token order; kept claims take
           slots 0.. in token order.  Counts, offsets and the loss do not
           change.
All random numbers come from one counter-based generator, Philox4x32-10
(Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3",
SC 2011), written here from its published definition: draw n of stream s
under a 64-bit seed is word (n mod 4) of Philox4x32-10 applied to the counter
(n div 4 low 32 bits, n div 4 high 32 bits, s, 0) with the key (seed low,
seed high).  Streams: 0 jitter (n = t*d + i), 1 RSample (n = t*E + e),
2 second-expert sampling (n = t*E + e), 3 RTS priority (n = t).
A 32-bit draw w becomes the fp32 uniform u = ((w >> 9) + 0.5) * 2^-23 in the
open interval (0, 1) (exactly representable), the Gumbel draw -log(-log u),
the jitter factor (1 - eps) + (2 eps) * u in two fp32 roundings.
"""

from __future__ import annotations

import numpy as np

from oracle import moe_oracle as O

NOISE_NONE, NOISE_JITTER, NOISE_RSAMPLE = 0, 1, 2
STREAM_JITTER, STREAM_RSAMPLE, STREAM_SECOND, STREAM_RTS = 0, 1, 2, 3
JITTER_EPS = 0.01

# Philox multipliers and key increments (the published constants, as the
# rounding-free integers of the definition), for 32- and 64-bit words.
PHILOX_M = {32: (0xD2511F53, 0xCD9E8D57), 64: (0xD2E7470EE14C6C93, 0xCA5A826395121157)}
PHILOX_W = {32: (0x9E3779B9, 0xBB67AE85), 64: (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)}


def philox4(ctr, key, bits=32, rounds=10):
    """Philox4xW-R on one counter (four W-bit words) and key (two words), in
    Python integers, the round as published: with the products
    M0*c0 = (hi0, lo0) and M1*c2 = (hi1, lo1), the new counter is
    (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key advances by the Weyl
    constants between rounds."""
    mask = (1 << bits) - 1
    (m0, m1), (w0, w1) = PHILOX_M[bits], PHILOX_W[bits]
    c0, c1, c2, c3 = (int(v) & mask for v in ctr)
    k0, k1 = (int(v) & mask for v in key)
    for r in range(rounds):
        if r:
            k0, k1 = (k0 + w0) & mask, (k1 + w1) & mask
        p0, p1 = m0 * c0, m1 * c2
        hi0, lo0 = p0 >> bits, p0 & mask
        hi1, lo1 = p1 >> bits, p1 & mask
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def philox4x32_np(c0, c1, c2, c3, k0, k1, rounds=10):
    """The same Philox4x32 round on arrays of counters (uint32 arithmetic in
    uint64 so that the 64-bit products are exact)."""
    M0, M1 = (np.uint64(v) for v in PHILOX_M[32])
    W0, W1 = (np.uint64(v) for v in PHILOX_W[32])
    m32 = np.uint64(0xFFFFFFFF)
    s32 = np.uint64(32)
    c0, c1, c2, c3 = (np.asarray(v, np.uint64) & m32 for v in (c0, c1, c2, c3))
    k0, k1 = np.uint64(int(k0) & 0xFFFFFFFF), np.uint64(int(k1) & 0xFFFFFFFF)
    for r in range(rounds):
        if r:
            k0, k1 = (k0 + W0) & m32, (k1 + W1) & m32
        p0, p1 = M0 * c0, M1 * c2
        hi0, lo0 = p0 >> s32, p0 & m32
        hi1, lo1 = p1 >> s32, p1 & m32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def draws(seed, stream, n):
    """32-bit draws number n (int array) of a stream: word n % 4 of
    Philox4x32-10((n // 4) lo, (n // 4) hi, stream, 0; seed lo, seed hi)."""
    n = np.asarray(n, np.int64)
    blk = (n >> 2).astype(np.uint64)
    seed = int(seed) & ((1 << 64) - 1)
    words = philox4x32_np(blk & np.uint64(0xFFFFFFFF), blk >> np.uint64(32),
                          np.full(n.shape, stream, np.uint64), np.zeros(n.shape, np.uint64),
                          seed & 0xFFFFFFFF, seed >> 32)
    sel = (n & 3).astype(np.int64)
    out = np.choose(sel, words)
    return out.astype(np.uint32)


def uniform01(w):
    """fp32 uniform in (0, 1) from 32-bit draws: ((w >> 9) + 0.5) * 2^-23."""
    w = np.asarray(w, np.uint32)
    return ((w >> np.uint32(9)).astype(np.float32) + np.float32(0.5)) * np.float32(2.0 ** -23)


def gumbel(u):
    """Standard Gumbel draws -log(-log u) (float64 from the fp32 uniforms)."""
    u = np.asarray(u, np.float64)
    return -np.log(-np.log(u))


def jitter_factors(seed, T, d, eps=JITTER_EPS, rows=None):
    """fp32 factors (1 - eps) + (2 eps) * u for every element of x [T, d]
    (or of the given token rows only): the product and the sum are each
    rounded to fp32 (no fused step)."""
    t = np.arange(T, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    n = t[:, None] * d + np.arange(d, dtype=np.int64)[None, :]
    u = uniform01(draws(seed, STREAM_JITTER, n))
    return np.float32(1.0 - eps) + np.float32(2.0 * eps) * u


def jittered_input(x, seed, eps=JITTER_EPS, rows=None):
    """The router's input under Jitter: x * factor in fp32, stored as bf16
    (round to nearest even), as the router product reads it.  With ``rows``,
    x holds those token rows only."""
    x = np.asarray(x, np.float32)
    T, d = x.shape
    return O.round_bf16((x * jitter_factors(seed, T, d, eps, rows)).astype(np.float64))


def noisy_keys(logits, seed, stream):
    """Selection keys logit + Gumbel in fp32: the fp32 logit plus the Gumbel
    draw rounded to fp32, one fp32 rounding of the sum."""
    l = np.asarray(logits, np.float32)
    T, E = l.shape
    n = np.arange(T * E, dtype=np.int64).reshape(T, E)
    g = gumbel(uniform01(draws(seed, stream, n))).astype(np.float32)
    return l + g


def _argbest(keys, exclude=None):
    """Per row, the index of the largest key, ties to the lower index (R2)."""
    k = np.asarray(keys, np.float64).copy()
    if exclude is not None:
        k[np.arange(k.shape[0]), exclude] = -np.inf
    T, E = k.shape
    order = np.lexsort((np.broadcast_to(np.arange(E), (T, E)), -k), axis=1)
    return order[:, 0].astype(np.int64)


def select_experts(logits, k, seed=0, rsample=False, second_sampling=False):
    """The k chosen experts per token under the options (R15); without them
    this is the deterministic top-k of ``moe_oracle.top_k``."""
    l = np.asarray(logits, np.float64)
    T, E = l.shape
    if T == 0:
        return np.zeros((0, k), np.int64)
    base = O.top_k(l, k)
    i0 = _argbest(noisy_keys(l, seed, STREAM_RSAMPLE)) if (rsample and k == 1) else base[:, 0]
    if k == 1:
        return i0[:, None]
    i1 = _argbest(noisy_keys(l, seed, STREAM_SECOND), exclude=i0) if second_sampling else base[:, 1]
    return np.stack([i0, i1], axis=1)


def rts_slots(idx, num_experts, cap, seed):
    """Slots of a k = 1 gate under Random Token Selection (R15), literally:
    for each expert, its claimants in token order; if there are more than C,
    the C with the largest priority (the stream-3 draw of the token; equal
    priorities to the lower token) are kept; kept claims are numbered 0.. in
    token order, the others get -1.  Also returns the demand, as
    ``moe_oracle.assign_slots`` does."""
    idx = np.asarray(idx, np.int64)
    T = idx.shape[0]
    prio = draws(seed, STREAM_RTS, np.arange(T, dtype=np.int64)).astype(np.int64)
    slot = np.full((T, 1), -1, np.int64)
    demand = np.zeros((1, num_experts), np.int64)
    for e in range(num_experts):
        toks = [t for t in range(T) if idx[t, 0] == e]
        demand[0, e] = len(toks)
        if cap is None or len(toks) <= cap:
            kept = set(toks)
        else:
            ranked = sorted(toks, key=lambda t: (-prio[t], t))
            kept = set(ranked[:cap])
        s = 0
        for t in toks:
            if t in kept:
                slot[t, 0] = s
                s += 1
    return slot, demand


def route(logits, k, capacity_factor=1.0, min_capacity=4, drop_tokens=True, normalize_topk=False,
          loss_kind=O.LOSS_BALANCE, seed=0, rsample=False, second_sampling=False, rts=False):
    """The gate with the random options (R15): choices by ``select_experts``,
    weights from the clean softmax (R1), slots by ``rts_slots`` (k = 1, RTS)
    or the deterministic claim order (R3), counts, offsets, and the loss on
    the chosen experts (R5)."""
    l = np.asarray(logits, np.float64)
    T, E = l.shape
    p = O.softmax(l)
    idx = select_experts(l, k, seed, rsample, second_sampling)
    w = O.gate_weights(p, idx, normalize_topk)
    C = O.capacity(k, T, E, capacity_factor, min_capacity, drop_tokens)
    if rts and k == 1:
        slot, demand = rts_slots(idx, E, C, seed)
    else:
        slot, demand = O.assign_slots(idx, E, C)
    count, offset = O.expert_count_and_offset(idx, slot, E)
    loss = O.gate_loss(p, idx, E, loss_kind)
    return dict(probs=p, expert_idx=idx, weight=w, capacity=C, slot=slot, demand=demand,
                expert_count=count, expert_offset=offset, gate_loss=loss)


def layer_backward_jitter(x, w_router, r, w1, w2, dout, dloss, *, act, dtype, seed, eps=JITTER_EPS,
                          normalize_topk=False, loss_kind=O.LOSS_BALANCE):
    """The layer backward when the router read the jittered input (R15):
    dW_r = dlogits^T x_j with x_j = ``jittered_input``, and the router's
    input gradient (dlogits W_r) times the factors; the bf16 rounding of
    x * factor is taken as the identity, as in R13 for stored tensors."""
    x = np.asarray(x, np.float64)
    T, d = x.shape
    return O.layer_backward(x, w_router, r, w1, w2, dout, dloss, act=act, dtype=dtype,
                            normalize_topk=normalize_topk, loss_kind=loss_kind,
                            router_input=jittered_input(x, seed, eps),
                            router_input_scale=jitter_factors(seed, T, d, eps).astype(np.float64))

"""CPU oracle for one GPU's share of a top-k gated Mixture-of-Experts layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It shares
no code, constant or helper with the HIP library, and imports nothing from it.

It is a plain, slow, obviously-correct restatement of what the layer computes,
in float64 NumPy, with the steps in the order the source pages give them.

Sources (cited below by the tag in brackets, then the section on that page):
  [ZeRO3-MoE]   "DeepSpeed ZeRO-3 与 MoE 训练" walkthrough, mhpq.cn/news/1113018
  [ds.moe]      "deepspeed.moe 模块" overview, adg.csdn.net/694deb285b9f5f31781ae763.html
  [DS-MoE-traps] DeepSeek-MoE fine-tuning article, lnwmold.com/news/1162317
  [AllToAll]    "DeepSpeed MoE 系列指南（二）：跨节点专家并行与 AllToAll 通信优化工程实践",
                bbs.songma.com/80271.html
  [MoE-sched]   "MoE混合专家架构：大模型高效推理的智能调度原理", lpnh.cn/news/725941

Readings taken where the pages are silent or disagree (each is repeated at the
function that applies it):
  R1  softmax over all E experts, select the top k on it, weight = that
      probability ([DS-MoE-traps] ch.1 moe_forward pseudocode); the
      renormalised-over-k variant of [MoE-sched] §3.1 Step 2 is a flag.
  R2  selection key is the fp32 logit, larger first, ties to the lower expert
      index; -0.0 equals +0.0.
  R3  capacity slots: every top-1 claim in token order, then every top-2 claim
      in token order; a claim whose slot reaches the capacity is dropped.
  R4  capacity = max(min_capacity, ceil((k*T/E)*capacity_factor)) evaluated in
      IEEE double; no capacity when drop_tokens is off.
  R5  gate_loss is returned without the caller's weight (lambda); two kinds:
      BALANCE = E * sum_e mean_t(p[t,e]) * frac_t(top1==e)   (the load-balancing
      loss of the GShard/Switch papers that [AllToAll] lists as references;
      its formula is not printed on the pages: parity unpinned against a page
      number, pinned by closed forms only)
      USAGE_STD = std_e(usage_e) + 1e-6 with usage over all k choices before
      capacity, population std ([DS-MoE-traps] ch.1 load-balance table).
  R6  a dropped claim contributes nothing; a token with every claim dropped
      gets a zero output row.
  R7  every Linear has a bias; GELU is the exact erf form.
  R8  storage rounding: bf16 (round to nearest even) at the points where the
      HIP path stores a bf16 tensor: pre-activation a, h, y, out, dA, dX, dW.
"""

from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf

ACT_NONE, ACT_RELU, ACT_GELU = 0, 1, 2
LOSS_BALANCE, LOSS_USAGE_STD = 0, 1


# --------------------------------------------------------------------------
# storage rounding
# --------------------------------------------------------------------------
def round_bf16(v):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits and float32's exponent range.  The value
    is split as m * 2**e with 0.5 <= |m| < 1, m is scaled to 8 integer bits and
    rounded half-to-even by ``np.rint``; below the normal range the quantum is
    fixed at 2**-133 (the bf16 subnormal step).  Overflow gives +-inf.
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    # quantum exponent: value = q * 2**(e-8) for normals; clamp for subnormals
    qexp = np.maximum(e - 8, -133)
    q = np.rint(np.ldexp(v, -qexp))
    r = np.ldexp(q, qexp)
    r = np.where(np.abs(r) > 3.3895313892515355e38, np.copysign(np.inf, v), r)
    return np.where(np.isfinite(v), r, v)


def store(v, dtype):
    """Value of ``v`` after it is stored as ``dtype`` ("bf16", "f32", or
    "f64" for no rounding at all)."""
    if dtype == "f64":
        return np.asarray(v, dtype=np.float64)
    if dtype == "bf16":
        return round_bf16(v)
    if dtype == "f32":
        return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# routing: [ds.moe] §2.1 (MoE arguments) and §3.1 steps 1 and 5,
#          [MoE-sched] §3.1 Steps 1-3, [DS-MoE-traps] ch.1 pseudocode
# --------------------------------------------------------------------------
def capacity(k, num_tokens, num_experts, capacity_factor, min_capacity, drop_tokens):
    """Expert capacity C, or None when tokens are never dropped (R4).

    C = max(min_capacity, ceil(k*T/E * capacity_factor)).  The pages compute
    it as assignments per expert times a factor: [ZeRO3-MoE] §2.2 (1024x512
    tokens, top-2, 8 experts -> 131072 each, factor 2.0 -> 262144) and
    [MoE-sched] §3.1 (32x2048x2 assignments over 64 experts -> 2048).
    Python floats are IEEE doubles, so the expression is the double one.
    """
    if not drop_tokens:
        return None
    return max(int(min_capacity), math.ceil((float(k * num_tokens) / num_experts) * capacity_factor))


def router_logits(x, w_router, b_router=None):
    """logits[t,e] = x[t,:] . W_r[e,:] (+ b_r[e])   ([MoE-sched] §3.1 Step 1:
    the router is a Linear(hidden -> num_experts))."""
    l = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T
    if b_router is not None:
        l = l + np.asarray(b_router, np.float64)[None, :]
    return l


def softmax(logits):
    """Row softmax over the experts ([DS-MoE-traps] ch.1: softmax of the
    router logits along the expert axis), float64."""
    l = np.asarray(logits, np.float64)
    if l.shape[0] == 0:
        return l.copy()
    z = np.exp(l - l.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def top_k(logits, k):
    """Indices of the k chosen experts per token, best first (R2).

    Order: logit descending, then expert index ascending.  ``np.lexsort``
    compares numerically, so -0.0 and +0.0 tie and the index decides.
    """
    l = np.asarray(logits, np.float64)
    T, E = l.shape
    if T == 0:
        return np.zeros((0, k), np.int64)
    idx_key = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx_key, -l), axis=1)
    return order[:, :k].astype(np.int64)


def gate_weights(probs, idx, normalize_topk):
    """Combine weight of each (token, choice) (R1).

    Default: the softmax probability of the chosen expert.  With
    ``normalize_topk`` the k chosen probabilities are rescaled to sum to one,
    which equals [MoE-sched] §3.1 Step 2 (softmax over the top-k logits).
    Computed before any capacity drop, so a drop never rescales a survivor.
    """
    w = np.take_along_axis(probs, idx, axis=1)
    if normalize_topk:
        w = w / w.sum(axis=1, keepdims=True)
    return w


def assign_slots(idx, num_experts, cap):
    """Capacity slot of every (token, choice); -1 when dropped (R3).

    Literal definition: a fill counter per expert; all choice-0 claims are
    taken in token order, then all choice-1 claims in token order; the claim
    gets the counter's value and the counter advances.  A claim whose value
    is >= C is dropped ([MoE-sched] §3.1 item 4 "Drop tokens": tokens beyond
    the capacity are discarded).  ``cap`` None means no capacity.
    Also returns the per-expert demand of each choice.
    """
    T, k = idx.shape
    fill = [0] * num_experts
    slot = np.empty((T, k), np.int64)
    demand = np.zeros((k, num_experts), np.int64)
    for j in range(k):
        col = idx[:, j].tolist()
        for t in range(T):
            e = col[t]
            s = fill[e]
            fill[e] = s + 1
            demand[j, e] += 1
            slot[t, j] = s if (cap is None or s < cap) else -1
    return slot, demand


def expert_count_and_offset(idx, slot, num_experts):
    """expert_count[e] = kept claims of expert e ([ds.moe] §2.1 return value:
    tokens each expert processed); expert_offset = exclusive prefix sum."""
    count = np.zeros(num_experts, np.int64)
    kept = slot >= 0
    np.add.at(count, idx[kept], 1)
    offset = np.zeros(num_experts + 1, np.int64)
    offset[1:] = np.cumsum(count)
    return count, offset


def gate_loss(probs, idx, num_experts, loss_kind):
    """Auxiliary gate loss (R5), float64; zero when there are no tokens."""
    T, k = idx.shape
    if T == 0:
        return 0.0
    E = num_experts
    if loss_kind == LOSS_BALANCE:
        me = probs.mean(axis=0)
        ce = np.bincount(idx[:, 0], minlength=E) / T
        return float(E * np.sum(me * ce))
    if loss_kind == LOSS_USAGE_STD:
        usage = np.bincount(idx.reshape(-1), minlength=E) / (k * T)
        return float(np.std(usage) + 1e-6)
    raise ValueError(loss_kind)


def route(logits, k, capacity_factor=1.0, min_capacity=4, drop_tokens=True,
          normalize_topk=False, loss_kind=LOSS_BALANCE):
    """Whole gate: softmax, top-k, weights, capacity slots, counts, loss."""
    logits = np.asarray(logits, np.float64)
    T, E = logits.shape
    if not (1 <= k <= E):
        raise ValueError("k must be in 1..E")
    p = softmax(logits)
    idx = top_k(logits, k)
    w = gate_weights(p, idx, normalize_topk)
    C = capacity(k, T, E, capacity_factor, min_capacity, drop_tokens)
    slot, demand = assign_slots(idx, E, C)
    count, offset = expert_count_and_offset(idx, slot, E)
    loss = gate_loss(p, idx, E, loss_kind)
    return dict(probs=p, expert_idx=idx, weight=w, capacity=C, slot=slot,
                demand=demand, expert_count=count, expert_offset=offset,
                gate_loss=loss)


# --------------------------------------------------------------------------
# dispatch, experts, combine: [MoE-sched] §3.1 Steps 3-5, [ds.moe] §3.1
# --------------------------------------------------------------------------
def dispatch(x, idx, slot, offset):
    """Packed expert-major buffer: row offset[e]+slot holds token t's input
    for every kept claim (t, j) of expert e ([MoE-sched] §3.1 Step 3: each
    expert receives a [tokens_for_this_expert, hidden] tensor)."""
    x = np.asarray(x)
    n = int(offset[-1])
    out = np.zeros((n, x.shape[1]), x.dtype)
    T, k = idx.shape
    for t in range(T):
        for j in range(k):
            s = slot[t, j]
            if s >= 0:
                out[offset[idx[t, j]] + s] = x[t]
    return out


def gelu(a):
    """Exact GELU, 0.5*a*(1+erf(a/sqrt 2)) ([MoE-sched] §3.1 expert FFN uses
    nn.GELU(), whose default is this erf form)."""
    return 0.5 * a * (1.0 + _erf(a / math.sqrt(2.0)))


def gelu_grad(a):
    """d/da GELU(a) = Phi(a) + a*phi(a)."""
    return 0.5 * (1.0 + _erf(a / math.sqrt(2.0))) + a * np.exp(-0.5 * a * a) / math.sqrt(2.0 * math.pi)


def activation(a, act):
    if act == ACT_NONE:
        return a
    if act == ACT_RELU:
        return np.maximum(a, 0.0)
    if act == ACT_GELU:
        return gelu(a)
    raise ValueError(act)


def expert_ffn(x_disp, offset, w1, b1, w2, b2, act, dtype):
    """Expert FFNs on the packed buffer ([MoE-sched] §3.1 Step 4; expert =
    Linear-act-Linear, or one Linear when ``w2`` is None as in [ds.moe] §2.1's
    nn.Linear(512, 512) expert).

    Weights are read per expert (``w1[e]`` is [out, in]), so any indexable
    stack works.  Returns (a, h, y): pre-activation and activation output
    (both stored as ``dtype``) and the expert output stored as ``dtype``.
    For a single Linear, y == h.
    """
    x_disp = np.asarray(x_disp, np.float64)
    n = x_disp.shape[0]
    E = len(offset) - 1
    hid = np.asarray(w1[0]).shape[0]
    d_out = hid if w2 is None else np.asarray(w2[0]).shape[0]
    a_all = np.zeros((n, hid))
    h_all = np.zeros((n, hid))
    y_all = np.zeros((n, d_out))
    for e in range(E):
        r0, r1 = int(offset[e]), int(offset[e + 1])
        if r1 == r0:
            continue
        a, h, y = _ffn_rows(x_disp[r0:r1], e, w1, b1, w2, b2, act, dtype)
        a_all[r0:r1], h_all[r0:r1], y_all[r0:r1] = a, h, y
    return a_all, h_all, y_all


def _ffn_rows(X, e, w1, b1, w2, b2, act, dtype):
    """One expert's FFN on rows X: (a, h, y) with the storage roundings."""
    a = X @ np.asarray(w1[e], np.float64).T
    if b1 is not None:
        a = a + np.asarray(b1[e], np.float64)
    h = store(activation(a, act), dtype)
    if w2 is None:
        return store(a, dtype), h, h
    y = h @ np.asarray(w2[e], np.float64).T
    if b2 is not None:
        y = y + np.asarray(b2[e], np.float64)
    return store(a, dtype), h, store(y, dtype)


def token_forward(x_t, experts, weights, w1, b1, w2, b2, act, dtype):
    """Layer output of one token given its kept (expert, weight) pairs in
    choice order: sum_j w_j * FFN_{e_j}(x_t), rounded once to ``dtype``
    ([DS-MoE-traps] ch.1 weighted sum, written per token)."""
    x_t = np.asarray(x_t, np.float64)[None, :]
    out = None
    for e, w in zip(experts, weights):
        _, _, y = _ffn_rows(x_t, int(e), w1, b1, w2, b2, act, dtype)
        out = w * y[0] if out is None else out + w * y[0]
    if out is None:
        d_out = x_t.shape[1] if w2 is None else np.asarray(w2[0]).shape[0]
        out = np.zeros(d_out)
    return store(out, dtype)


def combine(y_disp, idx, slot, weight, offset, num_tokens, dtype):
    """out[t] = sum over kept choices j (in order) of w[t,j] * y_disp[row]
    ([MoE-sched] §3.1 Step 5 gather-weighted-sum; [ds.moe] §3.1 step 4
    weighted merge by gate score).  A fully dropped token gives zeros (R6)."""
    y_disp = np.asarray(y_disp, np.float64)
    out = np.zeros((num_tokens, y_disp.shape[1]))
    T, k = idx.shape
    for t in range(T):
        for j in range(k):
            s = slot[t, j]
            if s >= 0:
                out[t] += weight[t, j] * y_disp[offset[idx[t, j]] + s]
    return store(out, dtype)


def layer_forward(x, logits, w1, b1, w2, b2, *, k, capacity_factor, min_capacity,
                  drop_tokens, act, dtype, normalize_topk=False,
                  loss_kind=LOSS_BALANCE):
    """(output, gate_loss, expert_count) of the layer ([ds.moe] §2.1 return
    values), with every intermediate, given the router logits."""
    r = route(logits, k, capacity_factor, min_capacity, drop_tokens,
              normalize_topk, loss_kind)
    xd = dispatch(np.asarray(x, np.float64), r["expert_idx"], r["slot"], r["expert_offset"])
    a, h, y = expert_ffn(xd, r["expert_offset"], w1, b1, w2, b2, act, dtype)
    out = combine(y, r["expert_idx"], r["slot"], r["weight"], r["expert_offset"],
                  np.asarray(x).shape[0], dtype)
    r.update(x_disp=xd, a=a, h=h, y_disp=y, out=out)
    return r


def direct_forward(x, logits, w1, b1, w2, b2, *, k, act, dtype, normalize_topk=False):
    """No-capacity layer written per token, as in [DS-MoE-traps] ch.1's
    moe_forward: out[t] = sum_j w[t,j] * FFN_{e_j}(x[t]).  Used as a second
    formulation of the forward when nothing is dropped."""
    p = softmax(logits)
    idx = top_k(logits, k)
    w = gate_weights(p, idx, normalize_topk)
    return np.stack([token_forward(x[t], idx[t], w[t], w1, b1, w2, b2, act, dtype)
                     for t in range(np.asarray(x).shape[0])])


# --------------------------------------------------------------------------
# backward of the expert FFNs (chain rule of Linear-GELU-Linear)
# --------------------------------------------------------------------------
def expert_ffn_backward(x_disp, offset, w1, w2, a_save, h, dy, act, dtype):
    """Gradients of the packed expert FFNs for an upstream gradient dy.

    Per expert, with rows X, saved pre-activation A and H = act(A):
      dH = dY W2;  dA = dH * act'(A) (stored as ``dtype``);  dX = dA W1;
      dW2 = dY^T H;  dW1 = dA^T X;  db2 = colsum dY;  db1 = colsum dA.
    Returns (dx, dw1, db1, dw2, db2); dx/dW stored as ``dtype``, biases f32
    (unrounded in the float64 mode).
    """
    x_disp = np.asarray(x_disp, np.float64)
    dy = np.asarray(dy, np.float64)
    E = len(offset) - 1
    hid, d = np.asarray(w1[0]).shape
    dx = np.zeros_like(x_disp)
    dw1 = np.zeros((E, hid, d))
    dw2 = np.zeros((E, d, hid))
    db1 = np.zeros((E, hid))
    db2 = np.zeros((E, d))
    for e in range(E):
        r0, r1 = int(offset[e]), int(offset[e + 1])
        if r1 == r0:
            continue
        X = x_disp[r0:r1]
        A = np.asarray(a_save[r0:r1], np.float64)
        H = np.asarray(h[r0:r1], np.float64)
        dY = dy[r0:r1]
        W1 = np.asarray(w1[e], np.float64)
        W2 = np.asarray(w2[e], np.float64)
        dH = dY @ W2
        if act == ACT_GELU:
            dA = dH * gelu_grad(A)
        elif act == ACT_RELU:
            dA = dH * (A > 0)
        else:
            dA = dH
        dA = store(dA, dtype)
        dx[r0:r1] = store(dA @ W1, dtype)
        dw2[e] = store(dY.T @ H, dtype)
        dw1[e] = store(dA.T @ X, dtype)
        db2[e] = store(dY.sum(axis=0), _f32_or_f64(dtype))
        db1[e] = store(dA.sum(axis=0), _f32_or_f64(dtype))
    return dx, dw1, db1, dw2, db2


# --------------------------------------------------------------------------
# backward of the whole layer (chain rule through combine, the expert FFNs,
# dispatch, the gate weights, softmax and the router Linear)
#
# Reading R13: the top-k choice and the capacity slots are piecewise constant
# in the inputs, so they pass no gradient: the top-k operation passes its
# gradient only to the chosen positions ([DS-MoE-traps] ch.3 §3.1, the
# TopKRouter backward) and experts without tokens get none (ch.2 §2.1, the
# gradient mask); the chosen values then reach all logits through the
# softmax over the experts (R1).  The gradient of gate_loss is taken through
# its probability term only (the counts are integers).  Precisions as the HIP
# path stores them: dY_disp (= w * dOut) as ``dtype``, the per-choice weight
# gradients and logit gradients in f32, dX stored once as ``dtype`` after
# summing the expert rows and the router term, router weight and bias
# gradients in f32 (nothing is rounded in the float64 mode, dtype "f64").
# --------------------------------------------------------------------------
def combine_backward(dout, y_disp, idx, slot, weight, offset, dtype):
    """Backward of ``combine``: for each kept claim (t, j) at packed row r,
    dY_disp[r] = w[t,j] * dOut[t] and dw[t,j] = <dOut[t], y_disp[r]>;
    dropped claims get dw = 0 and own no row."""
    dout = np.asarray(dout, np.float64)
    y_disp = np.asarray(y_disp, np.float64)
    T, k = idx.shape
    dy = np.zeros_like(y_disp)
    dw = np.zeros((T, k))
    for t in range(T):
        for j in range(k):
            s = slot[t, j]
            if s >= 0:
                r = offset[idx[t, j]] + s
                dy[r] = weight[t, j] * dout[t]
                dw[t, j] = float(dout[t] @ y_disp[r])
    return store(dy, dtype), store(dw, _f32_or_f64(dtype))


def _f32_or_f64(dtype):
    """The f32 intermediates of the backward, left unrounded in the pure
    float64 mode (dtype "f64") used by the mathematical pins."""
    return "f64" if dtype == "f64" else "f32"


def dispatch_backward(dx_disp, idx, slot, offset, num_tokens):
    """Backward of ``dispatch``: token t's input gradient is the sum over its
    kept claims (in choice order) of the rows they were copied to."""
    dx_disp = np.asarray(dx_disp, np.float64)
    dx = np.zeros((num_tokens, dx_disp.shape[1]))
    T, k = idx.shape
    for t in range(T):
        for j in range(k):
            s = slot[t, j]
            if s >= 0:
                dx[t] += dx_disp[offset[idx[t, j]] + s]
    return dx


def gate_backward(probs, idx, dw, normalize_topk, loss_kind, dloss, dtype="f32", top1_count=None,
                  num_tokens=None):
    """Gradient of the router logits from the weight gradients dw [T, k] and
    the upstream gradient dloss of gate_loss.  ``top1_count`` [E] and
    ``num_tokens`` describe the whole batch when ``probs`` holds only some of
    its tokens (default: the rows given are the batch).

    Weights: w_j = p[t, e_j], or w_j = p_j / S with S = sum_j p[t, e_j]
    (normalize_topk), whose derivative gives dp[t, e_i] += (dw_i - sum_j
    dw_j w_j) / S.  BALANCE loss E * sum_e mean_t(p[t,e]) * ce_e adds
    dloss * E * ce_e / T to every dp[t, e] (ce_e = share of top-1 choices);
    USAGE_STD depends on counts only.  Then the softmax backward
    dlogits = p * (dp - <p, dp>) per token.
    """
    p = np.asarray(probs, np.float64)
    T, E = p.shape
    k = idx.shape[1]
    dw = np.asarray(dw, np.float64)
    dp = np.zeros((T, E))
    for t in range(T):
        pe = [p[t, idx[t, j]] for j in range(k)]
        if normalize_topk:
            S = sum(pe)
            w = [v / S for v in pe]
            corr = sum(dw[t, j] * w[j] for j in range(k))
            for i in range(k):
                dp[t, idx[t, i]] += (dw[t, i] - corr) / S
        else:
            for j in range(k):
                dp[t, idx[t, j]] += dw[t, j]
    if T > 0 and loss_kind == LOSS_BALANCE:
        n = T if num_tokens is None else num_tokens
        cnt = np.bincount(idx[:, 0], minlength=E) if top1_count is None else np.asarray(top1_count)
        ce = cnt / n
        dp += dloss * E * ce[None, :] / n
    dl = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return store(dl, _f32_or_f64(dtype))


def router_backward(x, w_router, dlogits):
    """Backward of ``router_logits``: dx = dlogits W_r, dW_r = dlogits^T x,
    db_r = column sums of dlogits (all float64)."""
    x = np.asarray(x, np.float64)
    dl = np.asarray(dlogits, np.float64)
    wr = np.asarray(w_router, np.float64)
    return dl @ wr, dl.T @ x, dl.sum(axis=0)


def layer_backward(x, w_router, r, w1, w2, dout, dloss, *, act, dtype,
                   normalize_topk=False, loss_kind=LOSS_BALANCE, router_input=None, router_input_scale=None):
    """Gradients of <dOut, out> + dloss * gate_loss for the layer whose
    forward ``r`` is (``layer_forward``'s result, with ``probs`` from the
    same logits).  ``w_router`` None means the logits were inputs: the
    logit gradient is returned instead of router gradients.
    ``router_input`` / ``router_input_scale``: when the router read
    x * scale rather than x (the jitter option of ``stochastic_gate``), its
    weight gradient contracts with that input and its input gradient carries
    the scale (the chain rule of logits = (x * scale) W_r^T).

    Returns a dict: dx (stored ``dtype``), dlogits (f32), dw_router, db_router
    (f32, or None), dw1, db1, dw2, db2 (as ``expert_ffn_backward``), and the
    intermediates dy_disp, dw_gate, dx_disp.
    """
    T = np.asarray(x).shape[0]
    idx, slot, off = r["expert_idx"], r["slot"], r["expert_offset"]
    dy, dwg = combine_backward(dout, r["y_disp"], idx, slot, r["weight"], off, dtype)
    dxd, dw1, db1, dw2, db2 = expert_ffn_backward(r["x_disp"], off, w1, w2, r["a"], r["h"], dy, act, dtype)
    dx = dispatch_backward(dxd, idx, slot, off, T)
    dl = gate_backward(r["probs"], idx, dwg, normalize_topk, loss_kind, dloss, dtype)
    dwr = dbr = None
    if w_router is not None:
        dxr, dwr, dbr = router_backward(x if router_input is None else router_input, w_router, dl)
        if router_input_scale is not None:
            dxr = dxr * np.asarray(router_input_scale, np.float64)
        dx = dx + dxr
        dwr, dbr = store(dwr, _f32_or_f64(dtype)), store(dbr, _f32_or_f64(dtype))
    return dict(dx=store(dx, dtype), dlogits=dl, dw_router=dwr, db_router=dbr,
                dw1=dw1, db1=db1, dw2=dw2, db2=db2, dy_disp=dy, dw_gate=dwg, dx_disp=dxd)

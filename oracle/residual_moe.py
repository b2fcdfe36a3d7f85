"""CPU oracle for the residual MoE layer (PR-MoE's use_residual).

TEST INFRASTRUCTURE ONLY, like ``moe_oracle``: only the test suite, the smoke
check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may use
it.  It shares no code with the HIP library.

What the pages say ("deepspeed.moe 模块" overview [ds.moe]): use_residual
turns on PR-MoE, the residual MoE (§2.1 arguments); PR-MoE combines a fixed
MLP with the dynamic experts through a residual connection, and its pyramid
uses fewer experts in early layers and more in later ones, through a list of
expert counts (§2.3, §3.3); §4.2's example builds it from an nn.Linear expert
with num_experts=[4, 8, 16].

Reading R16 (the mix is not on the pages): the dense branch is an MLP of the
expert's own architecture with its own weights, applied to every token.  The
two outputs are mixed per token by coefficients c = softmax(x W_c^T + b_c)
over two entries, out = c0 * moe(x) + c1 * mlp(x), as in the published
DeepSpeed layer that the pages document (its coefficient is a Linear from
the hidden size to 2 followed by a softmax).  Without coefficient weights
the mix is the plain residual sum moe(x) + mlp(x) of the PR-MoE paper's
residual MoE.  The pyramid is a property of the model: each layer is its own
call with its own number of experts.

Precision (R8 extended): the MLP's activation output and output are stored
as bf16 like an expert's; the coefficient logits are bf16 inputs with exact
accumulation here; the MoE sum is kept unrounded and the mixed output is
rounded once.
"""

from __future__ import annotations

import numpy as np

from oracle import moe_oracle as O


def coefficients(x, coef_w=None, coef_b=None):
    """[T, 2] mixing coefficients softmax(x W_c^T + b_c), or ones (the plain
    residual sum) when ``coef_w`` is None."""
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    if coef_w is None:
        return np.ones((T, 2))
    l = x @ np.asarray(coef_w, np.float64).T
    if coef_b is not None:
        l = l + np.asarray(coef_b, np.float64)[None, :]
    return O.softmax(l)


def dense_mlp(x, mlp, act, dtype):
    """The dense branch: the expert architecture with weights ``mlp`` =
    (w1 [h, d], b1, w2 [d, h], b2), or one Linear (w2 None), on every token.
    Returns (a, h, y) as ``moe_oracle.expert_ffn`` does for one expert."""
    w1, b1, w2, b2 = mlp
    T = np.asarray(x).shape[0]
    wrap = lambda v: None if v is None else [np.asarray(v)]
    return O.expert_ffn(np.asarray(x, np.float64), np.array([0, T]), wrap(w1), wrap(b1), wrap(w2), wrap(b2),
                        act, dtype)


def forward(x, logits, w1, b1, w2, b2, mlp, coef_w=None, coef_b=None, *, k, capacity_factor, min_capacity,
            drop_tokens, act, dtype, normalize_topk=False, loss_kind=O.LOSS_BALANCE):
    """The residual MoE layer: ``moe_oracle.layer_forward``'s routing and
    experts, the dense branch, the coefficients and the mix (R16).  Returns
    the MoE layer's dict with out replaced by the mixed output, plus moe (the
    unrounded MoE sum), mlp_a, mlp_h, mlp_y and coef."""
    r = O.layer_forward(x, logits, w1, b1, w2, b2, k=k, capacity_factor=capacity_factor,
                        min_capacity=min_capacity, drop_tokens=drop_tokens, act=act, dtype=dtype,
                        normalize_topk=normalize_topk, loss_kind=loss_kind)
    T = np.asarray(x).shape[0]
    moe = O.combine(r["y_disp"], r["expert_idx"], r["slot"], r["weight"], r["expert_offset"], T, "f64")
    a, h, y = dense_mlp(x, mlp, act, dtype)
    c = coefficients(x, coef_w, coef_b)
    out = O.store(c[:, :1] * moe + c[:, 1:] * y, dtype)
    r.update(out=out, moe=moe, mlp_a=a, mlp_h=h, mlp_y=y, coef=c)
    return r


def backward(x, w_router, r, w1, w2, mlp, coef_w, dout, dloss, *, act, dtype, normalize_topk=False,
             loss_kind=O.LOSS_BALANCE):
    """Gradients of <dOut, out> + dloss * gate_loss for ``forward``'s result
    ``r`` (the chain rule through the mix):
      MoE branch   the layer backward with dOut scaled by c0;
      dense branch the MLP backward with dOut scaled by c1;
      coefficients dc = (<dOut, moe>, <dOut, mlp_y>), through the two-way
                   softmax dl = c * (dc - <c, dc>), then dW_c = dl^T x,
                   db_c = column sums, and dl W_c into dx.
    Returns the MoE layer backward's dict with dx the sum of all three
    input gradients (stored ``dtype``) and mlp_dw1, mlp_db1, mlp_dw2,
    mlp_db2, dcoef_w, dcoef_b, dcoef_logits added."""
    x = np.asarray(x, np.float64)
    dout = np.asarray(dout, np.float64)
    T = x.shape[0]
    c = r["coef"]
    g = O.layer_backward(x, w_router, r, w1, w2, c[:, :1] * dout, dloss, act=act, dtype="f64" if dtype == "f64"
                         else dtype, normalize_topk=normalize_topk, loss_kind=loss_kind)
    # the MoE layer backward rounds its dx; take it again unrounded
    dx = O.dispatch_backward(g["dx_disp"], r["expert_idx"], r["slot"], r["expert_offset"], T)
    if w_router is not None:
        dx = dx + g["dlogits"] @ np.asarray(w_router, np.float64)
    mw1, _, mw2, _ = mlp
    if mw2 is None:
        raise ValueError("the backward takes a two-Linear expert (as the expert FFN backward does)")
    dy_mlp = O.store(c[:, 1:] * dout, dtype)
    wrap = lambda v: [np.asarray(v)]
    dxm, dw1m, db1m, dw2m, db2m = O.expert_ffn_backward(x, np.array([0, T]), wrap(mw1), wrap(mw2), r["mlp_a"],
                                                        r["mlp_h"], dy_mlp, act, dtype)
    dcw = dcb = dl = None
    if coef_w is not None:
        dc = np.stack([(dout * r["moe"]).sum(axis=1), (dout * r["mlp_y"]).sum(axis=1)], axis=1)
        dl = c * (dc - (c * dc).sum(axis=1, keepdims=True))
        dcw = dl.T @ x
        dcb = dl.sum(axis=0)
        dx = dx + dl @ np.asarray(coef_w, np.float64)
    g.update(dx=O.store(dx + dxm, dtype), mlp_dw1=dw1m[0], mlp_db1=db1m[0], mlp_dw2=dw2m[0], mlp_db2=db2m[0],
             dy_mlp=dy_mlp, dcoef_w=dcw, dcoef_b=dcb, dcoef_logits=dl)
    return g

"""Top-k gated Mixture-of-Experts layer for one MI355X (gfx950) GPU.

The compute is the HIP library libmoe_mi355x.so behind the C ABI in
include/moe.h; ``binding`` exposes those calls with the same names and
``MoE`` is a small holder of the layer's weights whose ``forward`` returns
(output, gate_loss, expert_count) like the MoE layer of the deepspeed.moe
overview page (§2.1).  torch is used for device memory and streams only.
"""
from __future__ import annotations

from . import binding
from .binding import (MOE_ACT_GELU, MOE_ACT_NONE, MOE_ACT_RELU, MOE_BF16, MOE_F32,  # noqa: F401
                      MOE_LOSS_BALANCE, MOE_LOSS_USAGE_STD, MOE_NOISE_JITTER, MOE_NOISE_NONE, MOE_NOISE_RSAMPLE, MoeConfig, MoeError, make_config,
                      moe_capacity, moe_combine, moe_dispatch, moe_expert_ffn, moe_expert_ffn_backward,
                      moe_gate, moe_layer_forward, moe_max_rows, moe_workspace_size, moe_workspace_views)


class MoE:
    """Weights and workspace of one MoE layer; ``forward(x)`` runs the fused
    layer on the current stream and returns (output, gate_loss, expert_count).

    Arguments mirror MoE(hidden_size, num_experts, k, capacity_factor,
    eval_capacity_factor, min_capacity, drop_tokens) of the deepspeed.moe
    overview (§2.1): capacity_factor applies in training mode (the default,
    ``train()``), eval_capacity_factor after ``eval()``.  The expert is
    Linear(hidden, ffn_hidden) -> activation -> Linear(ffn_hidden, hidden),
    or one Linear(hidden, hidden) when ffn_hidden == 0.  Weights use the
    nn.Linear [out, in] layout, stacked over experts.  ``residual`` =
    (mlp_w1, mlp_b1, mlp_w2, mlp_b2, coef_w, coef_b) makes it the residual MoE
    of PR-MoE (use_residual): a dense MLP of the expert's shape mixed in by
    softmax(x coef_w^T + coef_b), or summed when coef_w is None; a pyramid
    is a stack of such layers with their own num_experts.  small_batch selects
    the one-launch forward for a few tokens (0 automatic, 1 always when it
    applies, -1 never).

    ``pack_weights()`` keeps copies of the expert weights in the packed
    layout (moe_pack_expert_weight), which the inference forward (after
    ``eval()``) then reads; call it again after the weights change.  Training
    forwards read the nn.Linear weights.

    The random gate options noisy_gate_policy ("Jitter" or "RSample"),
    use_rts and top2_2nd_expert_sampling act in training mode only and, as
    in the gate they come from, each where it applies: RSample and RTS with
    k = 1, second-expert sampling with k = 2, jitter with either.  Their
    Philox seed is ``seed`` plus the number of training forwards so far, so
    each step draws fresh noise and a run is reproducible.  They default to
    off (the deterministic gate).
    """

    def __init__(self, hidden_size, num_experts, w_router, w1, b1=None, w2=None, b2=None, b_router=None,
                 k=1, capacity_factor=1.0, eval_capacity_factor=1.0, min_capacity=4, drop_tokens=True,
                 ffn_hidden=0, activation=MOE_ACT_NONE, normalize_topk=False, loss_kind=MOE_LOSS_BALANCE,
                 small_batch=0, noisy_gate_policy=None, use_rts=False, top2_2nd_expert_sampling=False, seed=0,
                 residual=None):
        import torch
        self.hidden_size, self.num_experts, self.k = hidden_size, num_experts, k
        self.capacity_factor, self.min_capacity, self.drop_tokens = capacity_factor, min_capacity, drop_tokens
        self.eval_capacity_factor, self.small_batch, self.training = eval_capacity_factor, small_batch, True
        policies = {None: MOE_NOISE_NONE, "jitter": MOE_NOISE_JITTER, "rsample": MOE_NOISE_RSAMPLE}
        key = noisy_gate_policy.lower() if isinstance(noisy_gate_policy, str) else noisy_gate_policy
        if key not in policies:
            raise ValueError(f"noisy_gate_policy must be None, 'Jitter' or 'RSample', not {noisy_gate_policy!r}")
        self.noisy_gate_policy, self.use_rts = policies[key], bool(use_rts)
        self.top2_2nd_expert_sampling, self.seed, self.steps = bool(top2_2nd_expert_sampling), int(seed), 0
        # residual MoE (use_residual): (mlp_w1, mlp_b1, mlp_w2, mlp_b2, coef_w, coef_b) or None
        if residual is not None and len(residual) != 6:
            raise ValueError("residual is (mlp_w1, mlp_b1, mlp_w2, mlp_b2, coef_w, coef_b)")
        self.residual = residual
        self.ffn_hidden, self.activation = ffn_hidden, activation
        self.normalize_topk, self.loss_kind = normalize_topk, loss_kind
        self.w_router, self.b_router = w_router, b_router
        self.w1, self.b1, self.w2, self.b2 = w1, b1, w2, b2
        self.dtype = MOE_BF16 if w1.dtype == torch.bfloat16 else MOE_F32
        self._ws = None
        self._packed = None   # (w1, w2) in the packed layout, or None

    def pack_weights(self):
        """Packed copies of w1 and w2 for the inference forward (raises
        MoeError where the packed layout does not apply)."""
        probe = make_config(1, self.hidden_size, self.num_experts, self.k, 1.0, self.min_capacity, self.drop_tokens,
                            self.ffn_hidden, self.activation, self.dtype, packed_weights=True)
        moe_workspace_size(probe)   # validates the configuration
        w2 = binding.pack_expert_weight(self.w2) if self.w2 is not None else None
        self._packed = (binding.pack_expert_weight(self.w1), w2)
        return self

    def train(self, mode=True):
        self.training = bool(mode)
        return self

    def eval(self):
        return self.train(False)

    def config(self, num_tokens):
        cf = self.capacity_factor if self.training else self.eval_capacity_factor
        rnd = {}
        if self.training:
            noise = self.noisy_gate_policy
            if noise == MOE_NOISE_RSAMPLE and self.k != 1:
                noise = MOE_NOISE_NONE
            rnd = dict(noisy_gate_policy=noise, use_rts=self.use_rts and self.k == 1,
                       second_expert_sampling=self.top2_2nd_expert_sampling and self.k == 2,
                       seed=(self.seed + self.steps) % 2 ** 64)
        return make_config(num_tokens, self.hidden_size, self.num_experts, self.k, cf, self.min_capacity,
                           self.drop_tokens, self.ffn_hidden, self.activation, self.dtype, self.normalize_topk,
                           self.loss_kind, small_batch=self.small_batch, use_residual=self.residual is not None,
                           packed_weights=self._packed is not None and not self.training, **rnd)

    def forward(self, x, logits=None):
        import torch
        shape = x.shape
        x2 = x.reshape(-1, self.hidden_size).contiguous()
        cfg = self.config(x2.shape[0])
        nbytes = moe_workspace_size(cfg)
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
        out = torch.empty_like(x2)
        loss = torch.empty(1, dtype=torch.float32, device=x.device)
        count = torch.empty(self.num_experts, dtype=torch.int32, device=x.device)
        w1, w2 = self._packed if cfg.packed_weights else (self.w1, self.w2)
        if self.residual is None:
            moe_layer_forward(cfg, x2, self.w_router, self.b_router, logits, w1, self.b1, w2, self.b2,
                              out, loss, count, ws=self._ws)
        else:
            binding.moe_residual_layer_forward(cfg, x2, self.w_router, self.b_router, logits, w1, self.b1,
                                               w2, self.b2, *self.residual, out, loss, count, ws=self._ws)
        if self.training:
            self.steps += 1
        return out.reshape(shape), loss[0], count

    __call__ = forward

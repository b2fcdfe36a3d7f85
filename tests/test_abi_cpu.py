"""The C-ABI library on a machine without a GPU: it loads, exports every
function include/moe.h declares, the config struct layout matches the C
compiler's, and every host-only call (capacity, row bound, workspace size,
argument validation) behaves as documented.  No compute call reaches the GPU:
the device entry points are only called with arguments that fail validation,
which happens before anything is enqueued."""
import ctypes
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest
import torch

from mixture_experts_layer_39_amd import binding as B
from oracle import moe_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|const char\*)\s+(moe_\w+)\s*\(", txt, re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 11
    L = B.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(B.EXPORTED)


def test_config_struct_layout_matches_c():
    src = r'''
#include <stdio.h>
#include <stddef.h>
#include "moe.h"
int main(void) {
  printf("%zu", sizeof(moe_config));
#define F(n) printf(" %zu", offsetof(moe_config, n));
  F(num_tokens) F(capacity_factor) F(hidden_size) F(num_experts) F(k) F(min_capacity) F(drop_tokens)
  F(ffn_hidden) F(activation) F(dtype) F(normalize_topk) F(loss_kind) F(save_preact)
  F(small_batch) F(noisy_gate_policy) F(use_rts) F(second_expert_sampling) F(use_residual) F(seed)
  F(packed_weights)
  return 0;
}'''
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        exe = os.path.join(d, "t")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        vals = [int(v) for v in subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()]
    want = [ctypes.sizeof(B.MoeConfig)] + [getattr(B.MoeConfig, f[0]).offset for f in B.MoeConfig._fields_]
    assert vals == want


def _cfg(**kw):
    base = dict(num_tokens=4096, hidden_size=512, num_experts=8, k=2, capacity_factor=1.0, min_capacity=4,
                drop_tokens=True, ffn_hidden=0, activation=B.MOE_ACT_NONE, dtype=B.MOE_BF16)
    base.update(kw)
    return B.make_config(**base)


def test_capacity_matches_oracle_on_many_configs():
    rng = np.random.default_rng(0)
    factors = [0.25, 0.5, 1.0, 1.1, 1.2, 1.25, 1.5, 2.0, 2.2, 3.3, 0.1, 7.0]
    for _ in range(2000):
        T = int(rng.integers(0, 70000))
        E = int(rng.integers(1, 257))
        k = int(rng.integers(1, 3)) if E > 1 else 1
        cf = float(rng.choice(factors))
        mc = int(rng.integers(0, 9))
        got = B.moe_capacity(_cfg(num_tokens=T, num_experts=E, k=k, capacity_factor=cf, min_capacity=mc))
        assert got == O.capacity(k, T, E, cf, mc, True), (T, E, k, cf, mc)
    # the double-evaluation case: 50 * 1.1 = 55.00000000000001 -> 56
    assert B.moe_capacity(_cfg(num_tokens=100, num_experts=4, k=2, capacity_factor=1.1, min_capacity=0)) == 56
    assert B.moe_capacity(_cfg(drop_tokens=False)) == -1


def test_workload_capacities_and_rows():
    assert B.moe_capacity(_cfg(num_tokens=64, hidden_size=32, num_experts=4, k=1, dtype=B.MOE_F32)) == 16
    assert B.moe_capacity(_cfg()) == 1024
    assert B.moe_capacity(_cfg(num_tokens=16384, hidden_size=2048, num_experts=64, capacity_factor=1.25)) == 640
    assert B.moe_capacity(_cfg(num_tokens=32768, hidden_size=4096, num_experts=16, capacity_factor=2.0)) == 8192
    assert B.moe_max_rows(_cfg()) == 8192
    assert B.moe_max_rows(_cfg(num_tokens=16384, num_experts=64, capacity_factor=1.25)) == 32768
    assert B.moe_max_rows(_cfg(capacity_factor=0.5)) == 8 * 512
    assert B.moe_max_rows(_cfg(num_tokens=65536, num_experts=128, drop_tokens=False)) == 131072
    assert B.moe_max_rows(_cfg(num_tokens=0)) == 0


def test_workspace_size_grows_with_problem():
    a = B.moe_workspace_size(_cfg())
    b = B.moe_workspace_size(_cfg(num_tokens=8192))
    c = B.moe_workspace_size(_cfg(ffn_hidden=1024, activation=B.MOE_ACT_GELU))
    d = B.moe_workspace_size(_cfg(ffn_hidden=1024, activation=B.MOE_ACT_GELU, save_preact=True))
    assert 0 < a < b and a < c < d
    assert B.moe_workspace_size(_cfg(num_tokens=0)) > 0
    # the packed buffers alone: rows * d * 2 bytes for x_disp and y_disp
    assert a >= 2 * 8192 * 512 * 2


@pytest.mark.parametrize("kw,status", [
    (dict(k=3), B.MOE_ERR_INVALID_ARG),
    (dict(k=0), B.MOE_ERR_INVALID_ARG),
    (dict(num_experts=1, k=2), B.MOE_ERR_INVALID_ARG),
    (dict(num_experts=0), B.MOE_ERR_INVALID_ARG),
    (dict(num_experts=257), B.MOE_ERR_INVALID_ARG),
    (dict(num_tokens=-1), B.MOE_ERR_INVALID_ARG),
    (dict(num_tokens=1 << 30), B.MOE_ERR_INVALID_ARG),
    (dict(hidden_size=0), B.MOE_ERR_INVALID_ARG),
    (dict(capacity_factor=0.0), B.MOE_ERR_INVALID_ARG),
    (dict(capacity_factor=-1.0), B.MOE_ERR_INVALID_ARG),
    (dict(capacity_factor=float("inf")), B.MOE_ERR_INVALID_ARG),
    (dict(min_capacity=-1), B.MOE_ERR_INVALID_ARG),
    (dict(ffn_hidden=-8), B.MOE_ERR_INVALID_ARG),
    (dict(activation=3), B.MOE_ERR_INVALID_ARG),
    (dict(dtype=2), B.MOE_ERR_INVALID_ARG),
    (dict(loss_kind=2), B.MOE_ERR_INVALID_ARG),
    (dict(normalize_topk=2), B.MOE_ERR_INVALID_ARG),
    (dict(small_batch=2), B.MOE_ERR_INVALID_ARG),
    (dict(noisy_gate_policy=3), B.MOE_ERR_INVALID_ARG),
    (dict(noisy_gate_policy=B.MOE_NOISE_RSAMPLE, k=2), B.MOE_ERR_INVALID_ARG),
    (dict(use_rts=True, k=2), B.MOE_ERR_INVALID_ARG),
    (dict(second_expert_sampling=True, k=1), B.MOE_ERR_INVALID_ARG),
    (dict(noisy_gate_policy=B.MOE_NOISE_JITTER, dtype=B.MOE_F32), B.MOE_ERR_UNSUPPORTED),
    (dict(small_batch=-2), B.MOE_ERR_INVALID_ARG),
    (dict(use_residual=True, dtype=B.MOE_F32), B.MOE_ERR_UNSUPPORTED),
    (dict(hidden_size=500), B.MOE_ERR_UNSUPPORTED),
    (dict(ffn_hidden=100, activation=B.MOE_ACT_GELU), B.MOE_ERR_UNSUPPORTED),
    (dict(hidden_size=34, dtype=B.MOE_F32), B.MOE_ERR_UNSUPPORTED),
    (dict(packed_weights=True, dtype=B.MOE_F32), B.MOE_ERR_UNSUPPORTED),
    (dict(packed_weights=True, hidden_size=96), B.MOE_ERR_UNSUPPORTED),              # d % 64
    (dict(packed_weights=True, ffn_hidden=520, activation=B.MOE_ACT_GELU), B.MOE_ERR_UNSUPPORTED),  # h % 64
])
def test_invalid_configs_are_rejected(kw, status):
    cfg = _cfg(**kw)
    if "normalize_topk" in kw:
        cfg.normalize_topk = kw["normalize_topk"]
    with pytest.raises(B.MoeError) as ei:
        B.moe_workspace_size(cfg)
    assert ei.value.status == status
    with pytest.raises(B.MoeError):
        B.moe_capacity(cfg)


def test_eval_mode_uses_eval_capacity_factor():
    """The MoE holder takes capacity_factor in training mode and
    eval_capacity_factor after eval() (deepspeed.moe overview §2.1)."""
    import mixture_experts_layer_39_amd as pkg
    w = torch.zeros(4, 8, 16, dtype=torch.bfloat16)
    m = pkg.MoE(16, 4, None, w, k=2, capacity_factor=1.0, eval_capacity_factor=2.0, min_capacity=1,
                ffn_hidden=8, small_batch=-1)
    assert m.training
    assert B.moe_capacity(m.config(64)) == 32
    assert B.moe_capacity(m.eval().config(64)) == 64
    assert m.config(64).small_batch == -1
    assert B.moe_capacity(m.train().config(64)) == 32


def test_random_gate_options_follow_mode_and_k():
    """The holder passes the random gate options in training mode only, each
    where it applies (RSample and RTS for k = 1, second-expert sampling for
    k = 2, jitter for both), with a seed that advances per training step."""
    import mixture_experts_layer_39_amd as pkg
    w = torch.zeros(4, 8, 16, dtype=torch.bfloat16)
    for k in (1, 2):
        m = pkg.MoE(16, 4, None, w, k=k, ffn_hidden=8, noisy_gate_policy="RSample", use_rts=True,
                    top2_2nd_expert_sampling=True, seed=7)
        c = m.config(64)
        assert c.noisy_gate_policy == (B.MOE_NOISE_RSAMPLE if k == 1 else B.MOE_NOISE_NONE)
        assert c.use_rts == (k == 1) and c.second_expert_sampling == (k == 2) and c.seed == 7
        B.moe_workspace_size(c)   # a valid configuration
        m.steps = 3
        assert m.config(64).seed == 10
        e = m.eval().config(64)
        assert (e.noisy_gate_policy, e.use_rts, e.second_expert_sampling) == (0, 0, 0)
    j = pkg.MoE(16, 4, None, w, k=2, ffn_hidden=8, noisy_gate_policy="Jitter")
    assert j.config(8).noisy_gate_policy == B.MOE_NOISE_JITTER
    with pytest.raises(ValueError):
        pkg.MoE(16, 4, None, w, noisy_gate_policy="gaussian")


def test_capacity_factor_unused_without_drop():
    assert B.moe_capacity(_cfg(drop_tokens=False, capacity_factor=0.0)) == -1


def test_null_config_and_outputs():
    L = B.lib()
    assert L.moe_workspace_size(None, None) == B.MOE_ERR_INVALID_ARG
    cfg = _cfg()
    assert L.moe_capacity(ctypes.byref(cfg), None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_max_rows(ctypes.byref(cfg), None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_workspace_views(ctypes.byref(cfg), None, None, None, None, None, None) == B.MOE_ERR_INVALID_ARG


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def test_device_entry_points_validate_before_launch():
    L = B.lib()
    cfg = _cfg()
    ws_need = B.moe_workspace_size(cfg)
    c = ctypes.byref(cfg)
    # missing outputs
    assert L.moe_gate(c, FAKE, FAKE, None, None, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws_need, None) \
        == B.MOE_ERR_INVALID_ARG
    # neither x/w_router nor logits
    assert L.moe_gate(c, None, None, None, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws_need, None) \
        == B.MOE_ERR_INVALID_ARG
    # workspace too small
    assert L.moe_gate(c, FAKE, FAKE, None, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws_need - 1,
                      None) == B.MOE_ERR_WORKSPACE
    assert L.moe_dispatch(c, FAKE, FAKE, None, FAKE, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_combine(c, FAKE, FAKE, FAKE, None, FAKE, FAKE, None) == B.MOE_ERR_INVALID_ARG
    # single-Linear expert must not get w2
    assert L.moe_expert_ffn(c, FAKE, FAKE, FAKE, None, FAKE, None, None, None, 0, FAKE, None, 0, None) \
        == B.MOE_ERR_INVALID_ARG
    cfg2 = _cfg(ffn_hidden=1024, activation=B.MOE_ACT_GELU)
    c2 = ctypes.byref(cfg2)
    # two-Linear expert needs w2 and h_disp
    assert L.moe_expert_ffn(c2, FAKE, FAKE, FAKE, None, None, None, None, FAKE, 0, FAKE, None, 0, None) \
        == B.MOE_ERR_INVALID_ARG
    assert L.moe_expert_ffn(c2, FAKE, FAKE, FAKE, None, FAKE, None, None, None, 0, FAKE, None, 0, None) \
        == B.MOE_ERR_INVALID_ARG
    # h_disp's row pitch: h or h + 64 only
    for bad in (1023, 1025, 1024 + 32, 1024 + 128, -1):
        assert L.moe_expert_ffn(c2, FAKE, FAKE, FAKE, None, FAKE, None, None, FAKE, bad, FAKE, None, 0, None) \
            == B.MOE_ERR_INVALID_ARG, bad
    # a padded pitch needs the bf16 large-tile path (d and h multiples of 64)
    cfg3 = _cfg(hidden_size=96, ffn_hidden=1024, activation=B.MOE_ACT_GELU)
    assert L.moe_expert_ffn(ctypes.byref(cfg3), FAKE, FAKE, FAKE, None, FAKE, None, None, FAKE, 1088, FAKE, None, 0,
                            None) == B.MOE_ERR_UNSUPPORTED
    # backward needs a hidden layer and every gradient output
    assert L.moe_expert_ffn_backward(c, *([FAKE] * 12), FAKE, 1 << 40, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_expert_ffn_backward(c2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None,
                                     FAKE, 1 << 40, None) == B.MOE_ERR_INVALID_ARG
    ws2 = B.moe_workspace_size(cfg2)
    assert L.moe_expert_ffn_backward(c2, *([FAKE] * 12), FAKE, ws2 - 1, None) == B.MOE_ERR_WORKSPACE
    # backward kernels: bf16 only, d and h multiples of 16
    cfg3 = _cfg(hidden_size=24, ffn_hidden=32, activation=B.MOE_ACT_GELU)
    assert L.moe_expert_ffn_backward(ctypes.byref(cfg3), *([FAKE] * 12), FAKE, 1 << 40, None) == B.MOE_ERR_UNSUPPORTED
    cfg4 = _cfg(hidden_size=32, ffn_hidden=64, activation=B.MOE_ACT_GELU, dtype=B.MOE_F32)
    assert L.moe_expert_ffn_backward(ctypes.byref(cfg4), *([FAKE] * 12), FAKE, 1 << 40, None) == B.MOE_ERR_UNSUPPORTED
    # fused forward
    assert L.moe_layer_forward(c, FAKE, FAKE, None, None, FAKE, None, None, None, FAKE, FAKE, None, None, None,
                               None, None, FAKE, ws_need, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_layer_forward(c, FAKE, FAKE, None, None, FAKE, None, None, None, FAKE, FAKE, FAKE, None, None,
                               None, None, FAKE, ws_need - 1, None) == B.MOE_ERR_WORKSPACE
    assert L.moe_layer_forward(c, FAKE, None, None, None, FAKE, None, None, None, FAKE, FAKE, FAKE, None, None,
                               None, None, FAKE, ws_need, None) == B.MOE_ERR_INVALID_ARG


def test_backward_entry_points_validate_before_launch():
    L = B.lib()
    tr = _cfg(hidden_size=256, ffn_hidden=512, activation=B.MOE_ACT_GELU, save_preact=True)
    ws = B.moe_workspace_size(tr)
    c = ctypes.byref(tr)
    inf = _cfg(hidden_size=256, ffn_hidden=512, activation=B.MOE_ACT_GELU)
    ci = ctypes.byref(inf)
    # training workspace is larger (it holds the logits and the backward regions)
    assert ws > B.moe_workspace_size(inf)
    # combine backward: every pointer needed
    assert L.moe_combine_backward(c, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == B.MOE_ERR_INVALID_ARG
    # gate backward: training config, outputs, workspace size
    assert L.moe_gate_backward(ci, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1 << 40, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_gate_backward(c, FAKE, FAKE, FAKE, None, None, FAKE, ws, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_gate_backward(c, FAKE, FAKE, FAKE, None, FAKE, FAKE, ws - 1, None) == B.MOE_ERR_WORKSPACE
    # dispatch backward: dlogits needed with the router weight; bf16 and d % 32
    assert L.moe_dispatch_backward(c, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, ws, None) \
        == B.MOE_ERR_INVALID_ARG
    assert L.moe_dispatch_backward(c, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, ws - 1, None) \
        == B.MOE_ERR_WORKSPACE
    f32 = _cfg(hidden_size=256, ffn_hidden=512, activation=B.MOE_ACT_GELU, save_preact=True, dtype=B.MOE_F32)
    assert L.moe_dispatch_backward(ctypes.byref(f32), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, 1 << 40,
                                   None) == B.MOE_ERR_UNSUPPORTED
    # router backward: some output; d % 64 for the weight gradient
    assert L.moe_router_backward(c, FAKE, FAKE, None, None, FAKE, ws, None) == B.MOE_ERR_INVALID_ARG
    d96 = _cfg(hidden_size=96, ffn_hidden=64, activation=B.MOE_ACT_GELU, save_preact=True)
    assert L.moe_router_backward(ctypes.byref(d96), FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None) \
        == B.MOE_ERR_UNSUPPORTED
    # layer backward: training config with a hidden layer; router gradients need the router weight
    args = [FAKE] * 18
    assert L.moe_layer_backward(ci, *args, FAKE, 1 << 40, None) == B.MOE_ERR_INVALID_ARG
    no_router = list(args)
    no_router[1] = None
    assert L.moe_layer_backward(c, *no_router, FAKE, ws, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_layer_backward(c, *args, FAKE, ws - 1, None) == B.MOE_ERR_WORKSPACE
    one = _cfg(hidden_size=256, ffn_hidden=0, save_preact=True)
    assert L.moe_layer_backward(ctypes.byref(one), *args, FAKE, 1 << 40, None) == B.MOE_ERR_INVALID_ARG


def test_packed_weights_config_and_sizes():
    # accepted where both Linears take the large-tile path
    for kw in (dict(), dict(ffn_hidden=1024, activation=B.MOE_ACT_GELU), dict(hidden_size=128, ffn_hidden=192,
                                                                             activation=B.MOE_ACT_RELU)):
        assert B.moe_workspace_size(_cfg(packed_weights=True, **kw)) == B.moe_workspace_size(_cfg(**kw))
    cfg = _cfg(packed_weights=True)
    cfg.packed_weights = 2
    with pytest.raises(B.MoeError) as ei:
        B.moe_workspace_size(cfg)
    assert ei.value.status == B.MOE_ERR_INVALID_ARG
    # E * ceil(N / 256) * 256 * K * 2 bytes
    assert B.moe_packed_weight_bytes(64, 5120, 2048) == 64 * 5120 * 2048 * 2
    assert B.moe_packed_weight_bytes(3, 80, 128) == 3 * 256 * 128 * 2
    assert B.moe_packed_weight_bytes(1, 272, 64) == 512 * 64 * 2
    for args, st in (((0, 256, 64), B.MOE_ERR_INVALID_ARG), ((257, 256, 64), B.MOE_ERR_INVALID_ARG),
                     ((1, 0, 64), B.MOE_ERR_INVALID_ARG), ((1, 256, -64), B.MOE_ERR_INVALID_ARG),
                     ((1, 256, 96), B.MOE_ERR_UNSUPPORTED), ((1, 24, 64), B.MOE_ERR_UNSUPPORTED)):
        with pytest.raises(B.MoeError) as ei:
            B.moe_packed_weight_bytes(*args)
        assert ei.value.status == st, args
    with pytest.raises(B.MoeError) as ei:
        B.moe_packed_weight_bytes(1, 256, 64, B.MOE_F32)
    assert ei.value.status == B.MOE_ERR_UNSUPPORTED


def test_pack_expert_weight_validates_before_launch():
    L = B.lib()
    n = 2 * 256 * 128 * 2   # E = 2, N = 256, K = 128
    # missing pointers, misalignment, overlap of input and output
    assert L.moe_pack_expert_weight(2, 256, 128, B.MOE_BF16, None, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_pack_expert_weight(2, 256, 128, B.MOE_BF16, FAKE, None, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_pack_expert_weight(2, 256, 128, B.MOE_BF16, FAKE + 8, FAKE + 2 * n, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_pack_expert_weight(2, 256, 128, B.MOE_BF16, FAKE, FAKE + n - 16, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_pack_expert_weight(2, 256, 128, B.MOE_BF16, FAKE + n - 16, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_pack_expert_weight(2, 256, 96, B.MOE_BF16, FAKE, FAKE + 2 * n, None) == B.MOE_ERR_UNSUPPORTED
    assert L.moe_pack_expert_weight(2, 256, 128, B.MOE_F32, FAKE, FAKE + 2 * n, None) == B.MOE_ERR_UNSUPPORTED


def test_backward_refuses_packed_weights():
    L = B.lib()
    tr = _cfg(hidden_size=256, ffn_hidden=512, activation=B.MOE_ACT_GELU, save_preact=True, packed_weights=True)
    c = ctypes.byref(tr)
    assert L.moe_expert_ffn_backward(c, *([FAKE] * 12), FAKE, 1 << 40, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_layer_backward(c, *([FAKE] * 18), FAKE, 1 << 40, None) == B.MOE_ERR_INVALID_ARG
    res = _cfg(hidden_size=256, ffn_hidden=512, activation=B.MOE_ACT_GELU, save_preact=True, packed_weights=True,
               use_residual=True)
    assert L.moe_residual_layer_backward(ctypes.byref(res), *([FAKE] * 27), FAKE, 1 << 40, None) \
        == B.MOE_ERR_INVALID_ARG


def test_residual_entry_points_validate_before_launch():
    L = B.lib()
    res = _cfg(hidden_size=256, ffn_hidden=512, activation=B.MOE_ACT_GELU, use_residual=True, save_preact=True)
    plain = _cfg(hidden_size=256, ffn_hidden=512, activation=B.MOE_ACT_GELU, save_preact=True)
    r, p = ctypes.byref(res), ctypes.byref(plain)
    ws = B.moe_workspace_size(res)
    # the residual layer's dense branch and coefficients take workspace
    assert ws > B.moe_workspace_size(plain)
    fwd = [FAKE] * 22
    assert L.moe_residual_layer_forward(p, *fwd, FAKE, 1 << 40, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_residual_layer_forward(r, *fwd, FAKE, ws - 1, None) == B.MOE_ERR_WORKSPACE
    no_mlp = list(fwd)
    no_mlp[8] = None   # mlp_w1
    assert L.moe_residual_layer_forward(r, *no_mlp, FAKE, ws, None) == B.MOE_ERR_INVALID_ARG
    bias_only = list(fwd)
    bias_only[12] = None   # coef_w NULL with coef_b given
    assert L.moe_residual_layer_forward(r, *bias_only, FAKE, ws, None) == B.MOE_ERR_INVALID_ARG
    # the plain entry points refuse a residual configuration
    assert L.moe_layer_forward(r, *([FAKE] * 15), FAKE, 1 << 40, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_layer_backward(r, *([FAKE] * 18), FAKE, 1 << 40, None) == B.MOE_ERR_INVALID_ARG
    bwd = [FAKE] * 27
    assert L.moe_residual_layer_backward(p, *bwd, FAKE, 1 << 40, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_residual_layer_backward(r, *bwd, FAKE, ws - 1, None) == B.MOE_ERR_WORKSPACE
    no_coef = list(bwd)
    no_coef[6] = None   # coef_w NULL with dcoef_w given
    assert L.moe_residual_layer_backward(r, *no_coef, FAKE, ws, None) == B.MOE_ERR_INVALID_ARG
    inf = _cfg(hidden_size=256, ffn_hidden=512, activation=B.MOE_ACT_GELU, use_residual=True)
    assert L.moe_residual_layer_backward(ctypes.byref(inf), *bwd, FAKE, 1 << 40, None) == B.MOE_ERR_INVALID_ARG


def test_workspace_views_are_inside_workspace():
    cfg = _cfg(ffn_hidden=1024, activation=B.MOE_ACT_GELU, save_preact=True)
    n = B.moe_workspace_size(cfg)
    base = 1 << 20
    xd, a, h, y, off = B.moe_workspace_views(cfg, base)
    rows = B.moe_max_rows(cfg)
    for p, size in ((xd, rows * 512 * 2), (a, rows * 1024 * 2), (h, rows * 1024 * 2), (y, rows * 512 * 2),
                    (off, 9 * 4)):
        assert base <= p and p + size <= base + n
        assert p % 256 == 0
    spans = sorted([(xd, rows * 512 * 2), (a, rows * 1024 * 2), (h, rows * 1024 * 2), (y, rows * 512 * 2)])
    for (p0, s0), (p1, _) in zip(spans, spans[1:]):
        assert p0 + s0 <= p1
    cfg.save_preact = 0
    assert B.moe_workspace_views(cfg, base)[1] is None


def test_workspace_h_ld():
    """The forward pads h_disp's rows to an odd number of 128-byte lines only
    without save_preact and only on the bf16 large-tile path; the padded rows
    fit in the h_disp region, before the next one."""
    gelu = dict(ffn_hidden=1024, activation=B.MOE_ACT_GELU)
    assert B.moe_workspace_h_ld(_cfg(**gelu)) == 1088                       # 16 lines -> 17
    assert B.moe_workspace_h_ld(_cfg(save_preact=True, **gelu)) == 1024
    assert B.moe_workspace_h_ld(_cfg(ffn_hidden=1088, activation=B.MOE_ACT_GELU)) == 1088   # 17 lines already
    assert B.moe_workspace_h_ld(_cfg(dtype=B.MOE_F32, **gelu)) == 1024
    assert B.moe_workspace_h_ld(_cfg(hidden_size=96, **gelu)) == 1024          # d not a multiple of 64
    assert B.moe_workspace_h_ld(_cfg()) == 0
    cfg = _cfg(**gelu)
    n = B.moe_workspace_size(cfg)
    base = 1 << 20
    xd, _, h, y, _ = B.moe_workspace_views(cfg, base)
    rows = B.moe_max_rows(cfg)
    spans = sorted([(xd, rows * 512 * 2), (h, rows * 1088 * 2), (y, rows * 512 * 2)])
    for (p0, s0), (p1, _) in zip(spans, spans[1:]):
        assert p0 + s0 <= p1
    assert spans[-1][0] + spans[-1][1] <= base + n
    L = B.lib()
    assert L.moe_workspace_h_ld(ctypes.byref(cfg), None) == B.MOE_ERR_INVALID_ARG


def test_workspace_status_word():
    """The small-batch status word lies inside the workspace (4-byte aligned)
    for batches the one-launch path takes, and there is none past them."""
    for T in (1, 64, 256):
        cfg = _cfg(num_tokens=T, ffn_hidden=1024, activation=B.MOE_ACT_GELU)
        n = B.moe_workspace_size(cfg)
        base = 1 << 20
        p = B.moe_workspace_status(cfg, base)
        assert base <= p and p + 4 <= base + n and p % 4 == 0
    assert B.moe_workspace_status(_cfg(num_tokens=257), 1 << 20) is None
    L = B.lib()
    cfg = _cfg(num_tokens=8)
    assert L.moe_workspace_status(ctypes.byref(cfg), None, None) == B.MOE_ERR_INVALID_ARG


def test_gate_noalloc_rejects_what_its_scratch_cannot_hold():
    """The no-allocation gate refuses, before any device call, a config whose
    gate scratch exceeds its fixed array (the pointers are never read)."""
    L = B.lib()
    big = _cfg(num_tokens=1 << 20, num_experts=256)
    dummy = [ctypes.c_void_p(4096)] * 11
    assert L.moe_gate_noalloc(ctypes.byref(big), *dummy, None) == B.MOE_ERR_WORKSPACE
    assert L.moe_gate_noalloc(ctypes.byref(_cfg()), None, None, None, None, None, None, None, None, None, None,
                              None, None) == B.MOE_ERR_INVALID_ARG


def test_status_strings():
    for s in range(5):
        assert B.status_string(s).startswith("MOE_")


def test_build_scratch_guard_reads_resource_remarks():
    """The build refuses a decode kernel that spills: its grid barriers need
    every workgroup resident, which scratch allocation can prevent."""
    from mixture_experts_layer_39_amd import build
    remarks = ("x.hip:1:1: remark: Function Name: _ZN3moe12_GLOBAL__N_113decode_kernelENS_10DecodeArgsE [-Rpass]\n"
               "x.hip:1:1: remark:     VGPRs: 172 [-Rpass]\n"
               "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 240 [-Rpass]\n"
               "x.hip:9:1: remark: Function Name: _ZN3moe12_GLOBAL__N_118decode_init_kernelEPj [-Rpass]\n"
               "x.hip:9:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass]\n")
    sizes = build._scratch_sizes(remarks)
    assert sizes == {"_ZN3moe12_GLOBAL__N_113decode_kernelENS_10DecodeArgsE": 240,
                     "_ZN3moe12_GLOBAL__N_118decode_init_kernelEPj": 0}
    assert build.NO_SCRATCH["decode.hip"] == ("decode_kernel",)

"""The no-allocation gate (moe_gate_noalloc: the gate's scratch in a
library-owned device array instead of a caller workspace) against moe_gate,
through the C ABI.  Three calls in a row on one GPU, each smaller than the
one before and with other expert counts, so a call that read the previous
call's scratch contents instead of its own would show: every output
(logits, chosen experts, slots, weights, counts, offsets, loss) must equal
moe_gate's bit for bit, and the routing must equal the oracle's on the same
logits."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_39_amd import binding as B
from mixture_experts_layer_39_amd.synthetic import make_inputs, spec
from oracle import moe_oracle as O
from tests.gpu_util import alloc_gate, cfg_of, f64, i64, workspace

pytestmark = pytest.mark.gpu
DEV = "cuda"

CALLS = [  # workload, T, E, k, given logits, normalize
    ("top2_e64", 5000, 64, 2, False, False),
    ("skew_e16", 1200, 16, 2, False, True),
    ("top2_e8", 700, 256, 1, True, False),
]


def _run(fn, cfg, inp, logits_in):
    g = alloc_gate(cfg, DEV)
    args = (cfg, inp["x"], inp["w_router"], inp["b_router"], logits_in, g["logits"], g["idx"], g["slot"],
            g["weight"], g["count"], g["offset"], g["loss"])
    if fn is B.moe_gate:
        fn(*args, workspace(cfg, DEV))
    else:
        fn(*args)
    return g


def test_gate_noalloc_matches_gate_on_calls_in_a_row():
    for name, T, E, k, given, norm in CALLS:
        print(f"no-alloc gate: {name} T={T} E={E} k={k}", flush=True)
        sp = spec(name, T=T, E=E, k=k, d=512, h=0, logits_given=given)
        inp = make_inputs(sp, DEV)
        cfg = cfg_of(sp, normalize_topk=norm)
        logits_in = inp["logits"] if given else None
        want = _run(B.moe_gate, cfg, inp, logits_in)
        got = _run(B.moe_gate_noalloc, cfg, inp, logits_in)
        torch.cuda.synchronize()
        for key in ("logits", "idx", "slot", "weight", "count", "offset", "loss"):
            assert torch.equal(got[key], want[key]), (name, key)
        r = O.route(f64(got["logits"]), k, sp["cf"], sp["min_cap"], sp["drop"], normalize_topk=norm)
        np.testing.assert_array_equal(i64(got["idx"]), r["expert_idx"])
        np.testing.assert_array_equal(i64(got["slot"]), r["slot"])
        np.testing.assert_array_equal(i64(got["count"]), r["expert_count"])
        assert np.abs(f64(got["weight"]) - r["weight"]).max() <= 1e-5

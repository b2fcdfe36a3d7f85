#!/usr/bin/env python3
"""Throughput of the MoE layer forward on one MI355X.

One step is one full pass of the layer over one batch of synthetic input:
gate (router GEMM, softmax, top-k, capacity slots, counts, loss), dispatch,
expert FFN grouped GEMMs, combine -- the fused moe_layer_forward call -- plus,
for the no-drop workload, the backward of the expert FFNs (nodrop_e128) or of
the whole layer (nodrop_e128_layer: moe_layer_backward with the router, bias
and gate_loss gradients).  Inputs are seeded synthetic tensors already
resident in HBM.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload top2_e64]

Besides the headline value the line carries
  roofline:     the expert grouped GEMM (the dominant kernel) against the bf16
                dense MFMA peak, its per-launch time taken with HIP events on the
                stream the kernels run on;
  stages:       every stage's event time and its algorithmic bytes or flops;
  small_batch:  latency of the forward for 1, 16 and 64 tokens with the same
                weights, through the one-launch kernel and the multi-kernel
                path, and the fused kernel's read rate against HBM peak;
  cpu_baseline: the CPU oracle timed on this host on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# the expert GEMM's sources (the kernel, and the header holding its GELU)
GEMM_SRC = tuple(os.path.join(ROOT, "mixture_experts_layer_39_amd", "csrc", f)
                 for f in ("grouped_gemm.hip", "moe_internal.h"))
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


def describe(sp):
    ffn = f"{sp['d']}->{sp['h']}->{sp['d']} " + {0: "none", 1: "ReLU", 2: "GELU"}[sp["act"]] if sp["h"] else \
        f"Linear {sp['d']}->{sp['d']}"
    drop = f"cf {sp['cf']} min_cap {sp['min_cap']}" if sp["drop"] else "no drop"
    return f"{sp['name']}: T={sp['T']} d={sp['d']} E={sp['E']} top-{sp['k']} FFN {ffn}, {drop}, {sp['dtype']}"


def source_hash(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(workload):
    """HBM bytes per GEMM launch from committed rocprofv3 counter runs, or
    None when none were taken for this workload or the kernel source changed
    since."""
    try:
        with open(TRAFFIC_JSON) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get(workload)
    if not rec or rec.get("source_sha256") != source_hash(GEMM_SRC):
        return None
    return rec.get("bytes_per_launch")


def bwd_label(sp):
    b = sp.get("backward")
    if sp.get("random_gate"):
        return ", seeded random gate (router input jitter, sampled second expert)"
    if sp.get("residual"):
        return ", residual MoE (dense MLP mixed by softmax coefficients)"
    return "" if not b else (", layer backward" if b == "layer" else ", expert FFN backward")


def cpu_baseline(sp, inp, target_s=15.0):
    """The oracle (as it stands) on the first Ts tokens of the same workload:
    router logits, routing, dispatch, float64 expert FFNs, combine."""
    import numpy as np
    from oracle import moe_oracle as O

    def f(t):
        return None if t is None else t.float().cpu().numpy()

    x = f(inp["x"])
    wr = f(inp["w_router"])
    br = f(inp["b_router"])
    lg_given = f(inp["logits"])
    w1, b1, w2, b2 = f(inp["w1"]), f(inp["b1"]), f(inp["w2"]), f(inp["b2"])
    dy = f(inp.get("dy"))

    def run(ts):
        t0 = time.perf_counter()
        logits = lg_given[:ts] if lg_given is not None else O.router_logits(x[:ts], wr, br)
        if sp.get("random_gate"):
            from oracle import stochastic_gate as S
            xj = S.jittered_input(x[:ts], 12345, rows=np.arange(ts))
            rr = S.route(O.router_logits(xj, wr, br), sp["k"], sp["cf"], sp["min_cap"], sp["drop"], seed=12345,
                         second_sampling=True)
            xd = O.dispatch(x[:ts], rr["expert_idx"], rr["slot"], rr["expert_offset"])
            _, _, y = O.expert_ffn(xd, rr["expert_offset"], w1, b1, w2, b2, sp["act"], sp["dtype"])
            O.combine(y, rr["expert_idx"], rr["slot"], rr["weight"], rr["expert_offset"], ts, sp["dtype"])
            return time.perf_counter() - t0
        if sp.get("residual"):
            from oracle import residual_moe as R
            mlp = (f(inp["mlp_w1"]), f(inp["mlp_b1"]), f(inp["mlp_w2"]), f(inp["mlp_b2"]))
            r = R.forward(x[:ts], logits, w1, b1, w2, b2, mlp, f(inp["coef_w"]), f(inp["coef_b"]), k=sp["k"],
                          capacity_factor=sp["cf"], min_capacity=sp["min_cap"], drop_tokens=sp["drop"],
                          act=sp["act"], dtype=sp["dtype"])
            return time.perf_counter() - t0
        r = O.layer_forward(x[:ts], logits, w1, b1, w2, b2, k=sp["k"], capacity_factor=sp["cf"],
                            min_capacity=sp["min_cap"], drop_tokens=sp["drop"], act=sp["act"], dtype=sp["dtype"])
        if sp.get("backward") == "layer":
            O.layer_backward(x[:ts], wr, r, w1, w2, dy[:ts], 1.0, act=sp["act"], dtype=sp["dtype"])
        elif sp.get("backward"):
            n = int(r["expert_offset"][-1])
            O.expert_ffn_backward(r["x_disp"], r["expert_offset"], w1, w2, r["a"], r["h"], dy[:n], sp["act"],
                                  sp["dtype"])
        return time.perf_counter() - t0

    # grow the sample until it takes a good part of the target time (a small
    # sample's time is mostly per-expert overhead, so one extrapolation from
    # it undershoots)
    ts = min(sp["T"], 64)
    el = run(ts)
    for _ in range(4):
        if el >= target_s / 2 or ts >= sp["T"]:
            break
        ts = int(min(sp["T"], max(2 * ts, ts * target_s / max(el, 1e-3))))
        el = run(ts)
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    return {"value": ts / el, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {ts} of {sp['T']} tokens of {sp['name']} (capacity recomputed for {ts} tokens): "
                      f"router, routing, dispatch, float64 expert FFNs, combine"
                      f"{bwd_label(sp)}; {el:.1f} s"}


def small_batch_latency(B, torch, sp, inp, dt, stream, sizes=(1, 16, 64), iters=50, packed=None):
    """Latency of moe_layer_forward for a few tokens with the workload's
    weights, through the one-launch small-batch kernel and through the
    multi-kernel path, with the bytes the fused kernel must read (the chosen
    experts' weights and biases, x, the router weight, out).

    Two timings per size:
      *_us       the same T rows of x on every call (the chosen experts'
                 weights then stay in the 256 MB Infinity Cache: a cached
                 figure, not an HBM one);
      *_cold_us  each call takes the next T rows of x, so consecutive calls
                 route to other experts and read weights the cache does not
                 hold (a call's two experts at one token are 84 MB at the
                 headline shape; the last three calls' fill the cache).
    The HBM fraction is taken from the cold time, with the mean bytes of the
    calls (each call's own experts).  packed: (w1, w2) in the packed layout,
    which the calls then read (as the timed forward does)."""
    dev = inp["x"].device
    T0, d, E, k, h = sp["T"], sp["d"], sp["E"], sp["k"], sp["h"]
    esz = 2 if dt == B.MOE_BF16 else 4
    per_expert = (2 * h * d + h + d) * esz if h else (d * d + d) * esz
    res = {}
    for T in sizes:
        if T * iters > T0:
            continue
        row = {}
        touched_sum = 0
        for mode, name in ((1, "fused"), (-1, "multi_kernel")):
            cfg = B.make_config(T, d, E, k, sp["cf"], sp["min_cap"], sp["drop"], h, sp["act"], dt, small_batch=mode,
                                packed_weights=packed is not None)
            w1, w2 = packed if packed is not None else (inp["w1"], inp["w2"])
            ws = torch.empty(B.moe_workspace_size(cfg), dtype=torch.uint8, device=dev)
            out = torch.empty(T, d, dtype=inp["x"].dtype, device=dev)
            loss = torch.empty(1, dtype=torch.float32, device=dev)
            counts = torch.empty(iters, E, dtype=torch.int32, device=dev)

            def call(i, c):
                x = inp["x"][i * T:(i + 1) * T]
                B.moe_layer_forward(cfg, x, inp["w_router"], inp["b_router"], None, w1, inp["b1"], w2,
                                    inp["b2"], out, loss, c, ws=ws, stream=stream)
            for cold in (False, True):
                for i in range(5):
                    call(i if cold else 0, counts[0])
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for i in range(iters):
                    call(i if cold else 0, counts[i])
                e1.record(stream)
                torch.cuda.synchronize()
                row[name + ("_cold_us" if cold else "_us")] = e0.elapsed_time(e1) / iters * 1e3
                if cold and mode == 1:
                    touched_sum = int((counts > 0).sum())
        touched = touched_sum / iters
        nbytes = touched * per_expert + 2 * T * d * esz + E * d * esz
        gbs = nbytes / (row["fused_cold_us"] * 1e-6) / 1e9
        row.update({"experts_touched_mean": touched, "bytes": nbytes, "GB/s_cold": gbs, "frac_hbm_cold": gbs / PEAK_HBM_GBS})
        res[str(T)] = row
    return {"kernel": "decode_kernel (one launch, one workgroup per CU)", "bound": "hbm",
            "tokens": res}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="top2_e64")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-small-batch", action="store_true", help="skip the small-batch latency object")
    ap.add_argument("--small-batch-only", action="store_true",
                    help="only time the small-batch forward (1, 16, 64 tokens) and print that object")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (scales HBM byte counters)")
    a = ap.parse_args(argv)
    if a.copy_calibration:
        import torch
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read_per_launch": src.numel() * 4, "copy_bytes_written_per_launch": src.numel() * 4}))
        return 0
    if a.gpus != 1:
        print(f"bench.py measures one GPU's share of the layer; --gpus {a.gpus} is not supported "
              f"(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch

    from mixture_experts_layer_39_amd import binding as B
    from mixture_experts_layer_39_amd.synthetic import make_inputs, spec

    dev = torch.device("cuda:0")
    sp = spec(a.workload)
    inp = make_inputs(sp, dev)
    T, d, E, k, h = sp["T"], sp["d"], sp["E"], sp["k"], sp["h"]
    dt = B.MOE_BF16 if sp["dtype"] == "bf16" else B.MOE_F32
    esz = 2 if dt == B.MOE_BF16 else 4
    rnd = dict(noisy_gate_policy=B.MOE_NOISE_JITTER, second_expert_sampling=True, seed=12345) \
        if sp.get("random_gate") else {}
    # Inference workloads keep the expert weights packed (moe_pack_expert_weight, once, before timing, as a
    # server does after loading them); training workloads (backward, random gate) read the nn.Linear layout.
    packable = (not sp.get("backward") and not sp.get("random_gate") and dt == B.MOE_BF16)
    if packable:
        try:
            B.moe_workspace_size(B.make_config(T, d, E, k, sp["cf"], sp["min_cap"], sp["drop"], h, sp["act"], dt,
                                               use_residual=bool(sp.get("residual")), packed_weights=True))
        except B.MoeError:
            packable = False
    cfg_lin = B.make_config(T, d, E, k, sp["cf"], sp["min_cap"], sp["drop"], h, sp["act"], dt,
                            save_preact=bool(sp.get("backward")), use_residual=bool(sp.get("residual")), **rnd)
    cfg = B.make_config(T, d, E, k, sp["cf"], sp["min_cap"], sp["drop"], h, sp["act"], dt,
                        save_preact=bool(sp.get("backward")), use_residual=bool(sp.get("residual")),
                        packed_weights=packable, **rnd)
    if packable:
        wp = (B.pack_expert_weight(inp["w1"]), B.pack_expert_weight(inp["w2"]) if h else None)
    else:
        wp = (inp["w1"], inp["w2"])
    ws = torch.empty(B.moe_workspace_size(cfg), dtype=torch.uint8, device=dev)
    out = torch.empty_like(inp["x"])
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    count = torch.empty(E, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    if a.small_batch_only:
        print(json.dumps(small_batch_latency(B, torch, sp, inp, dt, stream, packed=wp if packable else None)),
              flush=True)
        return 0

    bwd = bool(sp.get("backward"))
    layer = sp.get("backward") == "layer"
    if bwd:
        rows = B.moe_max_rows(cfg)
        xd_p, a_p, h_p, _, off_p = B.moe_workspace_views(cfg, ws)
        dx = torch.empty(T if layer else rows, d, dtype=torch.bfloat16, device=dev)
        dw1 = torch.empty_like(inp["w1"])
        dw2 = torch.empty_like(inp["w2"])
    if layer:
        f32 = dict(dtype=torch.float32, device=dev)
        db1 = torch.empty(E, h, **f32)
        db2 = torch.empty(E, d, **f32)
        dwr = torch.empty(E, d, **f32)
        dbr = torch.empty(E, **f32)
        dlg = torch.empty(T, E, **f32)
        dwg = torch.empty(T, k, **f32)
        dloss = torch.ones(1, **f32)

    def backward():
        if layer:
            B.moe_layer_backward(cfg, inp["x"], inp["w_router"], inp["w1"], inp["w2"], inp["dy"], dloss, dx, dw1, dw2,
                                 dlogits=dlg, dw_router=dwr, db_router=dbr, db1=db1, db2=db2, ws=ws, stream=stream)
        else:
            B.moe_expert_ffn_backward(cfg, xd_p, off_p, inp["w1"], inp["w2"], a_p, h_p, inp["dy"], dx, dw1, None,
                                      dw2, None, ws, stream=stream)

    res = bool(sp.get("residual"))

    def step(c=cfg, w=wp):
        if res:
            B.moe_residual_layer_forward(c, inp["x"], inp["w_router"], inp["b_router"], inp["logits"], w[0],
                                         inp["b1"], w[1], inp["b2"], inp["mlp_w1"], inp["mlp_b1"],
                                         inp["mlp_w2"], inp["mlp_b2"], inp["coef_w"], inp["coef_b"], out, loss,
                                         count, ws=ws, stream=stream)
        else:
            B.moe_layer_forward(c, inp["x"], inp["w_router"], inp["b_router"], inp["logits"], w[0],
                                inp["b1"], w[1], inp["b2"], out, loss, count, ws=ws, stream=stream)
        if bwd:
            backward()

    def timed(*args):
        for _ in range(a.warmup):
            step(*args)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(a.steps):
            step(*args)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    el = timed()
    ms_step = el / a.steps * 1e3
    value = T * a.steps / el
    # the same forward on the nn.Linear weight layout (context for the packed figure)
    el_lin = timed(cfg_lin, (inp["w1"], inp["w2"])) if packable else el

    # ---- per-stage breakdown: the same kernels called stage by stage, HIP
    # events recorded on the stream they run on
    rows = max(B.moe_max_rows(cfg), 1)
    g = dict(idx=torch.empty(T, k, dtype=torch.int32, device=dev), slot=torch.empty(T, k, dtype=torch.int32, device=dev),
             weight=torch.empty(T, k, dtype=torch.float32, device=dev),
             offset=torch.empty(E + 1, dtype=torch.int32, device=dev))
    xd, a_p, hd_p, yd_p, _ = B.moe_workspace_views(cfg, ws)
    h_ld = B.moe_workspace_h_ld(cfg)   # the pitch the fused forward keeps h_disp at
    nst = 9 if layer else 5
    if res:
        # the dense branch on its own: the expert FFN entry point with one
        # expert holding all T rows
        cfg1 = B.make_config(T, d, 1, 1, 1.0, 0, False, h, sp["act"], dt)
        off1 = torch.tensor([0, T], dtype=torch.int32, device=dev)
        h1 = torch.empty(T, h, dtype=inp["x"].dtype, device=dev)
        y1 = torch.empty(T, d, dtype=inp["x"].dtype, device=dev)
        ws1 = torch.empty(max(B.moe_workspace_size(cfg1), 1), dtype=torch.uint8, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)]
    acc = [0.0] * nst
    lg_out = torch.empty(T, E, dtype=torch.float32, device=dev) if layer else None
    for it in range(a.warmup + a.steps):
        ev[0].record(stream)
        B.moe_gate(cfg, inp["x"], inp["w_router"], inp["b_router"], inp["logits"], lg_out, g["idx"], g["slot"],
                   g["weight"], count, g["offset"], loss, ws, stream=stream)
        ev[1].record(stream)
        B.moe_dispatch(cfg, inp["x"], g["idx"], g["slot"], g["offset"], xd, stream=stream)
        ev[2].record(stream)
        B.moe_expert_ffn(cfg, xd, g["offset"], wp[0], inp["b1"], wp[1], inp["b2"], a_p if bwd else None,
                         hd_p, yd_p, ws, stream=stream, h_ld=h_ld)
        ev[3].record(stream)
        B.moe_combine(cfg, yd_p, g["idx"], g["slot"], g["weight"], g["offset"], out, stream=stream)
        ev[4].record(stream)
        if layer:
            # the backward as its separate calls: combine, expert FFNs, gate,
            # dispatch + router input, router weights
            B.moe_combine_backward(cfg, inp["dy"], yd_p, g["idx"], g["slot"], g["weight"], g["offset"], yd_p, dwg,
                                   stream=stream)
            ev[5].record(stream)
            B.moe_expert_ffn_backward(cfg, xd, g["offset"], inp["w1"], inp["w2"], a_p, hd_p, yd_p, yd_p, dw1, db1,
                                      dw2, db2, ws, stream=stream)
            ev[6].record(stream)
            B.moe_gate_backward(cfg, lg_out, g["idx"], dwg, dloss, dlg, ws, stream=stream)
            ev[7].record(stream)
            B.moe_dispatch_backward(cfg, yd_p, g["idx"], g["slot"], g["offset"], inp["w_router"], dlg, dx, ws,
                                    stream=stream)
            ev[8].record(stream)
            B.moe_router_backward(cfg, inp["x"], dlg, dwr, dbr, ws, stream=stream)
        elif bwd:
            B.moe_expert_ffn_backward(cfg, xd, g["offset"], inp["w1"], inp["w2"], a_p, hd_p, inp["dy"], dx, dw1,
                                      None, dw2, None, ws, stream=stream)
        elif res:
            B.moe_expert_ffn(cfg1, inp["x"], off1, inp["mlp_w1"], inp["mlp_b1"], inp["mlp_w2"], inp["mlp_b2"], None,
                             h1, y1, ws1, stream=stream)
        ev[nst].record(stream)
        if it >= a.warmup:
            torch.cuda.synchronize()
            for i in range(nst):
                acc[i] += ev[i].elapsed_time(ev[i + 1])
    st_ms = [v / a.steps for v in acc]

    # ---- algorithmic work from the realised routing
    counts = count.cpu().long()
    slots = g["slot"].cpu().long()
    N = int(counts.sum())
    tok_kept = int((slots >= 0).any(dim=1).sum())
    gate_bytes = T * d * esz + E * d * esz + T * k * 12 + (T * E * 4 if inp["logits"] is not None else 0)
    disp_bytes = tok_kept * d * esz + N * d * esz + T * k * 8
    comb_bytes = N * d * esz + T * d * esz + T * k * 12
    ffn_flops = 4 * N * d * h if h else 2 * N * d * d
    n_gemm = 2 if h else 1

    def gbs(b, ms):
        return b / (ms * 1e-3) / 1e9

    stages = {
        "gate": {"ms": st_ms[0], "bytes": gate_bytes, "GB/s": gbs(gate_bytes, st_ms[0]),
                 "frac_hbm": gbs(gate_bytes, st_ms[0]) / PEAK_HBM_GBS},
        "dispatch": {"ms": st_ms[1], "bytes": disp_bytes, "GB/s": gbs(disp_bytes, st_ms[1]),
                     "frac_hbm": gbs(disp_bytes, st_ms[1]) / PEAK_HBM_GBS},
        "expert_ffn": {"ms": st_ms[2], "flops": ffn_flops, "TFLOP/s": ffn_flops / (st_ms[2] * 1e-3) / 1e12,
                       "frac_mfma": ffn_flops / (st_ms[2] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "launches": n_gemm},
        "combine": {"ms": st_ms[3], "bytes": comb_bytes, "GB/s": gbs(comb_bytes, st_ms[3]),
                    "frac_hbm": gbs(comb_bytes, st_ms[3]) / PEAK_HBM_GBS},
    }
    if res:
        dflops = 4 * T * d * h
        stages["dense_mlp"] = {"ms": st_ms[4], "flops": dflops, "TFLOP/s": dflops / (st_ms[4] * 1e-3) / 1e12,
                               "frac_mfma": dflops / (st_ms[4] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "launches": 2}
        stages["note"] = ("combine + mix is fused in the step (it reads x, the kept y rows and the dense output); "
                          "the combine stage above is the plain combine")
    bflops = 2 * ffn_flops   # dgrad (dH, dX) + wgrad (dW2, dW1): 4 GEMMs of 2*N*d*h
    if bwd and not layer:
        stages["expert_ffn_backward"] = {"ms": st_ms[4], "flops": bflops,
                                         "TFLOP/s": bflops / (st_ms[4] * 1e-3) / 1e12,
                                         "frac_mfma": bflops / (st_ms[4] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                         "launches": 4}
    if layer:
        ep = (E + 31) // 32 * 32
        cb_bytes = T * d * esz + 2 * N * d * esz + T * k * 16
        gb_bytes = 2 * T * E * 4 + T * k * 8
        ib_bytes = N * d * esz + T * d * esz + T * E * 4 + T * 2 * ep * 2 + T * k * 8
        rb_flops = 2 * T * E * d
        stages["combine_backward"] = {"ms": st_ms[4], "bytes": cb_bytes, "GB/s": gbs(cb_bytes, st_ms[4]),
                                      "frac_hbm": gbs(cb_bytes, st_ms[4]) / PEAK_HBM_GBS}
        stages["expert_ffn_backward"] = {"ms": st_ms[5], "flops": bflops,
                                         "TFLOP/s": bflops / (st_ms[5] * 1e-3) / 1e12,
                                         "frac_mfma": bflops / (st_ms[5] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                         "launches": 4, "with": "db1, db2"}
        stages["gate_backward"] = {"ms": st_ms[6], "bytes": gb_bytes, "GB/s": gbs(gb_bytes, st_ms[6]),
                                   "frac_hbm": gbs(gb_bytes, st_ms[6]) / PEAK_HBM_GBS}
        stages["dispatch_router_input_backward"] = {"ms": st_ms[7], "bytes": ib_bytes, "GB/s": gbs(ib_bytes, st_ms[7]),
                                                    "frac_hbm": gbs(ib_bytes, st_ms[7]) / PEAK_HBM_GBS}
        stages["router_weight_backward"] = {"ms": st_ms[8], "flops": rb_flops,
                                            "TFLOP/s": rb_flops / (st_ms[8] * 1e-3) / 1e12,
                                            "bytes": T * d * esz + T * E * 4,
                                            "GB/s": gbs(T * d * esz + T * E * 4, st_ms[8])}
    gemm_ms = st_ms[2] / n_gemm
    achieved = (ffn_flops / n_gemm) / (gemm_ms * 1e-3) / 1e12
    # the expert GEMM: one kernel template launched once per Linear (the GELU
    # and the plain instantiation for a two-Linear expert), equal FLOPs each
    roofline = {"bound": "mfma", "kernel": "gemm_bf16_big_kernel (expert FFN GEMM, per launch)" if dt == B.MOE_BF16
                else "gemm_f32_kernel",
                "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": load_traffic(a.workload),
                "flops_per_launch": ffn_flops / n_gemm, "avg_launch_ms": gemm_ms, "rows": N}

    line = {"metric": "MoE-layer fwd tokens/s (E=64,top-2,d=2048); MFMA util + HBM GB/s vs peak",
            "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
            "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": sp["dtype"], "data": "synthetic",
            "config": {"workload": describe(sp) + bwd_label(sp).replace(",", " +"),
                       "tokens_per_step": T, "rows_kept": N,
                       "expert_weights": ("packed (moe_pack_expert_weight, once before timing)" if packable
                                          else "nn.Linear [E, out, in]")},
            "roofline": roofline, "stages": stages}
    if packable:
        line["nn_linear_weights"] = {"value": T * a.steps / el_lin, "ms_per_step": el_lin / a.steps * 1e3}
    if not a.no_small_batch and not bwd and not res and not sp.get("random_gate") and sp["h"] and dt == B.MOE_BF16:
        line["small_batch"] = small_batch_latency(B, torch, sp, inp, dt, stream, packed=wp if packable else None)
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(sp, inp)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

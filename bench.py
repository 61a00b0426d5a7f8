"""Benchmark of the MoE layer hot path on one MI355X.

One step = route -> dispatch -> grouped SwiGLU FFN -> combine over one batch
of synthetic tokens, all four through the C ABI (libmoe_route.so), inputs
already resident in HBM.  Prints one JSON line:

  value            whole-layer tokens/s (N tokens per step / time per step)
  roofline         the grouped FFN call (the dominant stage: its tile-schedule,
                   gate/up and down kernels) against bf16 MFMA peak:
                   6*M*d*ffn flops per call / its event-timed duration.
                   bf16 layers stream expert weights packed in MFMA operand
                   order (moe_pack_ffn_weights, run once at setup like a
                   weight load, outside the timed steps); --plain-weights
                   times the row-major-weight kernel instead
  stages           per-stage times of the timed steps; dispatch and combine
                   also timed alone with a cold cache (HBM GB/s vs peak)
  cpu_baseline     the CPU oracle on a bounded sample of the same workload

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16
FP32_PEAK_TFLOPS = 157.3

DEFAULT_WORKLOAD = "dense8"
SCRUB_MIB = 512                  # > the 256 MB last-level (MALL) cache
CSRC = os.path.join(ROOT, "grouped_gemm_route_amd", "csrc")
# sources of the timed FFN kernels (their digest keys the traffic counters)
FFN_SOURCES = {
    "packed": [os.path.join(CSRC, "grouped_ffn_packed.hip"), os.path.join(CSRC, "ffn_tiles.h")],
    "plain": [os.path.join(CSRC, "grouped_ffn.hip"), os.path.join(CSRC, "ffn_tiles.h")],
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # the GEMM's clock settles over the first ~10 layer steps; 20 untimed
    # steps put the timed ones in steady state (the timed region stays well
    # under a second)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-tokens", type=int, default=4096)
    p.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"))
    p.add_argument("--cold-reps", type=int, default=10,
                   help="reps of the cold-cache dispatch/combine timing (0 skips it)")
    p.add_argument("--no-exchange", action="store_true",
                   help="skip the virtual multi-source exchange measurements")
    p.add_argument("--no-residual", action="store_true",
                   help="skip the Residual-MoE (top-1 + shared MLP) measurements")
    p.add_argument("--no-per-rank", action="store_true",
                   help="skip the per-virtual-rank FFN timing (it launches the same GEMM "
                        "kernels on one rank's rows, which would mix into a profile's averages)")
    p.add_argument("--plain-weights", action="store_true",
                   help="time the FFN on row-major weights (moe_grouped_ffn) instead of "
                        "packed ones")
    p.add_argument("--copy-ref-mib", type=int, default=0,
                   help="run one plain device-to-device copy of this many MiB first "
                        "(the reference kernel for scaling HBM byte counters)")
    return p.parse_args()


def algorithmic_bytes(cfg, M, b):
    """Dispatch and combine bytes the method must move.

    dispatch: read every token row once (N*d*b), write every kept row
    (M*d*b), plus the index traffic of the mapping table (12 bytes per
    assignment: topk_idx read, dest and perm_token written).
    combine: read every kept row (M*d*b), write every token row (N*d*b),
    plus dest and topk_w reads (8 bytes per assignment).
    """
    N, d, K = cfg["N"], cfg["d"], cfg["K"]
    disp = N * d * b + M * d * b + 12 * N * K
    comb = M * d * b + N * d * b + 8 * N * K
    return disp, comb


def ffn_flops(cfg, M):
    return 6.0 * M * cfg["d"] * cfg["ffn"]


def ffn_bytes(cfg, M, nonempty, b):
    """HBM bytes the grouped FFN must move: the three weight matrices of
    every expert that has rows (3 d ffn b each), the kept rows read
    (M d b), h written and read back (2 M ffn b) and y_perm written
    (M d b)."""
    d, ffn = cfg["d"], cfg["ffn"]
    return nonempty * 3 * d * ffn * b + 2 * M * d * b + 2 * M * ffn * b


def route_bytes(cfg, b_logit=4):
    """Routing reads every logit and writes K ids and K weights per token."""
    return cfg["N"] * cfg["E"] * b_logit + cfg["N"] * cfg["K"] * 8


def source_digest(paths):
    """sha256[:16] of C++ sources with their comments and blank space
    removed, so the digest names the code a counter run measured, not its
    prose."""
    import re

    texts = []
    for path in paths:
        with open(path, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        texts.append(" ".join(text.split()))
    return hashlib.sha256("\n".join(texts).encode()).hexdigest()[:16]


def load_traffic(path, workload, weights):
    """HBM bytes per grouped-FFN call from the counter summary, or None when
    the summary is missing, is for another workload or weight layout, or
    predates the current kernel source."""
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            tj = json.load(f)
    except (OSError, ValueError):
        return None
    if (tj.get("workload") != workload or tj.get("weights") != weights
            or tj.get("source_sha256_16") != source_digest(FFN_SOURCES[weights])):
        return None
    return tj.get("bytes_per_call")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the layer's "
              "multi-GPU exchange is not implemented here.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from grouped_gemm_route_amd import binding as B
    from grouped_gemm_route_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B.load_library()
    cfg = synth.config(args.workload)
    N, d, ffn, E, K, W = (cfg[k] for k in ("N", "d", "ffn", "E", "K", "W"))
    dtype = synth.TORCH_DTYPE[cfg["act"]]
    b = 2 if cfg["act"] == "bf16" else 4
    cap = B.moe_capacity(cfg["C"], N, K, E) if cfg["C"] is not None else -1
    stream = torch.cuda.current_stream(dev)

    if args.copy_ref_mib > 0:
        nbytes = args.copy_ref_mib << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    inp = synth.make_inputs(cfg, dev)
    layer = B.MoeLayer(N, d, ffn, E, K, W, cap, dtype, dev)
    weights = "packed" if cfg["act"] == "bf16" and not args.plain_weights else "plain"
    pack_ms = None
    if weights == "packed":   # once, as at weight-load time
        torch.cuda.synchronize()
        t_pack = time.perf_counter()
        ffn_args = (B.moe_pack_ffn_weights(inp["w_gate"], inp["w_up"], inp["w_down"]),)
        torch.cuda.synchronize()
        pack_ms = (time.perf_counter() - t_pack) * 1e3
    else:
        ffn_args = (inp["w_gate"], inp["w_up"], inp["w_down"])

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        layer.route(inp["logits"])
        if ev is not None:
            ev[1].record(stream)
        layer.dispatch(inp["x"])
        if ev is not None:
            ev[2].record(stream)
        layer.ffn(*ffn_args)
        if ev is not None:
            ev[3].record(stream)
        layer.combine()
        if ev is not None:
            ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    M = int(layer.disp["offsets"][-1].item())

    # timed region: exactly `steps` steps, synchronised on both sides
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps

    names = ["route", "dispatch", "ffn", "combine"]
    per_step = {n: [evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)]
                for j, n in enumerate(names)}
    per_step["step"] = [evs[i][0].elapsed_time(evs[i][4]) for i in range(args.steps)]
    st = {n: float(np.mean(per_step[n])) for n in names}
    disp_b, comb_b = algorithmic_bytes(cfg, M, b)
    flops = ffn_flops(cfg, M)
    achieved_tflops = flops / (st["ffn"] * 1e-3) / 1e12
    peak = MFMA_BF16_PEAK_TFLOPS if cfg["act"] == "bf16" else FP32_PEAK_TFLOPS
    # which roof binds the grouped FFN: the longer of its flops at peak and
    # its bytes at peak HBM bandwidth (weight streaming when experts get few
    # rows)
    nonempty = int((layer.disp["counts"] > 0).sum().item())
    fbytes = ffn_bytes(cfg, M, nonempty, b)
    ffn_gbps = fbytes / (st["ffn"] * 1e-3) / 1e9
    t_mfma = flops / (peak * 1e12)
    t_hbm = fbytes / (HBM_PEAK_GBPS * 1e9)
    ffn_bound = "hbm" if t_hbm > t_mfma else ("mfma" if cfg["act"] == "bf16" else "alu")
    rbytes = route_bytes(cfg)

    # Cold-cache timing of the two HBM-bound stages, outside the timed steps:
    # before each rep a 512 MiB buffer is written and then read, so neither
    # the stage's inputs nor dirty lines of its own are left in L2 or MALL.
    cold = {}
    if args.cold_reps > 0:
        scrub = torch.empty(SCRUB_MIB << 18, dtype=torch.float32, device=dev)

        def flush(i):
            scrub.fill_(float(i))
            scrub.sum()

        for name, fn in (("dispatch", lambda: layer.dispatch(inp["x"])),
                         ("combine", layer.combine)):
            times = []
            for i in range(args.cold_reps):
                flush(i)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                e1.synchronize()
                times.append(e0.elapsed_time(e1))
            cold[name] = float(np.median(times))
        del scrub
        cold_dc = (disp_b + comb_b) / ((cold["dispatch"] + cold["combine"]) * 1e-3) / 1e9
    hot_dc = (disp_b + comb_b) / ((st["dispatch"] + st["combine"]) * 1e-3) / 1e9

    # the other weight layout's FFN on the same rows, for comparison (outside
    # the timed steps, after them, 10 calls)
    other_ffn_ms = None
    if cfg["act"] == "bf16":
        other = ((inp["w_gate"], inp["w_up"], inp["w_down"]) if weights == "packed" else
                 (B.moe_pack_ffn_weights(inp["w_gate"], inp["w_up"], inp["w_down"]),))
        other_ffn_ms = _timed(stream, lambda: layer.ffn(*other), reps=10)
        del other

    stages = {
        "route_ms": st["route"],
        "dispatch_ms": st["dispatch"],
        "ffn_ms": st["ffn"],
        "combine_ms": st["combine"],
        "dispatch_bytes": disp_b,
        "combine_bytes": comb_b,
        "dispatch_combine_GBps_in_step": hot_dc,
        "ffn_TFLOPs": achieved_tflops,
        "ffn_mfma_frac": achieved_tflops / peak,
        "ffn_bytes": fbytes,
        "ffn_GBps": ffn_gbps,
        "ffn_hbm_frac": ffn_gbps / HBM_PEAK_GBPS,
        "ffn_bound": ffn_bound,
        "ffn_roof_frac": max(t_mfma, t_hbm) / (st["ffn"] * 1e-3),
        "route_bytes": rbytes,
        "route_GBps": rbytes / (st["route"] * 1e-3) / 1e9,
        "route_hbm_frac": rbytes / (st["route"] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "ffn_weights": weights,
        "weight_pack_ms": pack_ms,
        ("ffn_plain_weights_ms" if weights == "packed" else "ffn_packed_weights_ms"):
            other_ffn_ms,
        "tokens_per_s": {n: N / (st[n] * 1e-3) for n in names},
        # event-timed spread over the timed steps (the means above; `value`
        # is the host clock around all of them)
        "median_ms": {n: float(np.median(v)) for n, v in per_step.items()},
        "min_ms": {n: float(np.min(v)) for n, v in per_step.items()},
    }
    if cold:
        stages.update({
            "cold_dispatch_ms": cold["dispatch"],
            "cold_combine_ms": cold["combine"],
            "cold_dispatch_GBps": disp_b / (cold["dispatch"] * 1e-3) / 1e9,
            "cold_combine_GBps": comb_b / (cold["combine"] * 1e-3) / 1e9,
            "cold_dispatch_combine_GBps": cold_dc,
            "cold_dispatch_combine_hbm_frac": cold_dc / HBM_PEAK_GBPS,
        })

    result = {
        "metric": "MoE layer tokens/s on 1 MI355X; dispatch/combine GB/s; grouped-GEMM TFLOP/s",
        "value": N / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg["act"] == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) logits and hidden states, N(0,1/sqrt(fan_in)) "
                "weights)",
        "config": {
            "workload": f"{args.workload}: N={N} d={d} ffn={ffn} E={E} K={K} W={W} "
                        f"{cfg['act']} capacity={cap} (M={M} kept rows)",
            "global_batch": N,
            "parallelism": "single GPU; all-to-all replaced by local pack/unpack into W "
                           "virtual-rank slices",
        },
        "roofline": {
            "kernel": ("moe_grouped_ffn_packed" if weights == "packed" else "moe_grouped_ffn")
                      + " call (tile schedule + gate/up GEMM + down GEMM)",
            "bound": ffn_bound,
            "achieved": ffn_gbps if ffn_bound == "hbm" else achieved_tflops,
            "peak": HBM_PEAK_GBPS if ffn_bound == "hbm" else peak,
            "unit": "GB/s" if ffn_bound == "hbm" else "TFLOP/s",
            "frac": ffn_gbps / HBM_PEAK_GBPS if ffn_bound == "hbm" else achieved_tflops / peak,
            "traffic": load_traffic(args.traffic_json, args.workload, weights),
        },
        "stages": stages,
    }
    if cfg["act"] == "bf16":
        # the layer's performance targets, stated for the dense8 workload:
        # the grouped GEMM at >= 50% of bf16 MFMA peak and dispatch + combine
        # at >= 60% of HBM peak (cold caches; the in-step figure beside it)
        dc_frac = cold_dc / HBM_PEAK_GBPS if cold else None
        result["targets"] = {
            "workload": "dense8",
            "applies": args.workload == "dense8",
            "grouped_gemm_mfma_frac": {"value": achieved_tflops / peak, "target": 0.50,
                                       "met": achieved_tflops / peak >= 0.50},
            "dispatch_combine_hbm_frac_cold": {
                "value": dc_frac, "target": 0.60,
                "met": dc_frac is not None and dc_frac >= 0.60},
            "dispatch_combine_hbm_frac_in_step": {
                "value": hot_dc / HBM_PEAK_GBPS, "target": 0.60,
                "met": hot_dc / HBM_PEAK_GBPS >= 0.60},
        }

    result["graph"] = graph_block(layer, inp, ffn_args, N, stream, args.steps)
    result["metrics"] = routing_metrics(layer, cfg, cap, M)
    if weights == "packed" and not args.no_per_rank:
        result["metrics"]["per_rank_ffn"] = per_rank_ffn_block(B, layer, ffn_args[0], cfg,
                                                               stream)
    result["dispatch_paths"] = dispatch_paths_block(B, layer, inp, cfg, cap, stream,
                                                    args.cold_reps)
    if not args.no_exchange:
        result["exchange"] = exchange_block(B, layer, inp["x"], cfg, M, b, stream)
        result["router_projection"] = router_block(B, synth, inp["x"], cfg, b, stream)
        result["routing_variants"] = routing_variants_block(B, inp["logits"], cfg, cap, stream)
        if cfg["act"] == "bf16" and d % 128 == 0:
            result["fp8_payload"] = fp8_block(B, layer, inp["x"], cfg, M, stream,
                                              args.cold_reps)
    if not args.no_residual and cfg["act"] == "bf16":
        del layer
        packed = ffn_args[0] if weights == "packed" else None
        result["residual_moe"] = residual_block(B, synth, inp, cfg, b, stream, packed)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_sample_tokens)
    print(json.dumps(result))


XGMI_EGRESS_GBPS = 7 * 153.0   # MI355X: 7 xGMI links of about 153 GB/s each


def dispatch_paths_block(B, layer, inp, cfg, cap, stream, cold_reps):
    """Routing + dispatch both ways, timed alike: planned (moe_route_plan,
    which also ranks and counts the tokens per expert, then
    moe_dispatch_planned) and plain (moe_route_topk, then moe_dispatch with
    its own counting pass).  Warm: 20 calls (or pairs) queued behind a spin
    kernel, so that host call costs stay out, best of 3; cold: the dispatch
    alone after the same cache scrub as the stages' cold figures (median).
    step_path names the one the layer step runs (MoeLayer's default)."""
    import numpy as np
    import torch

    N, d, E, K, W = cfg["N"], cfg["d"], cfg["E"], cfg["K"], cfg["W"]
    dev = inp["x"].device
    lg, x = inp["logits"], inp["x"]

    def queued(fn, reps=20):
        fn()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(20_000_000)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            e1.synchronize()
            best = min(best, e0.elapsed_time(e1) / reps * 1e3)
        return best

    def cold(lay):
        scrub = torch.empty(SCRUB_MIB << 18, dtype=torch.float32, device=dev)
        times = []
        for i in range(max(cold_reps, 1)):
            scrub.fill_(float(i))
            scrub.sum()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            lay.dispatch(x)
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        del scrub
        return float(np.median(times)) * 1e3

    out = {"step_path": "planned" if layer.planned else "plain"}
    dests = {}
    for name, planned in (("planned", True), ("plain", False)):
        lay = B.MoeLayer(N, d, 16, E, K, W, cap, x.dtype, dev, planned=planned)
        lay.route(lg)
        lay.dispatch(x)
        out[name] = {
            "route_us": queued(lambda: lay.route(lg)),
            "dispatch_us": queued(lambda: lay.dispatch(x)),
            "route_dispatch_us": queued(lambda: (lay.route(lg), lay.dispatch(x))),
            "cold_dispatch_us": cold(lay),
        }
        dests[name] = lay.disp["dest"].clone()
        del lay
    out["same_dest"] = bool(torch.equal(dests["planned"], dests["plain"]))
    return out


def graph_block(layer, inp, ffn_args, N, stream, steps):
    """The same layer step captured once as a HIP graph (MoeLayer.capture)
    and replayed `steps` times, timed between two synchronisations like the
    eager steps: the launch costs of the four calls' kernels leave the
    step, which matters for decode-sized layers."""
    import torch

    graph = layer.capture(inp["logits"], inp["x"], *ffn_args)
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    del graph
    return {"steps": steps, "ms_per_step": ms, "tokens_per_s": N / (ms * 1e-3)}


def routing_metrics(layer, cfg, cap, M):
    """Load and drop metrics of the dispatch ("MoE 推理服务工程真相 2026",
    section 5.1: expert load per card std/mean, overflow rate, token drops),
    from the library's demand / counts outputs."""
    import numpy as np

    E, W, N, K = cfg["E"], cfg["W"], cfg["N"], cfg["K"]
    demand = layer.disp["demand"].cpu().numpy().astype(np.int64)
    counts = layer.disp["counts"].cpu().numpy().astype(np.int64)
    per_rank = counts.reshape(W, E // W).sum(axis=1)
    # capacity_factor_effective (section 5.1's dispatcher metric, "C_eff >
    # 0.8"): kept rows over the expert buffers' slots, M / (E c), c = the
    # capacity, or for a dropless layer the largest expert's rows (the
    # capacity a padded exchange would need): mean over largest load
    c = cap if cap >= 0 else int(counts.max())
    return {
        "kept_rows": M,
        "capacity_factor_effective": float(M / (E * c)) if c > 0 else 0.0,
        "dropped_pairs": int(N * K - M),
        "drop_rate": float((N * K - M) / (N * K)),
        "experts_overflowing": int((demand > cap).sum()) if cap >= 0 else 0,
        "expert_overflow_rate": float((demand > cap).mean()) if cap >= 0 else 0.0,
        "nonempty_experts": int((counts > 0).sum()),
        "max_rows_per_expert": int(counts.max()),
        "expert_rows": counts.tolist() if E <= 16 else None,
        "rank_load_std_over_mean": float(per_rank.std() / max(per_rank.mean(), 1e-9)),
        "rank_load_max_over_min": float(per_rank.max() / max(per_rank.min(), 1)),
    }


def per_rank_ffn_block(B, layer, packed, cfg, stream, reps=5):
    """Expert compute time per virtual rank ("MoE 专家并行的 All-to-All 通信瓶颈",
    section "可观测指标与故障定位": each card's expert time, to find the slowest
    card).  Rank r's experts [r E/W, (r+1) E/W) run as one grouped-FFN call
    on its own rows of the packed buffer, as they would on its own GPU; the
    EP step waits for the slowest rank."""
    import torch

    E, W = cfg["E"], cfg["W"]
    Ep = E // W
    offs = layer.disp["offsets"]
    ro = layer.disp["rank_offsets"].cpu().tolist()
    up_e = packed.up.numel() // E
    dn_e = packed.down.numel() // E
    ms = []
    for r in range(W):
        rows = ro[r + 1] - ro[r]
        if rows == 0:
            ms.append(0.0)
            continue
        sub = B.PackedFfnWeights(packed.up[r * Ep * up_e:(r + 1) * Ep * up_e],
                                 packed.down[r * Ep * dn_e:(r + 1) * Ep * dn_e], Ep,
                                 packed.d, packed.ffn)
        sub_offs = (offs[r * Ep:(r + 1) * Ep + 1] - ro[r]).contiguous()
        x_sub = layer.disp["x_perm"][ro[r]:ro[r + 1]]
        h_sub = layer.h[ro[r]:ro[r + 1]]
        y_sub = layer.y_perm[ro[r]:ro[r + 1]]
        ms.append(_timed(stream, lambda: B.moe_grouped_ffn_packed(
            x_sub, sub_offs, sub, rows, h_sub, y_sub, layer.ffn_ws), reps=reps))
    mean = sum(ms) / len(ms)
    return {"ms": ms, "slowest_rank": int(max(range(W), key=lambda i: ms[i])),
            "max_over_mean": float(max(ms) / mean) if mean > 0 else 0.0}


def exchange_block(B, layer, src_x, cfg, M, b, stream):
    """The virtual W-source exchange around the all-to-all: plan, pack,
    all-to-all (as a local gather), regroup; the W x W traffic matrix and
    Aurora's lower bound on the all-to-all time ("MoE Inference
    Communication", Theorem 4.2), in rows, bytes and at MI355X xGMI egress.
    Timed alone on warm buffers, outside the timed steps."""
    import numpy as np
    import torch

    E, W, d = cfg["E"], cfg["W"], cfg["d"]
    x = layer.disp["x_perm"]
    dev = x.device
    plan = B.moe_exchange_plan(layer.topk_idx, layer.disp, E, W)
    n_rows = layer.disp["offsets"][E:E + 1]
    send = torch.empty_like(x)
    recv = torch.empty_like(x)
    regrouped = torch.empty_like(x)

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / reps

    t_plan = timed(lambda: B.moe_exchange_plan(layer.topk_idx, layer.disp, E, W, plan))
    t_pack = timed(lambda: B.moe_rows_permute(src_x, send, plan["send_token"], n_rows))
    t_a2a = timed(lambda: B.moe_rows_permute(send, recv, plan["a2a_src"], n_rows))
    t_reg = timed(lambda: B.moe_rows_permute(recv, regrouped, plan["regroup_src"], n_rows))
    torch.cuda.synchronize()
    same = bool(torch.equal(regrouped[:M], layer.disp["x_perm"][:M]))
    D = plan["traffic"].cpu().numpy().astype(np.int64)
    off = D - np.diag(np.diag(D))
    tau_rows = int(max(off.sum(axis=1).max(), off.sum(axis=0).max()))
    row_bytes = d * b
    moved = 2.0 * M * row_bytes   # each permutation reads and writes M rows
    return {
        "plan_us": t_plan * 1e3,
        "pack_us": t_pack * 1e3,
        "a2a_local_us": t_a2a * 1e3,
        "regroup_us": t_reg * 1e3,
        "permute_GBps": moved / (t_a2a * 1e-3) / 1e9,
        "regrouped_equals_dispatch": same,
        "traffic_matrix_rows": D.tolist(),
        "cross_rank_fraction": float(off.sum() / max(D.sum(), 1)),
        "tau_min_rows": tau_rows,
        "tau_min_bytes": tau_rows * row_bytes,
        "tau_min_us_at_xgmi_egress": tau_rows * row_bytes / (XGMI_EGRESS_GBPS * 1e9) * 1e6,
    }


def _timed(stream, fn, reps=5):
    import torch

    fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


def routing_variants_block(B, logits, cfg, cap, stream):
    """Sigmoid gate and one-round re-route of capacity overflow ("MoE
    推理服务工程真相 2026", sections 2.3 and 4.3), timed alone on warm buffers.
    A dropless workload is re-routed at the capacity of C = 1.0."""
    import torch

    N, E, K = cfg["N"], cfg["E"], cfg["K"]
    c = cap if cap >= 0 else B.moe_capacity(1.0, N, K, E)
    idx = torch.empty(N, K, dtype=torch.int32, device=logits.device)
    w = torch.empty(N, K, dtype=torch.float32, device=logits.device)
    t_soft = _timed(stream, lambda: B.moe_route_topk(logits, K, False, idx, w))
    t_sig = _timed(stream, lambda: B.moe_route_topk(logits, K, False, idx, w, "sigmoid"))
    ws = torch.empty(max(1, B.moe_reroute_workspace_bytes(N, E, K)), dtype=torch.uint8,
                     device=logits.device)
    rr = torch.empty(E, dtype=torch.int32, device=logits.device)
    idx2, w2 = idx.clone(), w.clone()

    def reroute():
        idx2.copy_(idx)
        w2.copy_(w)
        B.moe_reroute_overflow(logits, idx2, w2, c, "softmax", False, rr, ws)

    B.moe_route_topk(logits, K, False, idx, w)
    t_copy = _timed(stream, lambda: (idx2.copy_(idx), w2.copy_(w)))
    t_rr = _timed(stream, reroute)
    demand = torch.bincount(idx.flatten().long(), minlength=E)
    kept = int(torch.clamp(demand, max=c).sum())
    admitted = int(rr.sum())
    return {
        "route_softmax_us": t_soft * 1e3,
        "route_sigmoid_us": t_sig * 1e3,
        "reroute_capacity": int(c),
        "reroute_us": max(t_rr - t_copy, 0.0) * 1e3,
        "dropped_without_reroute": N * K - kept,
        "reroute_admitted": admitted,
        "dropped_with_reroute": N * K - kept - admitted,
    }


def fp8_block(B, layer, x, cfg, M, stream, cold_reps):
    """FP8 (e4m3, one fp32 scale per 128 columns) exchange payload ("MoE
    推理服务工程真相 2026", section 6.3): the fp8 dispatch and combine timed
    with a cold cache like the bf16 ones, the quantize / dequantize passes at
    either end of an exchange timed warm, and the payload bytes per
    exchange direction in bf16 and fp8."""
    import numpy as np
    import torch

    N, d, E, K, W = cfg["N"], cfg["d"], cfg["E"], cfg["K"], cfg["W"]
    cap = layer.capacity
    dev = x.device
    out8 = B.alloc_dispatch_fp8_outputs(N, d, E, K, W, dev)
    n_rows = layer.disp["offsets"][E:E + 1]
    y8 = torch.empty(N * K, d, dtype=torch.uint8, device=dev)
    ys = torch.empty(N * K, d // 128, dtype=torch.float32, device=dev)
    out = torch.empty(N, d, dtype=torch.bfloat16, device=dev)
    xp = torch.empty(N * K, d, dtype=torch.bfloat16, device=dev)
    if layer.planned:   # the layer's plan (its routing ran last)
        def dispatch8():
            B.moe_dispatch_planned(x, layer.topk_idx, E, W, cap, layer.plan, out8, fp8=True)
    else:
        def dispatch8():
            B.moe_dispatch_fp8(x, layer.topk_idx, E, W, cap, out8)
    dispatch8()
    B.moe_fp8_quantize_rows(layer.y_perm, n_rows, N * K, y8, ys)
    torch.cuda.synchronize()

    scrub = torch.empty(SCRUB_MIB << 18, dtype=torch.float32, device=dev)
    cold = {}
    fns = {
        "dispatch": dispatch8,
        "combine": lambda: B.moe_combine_fp8(y8, ys, out8["dest"], layer.topk_w, out),
    }
    for name, fn in fns.items():
        times = []
        for i in range(max(cold_reps, 1)):
            scrub.fill_(float(i))
            scrub.sum()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        cold[name] = float(np.median(times))
    del scrub
    t_q = _timed(stream, lambda: B.moe_fp8_quantize_rows(layer.y_perm, n_rows, N * K, y8, ys))
    t_dq = _timed(stream, lambda: B.moe_fp8_dequantize_rows(out8["x8"], out8["x_scale"], n_rows,
                                                            N * K, xp))
    sb = M * (d // 128) * 4                        # scale bytes of M rows
    disp_b = N * d * 2 + M * d + sb + 12 * N * K
    comb_b = M * d + sb + N * d * 2 + 8 * N * K
    q_b = M * d * 2 + M * d + sb
    return {
        "format": "OCP e4m3 codes, one fp32 scale per 128 columns",
        "wire_bytes_per_direction_bf16": M * d * 2,
        "wire_bytes_per_direction_fp8": M * d + sb,
        "cold_dispatch_us": cold["dispatch"] * 1e3,
        "cold_combine_us": cold["combine"] * 1e3,
        "dispatch_bytes": disp_b,
        "combine_bytes": comb_b,
        "cold_dispatch_GBps": disp_b / (cold["dispatch"] * 1e-3) / 1e9,
        "cold_combine_GBps": comb_b / (cold["combine"] * 1e-3) / 1e9,
        "cold_dispatch_combine_GBps": (disp_b + comb_b) /
                                      ((cold["dispatch"] + cold["combine"]) * 1e-3) / 1e9,
        "quantize_rows_us": t_q * 1e3,
        "quantize_rows_GBps": q_b / (t_q * 1e-3) / 1e9,
        "dequantize_rows_us": t_dq * 1e3,
        "dequantize_rows_GBps": q_b / (t_dq * 1e-3) / 1e9,
    }


def residual_block(B, synth, inp, cfg, b, stream, packed=None, reps=10):
    """Residual-MoE ("MoE Inference Communication", section "PR-MoE：从”所有层
    一样多专家”到”哪里需要哪里多”", Phenomenon-II) at the workload's shape:
    top-1 routing plus a shared MLP as wide as an expert, on every token, its
    output added in the combine.  Times the whole layer step (route, dispatch,
    grouped FFN, shared MLP, residual combine; packed weights), the shared MLP
    and the residual combine alone, and compares the exchange's wire bytes
    with the workload's top-K layer (the reason for the design: top-1's
    all-to-all volume)."""
    import torch

    N, d, ffn, E, W, K = cfg["N"], cfg["d"], cfg["ffn"], cfg["E"], cfg["W"], cfg["K"]
    cap = -1
    if cfg.get("C") is not None:
        cap = B.moe_capacity(cfg["C"], N, 1, E)
    layer = B.MoeLayer(N, d, ffn, E, 1, W, cap, torch.bfloat16, "cuda:0", shared_ffn=ffn)
    experts = packed or B.moe_pack_ffn_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
    shared = B.moe_pack_ffn_weights(*synth.make_shared_weights(cfg, "cuda:0"))
    step_ms = _timed(stream, lambda: layer.forward(inp["logits"], inp["x"], experts,
                                                   shared=shared), reps=reps)
    shared_ms = _timed(stream, lambda: layer.shared(inp["x"], shared), reps=reps)
    comb_ms = _timed(stream, lambda: layer.combine(residual=True), reps=reps)
    M1 = int(layer.disp["offsets"][E].item())
    comb_bytes = M1 * d * b + 2 * N * d * b + 8 * N
    shared_flops = 6.0 * N * d * ffn
    M_k = N * K if cap < 0 else None
    return {
        "shape": f"top-1 routing + shared SwiGLU MLP (width {ffn}) on all {N} tokens, "
                 f"capacity {cap}",
        "kept_rows_top1": M1,
        "layer_ms": step_ms,
        "tokens_per_s": N / (step_ms * 1e-3),
        "shared_mlp_ms": shared_ms,
        "shared_mlp_TFLOPs": shared_flops / (shared_ms * 1e-3) / 1e12,
        "residual_combine_us": comb_ms * 1e3,
        "residual_combine_GBps": comb_bytes / (comb_ms * 1e-3) / 1e9,
        "wire_bytes_per_direction_top1": M1 * d * b,
        "wire_bytes_per_direction_topK_dropless": (M_k * d * b) if M_k is not None else None,
    }


def router_block(B, synth, x, cfg, b, stream):
    """Router projection logits = x @ w_router^T (fp32), timed alone on warm
    buffers: HBM bytes (x, w_router, logits) and flops.  The timed launches
    are queued behind a spin kernel, so the host's per-call overhead does not
    open gaps between them (a short kernel would otherwise be timed at the
    host's call rate); `us_host_paced` is the same loop without it."""
    import torch

    N, d, E = cfg["N"], cfg["d"], cfg["E"]
    wr = synth.make_router(cfg, x.device)
    logits = torch.empty(N, E, dtype=torch.float32, device=x.device)
    B.moe_router_logits(x, wr, logits)
    torch.cuda.synchronize()
    reps = 20

    def timed(queued):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        if queued:
            torch.cuda._sleep(2_000_000)
        e0.record(stream)
        for _ in range(reps):
            B.moe_router_logits(x, wr, logits)
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / reps

    ms = min(timed(True) for _ in range(3))
    host_ms = timed(False)
    nbytes = N * d * b + E * d * b + N * E * 4
    return {"us": ms * 1e3, "us_host_paced": host_ms * 1e3,
            "GBps": nbytes / (ms * 1e-3) / 1e9,
            "TFLOPs": 2.0 * N * d * E / (ms * 1e-3) / 1e12}


def cpu_baseline(cfg, inp, n_tok, runs=3):
    """The oracle, untouched, on the first n_tok tokens of the same workload,
    stage by stage: route, dispatch (histogram, capacity, layout and the row
    copies), the grouped FFN and combine, each timed with perf_counter, the
    median of `runs` runs.  Routing, dispatch and combine are single-threaded
    numpy; the FFN's products use the BLAS thread pool."""
    import numpy as np
    from oracle import moe_oracle as O

    n = min(n_tok, cfg["N"])
    logits = inp["logits"][:n].cpu().numpy()
    x = inp["x"][:n].float().cpu().numpy()
    cache = {}

    def weights(e):
        if e not in cache:
            cache.clear()
            cache[e] = tuple(inp[k][e].float().cpu().numpy() for k in ("w_gate", "w_up", "w_down"))
        return cache[e]

    # with few experts the weights are copied to the host before the clock starts
    host_w = {e: weights(e) for e in range(cfg["E"])} if cfg["E"] <= 16 else None
    fn = (lambda e: host_w[e]) if host_w is not None else weights
    cap_s = O.capacity(cfg["C"], n, cfg["K"], cfg["E"]) if cfg["C"] is not None else -1
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = 1
    times = {k: [] for k in ("route", "dispatch", "ffn", "combine")}
    for _ in range(runs):
        t = time.perf_counter()
        idx, w = O.route(logits, cfg["K"])
        times["route"].append(time.perf_counter() - t)
        t = time.perf_counter()
        disp = O.dispatch(idx, cfg["E"], cfg["W"], cap_s)
        x_perm = O.pack(x, disp["perm_token"])
        times["dispatch"].append(time.perf_counter() - t)
        t = time.perf_counter()
        _, y = O.grouped_ffn(x_perm, disp["offsets"], fn, cfg["act"])
        times["ffn"].append(time.perf_counter() - t)
        t = time.perf_counter()
        O.combine(y, disp["dest"], w, cfg["act"])
        times["combine"].append(time.perf_counter() - t)
    med = {k: float(np.median(v)) for k, v in times.items()}
    total = sum(med.values())
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return {
        "value": n / total,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {n} of {cfg['N']} tokens of the same workload (same logits, hidden "
                  f"states and weights; capacity recomputed for {n} tokens), whole oracle "
                  f"layer in float64 numpy stage by stage, median of {runs} runs per stage, "
                  f"{total:.1f} s per layer; route, dispatch and combine on 1 core, the FFN's "
                  f"products on {threads} BLAS threads",
        "stage_s": med,
        "stage_tokens_per_s": {k: (n / v if v > 0 else None) for k, v in med.items()},
        "os_cpu_count": os.cpu_count(),
        "affinity_cpus": affinity,
        "blas_threads": threads,
    }


if __name__ == "__main__":
    main()

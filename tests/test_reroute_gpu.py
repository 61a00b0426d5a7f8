"""Routing variants on the GPU against the oracle: the sigmoid gate
(moe_route_topk_gated) and the re-route of capacity overflow
(moe_reroute_overflow).  Expert ids, admitted counts and everything
dispatch derives from them must match bit for bit; gate weights to 1e-6."""
import json
import os

import numpy as np
import pytest
import torch

from grouped_gemm_route_amd import binding as B
from grouped_gemm_route_amd import synth
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
W_TOL = 1e-6
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _np(t):
    return t.detach().cpu().numpy()


def _logits(N, E, seed, kind="normal"):
    g = torch.Generator().manual_seed(seed)
    if kind == "ties":
        return (torch.randint(-3, 4, (N, E), generator=g) * 0.5).float()
    if kind == "uniform":
        return torch.zeros(N, E)
    return torch.randn(N, E, generator=g)


@pytest.mark.parametrize("N,E,K,renorm", [(300, 8, 2, False), (257, 64, 6, True),
                                          (100, 256, 8, False), (64, 1024, 16, True),
                                          (50, 5, 5, False)])
def test_sigmoid_route_matches_oracle(N, E, K, renorm):
    print(f"[reroute] sigmoid route N={N} E={E} K={K} renorm={renorm}", flush=True)
    l = _logits(N, E, E + K)
    l[::7] = 0.0
    idx, w = B.moe_route_topk(l.to(DEV), K, renorm, gate="sigmoid")
    torch.cuda.synchronize()
    ri, rw = O.route(_np(l), K, renorm, gate="sigmoid")
    assert np.array_equal(_np(idx), ri)
    assert np.abs(_np(w).astype(np.float64) - rw).max() <= W_TOL


def _check_reroute(l, K, cap, gate="softmax", renorm=False, W=1):
    N, E = l.shape
    ld = l.to(DEV)
    idx, w = B.moe_route_topk(ld, K, renorm, gate=gate)
    rr = B.moe_reroute_overflow(ld, idx, w, cap, gate, renorm)
    disp = B.moe_dispatch(torch.zeros(N, 8, dtype=torch.bfloat16, device=DEV), idx, E, W, cap)
    torch.cuda.synchronize()
    ri, rw = O.route(_np(l), K, renorm, gate)
    ni, nw, nrr = O.reroute_overflow(_np(l), ri, cap, gate, renorm)
    assert np.array_equal(_np(idx), ni)
    assert np.array_equal(_np(rr), nrr)
    assert np.abs(_np(w).astype(np.float64) - nw).max() <= W_TOL
    ref = O.dispatch(ni, E, W, cap)
    for k in ("demand", "counts", "offsets", "dest"):
        assert np.array_equal(_np(disp[k]), ref[k]), k
    return ni, nrr, ref


def test_reroute_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "reroute_hand.json")))
    l = torch.tensor(g["logits"], dtype=torch.float32)
    for gate in ("softmax", "sigmoid"):
        ni, nrr, ref = _check_reroute(l, g["K"], g["capacity"], gate, W=g["W"])
        assert ni.tolist() == g["reroute_topk_idx"]
        assert nrr.tolist() == g["rerouted"]
        assert ref["dest"].tolist() == g["after_dispatch"]["dest"]


@pytest.mark.parametrize("case", [
    dict(N=700, E=8, K=2, cap=150, kind="normal"),
    dict(N=700, E=8, K=2, cap=150, kind="ties", gate="sigmoid"),
    dict(N=513, E=32, K=4, cap=40, kind="ties", renorm=True),
    dict(N=513, E=32, K=4, cap=40, kind="normal", gate="sigmoid", renorm=True),
    dict(N=100, E=16, K=4, cap=10, kind="uniform"),
    dict(N=300, E=6, K=6, cap=20, kind="normal"),         # K == E: nowhere to go
    dict(N=200, E=16, K=2, cap=0, kind="normal"),         # no room anywhere
    dict(N=200, E=16, K=2, cap=-1, kind="normal"),        # dropless: no-op
    dict(N=90, E=1024, K=16, cap=1, kind="ties"),
    dict(N=1000, E=100, K=3, cap=25, kind="normal"),      # E not a power of two
])
def test_reroute_matches_oracle(case):
    print(f"[reroute] {case}", flush=True)
    l = _logits(case["N"], case["E"], case["N"] + case["E"], case["kind"])
    _check_reroute(l, case["K"], case["cap"], case.get("gate", "softmax"),
                   case.get("renorm", False))


@pytest.mark.parametrize("name", ["fine128_zipf_c1.25", "prefill256_hot_c1.0"])
def test_reroute_full_size_routing(name):
    cfg = synth.config(name)
    print(f"[reroute] full size {name}", flush=True)
    logits = synth.make_logits(cfg, "cpu")
    cap = O.capacity(cfg["C"], cfg["N"], cfg["K"], cfg["E"])
    ni, nrr, ref = _check_reroute(logits, cfg["K"], cap, W=cfg["W"])
    print(f"[reroute] {name}: admitted {int(nrr.sum())}, dropped after {ref['dropped']}",
          flush=True)


def test_reroute_layer_matches_oracle():
    cfg = synth.config("reroute_layer", N=600, d=128, ffn=192, E=16, K=4, W=4, act="bf16",
                       C=0.8, bias="zipf")
    inp = synth.make_inputs(cfg, DEV)
    cap = O.capacity(cfg["C"], cfg["N"], cfg["K"], cfg["E"])
    layer = B.MoeLayer(cfg["N"], cfg["d"], cfg["ffn"], cfg["E"], cfg["K"], cfg["W"], cap,
                       torch.bfloat16, DEV, gate="sigmoid", reroute=True)
    layer.forward(inp["logits"], inp["x"], inp["w_gate"], inp["w_up"], inp["w_down"])
    torch.cuda.synchronize()

    def weights(e):
        return tuple(inp[k][e].float().cpu().numpy() for k in ("w_gate", "w_up", "w_down"))
    ref = O.layer(_np(inp["logits"]), inp["x"].float().cpu().numpy(), weights, cfg["K"],
                  cfg["W"], cap, "bf16", gate="sigmoid", reroute=True)
    assert np.array_equal(_np(layer.topk_idx), ref["topk_idx"])
    assert np.array_equal(_np(layer.rerouted), ref["rerouted"])
    assert ref["rerouted"].sum() > 0
    got = layer.out.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref["out"])
    assert (err <= 2e-2 + 1e-2 * np.abs(ref["out"])).all(), err.max()


def test_reroute_sigmoid_renormalised_far_negative_logits():
    # renormalised sigmoid weights of re-routed slots stay finite when every
    # logit is far below zero (plain fp32 scores all round to 0 there)
    N, E, K, cap = 300, 16, 2, 60
    g = torch.Generator().manual_seed(11)
    l = -110.0 - 20.0 * torch.rand(N, E, generator=g)
    l[:, 0] += 5.0                   # a hot expert that overflows
    ni, nrr, _ = _check_reroute(l, K, cap, "sigmoid", True)
    assert nrr.sum() > 0

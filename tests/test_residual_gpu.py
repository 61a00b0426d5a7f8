"""Residual-MoE layer on the GPU ("MoE Inference Communication", section
"PR-MoE：从”所有层一样多专家”到”哪里需要哪里多”", Phenomenon-II: a shared dense
MLP on every token, its output added to the routed expert's) against the
oracle: routing and dispatch bit-exact, y_shared and out within the layer
tolerances (bf16: |err| <= 2e-2 + 1e-2 |ref|; fp32: 1e-4 + 1e-4 |ref|), with
the shared MLP's weights row-major and packed.  moe_combine_residual alone:
one rounding of the whole sum and the shared term unweighted (bit-exact on a
built input), every pair dropped (out = the shared rows, bitwise), and the
full-size dense8 shape with top-1 routing on sampled tokens."""
import numpy as np
import pytest
import torch

from grouped_gemm_route_amd import binding as B
from grouped_gemm_route_amd import synth
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-4)}


def _np(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def _close(name, got, ref, act):
    atol, rtol = TOL[act]
    err = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    bad = err > atol + rtol * np.abs(ref)
    assert not bad.any(), f"{name}: {int(bad.sum())} bad of {bad.size}, max err {err.max():.3e}"


def _weights_np(inp):
    return {e: tuple(_np(inp[k][e]) for k in ("w_gate", "w_up", "w_down"))
            for e in range(inp["w_gate"].shape[0])}


CASES = [
    dict(name="tiny_f32", K=1, ffn_s=256),
    dict(name="res_bf16_drop", N=300, d=128, ffn=192, E=8, K=1, W=4, act="bf16", C=1.0,
         ffn_s=320),
    dict(name="res_bf16_k2", N=257, d=256, ffn=128, E=16, K=2, W=8, act="bf16", C=None,
         ffn_s=256),
]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_residual_layer_matches_oracle(case):
    case = dict(case)
    ffn_s = case.pop("ffn_s")
    cfg = synth.config(case.pop("name"), **case)
    print(f"[residual] {cfg} ffn_s={ffn_s}", flush=True)
    inp = synth.make_inputs(cfg, DEV)
    sh = synth.make_shared_weights(cfg, DEV, ffn_s)
    cap = O.capacity(cfg["C"], cfg["N"], cfg["K"], cfg["E"]) if cfg["C"] is not None else -1
    wts = _weights_np(inp)
    sh_np = tuple(_np(a[0]) for a in sh)
    ref = O.layer(_np(inp["logits"]), _np(inp["x"]), lambda e: wts[e], cfg["K"], cfg["W"], cap,
                  cfg["act"], shared_weights=sh_np)
    kinds = [("row-major", sh)]
    if cfg["act"] == "bf16":
        kinds.append(("packed", B.moe_pack_ffn_weights(*sh)))
    for kind, shared in kinds:
        layer = B.MoeLayer(cfg["N"], cfg["d"], cfg["ffn"], cfg["E"], cfg["K"], cfg["W"], cap,
                           synth.TORCH_DTYPE[cfg["act"]], DEV, shared_ffn=ffn_s)
        experts = (B.moe_pack_ffn_weights(inp["w_gate"], inp["w_up"], inp["w_down"]),) \
            if kind == "packed" else (inp["w_gate"], inp["w_up"], inp["w_down"])
        out = layer.forward(inp["logits"], inp["x"], *experts, shared=shared)
        torch.cuda.synchronize()
        assert np.array_equal(_np(layer.topk_idx), ref["topk_idx"])
        for k in ("counts", "offsets", "dest"):
            assert np.array_equal(_np(layer.disp[k]), ref[k]), (kind, k)
        _close(f"{kind} y_shared", _np(layer.y_shared), ref["y_shared"], cfg["act"])
        _close(f"{kind} out", _np(out), ref["out"], cfg["act"])


def test_residual_combine_rounds_once_and_adds_shared_unweighted():
    bf = torch.bfloat16
    y_perm = torch.zeros(3, 8, dtype=bf, device=DEV)
    y_perm[0] = 2.0 ** -8
    y_perm[1] = 2.0 ** -17
    dest = torch.tensor([[0, 1], [2, -1]], dtype=torch.int32, device=DEV)
    w = torch.tensor([[1.0, 1.0], [0.25, 0.5]], dtype=torch.float32, device=DEV)
    shared = torch.tensor([[1.0] * 8, [3.0] * 8], dtype=bf, device=DEV)
    out = B.moe_combine_residual(y_perm, dest, w, shared)
    torch.cuda.synchronize()
    ref = O.combine(_np(y_perm), _np(dest), _np(w), "bf16", shared=_np(shared))
    assert np.array_equal(_np(out), ref)
    assert (_np(out)[0] == 1.0 + 2.0 ** -7).all() and (_np(out)[1] == 3.0).all()


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_residual_combine_with_every_pair_dropped_is_the_shared_rows(act):
    dt = synth.TORCH_DTYPE[act]
    N, K, d = 77, 4, 136 if act == "bf16" else 132
    g = torch.Generator(device=DEV).manual_seed(5)
    shared = torch.randn(N, d, generator=g, device=DEV).to(dt)
    y_perm = torch.randn(16, d, generator=g, device=DEV).to(dt)
    dest = torch.full((N, K), -1, dtype=torch.int32, device=DEV)
    w = torch.rand(N, K, generator=g, device=DEV)
    out = B.moe_combine_residual(y_perm, dest, w, shared)
    torch.cuda.synchronize()
    assert torch.equal(out, shared)


@pytest.mark.parametrize("K", [1, 3, 8, 16])
def test_residual_combine_matches_oracle(K):
    N, d, rows = 501, 1032, 700
    g = torch.Generator(device=DEV).manual_seed(K)
    y_perm = torch.randn(rows, d, generator=g, device=DEV).to(torch.bfloat16)
    shared = torch.randn(N, d, generator=g, device=DEV).to(torch.bfloat16)
    dest = torch.randint(-1, rows, (N, K), generator=g, device=DEV, dtype=torch.int32)
    w = torch.rand(N, K, generator=g, device=DEV)
    out = B.moe_combine_residual(y_perm, dest, w, shared)
    torch.cuda.synchronize()
    ref = O.combine(_np(y_perm), _np(dest), _np(w), "bf16", shared=_np(shared))
    _close(f"combine K={K}", _np(out), ref, "bf16")


def test_full_size_residual_top1_layer_matches_oracle():
    # the dense8 shape with the Residual-MoE pairing: top-1 routing plus a
    # shared MLP as wide as an expert, packed weights as in the bench
    cfg = synth.config("dense8", K=1)
    print(f"[residual] full size {cfg}", flush=True)
    inp = synth.make_inputs(cfg, DEV)
    sh = synth.make_shared_weights(cfg, DEV)
    layer = B.MoeLayer(cfg["N"], cfg["d"], cfg["ffn"], cfg["E"], 1, cfg["W"], -1,
                       torch.bfloat16, DEV, shared_ffn=cfg["ffn"])
    pw = B.moe_pack_ffn_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
    layer.forward(inp["logits"], inp["x"], pw, shared=B.moe_pack_ffn_weights(*sh))
    torch.cuda.synchronize()
    idx, w = O.route(_np(inp["logits"]), 1)
    ref = O.dispatch(idx, cfg["E"], cfg["W"], -1)
    assert np.array_equal(_np(layer.topk_idx), idx)
    assert np.array_equal(_np(layer.disp["dest"]), ref["dest"])
    toks = [0, 17, 1000, 2049, 3333, cfg["N"] - 1]
    xs = _np(inp["x"][torch.tensor(toks, device=DEV)])
    wts = {}

    def expert(e):
        if e not in wts:
            wts[e] = tuple(_np(inp[k][e]) for k in ("w_gate", "w_up", "w_down"))
        return wts[e]
    sh_np = tuple(_np(a[0]) for a in sh)
    _, out_ref = O.token_outputs(toks, xs, idx, w, ref["dest"], expert, "bf16",
                                 shared_weights=sh_np)
    _close("y_shared", _np(layer.y_shared[torch.tensor(toks, device=DEV)]),
           O.shared_expert(xs, *sh_np, "bf16"), "bf16")
    _close("out", _np(layer.out[torch.tensor(toks, device=DEV)]), out_ref, "bf16")


@pytest.mark.parametrize("case", [
    dict(N=1, d=64, ffn=64, E=4, K=2, W=2, cap=-1),      # one token
    dict(N=40, d=128, ffn=64, E=1, K=1, W=1, cap=-1),    # one expert: weight 1
    dict(N=64, d=64, ffn=128, E=8, K=3, W=4, cap=0),     # every pair dropped
])
def test_residual_layer_edge_cases(case):
    cfg = synth.config("res_edge", act="bf16", C=None,
                       **{k: v for k, v in case.items() if k != "cap"})
    cap = case["cap"]
    print(f"[residual] edge {case}", flush=True)
    inp = synth.make_inputs(cfg, DEV)
    sh = synth.make_shared_weights(cfg, DEV, 192)
    wts = _weights_np(inp)
    sh_np = tuple(_np(a[0]) for a in sh)
    ref = O.layer(_np(inp["logits"]), _np(inp["x"]), lambda e: wts[e], cfg["K"], cfg["W"], cap,
                  "bf16", shared_weights=sh_np)
    layer = B.MoeLayer(cfg["N"], cfg["d"], cfg["ffn"], cfg["E"], cfg["K"], cfg["W"], cap,
                       torch.bfloat16, DEV, shared_ffn=192)
    out = layer.forward(inp["logits"], inp["x"], inp["w_gate"], inp["w_up"], inp["w_down"],
                        shared=B.moe_pack_ffn_weights(*sh))
    torch.cuda.synchronize()
    assert np.array_equal(_np(layer.disp["dest"]), ref["dest"])
    _close("y_shared", _np(layer.y_shared), ref["y_shared"], "bf16")
    _close("out", _np(out), ref["out"], "bf16")
    if cap == 0:
        assert torch.equal(out, layer.y_shared)     # nothing kept: the shared rows, bitwise


def test_shared_ffn_rejects_more_than_one_expert():
    cfg = synth.config("res_reject", N=8, d=64, ffn=64, E=2, K=1, W=1, act="bf16", C=None)
    inp = synth.make_inputs(cfg, DEV)
    offsets = torch.tensor([0, 8], dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        B.moe_shared_ffn(inp["x"], offsets, inp["w_gate"], inp["w_up"], inp["w_down"])

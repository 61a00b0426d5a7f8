"""The layer's four calls captured as one HIP graph (MoeLayer.capture) and
replayed: every replay, with new inputs written into the captured buffers
and eager work and synchronisations between replays, must give bit for bit
what an eager layer gives on the same inputs (the kernels are deterministic,
split reductions included), and the eager layer matches the oracle.  The
bf16 layers route and dispatch on the planned path (MoeLayer's default):
the small tables are scanned in the scatter, plan_in_route's by the routing
launch's last block and plan_scan_kernel's by the scan kernel."""
import numpy as np
import pytest
import torch

from grouped_gemm_route_amd import binding as B
from grouped_gemm_route_amd import synth
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = {
    "tiny_f32": (synth.config("tiny_f32"), False),
    "decode_like": (synth.config("gr_decode", N=16, d=1024, ffn=512, E=64, K=8, W=8,
                                 act="bf16", C=None), True),
    "capped_bf16": (synth.config("gr_capped", N=300, d=256, ffn=320, E=8, K=2, W=4,
                                 act="bf16", C=0.9), True),
    # splits along the reduction in both passes (the arrival counters and
    # partial slots are reused by every replay)
    "split": (synth.config("gr_split", N=48, d=4096, ffn=4096, E=2, K=2, W=2, act="bf16",
                           C=None), True),
    # the planned routing's count table (32 x 128) scanned by the routing
    # launch's last block: its arrival counter is reused by every replay
    "plan_in_route": (synth.config("gr_plan_route", N=2048, d=256, ffn=256, E=128, K=4, W=8,
                                   act="bf16", C=1.0), True),
    # a count table (71 x 600) scanned by the dispatch's scan kernel
    "plan_scan_kernel": (synth.config("gr_plan_kernel", N=4500, d=128, ffn=128, E=600, K=2,
                                      W=8, act="bf16", C=None), True),
}


def _outputs(layer):
    M = int(layer.disp["offsets"][-1])
    return {"topk_idx": layer.topk_idx.clone(), "topk_w": layer.topk_w.clone(),
            "dest": layer.disp["dest"].clone(), "offsets": layer.disp["offsets"].clone(),
            "y_perm": layer.y_perm[:M].clone(), "out": layer.out.clone()}


# packed weights exist for bf16 layers only
@pytest.mark.parametrize("name,packed",
                         [(n, p) for n, (_, bf16) in CASES.items() for p in (False, True)
                          if bf16 or not p])
def test_graph_replays_match_eager(name, packed):
    cfg, _ = CASES[name]
    print(f"[graph] {name} packed={packed}", flush=True)
    N, d, ffn, E, K, W = (cfg[k] for k in ("N", "d", "ffn", "E", "K", "W"))
    cap = O.capacity(cfg["C"], N, K, E) if cfg["C"] is not None else -1
    dt = synth.TORCH_DTYPE[cfg["act"]]
    inp = synth.make_inputs(cfg, DEV)
    wargs = ((B.moe_pack_ffn_weights(inp["w_gate"], inp["w_up"], inp["w_down"]),) if packed
             else (inp["w_gate"], inp["w_up"], inp["w_down"]))
    logits = inp["logits"].clone()
    x = inp["x"].clone()
    layer = B.MoeLayer(N, d, ffn, E, K, W, cap, dt, DEV)
    graph = layer.capture(logits, x, *wargs)
    eager = B.MoeLayer(N, d, ffn, E, K, W, cap, dt, DEV)
    g = torch.Generator(device=DEV).manual_seed(3)
    for rep in range(4):
        if rep > 0:   # new inputs in the captured buffers, written eagerly
            logits.copy_(torch.randn(N, E, generator=g, device=DEV))
            x.copy_(torch.randn(N, d, generator=g, device=DEV).to(dt))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _outputs(layer)
        eager.forward(logits, x, *wargs)
        torch.cuda.synchronize()
        ref = _outputs(eager)
        for k in ref:
            assert torch.equal(got[k], ref[k]), (name, rep, k)
        if rep == 0:
            # the eager layer against the oracle on the original inputs
            wts = {e: tuple(inp[k][e].float().cpu().numpy() for k in ("w_gate", "w_up", "w_down"))
                   for e in range(E)}
            o = O.layer(logits.cpu().numpy(), x.float().cpu().numpy(), lambda e: wts[e], K, W,
                        cap, cfg["act"])
            assert np.array_equal(eager.topk_idx.cpu().numpy(), o["topk_idx"])
            atol, rtol = (2e-2, 1e-2) if cfg["act"] == "bf16" else (1e-4, 1e-4)
            err = np.abs(eager.out.float().cpu().numpy() - o["out"])
            assert (err <= atol + rtol * np.abs(o["out"])).all()

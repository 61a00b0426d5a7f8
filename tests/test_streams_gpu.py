"""Calls on two streams at once: two layers, each enqueued on its own
non-default stream and interleaved call by call, give bit for bit what
each gives alone on the default stream.  Every call launches on the stream
it is given and keeps no state between calls outside its own buffers
(workspaces, counters and split partials are per layer), so concurrent
layers cannot disturb each other.  Row-major and packed weights, a
dropless and a capped layer, and split reductions in the packed FFN."""
import pytest
import torch

from grouped_gemm_route_amd import binding as B
from grouped_gemm_route_amd import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

CFGS = [
    synth.config("streams_a", N=600, d=256, ffn=512, E=8, K=2, W=4, act="bf16", C=None),
    synth.config("streams_b", N=900, d=256, ffn=512, E=16, K=4, W=4, act="bf16", C=1.0),
    # one expert whose 512 rows make every packed pass split its last round
    synth.config("streams_split", N=512, d=4096, ffn=4096, E=1, K=1, W=1, act="bf16", C=None),
]


def _layer(cfg, packed):
    inp = synth.make_inputs(cfg, DEV)
    N, d, ffn, E, K, W = (cfg[k] for k in ("N", "d", "ffn", "E", "K", "W"))
    cap = B.moe_capacity(cfg["C"], N, K, E) if cfg["C"] is not None else -1
    layer = B.MoeLayer(N, d, ffn, E, K, W, cap, torch.bfloat16, DEV)
    w = ((B.moe_pack_ffn_weights(inp["w_gate"], inp["w_up"], inp["w_down"]),) if packed
         else (inp["w_gate"], inp["w_up"], inp["w_down"]))
    return layer, inp, w


def _calls(layer, inp, w):
    return [lambda: layer.route(inp["logits"]), lambda: layer.dispatch(inp["x"]),
            lambda: layer.ffn(*w), lambda: layer.combine()]


def _snapshot(layer):
    M = int(layer.disp["offsets"][-1])
    return (layer.topk_idx.clone(), layer.disp["x_perm"][:M].clone(), layer.y_perm[:M].clone(),
            layer.out.clone())


@pytest.mark.parametrize("packed", [False, True])
def test_two_layers_on_two_streams_match_each_alone(packed):
    print(f"[streams] packed={packed}", flush=True)
    layers = [_layer(c, packed) for c in CFGS]
    alone = []
    for layer, inp, w in layers:
        for f in _calls(layer, inp, w):
            f()
        torch.cuda.synchronize()
        alone.append(_snapshot(layer))
        layer.out.zero_()
        layer.y_perm.zero_()
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(DEV) for _ in layers]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream(DEV))
    calls = [_calls(*lw) for lw in layers]
    for rep in range(3):
        for step in range(4):
            for s, c in zip(streams, calls):
                with torch.cuda.stream(s):
                    c[step]()
        torch.cuda.synchronize()
        for (layer, _, _), ref in zip(layers, alone):
            got = _snapshot(layer)
            for a, b in zip(got, ref):
                assert torch.equal(a, b), rep

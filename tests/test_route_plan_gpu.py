"""moe_route_plan (routing that also ranks and counts the tokens per expert,
in one launch) and moe_dispatch_planned (the dispatch without a counting
pass), HIP path vs the oracle: expert ids and every dispatch output
bit-exact, gate weights within 1e-6.

The plan's count table is scanned in one of three places by its size, and
the cases reach each: by every scatter block (up to 1024 counts and 256
experts: 8 experts over 32 blocks of 128 tokens, one token, a decode-sized
block, one expert, the sigmoid case), by the routing launch's last block
(up to 32768 counts: 128 experts over 128 blocks, 16 counts per thread;
600 experts over 47 blocks, one part per expert and a second batch of
loads; 1024 experts; capacity 0), and by the dispatch's scan kernel (256
experts over 512 blocks, four batches; 600 experts over 63 blocks).  Every
case calls twice on one plan buffer whose contents past the arrival counter
start as garbage, with output buffers filled with stale values, and the
counter must be back at zero after each call; one test reuses a plan across
sizes that switch between the modes, one checks the fp8 payload.
"""
import numpy as np
import pytest
import torch

from grouped_gemm_route_amd import binding as B
from grouped_gemm_route_amd import synth
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
W_TOL = 1e-6

# (N, E, K, W, C, gate, renormalize); C: capacity factor, None (dropless) or
# "cap0" (a capacity of 0 rows)
CASES = [
    pytest.param(4096, 8, 2, 8, None, "softmax", False, id="e8_dropless"),
    pytest.param(4097, 8, 2, 8, 1.0, "softmax", False, id="e8_ragged_c1.0"),
    pytest.param(1, 8, 2, 1, None, "softmax", True, id="one_token"),
    pytest.param(16, 256, 8, 8, None, "softmax", False, id="decode_one_block"),
    pytest.param(8192, 128, 8, 8, 1.25, "softmax", False, id="e128_c1.25"),
    pytest.param(32768, 256, 8, 8, 1.0, "softmax", False, id="e256_512_blocks"),
    pytest.param(3000, 600, 4, 8, 0.7, "softmax", True, id="e600_second_batch"),
    pytest.param(4000, 600, 4, 8, 1.0, "softmax", False, id="e600_scan_kernel"),
    pytest.param(700, 1024, 16, 8, None, "softmax", False, id="e1024"),
    pytest.param(9000, 1, 1, 1, None, "softmax", False, id="one_expert"),
    pytest.param(2000, 64, 6, 4, "cap0", "softmax", False, id="capacity_0"),
    pytest.param(1000, 64, 4, 4, 1.0, "sigmoid", True, id="sigmoid_renorm"),
]


def _np(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def _plan_counter(plan):
    return int(plan[:4].view(torch.int32).item())


def _run(inp, E, K, W, cap, plan, gate, renorm):
    N, d = inp["x"].shape
    out = B.alloc_dispatch_outputs(N, d, E, K, W, inp["x"].dtype, DEV)
    for k in B.DISPATCH_OUTPUTS:
        if out[k].dtype == torch.int32:
            out[k].fill_(-7)               # stale values a call must overwrite
    idx, w, _ = B.moe_route_plan(inp["logits"], K, W, cap, plan, out, renorm, gate=gate)
    B.moe_dispatch_planned(inp["x"], idx, E, W, cap, plan, out)
    torch.cuda.synchronize()
    out.update(topk_idx=idx, topk_w=w)
    return out


def _check(out, inp, ri, rw, ref):
    assert np.array_equal(_np(out["topk_idx"]), ri)
    assert np.abs(_np(out["topk_w"]).astype(np.float64) - rw).max() <= W_TOL
    for k in ("demand", "counts", "offsets", "rank_offsets", "dest"):
        assert np.array_equal(_np(out[k]), ref[k]), k
    M = int(ref["offsets"][-1])
    assert np.array_equal(_np(out["perm_token"])[:M], ref["perm_token"])
    perm = torch.from_numpy(ref["perm_token"].astype(np.int64)).to(DEV)
    assert torch.equal(out["x_perm"][:M], inp["x"][perm])   # bitwise row copies


@pytest.mark.parametrize("N,E,K,W,C,gate,renorm", CASES)
def test_route_plan_and_planned_dispatch_match_oracle(N, E, K, W, C, gate, renorm):
    d = 64
    factor = C if isinstance(C, float) else None
    cfg = synth.config(f"plan_{N}_{E}_{K}", N=N, d=d, ffn=64, E=E, K=K, W=W, act="bf16",
                       C=factor)
    print(f"[route_plan] N={N} E={E} K={K} W={W} C={C} gate={gate}", flush=True)
    cap = 0 if C == "cap0" else O.capacity(C, N, K, E) if C is not None else -1
    inp = synth.make_inputs(cfg, DEV, weights=False)
    ri, rw = O.route(_np(inp["logits"]), K, renorm, gate=gate)
    ref = O.dispatch(ri, E, W, cap)
    plan = B.alloc_route_plan(N, E, K, DEV)
    plan[256:].fill_(0xA5)               # all but the arrival counter: garbage
    for _ in range(2):
        out = _run(inp, E, K, W, cap, plan, gate, renorm)
        _check(out, inp, ri, rw, ref)
        assert _plan_counter(plan) == 0


def test_one_plan_across_sizes():
    # a plan sized for the largest call serves smaller ones
    E, K, W, d = 128, 4, 8, 64
    plan = B.alloc_route_plan(6000, E, K, DEV)
    for N, C in ((6000, 1.0), (300, None), (4097, 0.5), (6000, None)):
        cfg = synth.config(f"plan_sizes_{N}", N=N, d=d, ffn=64, E=E, K=K, W=W, act="bf16", C=C)
        print(f"[route_plan] shared plan N={N} C={C}", flush=True)
        cap = O.capacity(C, N, K, E) if C is not None else -1
        inp = synth.make_inputs(cfg, DEV, weights=False)
        ri, rw = O.route(_np(inp["logits"]), K)
        out = _run(inp, E, K, W, cap, plan, "softmax", False)
        _check(out, inp, ri, rw, O.dispatch(ri, E, W, cap))
        assert _plan_counter(plan) == 0


@pytest.mark.parametrize("N,E,K,W", [(300, 8, 2, 4), (2100, 128, 4, 8)])
def test_planned_dispatch_fp8_payload(N, E, K, W):
    d = 2048
    cfg = synth.config(f"plan_fp8_{N}_{E}", N=N, d=d, ffn=64, E=E, K=K, W=W, act="bf16", C=0.8)
    print(f"[route_plan] fp8 N={N} E={E}", flush=True)
    cap = O.capacity(0.8, N, K, E)
    inp = synth.make_inputs(cfg, DEV, weights=False)
    plan = B.alloc_route_plan(N, E, K, DEV)
    out = B.alloc_dispatch_fp8_outputs(N, d, E, K, W, DEV)
    idx, _, _ = B.moe_route_plan(inp["logits"], K, W, cap, plan, out)
    B.moe_dispatch_planned(inp["x"], idx, E, W, cap, plan, out, fp8=True)
    torch.cuda.synchronize()
    ri, _ = O.route(_np(inp["logits"]), K)
    ref = O.dispatch(ri, E, W, cap)
    for k in ("demand", "counts", "offsets", "rank_offsets", "dest"):
        assert np.array_equal(_np(out[k]), ref[k]), k
    M = int(ref["offsets"][-1])
    assert np.array_equal(_np(out["perm_token"])[:M], ref["perm_token"])
    tq, ts = O.quantize_fp8(_np(inp["x"]))
    pt = ref["perm_token"].astype(np.int64)
    assert np.array_equal(_np(out["x8"])[:M], tq[pt])
    assert np.array_equal(_np(out["x_scale"])[:M], ts[pt])

"""Dispatch alone, HIP path vs the oracle, across row widths and count-table sizes.

The scatter kernel holds 1, 2 or 4 of a token's 16-byte row pieces per thread
before it knows the token's rows, and copies any further pieces one by one
afterwards; it runs 256 threads per token below 1024 tokens, and from 1024
tokens 64, 128 or 256 by row width (about a quarter of the row's pieces).
The widths below reach every one of those paths, fully and partly filled,
for bf16 and fp32 rows and for the fp8 payload, at 300 tokens (256 threads)
and at 2100 (the narrower blocks).  Two expert counts cover both ways of finding the expert offsets:
each scatter block scanning the small per-block count table itself (8
experts), and the one-block scan kernel (128 experts over 9 blocks of
tokens: a table of 1152 counts).  Further cases take both paths at their
edges (one block of tokens, whole blocks and a ragged last one, one expert,
the largest expert count, the largest table the scatter scans itself) and
repeat each call three times on one workspace.  Everything compared is an
integer or a bit copy, so it must match exactly.
"""
import numpy as np
import pytest
import torch

from grouped_gemm_route_amd import binding as B
from grouped_gemm_route_amd import synth
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (activation dtype, d): a row is d * (2 or 4) / 16 pieces
WIDTHS = [
    ("bf16", 8),      # 1 piece
    ("bf16", 2048),   # 256: one held piece per thread, every thread
    ("bf16", 2056),   # 257: two held, the second on one thread only
    ("bf16", 4104),   # 513: four held, partly filled
    ("bf16", 8192),   # 1024: four held, full
    ("bf16", 8200),   # 1025: four held, then one piece copied after them
    ("f32", 4100),    # 1025 fp32 pieces
    ("f32", 9000),    # 2250: several rounds after the held pieces
]
# (N, E, K, W): fused table scan / scan kernel
ROUTINGS = [(300, 8, 2, 4), (2100, 128, 4, 8)]


def _np(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def _dispatch_reference(cfg, inp, idx, cap):
    ri, _ = O.route(_np(inp["logits"]), cfg["K"])
    assert np.array_equal(_np(idx), ri)
    return O.dispatch(ri, cfg["E"], cfg["W"], cap)


def _check_indices(out, ref):
    for k in ("demand", "counts", "offsets", "rank_offsets", "dest"):
        assert np.array_equal(_np(out[k]), ref[k]), k
    M = int(ref["offsets"][-1])
    assert np.array_equal(_np(out["perm_token"])[:M], ref["perm_token"])
    return M


# every width at 8 experts; at 128 experts (the scan kernel's path) only the
# rows up to 4104 elements, since the wide rows exercise the same copy loop
WIDTH_CASES = [
    pytest.param(act, d, C, routing, id=f"{act}_{d}-{cid}-{rid}")
    for act, d in WIDTHS
    for C, cid in ((None, "dropless"), (0.8, "c0.8"))
    for routing, rid in zip(ROUTINGS, ("e8", "e128"))
    if not (routing[1] == 128 and d > 4104)
]


@pytest.mark.parametrize("act,d,C,routing", WIDTH_CASES)
def test_dispatch_row_widths_match_oracle(act, d, C, routing):
    N, E, K, W = routing
    cfg = synth.config(f"width_{act}_{d}_{E}", N=N, d=d, ffn=64, E=E, K=K, W=W, act=act, C=C)
    print(f"[dispatch] {act} d={d} N={N} E={E} K={K} C={C}", flush=True)
    cap = O.capacity(C, N, K, E) if C is not None else -1
    inp = synth.make_inputs(cfg, DEV, weights=False)
    idx, _ = B.moe_route_topk(inp["logits"], K)
    out = B.moe_dispatch(inp["x"], idx, E, W, cap)
    torch.cuda.synchronize()
    ref = _dispatch_reference(cfg, inp, idx, cap)
    M = _check_indices(out, ref)
    perm = torch.from_numpy(ref["perm_token"].astype(np.int64)).to(DEV)
    assert torch.equal(out["x_perm"][:M], inp["x"][perm])      # bitwise row copies


# fp8 payload: d a multiple of 128; a row is d / 8 pieces of the bf16 row
FP8_WIDTHS = [128, 2048, 4224, 8320]   # 16, 256, 528 and 1040 pieces


@pytest.mark.parametrize("routing", ROUTINGS, ids=("e8", "e128"))
@pytest.mark.parametrize("d", FP8_WIDTHS)
def test_dispatch_fp8_row_widths_match_oracle(d, routing):
    N, E, K, W = routing
    cfg = synth.config(f"width_fp8_{d}_{E}", N=N, d=d, ffn=64, E=E, K=K, W=W, act="bf16",
                       C=0.8)
    print(f"[dispatch] fp8 d={d} N={N} E={E}", flush=True)
    cap = O.capacity(0.8, N, K, E)
    inp = synth.make_inputs(cfg, DEV, weights=False)
    idx, _ = B.moe_route_topk(inp["logits"], K)
    out = B.moe_dispatch_fp8(inp["x"], idx, E, W, cap)
    torch.cuda.synchronize()
    ref = _dispatch_reference(cfg, inp, idx, cap)
    M = _check_indices(out, ref)
    tq, ts = O.quantize_fp8(_np(inp["x"]))
    pt = ref["perm_token"].astype(np.int64)
    assert np.array_equal(_np(out["x8"])[:M], tq[pt])
    assert np.array_equal(_np(out["x_scale"])[:M], ts[pt])


# (N, E, K, W, C): the two paths at their edges (the scatter scans the
# per-block count table itself while it holds at most 1024 counts)
EDGE_ROUTINGS = [
    (4096, 8, 2, 8, None),     # 16 x 8 counts
    (4097, 8, 2, 8, None),     # a ragged last block of one token
    (6000, 4, 2, 2, 1.1),      # with a capacity
    (256, 16, 4, 4, None),     # one whole block
    (16384, 64, 8, 8, 0.9),    # 64 x 64 counts: the scan kernel
    (9000, 1, 1, 1, None),     # one expert
    (32768, 32, 4, 8, None),   # 128 x 32 = 4096 counts: the scan kernel
    (700, 1024, 16, 8, None),  # the largest expert count
]


@pytest.mark.parametrize("N,E,K,W,C", EDGE_ROUTINGS)
def test_dispatch_paths_match_oracle(N, E, K, W, C):
    cfg = synth.config(f"edge_{N}_{E}_{K}", N=N, d=64, ffn=64, E=E, K=K, W=W, act="bf16", C=C)
    print(f"[dispatch] edge N={N} E={E} K={K} W={W} C={C}", flush=True)
    cap = O.capacity(C, N, K, E) if C is not None else -1
    inp = synth.make_inputs(cfg, DEV, weights=False)
    idx, _ = B.moe_route_topk(inp["logits"], K)
    ref = _dispatch_reference(cfg, inp, idx, cap)
    out = None
    for _ in range(3):            # one workspace, three calls in a row
        out = B.moe_dispatch(inp["x"], idx, E, W, cap, out)
        torch.cuda.synchronize()
        M = _check_indices(out, ref)
        perm = torch.from_numpy(ref["perm_token"].astype(np.int64)).to(DEV)
        assert torch.equal(out["x_perm"][:M], inp["x"][perm])

"""Virtual multi-source exchange on the GPU vs the oracle: the plan (counts,
traffic matrix, row maps) bit for bit, the three row permutations against
the one-source dispatch, and the reverse direction through combine."""
import numpy as np
import pytest
import torch

from grouped_gemm_route_amd import binding as B
from grouped_gemm_route_amd import synth
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = {
    "small_w4": synth.config("ex_small_w4", N=300, d=64, ffn=64, E=8, K=2, W=4, act="bf16",
                             C=None),
    "skew_w8_c1": synth.config("ex_skew_w8", N=517, d=128, ffn=64, E=32, K=4, W=8,
                               act="bf16", bias="zipf", C=1.0),
    "tiny_f32_w4": synth.config("tiny_f32"),
    "w1": synth.config("ex_w1", N=64, d=64, ffn=64, E=4, K=2, W=1, act="bf16", C=None),
    "ragged_shards": synth.config("ex_ragged", N=13, d=64, ffn=64, E=16, K=3, W=16,
                                  act="bf16", C=None),
    "dense8": synth.config("dense8"),
    "prefill256_hot_c1.0": synth.config("prefill256_hot_c1.0"),
}


def _np(t):
    return t.detach().cpu().numpy()


@pytest.mark.parametrize("name", list(CASES))
def test_exchange_matches_oracle(name):
    cfg = CASES[name]
    print(f"[exchange] {name}", flush=True)
    N, d, E, K, W = (cfg[k] for k in ("N", "d", "E", "K", "W"))
    dt = synth.TORCH_DTYPE[cfg["act"]]
    inp = synth.make_inputs(cfg, DEV, weights=False)
    cap = O.capacity(cfg["C"], N, K, E) if cfg["C"] is not None else -1
    idx, w = B.moe_route_topk(inp["logits"], K)
    disp = B.moe_dispatch(inp["x"], idx, E, W, cap)
    plan = B.moe_exchange_plan(idx, disp, E, W)
    torch.cuda.synchronize()

    # the oracle's own route and dispatch feed its exchange plan; the GPU's
    # routing and dispatch must equal them first
    ri, _ = O.route(_np(inp["logits"]), K)
    rd = O.dispatch(ri, E, W, cap)
    assert np.array_equal(_np(idx), ri)
    assert np.array_equal(_np(disp["dest"]), rd["dest"])
    ex = O.exchange(ri, rd["dest"], E, W)
    M = int(rd["offsets"][-1])
    assert int(_np(disp["offsets"])[-1]) == M
    assert np.array_equal(_np(plan["src_counts"]), ex["C"])
    assert np.array_equal(_np(plan["traffic"]), ex["D"])
    assert np.array_equal(_np(plan["send_row"]), ex["send_row"])
    for k in ("send_token", "a2a_src", "regroup_src"):
        assert np.array_equal(_np(plan[k])[:M], ex[k]), k

    # forward: pack, all-to-all, regroup -> bit copy of the dispatch's x_perm
    n_rows = disp["offsets"][E:E + 1]
    send = torch.full((N * K, d), -1.0, dtype=dt, device=DEV)
    recv = torch.empty_like(send)
    regrouped = torch.empty_like(send)
    B.moe_rows_permute(inp["x"], send, plan["send_token"], n_rows)
    B.moe_rows_permute(send, recv, plan["a2a_src"], n_rows)
    B.moe_rows_permute(recv, regrouped, plan["regroup_src"], n_rows)
    torch.cuda.synchronize()
    st = torch.from_numpy(ex["send_token"].astype(np.int64)).to(DEV)
    assert torch.equal(send[:M], inp["x"][st])
    assert torch.equal(regrouped[:M], disp["x_perm"][:M])
    assert bool((send[M:] == -1).all())          # rows past M untouched

    # reverse: the same maps as scatters bring rows back to the send layout;
    # combining there with send_row gives the one-source combine bit for bit
    y = torch.randn(N * K, d, device=DEV).to(dt)
    recv_y = torch.empty_like(y)
    send_y = torch.empty_like(y)
    B.moe_rows_permute(y, recv_y, plan["regroup_src"], n_rows, scatter=True)
    B.moe_rows_permute(recv_y, send_y, plan["a2a_src"], n_rows, scatter=True)
    out_a = B.moe_combine(y, disp["dest"], w)
    out_b = B.moe_combine(send_y, plan["send_row"], w)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)
    # Aurora's lower bound from the traffic matrix, in rows
    tau = O.tau_min(_np(plan["traffic"]))
    assert tau <= M
    print(f"[exchange] {name}: M={M} tau_min={tau:.0f} rows "
          f"cross-rank={1 - np.trace(ex['D']) / max(M, 1):.3f}", flush=True)

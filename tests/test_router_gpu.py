"""Router projection on the GPU vs the oracle: logits within the fp32
summation bound of the exact sums; Top-K on the GPU's logits bit-exact with
the oracle's route of those logits, and equal to the route of the exact
logits wherever the K-th / (K+1)-th gap exceeds twice the bound."""
import numpy as np
import pytest
import torch

from grouped_gemm_route_amd import binding as B
from grouped_gemm_route_amd import synth
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = {
    "tiny_f32": (synth.config("tiny_f32"), None),
    "dense8": (synth.config("dense8"), 512),
    "fine128": (synth.config("fine128_zipf_c1.25"), 512),
    "decode256": (synth.config("decode256"), None),
    "prefill256": (synth.config("prefill256_hot"), 256),
    "ragged_n_e": (synth.config("rt_ragged", N=333, d=192, ffn=64, E=70, K=3, W=2,
                                act="bf16"), None),
    "e1024": (synth.config("rt_e1024", N=97, d=128, ffn=64, E=1024, K=16, W=8, act="bf16"),
              None),
    # the skinny kernel (up to 64 experts per block): every expert-tile count,
    # token counts off the 16-token block, and d a multiple of 8 but not of
    # 64 or 32 (the last step of a row is partly past its end), also with
    # more than 64 experts (two expert groups)
    "skinny_e3_d200": (synth.config("rt_sk1", N=45, d=200, ffn=64, E=3, K=2, W=1, act="bf16"),
                       None),
    "skinny_e20_d72": (synth.config("rt_sk2", N=130, d=72, ffn=64, E=20, K=4, W=4, act="bf16"),
                       None),
    "skinny_e64_d1000": (synth.config("rt_sk4", N=77, d=1000, ffn=64, E=64, K=8, W=8,
                                      act="bf16"), None),
    "skinny_e70_d200": (synth.config("rt_sk70", N=50, d=200, ffn=64, E=70, K=6, W=2,
                                     act="bf16"), None),
    "skinny_e8_d8": (synth.config("rt_sk_d8", N=33, d=8, ffn=64, E=8, K=2, W=2, act="bf16"),
                     None),
    # the tiled kernel: 128 x 256 tiles with the last token block and the
    # expert tile ragged (E not a multiple of 4: scalar stores), and with two
    # expert blocks and a single 64-wide stage; 64 x 64 tiles with ragged
    # tokens and experts
    "tiled_big_ragged": (synth.config("rt_tb", N=16001, d=192, ffn=64, E=250, K=8, W=2,
                                      act="bf16"), None),
    "tiled_big_e260_d64": (synth.config("rt_tb2", N=20000, d=64, ffn=64, E=260, K=4, W=4,
                                        act="bf16"), None),
    "tiled_small_ragged": (synth.config("rt_ts", N=2500, d=320, ffn=64, E=130, K=8, W=2,
                                        act="bf16"), None),
    # few tokens and many experts: the skinny kernel on blocks of 2 and of 4
    # experts, the last block ragged
    "skinny_epb2": (synth.config("rt_e2", N=20, d=256, ffn=64, E=130, K=8, W=2, act="bf16"),
                    None),
    "skinny_epb4": (synth.config("rt_e4", N=40, d=256, ffn=64, E=202, K=8, W=2, act="bf16"),
                    None),
}


def _np(t):
    return (t.float() if t.dtype == torch.bfloat16 else t).detach().cpu().numpy()


@pytest.mark.parametrize("name", list(CASES))
def test_router_logits_and_route(name):
    cfg, sample = CASES[name]
    print(f"[router] {name}", flush=True)
    x = synth.make_x(cfg, DEV)
    wr = synth.make_router(cfg, DEV)
    logits = B.moe_router_logits(x, wr)
    idx, w = B.moe_route_topk(logits, cfg["K"])
    torch.cuda.synchronize()
    N = cfg["N"]
    rows = np.arange(N) if sample is None else np.unique(
        np.concatenate([[0, N - 1], np.random.default_rng(1).choice(N, sample, replace=False)]))
    xs = _np(x)[rows]
    wn = _np(wr)
    exact = xs.astype(np.float64) @ wn.astype(np.float64).T
    got = _np(logits)[rows].astype(np.float64)
    bound = O.router_logits_error_bound(xs, wn)
    assert (np.abs(got - exact) <= bound).all(), float((np.abs(got - exact) - bound).max())
    ref32 = O.router_logits(xs, wn)
    assert (np.abs(got - ref32) <= bound + np.abs(ref32) * 2.0 ** -24).all()
    # route of the GPU's logits: bit-exact with the oracle's route of them
    gi, gw = O.route(_np(logits)[rows], cfg["K"])
    assert np.array_equal(_np(idx)[rows], gi)
    assert np.abs(_np(w)[rows] - gw).max() <= 1e-6
    # where the exact top-K is separated by more than the error, it is the same
    ei, _ = O.route(ref32, cfg["K"])
    srt = -np.sort(-exact, axis=1)
    K, E = cfg["K"], cfg["E"]
    if K < E:
        gap = srt[:, K - 1] - srt[:, K]
        clear = gap > 2 * bound.max(axis=1)
        assert clear.any()  # the check below must cover some tokens
        assert np.array_equal(np.sort(_np(idx)[rows][clear], 1), np.sort(ei[clear], 1))
    print(f"[router] {name}: rows checked {len(rows)} max err {np.abs(got - exact).max():.3e}",
          flush=True)


@pytest.mark.parametrize("name", ["dense8", "fine128", "decode256", "tiled_big_ragged",
                                  "skinny_epb4"])
def test_router_logits_bitwise_repeatable(name):
    """Two calls on the same inputs give the same bits (the split-reduction
    waves and the skinny kernel's partial tiles meet in a fixed order)."""
    cfg, _ = CASES[name]
    print(f"[router repeat] {name}", flush=True)
    x = synth.make_x(cfg, DEV)
    wr = synth.make_router(cfg, DEV)
    a = B.moe_router_logits(x, wr)
    b = B.moe_router_logits(x, wr)
    torch.cuda.synchronize()
    assert torch.equal(a, b)

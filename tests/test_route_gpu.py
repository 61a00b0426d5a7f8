"""moe_route_topk on every lane-group shape of the routing kernel (groups of
8 or 16 lanes per token, 1 to 64 logits per lane), on logits drawn
from a few values so that most rounds end in ties, with -0.0 beside +0.0:
expert ids bit-exact against the oracle (lowest index among equal logits),
weights within 1e-6, for the softmax and the sigmoid gate, raw and
renormalised.  A ragged last wave (N not a multiple of the groups per wave)
is in every case."""
import numpy as np
import pytest
import torch

from grouped_gemm_route_amd import binding as B
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
W_TOL = 1e-6

# E: one or more per kernel shape (8 lanes x 1 logit; 16 lanes x 1, 2, 4, 8,
# 16, 32, 64 logits) with padded lanes (E below the shape's capacity)
SHAPES = [3, 8, 13, 16, 24, 32, 50, 64, 100, 128, 200, 256, 300, 512, 1000, 1024]


def _tied_logits(N, E, seed):
    g = torch.Generator().manual_seed(seed)
    vals = torch.tensor([-1.5, -0.0, 0.0, 0.25, 1.0, 2.0])
    return vals[torch.randint(0, len(vals), (N, E), generator=g)]


@pytest.mark.parametrize("E", SHAPES)
@pytest.mark.parametrize("gate", ["softmax", "sigmoid"])
def test_route_ties_every_group_shape(E, gate):
    for K, renorm in sorted({(1, False), (min(E, 2), True), (min(E, 16), False)}):
        N = 333
        print(f"[route] E={E} K={K} gate={gate} renorm={renorm}", flush=True)
        l = _tied_logits(N, E, 1000 * E + K)
        l[5] = 0.0                       # one token of all-equal logits
        idx, w = B.moe_route_topk(l.to(DEV), K, renorm, gate=gate)
        torch.cuda.synchronize()
        ri, rw = O.route(l.numpy(), K, renorm, gate=gate)
        assert np.array_equal(idx.cpu().numpy(), ri), (E, K, gate, renorm)
        err = np.abs(w.cpu().numpy().astype(np.float64) - rw).max()
        assert err <= W_TOL, (E, K, gate, renorm, err)
        # the all-equal token takes experts 0 .. K - 1
        assert np.array_equal(ri[5], np.arange(K))


@pytest.mark.parametrize("E,K", [(8, 2), (64, 6), (256, 8), (1024, 16)])
def test_sigmoid_renormalised_far_negative_logits(E, K):
    # Every chosen logit far below zero: the plain fp32 sigmoid scores round
    # to 0 (below about -103.9) or come out subnormal, yet the renormalised
    # weights are finite ratios that the float64 oracle gives exactly.
    N = 97
    g = torch.Generator().manual_seed(E + K)
    l = -100.0 - 30.0 * torch.rand(N, E, generator=g)
    l[3] = -120.0                    # all-equal token: K equal weights 1/K
    l[4, :K] = -90.0 - torch.arange(K, dtype=torch.float32)
    idx, w = B.moe_route_topk(l.to(DEV), K, True, gate="sigmoid")
    torch.cuda.synchronize()
    ri, rw = O.route(l.numpy(), K, True, gate="sigmoid")
    assert np.array_equal(idx.cpu().numpy(), ri)
    got = w.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    assert np.abs(got - rw).max() <= W_TOL
    assert np.abs(got[3] - 1.0 / K).max() <= W_TOL

"""Pins of the oracle's virtual multi-source exchange and tau_min."""
import itertools

import numpy as np
import pytest

from oracle import moe_oracle as O


def _layer_ids(seed, N, E, K, W, cap_C=None, bias=0.0):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((N, E)).astype(np.float32)
    logits[:, 0] += bias
    idx, w = O.route(logits, K)
    cap = -1 if cap_C is None else O.capacity(cap_C, N, K, E)
    disp = O.dispatch(idx, E, W, cap)
    return idx, w, disp


@pytest.mark.parametrize("N,E,K,W,C,bias", [(40, 8, 2, 4, None, 0.0), (33, 12, 3, 3, 1.0, 1.5),
                                            (7, 4, 2, 4, None, 0.0), (50, 16, 4, 8, 0.75, 2.0),
                                            (1, 8, 2, 2, None, 0.0)])
def test_exchange_composes_to_the_one_source_dispatch(N, E, K, W, C, bias):
    idx, _, disp = _layer_ids(N * 7 + E, N, E, K, W, C, bias)
    ex = O.exchange(idx, disp["dest"], E, W)
    M = int(disp["offsets"][-1])
    # pack, all-to-all and regroup, applied to token ids, give the dispatch's
    # token order row by row (an independent construction of the same layout)
    send = ex["send_token"]
    recv = send[ex["a2a_src"]]
    regrouped = recv[ex["regroup_src"]]
    assert len(send) == len(recv) == len(regrouped) == M
    assert np.array_equal(regrouped, disp["perm_token"])
    # send_row is consistent with send_token
    for t in range(N):
        for k in range(K):
            q = ex["send_row"][t, k]
            assert (q >= 0) == (disp["dest"][t, k] >= 0)
            if q >= 0:
                assert send[q] == t
    # every map is a permutation of [0, M)
    for key in ("a2a_src", "regroup_src"):
        assert sorted(ex[key].tolist()) == list(range(M))


def test_traffic_matrix_sums():
    N, E, K, W = 64, 16, 4, 4
    idx, _, disp = _layer_ids(3, N, E, K, W, 1.0, 1.0)
    ex = O.exchange(idx, disp["dest"], E, W)
    C, D = ex["C"], ex["D"]
    lo = O.shard_bounds(N, W)
    # C by brute force over pairs
    for s in range(W):
        for e in range(E):
            n = sum(1 for t in range(lo[s], lo[s + 1]) for k in range(K)
                    if idx[t, k] == e and disp["dest"][t, k] >= 0)
            assert C[s, e] == n
    assert np.array_equal(C.sum(axis=0), disp["counts"])            # per expert
    assert np.array_equal(D.sum(axis=0), np.diff(disp["rank_offsets"]))  # received per rank
    kept_per_shard = [int((disp["dest"][lo[s]:lo[s + 1]] >= 0).sum()) for s in range(W)]
    assert D.sum(axis=1).tolist() == kept_per_shard                 # sent per source
    assert D.sum() == disp["offsets"][-1]


def test_send_buffer_is_rank_major_per_source():
    N, E, K, W = 30, 8, 2, 4
    idx, _, disp = _layer_ids(5, N, E, K, W)
    ex = O.exchange(idx, disp["dest"], E, W)
    # in the send buffer, each source's rows are grouped by destination rank
    lo = O.shard_bounds(N, W)
    send = ex["send_token"]
    start = 0
    for s in range(W):
        n = int(ex["D"][s].sum())
        toks = send[start:start + n]
        assert all(lo[s] <= t < lo[s + 1] for t in toks)
        start += n


def test_shards():
    assert O.shard_bounds(10, 4) == [0, 2, 5, 7, 10]
    assert O.shard_bounds(3, 4) == [0, 0, 1, 2, 3]


def test_tau_min_closed_forms():
    # Theorem 4.2: max over the busiest sender / receiver, off-diagonal only
    D = np.array([[5, 1, 2], [0, 9, 4], [3, 3, 1]])
    # off-diagonal row sums 3, 4, 6; column sums 3, 4, 6
    assert O.tau_min(D, 2.0) == 3.0
    D2 = np.array([[0, 10], [1, 0]])
    assert O.tau_min(D2) == 10.0
    # uniform all-to-all of x rows per pair: (W-1) x per GPU
    W, x = 8, 7
    assert O.tau_min(np.full((W, W), x)) == (W - 1) * x
    # brute force on small matrices: the bound equals the slowest port
    rng = np.random.default_rng(1)
    for _ in range(20):
        D = rng.integers(0, 9, size=(4, 4))
        ports = [sum(D[i, j] for j in range(4) if j != i) for i in range(4)] + \
                [sum(D[i, j] for i in range(4) if i != j) for j in range(4)]
        assert O.tau_min(D) == max(ports)

"""Pins of the oracle's routing variants: the sigmoid gate and the one-round
re-route of capacity overflow.  None of these reuses the oracle's code:
library routines, closed forms, a hand-worked fixture and an independent
brute-force restatement built from Python sets and sorted lists."""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit, softmax

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# sigmoid gate
# --------------------------------------------------------------------------

def test_sigmoid_scores_match_library():
    rng = np.random.default_rng(3)
    l = (rng.standard_normal((50, 40)) * 6).astype(np.float32)
    l[0, :5] = [0.0, -80.0, 80.0, 1e-8, -1e-8]
    got = O.gate_scores(l, "sigmoid")
    ref = expit(l.astype(np.float64))
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-300)
    # the softmax gate against the library softmax
    assert np.allclose(O.gate_scores(l, "softmax"), softmax(l.astype(np.float64), axis=1),
                       rtol=1e-12, atol=1e-300)


def test_sigmoid_route_special_cases():
    N, E, K = 7, 9, 3
    idx, w = O.route(np.zeros((N, E), np.float32), K, gate="sigmoid")
    assert (idx == np.arange(K)).all()            # ties -> lowest indices
    assert (w == np.float32(0.5)).all()           # sigmoid(0) = 1/2
    _, w = O.route(np.zeros((N, E), np.float32), K, renormalize=True, gate="sigmoid")
    assert np.allclose(w, 1.0 / K, rtol=0, atol=1e-7)
    rng = np.random.default_rng(4)
    l = rng.standard_normal((30, E)).astype(np.float32)
    i_sig, w_sig = O.route(l, K, gate="sigmoid")
    i_soft, _ = O.route(l, K)
    assert np.array_equal(i_sig, i_soft)          # both gates rise with the logit
    _, w_neg = O.route(-l, E, gate="sigmoid")
    i_all, w_all = O.route(l, E, gate="sigmoid")
    # sigma(x) + sigma(-x) = 1, expert by expert
    s_pos = np.zeros((30, E)); s_neg = np.zeros((30, E))
    np.put_along_axis(s_pos, i_all.astype(np.int64), w_all.astype(np.float64), 1)
    i_neg, _ = O.route(-l, E, gate="sigmoid")
    np.put_along_axis(s_neg, i_neg.astype(np.int64), w_neg.astype(np.float64), 1)
    assert np.allclose(s_pos + s_neg, 1.0, atol=2e-7)


# --------------------------------------------------------------------------
# re-route: hand example
# --------------------------------------------------------------------------

def test_reroute_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "reroute_hand.json")))
    l = np.array(g["logits"], np.float32)
    idx, _ = O.route(l, g["K"])
    assert idx.tolist() == g["route_topk_idx"]
    for gate, key in (("softmax", "t1_slot1_weight_softmax_7dp"),
                      ("sigmoid", "t1_slot1_weight_sigmoid_7dp")):
        ni, nw, rr = O.reroute_overflow(l, idx, g["capacity"], gate=gate)
        assert ni.tolist() == g["reroute_topk_idx"]
        assert rr.tolist() == g["rerouted"]
        assert round(float(nw[1, 1]), 7) == g[key]
        # untouched slots keep route()'s weights
        _, w0 = O.route(l, g["K"], gate=gate)
        mask = np.ones_like(nw, bool)
        mask[1, 1] = False
        assert np.array_equal(nw[mask], w0[mask])
    d = O.dispatch(ni, g["E"], g["W"], g["capacity"])
    a = g["after_dispatch"]
    assert d["demand"].tolist() == a["demand"]
    assert d["counts"].tolist() == a["counts"]
    assert d["dest"].tolist() == a["dest"]
    assert d["dropped"] == a["dropped"]
    assert O.dispatch(idx, g["E"], g["W"], g["capacity"])["dropped"] == a["dropped_without_reroute"]


# --------------------------------------------------------------------------
# re-route: closed forms and no-op cases
# --------------------------------------------------------------------------

@pytest.mark.parametrize("N,cap,K,E", [(10, 3, 2, 6), (10, 7, 2, 4), (5, 9, 3, 8),
                                       (12, 4, 3, 6), (9, 2, 1, 5), (6, 0, 2, 5)])
def test_reroute_uniform_closed_form(N, cap, K, E):
    # Equal logits: every token ranks the experts 0, 1, 2, ... so all take
    # 0..K-1, and each token t >= cap overflows in every slot; slot k is
    # offered expert K + k (if it exists), which admits the first cap of them.
    l = np.zeros((N, E), np.float32)
    idx, _ = O.route(l, K)
    ni, _, rr = O.reroute_overflow(l, idx, cap)
    over = max(N - cap, 0)
    n_alt = min(K, E - K)                     # slots that have an alternative
    want = np.zeros(E, np.int64)
    want[K:K + n_alt] = min(over, cap)
    assert np.array_equal(rr, want)
    kept = O.dispatch(ni, E, 1, cap)["counts"].sum()
    assert kept == K * min(N, cap) + n_alt * min(over, cap)


def test_reroute_is_a_no_op_without_overflow():
    rng = np.random.default_rng(5)
    l = rng.standard_normal((40, 8)).astype(np.float32)
    idx, w = O.route(l, 3)
    demand = np.bincount(idx.ravel(), minlength=8)
    for cap in (-1, int(demand.max()), int(demand.max()) + 5):
        ni, nw, rr = O.reroute_overflow(l, idx, cap)
        assert np.array_equal(ni, idx) and np.array_equal(nw, w) and rr.sum() == 0
    # K == E: no expert outside the token's own top K
    idx, w = O.route(l, 8)
    ni, _, rr = O.reroute_overflow(l, idx, 2)
    assert np.array_equal(ni, idx) and rr.sum() == 0


# --------------------------------------------------------------------------
# re-route: brute force
# --------------------------------------------------------------------------

def _brute_reroute(l, idx, cap):
    """Restates the re-route with sets and sorted lists."""
    N, E = l.shape
    K = idx.shape[1]
    pairs = [(t, k, int(idx[t, k])) for t in range(N) for k in range(K)]
    survivors = {e: [] for e in range(E)}
    overflow = []
    for t, k, e in pairs:                     # (t, k) order
        if len(survivors[e]) < cap:
            survivors[e].append(t)
        else:
            overflow.append((t, k))
    room = {e: cap - len(survivors[e]) for e in range(E)}
    new = idx.astype(np.int64).copy()
    got = np.zeros(E, np.int64)
    per_token = {}
    for t, k in overflow:
        per_token.setdefault(t, []).append(k)
    for t in sorted(per_token):
        ranking = sorted(range(E), key=lambda e: (-float(l[t, e]), e))
        outside = [e for e in ranking if e not in set(idx[t].tolist())]
        for j, k in enumerate(per_token[t]):
            if j < len(outside) and room[outside[j]] > 0:
                room[outside[j]] -= 1
                got[outside[j]] += 1
                new[t, k] = outside[j]
    return new, got


@pytest.mark.parametrize("seed", range(12))
def test_reroute_against_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    N = int(rng.integers(1, 40))
    E = int(rng.integers(2, 12))
    K = int(rng.integers(1, E + 1))
    # small integer logits make ties common
    l = rng.integers(-3, 4, size=(N, E)).astype(np.float32)
    idx, _ = O.route(l, K)
    cap = int(rng.integers(0, max(2, N * K // E + 2)))
    ni, nw, rr = O.reroute_overflow(l, idx, cap)
    bi, bg = _brute_reroute(l, idx, cap)
    assert np.array_equal(ni, bi)
    assert np.array_equal(rr, bg)
    # invariants of the re-routed layout
    for t in range(N):
        assert len(set(ni[t].tolist())) == K   # distinct experts per token
    moved = ni != idx
    for t, k in zip(*np.nonzero(moved)):
        assert ni[t, k] not in idx[t]            # a new expert, outside its top K
    d_new = O.dispatch(ni, E, 1, cap)
    d_old = O.dispatch(idx, E, 1, cap)
    assert (d_new["counts"] <= cap).all()
    assert d_new["counts"].sum() == d_old["counts"].sum() + rr.sum()
    assert (d_new["dest"][moved] >= 0).all()     # every admitted slot is kept
    scores = O.gate_scores(l)
    for t, k in zip(*np.nonzero(moved)):
        assert math.isclose(float(nw[t, k]), float(np.float32(scores[t, ni[t, k]])),
                            rel_tol=0, abs_tol=0)

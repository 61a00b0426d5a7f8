"""Pins for the CPU oracle, checked against things other than itself.

Each test re-derives a result by an independent route: brute force over
expert subsets, a dense every-expert-for-every-token recompute (the O(S*E*M)
"sparse einsum" form that "MoE Inference Communication", section
"MoE 计算核优化", replaces by a mapping table), closed forms, invariants,
a hand-worked 4-token example, and library routines (torch's bf16 cast,
torch's SiLU).
"""
import math
import itertools

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O


# --------------------------------------------------------------------------
# bf16 storage rounding
# --------------------------------------------------------------------------

def test_round_bf16_matches_torch_cast_on_fp32_values():
    rng = np.random.default_rng(1)
    parts = [
        rng.standard_normal(200000).astype(np.float32) * np.float32(7.0),
        (rng.standard_normal(20000) * 1e-39).astype(np.float32),   # subnormal
        (rng.standard_normal(20000) * 1e37).astype(np.float32),
    ]
    a = np.concatenate(parts)
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(a.astype(np.float64))
    assert np.array_equal(got, ref)


def test_round_bf16_closed_forms():
    one = 1.0
    ulp = 2.0 ** -7                       # bf16 spacing in [1, 2)
    cases = {
        one + ulp / 2: one,               # tie -> even (1.0)
        one + 3 * ulp / 2: one + 2 * ulp,  # tie -> even (mantissa ...10)
        one + ulp / 2 + 2.0 ** -30: one + ulp,   # above the tie: up
        -(one + ulp / 2): -one,
        2.0 ** -133 * 0.5: 0.0,           # half the smallest subnormal, tie -> 0
        2.0 ** -133 * 1.5: 2.0 ** -132,   # tie -> even
        3.3895313892515355e38: 3.3895313892515355e38,   # largest bf16
        3.4e38: math.inf,
    }
    got = O.round_bf16(np.array(list(cases.keys())))
    assert np.array_equal(got, np.array(list(cases.values())))
    # A value just above 2**-126 * 1.5 rounds within the normal range; the
    # sign of zero is kept.
    z = O.round_bf16(np.array([-0.0]))
    assert z[0] == 0.0 and math.copysign(1.0, z[0]) == -1.0


# --------------------------------------------------------------------------
# capacity
# --------------------------------------------------------------------------

def test_capacity_values():
    assert O.capacity(1.25, 8192, 8, 128) == 640
    assert O.capacity(1.0, 32768, 8, 256) == 1024
    assert O.capacity(1.0, 4, 2, 4) == 2
    assert O.capacity(None, 10, 2, 4) == -1
    # exact rational arithmetic on the double C: the double nearest 1.1 is
    # slightly above 1.1, and the double just above 1.0 rounds 1024 up.
    assert O.capacity(1.1, 10, 1, 1) == 12        # 11.000000000000000888 -> 12
    assert O.capacity(float(np.nextafter(1.0, 2.0)), 1024, 1, 1) == 1025
    assert O.capacity(0.5, 3, 1, 1) == 2          # 1.5 -> 2
    with pytest.raises(ValueError):
        O.capacity(0.0, 1, 1, 1)
    with pytest.raises(ValueError):
        O.capacity(float("nan"), 1, 1, 1)


# --------------------------------------------------------------------------
# route
# --------------------------------------------------------------------------

def _beats(la, a, lb, b):
    return la > lb or (la == lb and a < b)


def _brute_topk(row, K):
    """The unique K-subset every member of which beats every non-member,
    listed best first -- found by trying every subset."""
    E = len(row)
    for S in itertools.combinations(range(E), K):
        rest = [e for e in range(E) if e not in S]
        if all(_beats(row[a], a, row[b], b) for a in S for b in rest):
            # order the subset by pairwise wins
            return sorted(S, key=lambda a: -sum(_beats(row[a], a, row[b], b) for b in S))
    raise AssertionError("no dominating subset")


def _softmax_closed_form(row):
    m = max(row)
    den = math.fsum(math.exp(v - m) for v in row)
    return [math.exp(v - m) / den for v in row]


@pytest.mark.parametrize("E,K", [(4, 2), (6, 3), (8, 2), (5, 5), (7, 1)])
def test_route_against_brute_force(E, K):
    rng = np.random.default_rng(E * 10 + K)
    # quantised logits so that ties are common
    logits = (rng.integers(-3, 4, size=(60, E)) * 0.5).astype(np.float32)
    logits[::7] = 0.0                         # all-tie rows
    logits[1::11, :] = -0.0                   # negative zeros tie with zeros
    idx, w = O.route(logits, K)
    for t in range(logits.shape[0]):
        row = [float(v) for v in logits[t]]
        assert list(idx[t]) == _brute_topk(row, K)
        p = _softmax_closed_form(row)
        for k in range(K):
            assert abs(float(w[t, k]) - p[idx[t, k]]) <= 1e-7


def test_route_special_cases():
    N, E, K = 9, 16, 4
    idx, w = O.route(np.zeros((N, E), np.float32), K)      # uniform logits
    assert (idx == np.arange(K)).all()
    assert np.array_equal(w, np.full((N, K), 1.0 / E, np.float32))
    idx, w = O.route(np.full((5, 1), 3.25, np.float32), 1)  # E = 1
    assert (idx == 0).all() and (w == 1.0).all()
    rng = np.random.default_rng(3)
    l = rng.standard_normal((7, 6)).astype(np.float32)
    idx, w = O.route(l, 6)                                  # K = E
    assert (np.diff(np.take_along_axis(l, idx.astype(np.int64), 1), axis=1) <= 0).all()
    assert np.allclose(w.astype(np.float64).sum(1), 1.0, atol=1e-6)
    idx, w = O.route(l, 3, renormalize=True)
    assert np.allclose(w.astype(np.float64).sum(1), 1.0, atol=1e-6)
    with pytest.raises(ValueError):
        O.route(np.array([[np.nan, 0.0]], np.float32), 1)


# --------------------------------------------------------------------------
# dispatch
# --------------------------------------------------------------------------

def _brute_dispatch(idx, E, W, cap):
    """kept(t,e) <=> e in topk(t) and #{t' < t : e in topk(t')} < cap, via a
    dense [N, E] membership matrix and a running count down the tokens."""
    N, K = idx.shape
    member = np.zeros((N, E), dtype=np.int64)
    for t in range(N):
        member[t, idx[t]] = 1
    before = np.cumsum(member, axis=0) - member          # tokens t' < t on e
    kept = member.astype(bool)
    if cap >= 0:
        kept &= before < cap
    counts = kept.sum(axis=0)
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + int(c))
    row = np.full((N, E), -1)
    for e in range(E):
        ts = np.nonzero(kept[:, e])[0]
        row[ts, e] = offsets[e] + np.arange(len(ts))
    dest = np.array([[row[t, idx[t, k]] for k in range(K)] for t in range(N)])
    return member.sum(0), counts, np.array(offsets), dest


@pytest.mark.parametrize("cap", [-1, 0, 1, 3, 7, 1000])
def test_dispatch_against_brute_force(cap):
    rng = np.random.default_rng(cap + 5)
    N, E, K, W = 40, 8, 3, 4
    logits = rng.standard_normal((N, E)).astype(np.float32)
    logits[:, 2] += 1.5                                  # a hot expert
    idx, _ = O.route(logits, K)
    r = O.dispatch(idx, E, W, cap)
    demand, counts, offsets, dest = _brute_dispatch(idx, E, W, cap)
    assert np.array_equal(r["demand"], demand)
    assert np.array_equal(r["counts"], counts)
    assert np.array_equal(r["offsets"], offsets)
    assert np.array_equal(r["rank_offsets"], offsets[::E // W])
    assert np.array_equal(r["dest"], dest)
    M = int(offsets[-1])
    # invariants: sum(counts) = N*K - dropped; counts = min(demand, cap);
    # perm is a bijection onto [0, M) and inverts dest; rows ascend in t
    dropped = int(np.maximum(0, demand - cap).sum()) if cap >= 0 else 0
    assert M == N * K - dropped == N * K - r["dropped"]
    if cap >= 0:
        assert np.array_equal(r["counts"], np.minimum(demand, cap))
    kept_rows = r["dest"][r["dest"] >= 0]
    assert sorted(kept_rows.tolist()) == list(range(M))
    for t in range(N):
        for k in range(K):
            if r["dest"][t, k] >= 0:
                assert r["perm_token"][r["dest"][t, k]] == t
    for e in range(E):
        seg = r["perm_token"][offsets[e]:offsets[e + 1]]
        assert (np.diff(seg) > 0).all()


def test_dispatch_closed_forms():
    N, E, K, W = 30, 8, 3, 2
    idx, _ = O.route(np.zeros((N, E), np.float32), K)    # uniform logits
    for cap in (-1, 0, 5, 30, 31):
        r = O.dispatch(idx, E, W, cap)
        c = N if cap < 0 else min(N, cap)
        assert r["counts"].tolist() == [c] * K + [0] * (E - K)
        assert r["dropped"] == K * (N - c)
    r0 = O.dispatch(idx, E, W, 0)
    assert r0["offsets"][-1] == 0 and (r0["dest"] == -1).all()
    # cap >= max demand reproduces the dropless result exactly
    rng = np.random.default_rng(9)
    idx, _ = O.route(rng.standard_normal((50, E)).astype(np.float32), K)
    a = O.dispatch(idx, E, W, -1)
    b = O.dispatch(idx, E, W, int(a["demand"].max()))
    for key in ("counts", "offsets", "rank_offsets", "dest", "perm_token"):
        assert np.array_equal(a[key], b[key])


# --------------------------------------------------------------------------
# FFN and combine
# --------------------------------------------------------------------------

def _rand_weights(rng, E, d, ffn):
    wg = rng.standard_normal((E, ffn, d)) / math.sqrt(d)
    wu = rng.standard_normal((E, ffn, d)) / math.sqrt(d)
    wd = rng.standard_normal((E, d, ffn)) / math.sqrt(ffn)
    return wg, wu, wd


def _dense_every_expert(x, wg, wu, wd):
    """Every expert applied to every token: [N, E, d], float64."""
    G = np.einsum("nd,efd->nef", x, wg)
    U = np.einsum("nd,efd->nef", x, wu)
    H = G / (1.0 + np.exp(-G)) * U
    return np.einsum("nef,edf->ned", H, wd)


@pytest.mark.parametrize("cap", [-1, 2, 0])
def test_layer_against_dense_masked_recompute(cap):
    rng = np.random.default_rng(11 + cap)
    N, E, K, W, d, ffn = 24, 6, 2, 3, 8, 16
    logits = rng.standard_normal((N, E)).astype(np.float32)
    logits[:, 4] += 1.0
    x = rng.standard_normal((N, d))
    wg, wu, wd = _rand_weights(rng, E, d, ffn)
    res = O.layer(logits, x, lambda e: (wg[e], wu[e], wd[e]), K, W, cap, "f64")
    Y = _dense_every_expert(x, wg, wu, wd)
    # mask with kept * gate weight
    _, counts, _, dest = _brute_dispatch(res["topk_idx"], E, W, cap)
    mask = np.zeros((N, E))
    for t in range(N):
        for k in range(K):
            if dest[t, k] >= 0:
                mask[t, res["topk_idx"][t, k]] = float(res["topk_w"][t, k])
    ref = np.einsum("ne,ned->nd", mask, Y)
    assert np.allclose(res["out"], ref, rtol=1e-12, atol=1e-12)
    for t in range(N):
        for k in range(K):
            row = res["dest"][t, k]
            if row >= 0:
                e = res["topk_idx"][t, k]
                assert np.allclose(res["y_perm"][row], Y[t, e], rtol=1e-12, atol=1e-12)
    if cap == 0:
        assert (res["out"] == 0).all()


def test_single_expert_is_textbook_swiglu():
    rng = np.random.default_rng(5)
    N, d, ffn = 10, 16, 32
    x = rng.standard_normal((N, d))
    wg, wu, wd = _rand_weights(rng, 1, d, ffn)
    res = O.layer(np.zeros((N, 1), np.float32), x,
                  lambda e: (wg[e], wu[e], wd[e]), 1, 1, -1, "f64")
    xt = torch.from_numpy(x)
    ref = (torch.nn.functional.silu(xt @ torch.from_numpy(wg[0]).T)
           * (xt @ torch.from_numpy(wu[0]).T)) @ torch.from_numpy(wd[0]).T
    assert np.allclose(res["out"], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_dispatch_then_combine_with_identity_ffn_is_identity():
    rng = np.random.default_rng(21)
    N, E, K, W, d = 33, 8, 3, 4, 5
    idx, _ = O.route(rng.standard_normal((N, E)).astype(np.float32), K)
    x = O.round_bf16(rng.standard_normal((N, d)))
    onehot = np.zeros((N, K), np.float32)
    onehot[:, 0] = 1.0
    for cap in (-1, 4):
        r = O.dispatch(idx, E, W, cap)
        xp = O.pack(x, r["perm_token"])
        out = O.combine(xp, r["dest"], onehot, "bf16")
        kept0 = r["dest"][:, 0] >= 0
        assert np.array_equal(out[kept0], x[kept0])      # bitwise
        assert (out[~kept0] == 0).all()
        if cap < 0:
            assert kept0.all()


def test_token_outputs_equal_full_layer_rows():
    rng = np.random.default_rng(8)
    N, E, K, W, d, ffn = 20, 4, 2, 2, 8, 8
    logits = rng.standard_normal((N, E)).astype(np.float32)
    x = O.round_bf16(rng.standard_normal((N, d)))
    wg, wu, wd = (O.round_bf16(a) for a in _rand_weights(rng, E, d, ffn))
    fn = lambda e: (wg[e], wu[e], wd[e])
    full = O.layer(logits, x, fn, K, W, 6, "bf16")
    toks = [0, 3, 7, 19]
    y_rows, out = O.token_outputs(toks, x[toks], full["topk_idx"], full["topk_w"],
                                  full["dest"], fn, "bf16")
    assert np.array_equal(out, full["out"][toks])
    for (t, k), y in y_rows.items():
        assert np.array_equal(y, full["y_perm"][full["dest"][t, k]])


# --------------------------------------------------------------------------
# hand-worked example: N=4, E=4, K=2, W=2, d=2, ffn=1
# --------------------------------------------------------------------------
#
# logits  t0=[2,1,0,0]  t1=[0,0,3,3]  t2=[1,1,1,1]  t3=[0,5,0,4]
# x       t0=[1,1]      t1=[1,2]      t2=[-1,1]     t3=[2,-1]
# expert e: Wg=[[1,0]], Wu=[[0,e+1]], Wd=[[1],[-1]], so the expert's output
# on a row x is [h, -h] with h = silu(x0) * (e+1) * x1.
#
# By hand: t0 picks 0 then 1; t1 ties 2/3 -> 2 first; t2 all tie -> 0, 1;
# t3 picks 1 (5) then 3 (4).  Expert loads: e0 {t0,t2}, e1 {t0,t2,t3},
# e2 {t1}, e3 {t1,t3}.  Rows in (expert, token) order:
#   e0: t0->0, t2->1 | e1: t0->2, t2->3, t3->4 | e2: t1->5 | e3: t1->6, t3->7
# With capacity ceil(1.0*4*2/4) = 2 the third token of expert 1 (t3) drops:
#   e0: 0,1 | e1: t0->2, t2->3 | e2: t1->4 | e3: t1->5, t3->6

HAND_LOGITS = np.array([[2, 1, 0, 0], [0, 0, 3, 3], [1, 1, 1, 1], [0, 5, 0, 4]], np.float32)
HAND_X = np.array([[1, 1], [1, 2], [-1, 1], [2, -1]], np.float64)


def _hand_weights(e):
    return (np.array([[1.0, 0.0]]), np.array([[0.0, e + 1.0]]), np.array([[1.0], [-1.0]]))


def test_hand_example():
    e = math.e
    exp_w = [
        [e ** 2 / (e ** 2 + e + 2), e / (e ** 2 + e + 2)],
        [e ** 3 / (2 * e ** 3 + 2)] * 2,
        [0.25, 0.25],
        [e ** 5 / (e ** 5 + e ** 4 + 2), e ** 4 / (e ** 5 + e ** 4 + 2)],
    ]
    idx, w = O.route(HAND_LOGITS, 2)
    assert idx.tolist() == [[0, 1], [2, 3], [0, 1], [1, 3]]
    assert np.allclose(w, exp_w, atol=1e-7, rtol=0)

    r = O.dispatch(idx, 4, 2, -1)
    assert r["demand"].tolist() == [2, 3, 1, 2]
    assert r["counts"].tolist() == [2, 3, 1, 2]
    assert r["offsets"].tolist() == [0, 2, 5, 6, 8]
    assert r["rank_offsets"].tolist() == [0, 5, 8]
    assert r["perm_token"].tolist() == [0, 2, 0, 2, 3, 1, 1, 3]
    assert r["dest"].tolist() == [[0, 2], [5, 6], [1, 3], [4, 7]]

    cap = O.capacity(1.0, 4, 2, 4)
    assert cap == 2
    rc = O.dispatch(idx, 4, 2, cap)
    assert rc["counts"].tolist() == [2, 2, 1, 2]
    assert rc["offsets"].tolist() == [0, 2, 4, 5, 7]
    assert rc["rank_offsets"].tolist() == [0, 4, 7]
    assert rc["perm_token"].tolist() == [0, 2, 0, 2, 1, 1, 3]
    assert rc["dest"].tolist() == [[0, 2], [4, 5], [1, 3], [-1, 6]]
    assert rc["dropped"] == 1

    def sig_lu(z):
        return z / (1 + math.exp(-z))

    def y_first(t, ex):
        return sig_lu(HAND_X[t, 0]) * (ex + 1) * HAND_X[t, 1]

    for cap_, disp in ((-1, r), (cap, rc)):
        res = O.layer(HAND_LOGITS, HAND_X, _hand_weights, 2, 2, cap_, "f64")
        for t in range(4):
            ref = 0.0
            for k in range(2):
                if disp["dest"][t, k] >= 0:
                    ref += float(w[t, k]) * y_first(t, int(idx[t, k]))
            assert abs(res["out"][t, 0] - ref) < 1e-12
            assert abs(res["out"][t, 1] + ref) < 1e-12
    # the one value that the drop changes: t3 keeps only expert 3
    res_c = O.layer(HAND_LOGITS, HAND_X, _hand_weights, 2, 2, cap, "f64")
    assert abs(res_c["out"][3, 0] - float(w[3, 1]) * y_first(3, 3)) < 1e-12

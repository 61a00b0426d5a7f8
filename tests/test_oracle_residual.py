"""Pins of the oracle's Residual-MoE layer ("MoE Inference Communication",
section "PR-MoE：从”所有层一样多专家”到”哪里需要哪里多”", Phenomenon-II: a
fixed dense MLP that every token passes through, plus the gate-routed
expert, the two outputs added).  None of these reuses the oracle's code: a
dense every-expert recompute written with einsum, torch's SiLU, closed forms
(all pairs dropped; the shared MLP equal to the only expert), and combine
inputs built so that one rounding of the whole sum differs from rounding
after each term."""
import math

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O


def _rand_weights(rng, E, d, ffn):
    wg = rng.standard_normal((E, ffn, d)) / math.sqrt(d)
    wu = rng.standard_normal((E, ffn, d)) / math.sqrt(d)
    wd = rng.standard_normal((E, d, ffn)) / math.sqrt(ffn)
    return wg, wu, wd


def _textbook_swiglu(x, wg, wu, wd):
    xt = torch.from_numpy(np.asarray(x, np.float64))
    g = xt @ torch.from_numpy(wg).T
    u = xt @ torch.from_numpy(wu).T
    return ((torch.nn.functional.silu(g) * u) @ torch.from_numpy(wd).T).numpy()


@pytest.mark.parametrize("cap", [-1, 2, 0])
def test_residual_layer_against_dense_recompute(cap):
    rng = np.random.default_rng(31 + cap)
    N, E, K, W, d, ffn, ffn_s = 20, 5, 2, 5, 8, 12, 20
    logits = rng.standard_normal((N, E)).astype(np.float32)
    x = rng.standard_normal((N, d))
    wg, wu, wd = _rand_weights(rng, E, d, ffn)
    sg, su, sd = (a[0] for a in _rand_weights(rng, 1, d, ffn_s))
    res = O.layer(logits, x, lambda e: (wg[e], wu[e], wd[e]), K, W, cap, "f64",
                  shared_weights=(sg, su, sd))
    # every expert for every token, masked by kept * gate weight
    G = np.einsum("nd,efd->nef", x, wg)
    U = np.einsum("nd,efd->nef", x, wu)
    Y = np.einsum("nef,edf->ned", G / (1.0 + np.exp(-G)) * U, wd)
    mask = np.zeros((N, E))
    seen = np.zeros(E, int)
    for t in range(N):
        for k in range(K):
            e = res["topk_idx"][t, k]
            if cap < 0 or seen[e] < cap:
                mask[t, e] = float(res["topk_w"][t, k])
            seen[e] += 1
    shared = _textbook_swiglu(x, sg, su, sd)
    assert np.allclose(res["y_shared"], shared, rtol=1e-12, atol=1e-12)
    ref = shared + np.einsum("ne,ned->nd", mask, Y)
    assert np.allclose(res["out"], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_residual_all_dropped_is_the_shared_mlp(act):
    rng = np.random.default_rng(7)
    N, E, K, W, d, ffn = 16, 4, 2, 2, 8, 8
    logits = rng.standard_normal((N, E)).astype(np.float32)
    x = O.round_storage(rng.standard_normal((N, d)), act)
    wg, wu, wd = (O.round_storage(a, act) for a in _rand_weights(rng, E, d, ffn))
    sh = tuple(O.round_storage(a[0], act) for a in _rand_weights(rng, 1, d, ffn))
    res = O.layer(logits, x, lambda e: (wg[e], wu[e], wd[e]), K, W, 0, act,
                  shared_weights=sh)
    assert (res["dest"] < 0).all()
    # nothing kept: each row is exactly the stored shared-MLP row
    assert np.array_equal(res["out"], res["y_shared"])
    assert np.allclose(res["y_shared"], _textbook_swiglu(x, *sh),
                       rtol=1e-2 if act == "bf16" else 1e-5, atol=1e-2 if act == "bf16" else 1e-5)


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_shared_mlp_equal_to_the_only_expert_doubles_the_output(act):
    rng = np.random.default_rng(9)
    N, d, ffn = 12, 16, 24
    x = O.round_storage(rng.standard_normal((N, d)), act)
    w = tuple(O.round_storage(a[0], act) for a in _rand_weights(rng, 1, d, ffn))
    plain = O.layer(np.zeros((N, 1), np.float32), x, lambda e: w, 1, 1, -1, act)
    res = O.layer(np.zeros((N, 1), np.float32), x, lambda e: w, 1, 1, -1, act,
                  shared_weights=w)
    # one expert: gate weight exactly 1, so out = y + 1 * y = 2 y, exact
    assert (plain["topk_w"] == 1.0).all()
    assert np.array_equal(res["out"], 2.0 * plain["out"])
    assert np.array_equal(res["y_shared"], plain["y_perm"])


def test_zero_shared_output_leaves_the_layer_unchanged():
    rng = np.random.default_rng(3)
    N, E, K, W, d, ffn = 18, 6, 3, 3, 8, 8
    logits = rng.standard_normal((N, E)).astype(np.float32)
    x = O.round_bf16(rng.standard_normal((N, d)))
    wg, wu, wd = (O.round_bf16(a) for a in _rand_weights(rng, E, d, ffn))
    zero = (np.zeros((ffn, d)), np.zeros((ffn, d)), np.zeros((d, ffn)))
    for cap in (-1, 4):
        a = O.layer(logits, x, lambda e: (wg[e], wu[e], wd[e]), K, W, cap, "bf16")
        b = O.layer(logits, x, lambda e: (wg[e], wu[e], wd[e]), K, W, cap, "bf16",
                    shared_weights=zero)
        assert np.array_equal(a["out"], b["out"])


def test_residual_combine_rounds_once_and_adds_shared_unweighted():
    # bf16 keeps 8 significant bits: the spacing is 2^-7 at 1.0, 2^-15 at 2^-8
    y_perm = np.array([[2.0 ** -8], [2.0 ** -17], [0.0]])
    dest = np.array([[0, 1], [2, -1]], np.int32)
    w = np.array([[1.0, 1.0], [0.25, 0.5]], np.float32)
    shared = np.array([[1.0], [3.0]])
    out = O.combine(y_perm, dest, w, "bf16", shared=shared)
    # token 0: 1 + 2^-8 + 2^-17 lies just above the midpoint of 1 and
    # 1 + 2^-7, so one rounding of the whole sum gives 1 + 2^-7; rounding the
    # routed part first (2^-8 + 2^-17 -> 2^-8) would leave the tie 1 + 2^-8,
    # which rounds to even, 1.0
    assert out[0, 0] == 1.0 + 2.0 ** -7
    # token 1: its kept row is zero and its other pair dropped: the shared
    # output, not scaled by any gate weight
    assert out[1, 0] == 3.0


def test_sampled_token_outputs_equal_full_residual_layer_rows():
    rng = np.random.default_rng(12)
    N, E, K, W, d, ffn, ffn_s = 20, 4, 1, 2, 8, 8, 16
    logits = rng.standard_normal((N, E)).astype(np.float32)
    x = O.round_bf16(rng.standard_normal((N, d)))
    wg, wu, wd = (O.round_bf16(a) for a in _rand_weights(rng, E, d, ffn))
    sh = tuple(O.round_bf16(a[0]) for a in _rand_weights(rng, 1, d, ffn_s))
    for cap in (-1, 3):
        res = O.layer(logits, x, lambda e: (wg[e], wu[e], wd[e]), K, W, cap, "bf16",
                      shared_weights=sh)
        toks = [0, 5, 6, 19]
        _, out = O.token_outputs(toks, x[toks], res["topk_idx"], res["topk_w"], res["dest"],
                                 lambda e: (wg[e], wu[e], wd[e]), "bf16", shared_weights=sh)
        assert np.array_equal(out, res["out"][toks])

"""Pins of the oracle's router projection."""
import numpy as np
import torch

from oracle import moe_oracle as O


def test_router_logits_against_torch_float64_and_closed_forms():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((17, 24))
    w = rng.standard_normal((5, 24))
    ref = (torch.from_numpy(x) @ torch.from_numpy(w).T).numpy().astype(np.float32)
    assert np.array_equal(O.router_logits(x, w), ref)
    # one-hot inputs pick single weights exactly
    eye = np.eye(24)[:5]
    assert np.array_equal(O.router_logits(eye, w), w[:, :5].T.astype(np.float32))
    # a constant row of ones sums the weights
    ones = np.ones((1, 24))
    assert np.allclose(O.router_logits(ones, w)[0], w.sum(axis=1), rtol=1e-7)


def test_error_bound_covers_fp32_accumulation_in_any_order():
    rng = np.random.default_rng(3)
    d = 512
    x = rng.standard_normal((8, d)).astype(np.float32)
    w = (rng.standard_normal((4, d)) / np.sqrt(d)).astype(np.float32)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    bound = O.router_logits_error_bound(x, w)
    for order in (np.arange(d), np.arange(d)[::-1], rng.permutation(d)):
        acc = np.zeros((8, 4), dtype=np.float32)
        for i in order:
            acc = (acc + np.outer(x[:, i], w[:, i]).astype(np.float32)).astype(np.float32)
        assert (np.abs(acc.astype(np.float64) - exact) <= bound).all()
    # a dropped term breaks the bound somewhere
    acc = (x[:, 1:].astype(np.float32) @ w[:, 1:].T.astype(np.float32))
    assert (np.abs(acc.astype(np.float64) - exact) > bound).any()

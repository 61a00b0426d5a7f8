"""Plant plausible mistakes in the oracle (on the CPU) and check that its pins
catch every one of them.  Each mutant replaces one oracle function; the pin
suite in test_oracle must then fail somewhere."""
import numpy as np
import pytest

from oracle import moe_oracle as O
import test_oracle as P

_route = O.route
_dispatch = O.dispatch
_expert_ffn = O.expert_ffn
_combine = O.combine


def _route_tie_high(logits, K, renormalize=False):
    idx, w = _route(logits, K, renormalize)
    l = np.asarray(logits, np.float32)
    # ties broken toward the higher index
    order = np.argsort(-l[:, ::-1], axis=1, kind="stable")
    idx2 = (l.shape[1] - 1 - order[:, :K]).astype(np.int32)
    p = np.exp(l - l.max(1, keepdims=True))
    p = p / p.sum(1, keepdims=True)
    return idx2, np.take_along_axis(p, idx2.astype(np.int64), 1).astype(np.float32)


def _route_renorm_always(logits, K, renormalize=False):
    return _route(logits, K, True)


def _dispatch_drop_earlier(topk_idx, E, W, cap):
    # keeps the last `cap` tokens of each expert instead of the first
    flipped = _dispatch(np.asarray(topk_idx)[::-1], E, W, cap)
    return flipped if cap >= 0 else _dispatch(topk_idx, E, W, cap)


def _dispatch_rank_offsets_off_by_one(topk_idx, E, W, cap):
    r = _dispatch(topk_idx, E, W, cap)
    per = E // W
    r["rank_offsets"] = np.array([r["offsets"][min(E, i * per + 1)] for i in range(W + 1)],
                                 np.int32)
    return r


def _ffn_swapped_gate_up(R, wg, wu, wd, act):
    return _expert_ffn(R, wu, wg, wd, act)


def _ffn_no_silu(R, wg, wu, wd, act):
    R = np.asarray(R, np.float64)
    h = O.round_storage((R @ np.asarray(wg).T) * (R @ np.asarray(wu).T), act)
    return h, O.round_storage(h @ np.asarray(wd, np.float64).T, act)


def _combine_unweighted(y_perm, dest, topk_w, act):
    return _combine(y_perm, dest, np.ones_like(np.asarray(topk_w)), act)


def _combine_includes_dropped(y_perm, dest, topk_w, act):
    dest = np.where(np.asarray(dest) < 0, 0, dest)
    return _combine(y_perm, dest, topk_w, act)


MUTANTS = {
    "route_tie_high": ("route", _route_tie_high),
    "route_renorm_always": ("route", _route_renorm_always),
    "dispatch_drop_earlier": ("dispatch", _dispatch_drop_earlier),
    "dispatch_rank_offsets": ("dispatch", _dispatch_rank_offsets_off_by_one),
    "ffn_swapped_gate_up": ("expert_ffn", _ffn_swapped_gate_up),
    "ffn_no_silu": ("expert_ffn", _ffn_no_silu),
    "combine_unweighted": ("combine", _combine_unweighted),
    "combine_includes_dropped": ("combine", _combine_includes_dropped),
}

PINS = [
    lambda: P.test_route_against_brute_force(6, 3),
    lambda: P.test_route_special_cases(),
    lambda: [P.test_dispatch_against_brute_force(c) for c in (-1, 0, 3)],
    lambda: P.test_dispatch_closed_forms(),
    lambda: [P.test_layer_against_dense_masked_recompute(c) for c in (-1, 2)],
    lambda: P.test_single_expert_is_textbook_swiglu(),
    lambda: P.test_dispatch_then_combine_with_identity_ffn_is_identity(),
    lambda: P.test_hand_example(),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    failures = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, IndexError):
            failures += 1
    assert failures > 0, f"mutant {name} survived every pin"

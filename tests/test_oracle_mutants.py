"""Plant plausible mistakes in the oracle (on the CPU) and check that its pins
catch every one of them.  Each mutant replaces one oracle function; the pin
suite in test_oracle must then fail somewhere."""
import numpy as np
import pytest

from oracle import moe_oracle as O
import test_oracle as P
import test_oracle_reroute as PR
import test_oracle_fp8 as PF
import test_oracle_residual as PRS

_route = O.route
_dispatch = O.dispatch
_expert_ffn = O.expert_ffn
_combine = O.combine
_reroute = O.reroute_overflow
_gate_scores = O.gate_scores
_e4m3_encode = O.e4m3_encode
_quantize_fp8 = O.quantize_fp8


def _route_tie_high(logits, K, renormalize=False, gate="softmax"):
    idx, w = _route(logits, K, renormalize, gate)
    l = np.asarray(logits, np.float32)
    # ties broken toward the higher index
    order = np.argsort(-l[:, ::-1], axis=1, kind="stable")
    idx2 = (l.shape[1] - 1 - order[:, :K]).astype(np.int32)
    p = np.exp(l - l.max(1, keepdims=True))
    p = p / p.sum(1, keepdims=True)
    return idx2, np.take_along_axis(p, idx2.astype(np.int64), 1).astype(np.float32)


def _route_renorm_always(logits, K, renormalize=False, gate="softmax"):
    return _route(logits, K, True, gate)


def _gate_sigmoid_sign(logits, gate="softmax"):
    if gate == "sigmoid":
        return 1.0 / (1.0 + np.exp(np.asarray(logits, np.float64)))
    return _gate_scores(logits, gate)


def _e4m3_ties_away(v):
    # rounds halfway cases away from zero instead of to the even code
    v = np.asarray(v, np.float64)
    code = _e4m3_encode(v)
    table = O.e4m3_value(np.arange(0x7F))
    mids = (table[1:] + table[:-1]) / 2
    a = np.abs(v)
    tie = np.isin(a, mids)
    up = np.searchsorted(table, a)
    return np.where(tie, (up | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8), code)


def _quantize_scale_447(x, group=128):
    codes, scales = _quantize_fp8(x, group)
    return codes, (scales * np.float32(448) / np.float32(447)).astype(np.float32)


def _reroute_candidate_off_by_one(logits, topk_idx, cap, gate="softmax", renormalize=False):
    # offers position K + j - 1: the token's own worst top-K expert first
    l = np.asarray(logits, np.float32)
    idx = np.asarray(topk_idx)
    shifted = np.concatenate([idx[:, :-1], idx[:, -1:]], axis=1)
    ni, nw, rr = _reroute(l, shifted, cap, gate, renormalize)
    if cap >= 0 and idx.shape[1] < l.shape[1]:
        order = np.argsort(-l, axis=1, kind="stable")
        for t in range(l.shape[0]):
            for k in range(idx.shape[1]):
                if ni[t, k] != idx[t, k]:
                    ni[t, k] = order[t, idx.shape[1] - 1]
    return ni, nw, rr


def _reroute_ignores_room(logits, topk_idx, cap, gate="softmax", renormalize=False):
    # admits every candidate: the first pass's survivors are not counted
    if cap <= 0:
        return _reroute(logits, topk_idx, cap, gate, renormalize)
    return _reroute_unbounded(logits, topk_idx, cap, gate, renormalize)


def _reroute_unbounded(logits, topk_idx, cap, gate, renormalize):
    l = np.asarray(logits, np.float32)
    idx = np.asarray(topk_idx).astype(np.int64)
    N, E = l.shape
    K = idx.shape[1]
    ni, nw, _ = _reroute(l, idx, -1, gate, renormalize)
    rr = np.zeros(E, np.int64)
    seen = [0] * E
    order = np.argsort(-l, axis=1, kind="stable")
    p = O.gate_scores(l, gate)
    for t in range(N):
        j = 0
        for k in range(K):
            e = int(idx[t, k])
            if seen[e] >= cap and K + j < E:
                c = int(order[t, K + j])
                ni[t, k] = c
                nw[t, k] = np.float32(p[t, c])
                rr[c] += 1
            if seen[e] >= cap:
                j += 1
            seen[e] += 1
    return ni.astype(np.int32), nw, rr.astype(np.int32)


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


def _combine_unweighted(y_perm, dest, topk_w, act, shared=None):
    return _combine(y_perm, dest, np.ones_like(np.asarray(topk_w)), act, shared)


def _combine_includes_dropped(y_perm, dest, topk_w, act, shared=None):
    dest = np.where(np.asarray(dest) < 0, 0, dest)
    return _combine(y_perm, dest, topk_w, act, shared)


def _combine_shared_weighted(y_perm, dest, topk_w, act, shared=None):
    if shared is not None:
        shared = np.asarray(shared, np.float64) * np.asarray(topk_w, np.float64)[:, :1]
    return _combine(y_perm, dest, topk_w, act, shared)


def _combine_shared_rounded_apart(y_perm, dest, topk_w, act, shared=None):
    out = _combine(y_perm, dest, topk_w, act)
    if shared is not None:
        out = O.round_storage(out + np.asarray(shared, np.float64), act)
    return out


def _shared_expert_no_silu(x, wg, wu, wd, act):
    R = np.asarray(x, np.float64)
    h = O.round_storage((R @ np.asarray(wg, np.float64).T) * (R @ np.asarray(wu, np.float64).T), act)
    return O.round_storage(h @ np.asarray(wd, np.float64).T, act)


MUTANTS = {
    "route_tie_high": ("route", _route_tie_high),
    "route_renorm_always": ("route", _route_renorm_always),
    "dispatch_drop_earlier": ("dispatch", _dispatch_drop_earlier),
    "dispatch_rank_offsets": ("dispatch", _dispatch_rank_offsets_off_by_one),
    "ffn_swapped_gate_up": ("expert_ffn", _ffn_swapped_gate_up),
    "ffn_no_silu": ("expert_ffn", _ffn_no_silu),
    "combine_unweighted": ("combine", _combine_unweighted),
    "combine_includes_dropped": ("combine", _combine_includes_dropped),
    "gate_sigmoid_sign": ("gate_scores", _gate_sigmoid_sign),
    "reroute_candidate_off_by_one": ("reroute_overflow", _reroute_candidate_off_by_one),
    "reroute_ignores_room": ("reroute_overflow", _reroute_ignores_room),
    "e4m3_ties_away": ("e4m3_encode", _e4m3_ties_away),
    "quantize_scale_447": ("quantize_fp8", _quantize_scale_447),
    "combine_shared_weighted": ("combine", _combine_shared_weighted),
    "combine_shared_rounded_apart": ("combine", _combine_shared_rounded_apart),
    "shared_expert_no_silu": ("shared_expert", _shared_expert_no_silu),
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
    lambda: PR.test_sigmoid_scores_match_library(),
    lambda: PR.test_sigmoid_route_special_cases(),
    lambda: PR.test_reroute_hand_example(),
    lambda: [PR.test_reroute_uniform_closed_form(*c) for c in ((10, 3, 2, 6), (12, 4, 3, 6))],
    lambda: PR.test_reroute_is_a_no_op_without_overflow(),
    lambda: [PR.test_reroute_against_brute_force(s) for s in range(4)],
    lambda: PF.test_e4m3_closed_forms(),
    lambda: PF.test_e4m3_encode_matches_torch_cast(),
    lambda: PF.test_quantize_group_properties(),
    lambda: PF.test_quantize_is_exact_on_representable_groups(),
    lambda: [PRS.test_residual_layer_against_dense_recompute(c) for c in (-1, 2)],
    lambda: [PRS.test_residual_all_dropped_is_the_shared_mlp(a) for a in ("bf16", "f32")],
    lambda: PRS.test_shared_mlp_equal_to_the_only_expert_doubles_the_output("bf16"),
    lambda: PRS.test_zero_shared_output_leaves_the_layer_unchanged(),
    lambda: PRS.test_residual_combine_rounds_once_and_adds_shared_unweighted(),
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

"""Plain CPU oracle for one MoE expert-parallel layer on one GPU's share.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
run this module: only the tests, the smoke check of ``__graft_entry__`` and
the CPU-baseline leg of ``bench.py`` use it.  It shares no code, constant or
helper with the HIP library and never imports it.

What it computes (the layer is the four stages of the data flow drawn in
"MoE 专家并行的 All-to-All 通信瓶颈" (wiblog.cn), section "All-to-All
分发与回收的机制", flowchart: route -> pack by destination -> per-expert
grouped GEMM -> merge back to token order with the gate weights; the same
stage list is "Gate -> dispatch -> Expert FFN -> combine -> Aggregation" in
"MoE Inference Communication", section "系统剖析"):

  route     per token: softmax over the E router logits; the K experts with
            the largest logits (ties -> lower expert index), best first;
            gate weight = that expert's softmax probability.
  dispatch  histogram of expert ids (the ``bincount`` line of the dispatch
            pseudocode in "MoE 推理服务工程真相 2026", section 2.3), a
            per-expert capacity that drops the later tokens of an overflowing
            expert (same page, section 2.2; zeroed router output, section
            4.3 "Expert drop"), an exclusive prefix sum of the kept counts
            ("MoE Inference Communication", section "MoE 计算核优化",
            cumsum) and the dense token<->row mapping table of that same
            section, which places every kept (token, expert) pair in an
            expert-contiguous buffer ordered by (expert, token).  Experts are
            owned by W virtual ranks in contiguous blocks of E/W, so the
            buffer is also rank-major: rank r's send slice starts at
            offsets[r*E/W].
  ffn       per expert, on its rows: h = silu(x Wg^T) * (x Wu^T),
            y = h Wd^T (SwiGLU, no biases).
  combine   out[t] = sum over kept slots k (ascending) of w[t,k] * y[row(t,k)].

Routing variants (section 2.3 of "MoE 推理服务工程真相 2026" names sigmoid
routing as a balance remedy and re-maps overflowing expert ids in its
dispatch pseudocode; its section 4.3 sends an over-capacity token to a
next-best expert instead of dropping it):

  gate      "sigmoid": the gate score of expert e is 1 / (1 + exp(-l_e))
            instead of the softmax probability; the top-K choice is the same
            (both scores rise with the logit).
  reroute   one round of re-routing after the capacity check: a token's
            j-th overflowing slot is offered its (K + j)-th best expert and
            takes it if that expert still has room, in token order.

FP8 payload ("MoE 推理服务工程真相 2026", section 6.3: the all-to-all token
data goes as FP8 instead of BF16, halving the bytes):

  fp8       rows are cut into groups of 128 columns; each group is stored
            as OCP e4m3 codes of x * (448 / amax) (fp32 arithmetic,
            round-to-nearest-even) with the fp32 scale amax / 448, and read
            back as code value * scale.

Residual-MoE ("MoE Inference Communication", section "PR-MoE：从”所有层一样多
专家”到”哪里需要哪里多”", Phenomenon-II: one fixed dense MLP that every token
passes through, plus the routed expert, with the two outputs added; it
matches top-2 routing in quality at top-1's exchange volume):

  shared    y_shared = the SwiGLU MLP with its own weights on every token
            row, rounded to storage; combine starts each token's sum from
            y_shared[t] (unweighted) and adds the kept pairs in ascending k.

Where the pages say nothing (the gate function, the tie-break, the order
inside an expert, the capacity formula, the FFN form) the oracle takes the
plain reading: fp32-input softmax, lowest index wins ties, ascending token
order, capacity = ceil(C*N*K/E), SwiGLU.

Precision: arithmetic is float64 throughout.  A value is rounded to the
activation storage type (bf16 round-to-nearest-even, or fp32) exactly where
the layer stores it: h, y_perm and out; gate weights are stored as fp32.
The top-K choice compares the raw fp32 logits, so it never depends on how
``exp`` is rounded.

Every function here is pinned by tests that do not reuse its code:
brute-force subset checks, a dense every-expert-for-every-token recompute,
closed forms, invariants, a hand-worked example, and library routines.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

__all__ = [
    "round_bf16",
    "round_storage",
    "capacity",
    "gate_scores",
    "route",
    "reroute_overflow",
    "dispatch",
    "pack",
    "silu",
    "expert_ffn",
    "grouped_ffn",
    "combine",
    "layer",
    "token_outputs",
    "router_logits",
    "router_logits_error_bound",
    "e4m3_value",
    "e4m3_encode",
    "quantize_fp8",
    "dequantize_fp8",
    "shard_bounds",
    "exchange",
    "tau_min",
]


# --------------------------------------------------------------------------
# storage rounding
# --------------------------------------------------------------------------

def round_bf16(a):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits and fp32's exponent range (normal
    numbers down to 2**-126, subnormal spacing 2**-133).  For |a| in
    [2**(q-1), 2**q) the representable spacing is 2**(q-8); scaling by a power
    of two is exact in float64, so ``rint`` (half to even) performs the
    rounding exactly.  Results of magnitude 2**128 or more overflow to inf.
    Returns float64 holding the rounded values.
    """
    a = np.asarray(a, dtype=np.float64)
    out = np.zeros_like(a)
    nz = (a != 0) & np.isfinite(a)
    _, q = np.frexp(a[nz])
    q = np.maximum(q, -125)            # below 2**-126 the spacing stays 2**-133
    scale = np.ldexp(1.0, 8 - q)
    r = np.rint(a[nz] * scale) / scale
    r[np.abs(r) >= 2.0 ** 128] = np.inf * np.sign(r[np.abs(r) >= 2.0 ** 128])
    out[nz] = r
    out[~np.isfinite(a)] = a[~np.isfinite(a)]
    out[a == 0] = a[a == 0]            # keeps the sign of zero
    return out


def round_storage(a, act):
    """Round to the activation storage type: ``"bf16"`` or ``"f32"``.

    ``"f64"`` keeps float64 values unrounded; it exists so that tests can
    check the layer's structure without any storage rounding.
    """
    if act == "f64":
        return np.asarray(a, dtype=np.float64)
    if act == "bf16":
        return round_bf16(a)
    if act == "f32":
        return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(f"unknown activation type {act!r}")


# --------------------------------------------------------------------------
# capacity
# --------------------------------------------------------------------------

def capacity(C, N, K, E):
    """Per-expert token budget ceil(C*N*K/E), computed exactly.

    "MoE 推理服务工程真相 2026", section 2.2: an expert receiving more tokens
    than its capacity drops the excess; the page's formula lost its symbols,
    so the budget is the expected per-expert load N*K/E scaled by the
    capacity factor C, rounded up.  C is taken as the exact rational value of
    the given double.  Returns -1 (dropless) when C is None.
    """
    if C is None:
        return -1
    if not (isinstance(C, (int, float)) and math.isfinite(C) and C > 0):
        raise ValueError("capacity factor must be finite and > 0")
    v = Fraction(C) * N * K / E
    return int(math.ceil(v))


# --------------------------------------------------------------------------
# router projection
# --------------------------------------------------------------------------

def router_logits(x, w_router):
    """Router logits of every token: logits[t, e] = sum_i x[t, i] * w[e, i].

    The router yields each token's expert scores from its hidden state ("MoE
    推理服务工程真相 2026", section 一: the token passes through the router
    network before top-k selection; "MoE 专家并行的 All-to-All 通信瓶颈",
    flowchart step "路由器选 Top-K 专家").  Computed exactly in float64 (the
    products of bf16 or fp32 inputs and their sums up to d terms are exact
    or nearly so) and rounded once to fp32, the logits' storage type.
    x [N, d], w_router [E, d] hold values of the activation type.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_router, dtype=np.float64)
    return (x @ w.T).astype(np.float32)


def router_logits_error_bound(x, w_router):
    """Per-logit bound on |fp32-accumulated sum - exact sum| for any order of
    the d-term summation: gamma_{d} * sum_i |x_i w_i| with gamma_n =
    n u / (1 - n u), u = 2**-24 (the standard bound for floating-point
    summation, products being exact), plus half an ulp for the final fp32
    rounding of the reference."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    w = np.abs(np.asarray(w_router, dtype=np.float64))
    d = x.shape[1]
    u = 2.0 ** -24
    gamma = d * u / (1 - d * u)
    mag = x @ w.T
    return gamma * mag + u * mag


# --------------------------------------------------------------------------
# route
# --------------------------------------------------------------------------

def gate_scores(logits, gate="softmax"):
    """Gate score of every expert for every token, float64 [N, E].

    "softmax": exp(l_e - max) / sum_e' exp(l_e' - max), the default gate.
    "sigmoid": 1 / (1 + exp(-l_e)), the sigmoid routing that "MoE 推理服务工程
    真相 2026", section 2.3, names as a remedy for router-level imbalance;
    each expert's score is independent of the others'.
    """
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    if gate == "softmax":
        m = l.max(axis=1, keepdims=True)
        ex = np.exp(l - m)
        return ex / ex.sum(axis=1, keepdims=True)
    if gate == "sigmoid":
        return 1.0 / (1.0 + np.exp(-l))
    raise ValueError("gate must be 'softmax' or 'sigmoid'")


def route(logits, K, renormalize=False, gate="softmax"):
    """Top-K routing of every token.

    "MoE 专家并行的 All-to-All 通信瓶颈", section "一个反直觉的扩容结果": the
    router picks the Top-K experts of every token; "MoE 推理服务工程真相
    2026", section 一: the router yields top-k expert weights.

    logits: float32 [N, E] (finite).  Returns (topk_idx int32 [N, K],
    topk_w float32 [N, K]).  Slot 0 is the best expert.  A larger logit wins;
    equal logits go to the lower expert index.  The weight of slot k is the
    gate score of its expert (gate_scores: the softmax probability over all E
    logits, or the sigmoid of its logit), optionally divided by the sum of
    the K selected scores.  Both gates rise with the logit, so the choice is
    the same for either.
    """
    l32 = np.asarray(logits, dtype=np.float32)
    N, E = l32.shape
    if not (1 <= K <= E):
        raise ValueError("need 1 <= K <= E")
    if not np.all(np.isfinite(l32)):
        raise ValueError("logits must be finite")
    p = gate_scores(l32, gate)
    # Stable sort on the negated fp32 logit: descending logit, and among
    # equal logits the original (ascending expert) order survives.
    order = np.argsort(-l32, axis=1, kind="stable")
    idx = order[:, :K].astype(np.int32)
    w = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return idx, w.astype(np.float32)


def reroute_overflow(logits, topk_idx, cap, gate="softmax", renormalize=False):
    """One round of token re-routing of capacity overflow.

    "MoE 推理服务工程真相 2026", section 2.3: the dispatch pseudocode counts
    each expert's tokens, compares them with the capacity and re-maps the
    expert ids of the overflow before the all-to-all; section 4.3 ("Token
    drop"): an over-capacity token is sent to a next-best expert rather than
    losing that expert's output.  The pages fix neither which expert nor
    what happens when it is full; the reading here:

      1. Overflow: walk t = 0..N-1 and k = 0..K-1; slot (t, k) with expert
         e = topk_idx[t, k] overflows iff cap >= 0 and e has already been
         named by cap earlier slots (the same rule that drops it in
         ``dispatch``).  kept1[e] = min(demand[e], cap).
      2. Candidate: token t's j-th overflowing slot (j = 0, 1, .. in slot
         order) is offered the expert at position K + j of the token's full
         order (descending logit, ties to the lower index), i.e. its best
         experts outside its own top K; there is none if K + j >= E.
      3. Admission: walk the candidates in the same (t, k) order; expert c
         admits a candidate while it has admitted fewer than cap - kept1[c],
         so admitted slots only fill room the first pass left.
      4. An admitted slot takes expert c and weight score(c) (gate_scores),
         divided by the sum of the scores of the token's original K experts
         if renormalize.  Every other slot is left as it was: a slot that
         overflowed and was not admitted keeps its expert, and ``dispatch``
         with the same cap drops it again.

    With these rules ``dispatch(new_idx, E, W, cap)`` keeps exactly the
    first-pass survivors plus the admitted slots (an expert that overflowed
    has no room, and an expert with room had no overflow).

    Returns (new_idx int32 [N, K], new_w float32 [N, K], rerouted int32 [E]:
    admitted slots per expert).  topk_idx: int32 [N, K] as ``route`` gives.
    """
    l32 = np.asarray(logits, dtype=np.float32)
    idx = np.asarray(topk_idx).astype(np.int64)
    N, E = l32.shape
    K = idx.shape[1]
    p = gate_scores(l32, gate)
    # original weights (as route computes them) for the slots left alone
    w = np.take_along_axis(p, idx, axis=1)
    norm = w.sum(axis=1) if renormalize else np.ones(N)
    new_idx = idx.copy()
    new_w = (w / norm[:, None]).astype(np.float32)
    rerouted = np.zeros(E, dtype=np.int64)
    if cap < 0:
        return new_idx.astype(np.int32), new_w, rerouted.astype(np.int32)

    # 1. overflow in token order
    seen = [0] * E
    over = [[False] * K for _ in range(N)]
    for t in range(N):
        for k in range(K):
            e = int(idx[t, k])
            over[t][k] = seen[e] >= cap
            seen[e] += 1
    room = [cap - min(seen[e], cap) for e in range(E)]

    # 2 + 3. candidates and admission, in token order
    order = np.argsort(-l32, axis=1, kind="stable")
    for t in range(N):
        j = 0
        for k in range(K):
            if not over[t][k]:
                continue
            pos = K + j
            j += 1
            if pos >= E:
                continue
            c = int(order[t, pos])
            if room[c] > 0:
                room[c] -= 1
                rerouted[c] += 1
                new_idx[t, k] = c
                new_w[t, k] = np.float32(p[t, c] / norm[t])
    return new_idx.astype(np.int32), new_w, rerouted.astype(np.int32)


# --------------------------------------------------------------------------
# dispatch
# --------------------------------------------------------------------------

def dispatch(topk_idx, E, W, cap):
    """Histogram, capacity drop, prefix sum and the token<->row mapping.

    topk_idx int32 [N, K] (distinct experts per token); E experts owned by W
    virtual ranks in contiguous blocks of E/W; cap = -1 for dropless, else
    the per-expert budget (>= 0).

    Steps, in the order the dispatch pseudocode of "MoE 推理服务工程真相
    2026" (section 2.3) takes them:
      1. demand = bincount(expert ids, minlength=E)   (that page's own line)
      2. keep: walk tokens t = 0..N-1 and their slots k = 0..K-1; the
         r-th token seen by expert e (r counted from 0) is kept iff
         cap < 0 or r < cap, so an overflowing expert drops its later
         tokens (section 2.2) and the dropped pair's router output is zero
         (section 4.3 "Expert drop").
      3. counts = kept per expert; offsets = exclusive cumsum (E+1 entries)
         ("MoE Inference Communication", section "MoE 计算核优化", cumsum);
         rank_offsets[r] = offsets[r*E/W] (W+1 entries): rank r's contiguous
         send slice ("MoE 专家并行的 All-to-All 通信瓶颈", flowchart step
         "按目标卡分组打包").
      4. the dense mapping table of "MoE 计算核优化": a kept pair (t,k) with
         expert e and rank r goes to row offsets[e] + r; dest[t,k] is that
         row (-1 when dropped) and perm_token[row] = t.

    Returns a dict of int32 arrays: demand [E], counts [E], offsets [E+1],
    rank_offsets [W+1], dest [N, K], perm_token [M] with M = offsets[E],
    plus the int ``dropped``.
    """
    idx = np.asarray(topk_idx)
    N, K = idx.shape
    if E % W != 0:
        raise ValueError("E must be a multiple of W")
    if cap < -1:
        raise ValueError("cap must be >= -1")
    demand = np.bincount(idx.ravel().astype(np.int64), minlength=E).astype(np.int32)

    seen = [0] * E
    rank = [[0] * K for _ in range(N)]
    kept = [[False] * K for _ in range(N)]
    for t in range(N):
        for k in range(K):
            e = int(idx[t, k])
            r = seen[e]
            seen[e] = r + 1
            rank[t][k] = r
            kept[t][k] = cap < 0 or r < cap

    counts = np.zeros(E, dtype=np.int64)
    for t in range(N):
        for k in range(K):
            if kept[t][k]:
                counts[int(idx[t, k])] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    per_rank = E // W
    rank_offsets = np.array([offsets[r * per_rank] for r in range(W + 1)], dtype=np.int64)

    M = int(offsets[E])
    dest = np.full((N, K), -1, dtype=np.int64)
    perm_token = np.full(M, -1, dtype=np.int64)
    for t in range(N):
        for k in range(K):
            if kept[t][k]:
                row = int(offsets[int(idx[t, k])]) + rank[t][k]
                dest[t, k] = row
                perm_token[row] = t
    return {
        "demand": demand,
        "counts": counts.astype(np.int32),
        "offsets": offsets.astype(np.int32),
        "rank_offsets": rank_offsets.astype(np.int32),
        "dest": dest.astype(np.int32),
        "perm_token": perm_token.astype(np.int32),
        "dropped": int(N * K - M),
    }


def pack(x, perm_token):
    """Rank-major send buffer: row p holds a bit copy of x[perm_token[p]]."""
    return np.asarray(x)[np.asarray(perm_token, dtype=np.int64)]


# --------------------------------------------------------------------------
# expert FFN
# --------------------------------------------------------------------------

def silu(z):
    """z * sigmoid(z) = z / (1 + exp(-z)), float64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(R, wg, wu, wd, act):
    """One expert's SwiGLU FFN on its rows R [m, d].

    wg, wu: [ffn, d]; wd: [d, ffn] (all exactly representable in the
    activation type).  G = R wg^T and U = R wu^T in float64; h = silu(G)*U
    rounded to storage; y = h wd^T rounded to storage.  Returns (h, y).
    The grouped-GEMM stage of "MoE 专家并行的 All-to-All 通信瓶颈" (flowchart
    "Grouped GEMM 专家计算") applies this to each expert's contiguous rows.
    """
    R = np.asarray(R, dtype=np.float64)
    G = R @ np.asarray(wg, dtype=np.float64).T
    U = R @ np.asarray(wu, dtype=np.float64).T
    h = round_storage(silu(G) * U, act)
    y = round_storage(h @ np.asarray(wd, dtype=np.float64).T, act)
    return h, y


def grouped_ffn(x_perm, offsets, expert_weights, act):
    """Apply every non-empty expert to its slice of the packed buffer.

    x_perm [M, d]; offsets [E+1]; expert_weights(e) -> (wg, wu, wd).
    Returns (h [M, ffn], y_perm [M, d]) float64 holding storage values.
    """
    x_perm = np.asarray(x_perm, dtype=np.float64)
    E = len(offsets) - 1
    M = int(offsets[E])
    h_all = None
    y_all = np.zeros((M, x_perm.shape[1]), dtype=np.float64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b == a:
            continue
        wg, wu, wd = expert_weights(e)
        h, y = expert_ffn(x_perm[a:b], wg, wu, wd, act)
        if h_all is None:
            h_all = np.zeros((M, h.shape[1]), dtype=np.float64)
        h_all[a:b] = h
        y_all[a:b] = y
    if h_all is None:
        h_all = np.zeros((M, 0), dtype=np.float64)
    return h_all, y_all


def shared_expert(x, wg, wu, wd, act):
    """The dense MLP of a Residual-MoE layer ("MoE Inference Communication",
    section "PR-MoE：从”所有层一样多专家”到”哪里需要哪里多”", Phenomenon-II and
    the Residual bullet: every token passes through one fixed dense MLP
    beside its routed expert).  Read here as an expert of the same SwiGLU
    form with its own weights (wg, wu [ffn_s, d]; wd [d, ffn_s]) applied to
    every token row of x [N, d]; returns y_shared [N, d] rounded to storage.
    """
    return expert_ffn(x, wg, wu, wd, act)[1]


# --------------------------------------------------------------------------
# combine
# --------------------------------------------------------------------------

def combine(y_perm, dest, topk_w, act, shared=None):
    """Weighted merge back to token order.

    "MoE 专家并行的 All-to-All 通信瓶颈", flowchart "加权合并回原 token 顺序":
    out[t] = sum over k ascending with dest[t,k] >= 0 of w[t,k] * y[dest[t,k]]
    in float64, rounded to storage.  A dropped pair adds nothing ("MoE 推理
    服务工程真相 2026", section 4.3: the dropped expert's output is zero); a
    token with every pair dropped gets a zero row.

    shared [N, d] (storage values), for a Residual-MoE layer ("MoE Inference
    Communication", section "PR-MoE：从”所有层一样多专家”到”哪里需要哪里多”",
    Phenomenon-II: a fixed dense MLP that every token passes through, whose
    output is added to the routed expert's): the sum starts from shared[t],
    unweighted, and the kept pairs are added to it in ascending k; a token
    with every pair dropped gets shared[t].
    """
    y_perm = np.asarray(y_perm, dtype=np.float64)
    dest = np.asarray(dest)
    w = np.asarray(topk_w, dtype=np.float32).astype(np.float64)
    N, K = dest.shape
    d = y_perm.shape[1]
    out = np.zeros((N, d), dtype=np.float64)
    if shared is not None:
        out += np.asarray(shared, dtype=np.float64)
    for k in range(K):
        rows = dest[:, k]
        ok = rows >= 0
        out[ok] += w[ok, k:k + 1] * y_perm[rows[ok].astype(np.int64)]
    return round_storage(out, act)


# --------------------------------------------------------------------------
# the whole layer
# --------------------------------------------------------------------------

# --------------------------------------------------------------------------
# fp8 payload
# --------------------------------------------------------------------------

FP8_GROUP = 128
E4M3_MAX = 448.0


def e4m3_value(code):
    """Value of OCP FP8 E4M3 codes (uint8 array) as float64, from the format's
    definition: sign bit, 4-bit exponent with bias 7, 3-bit mantissa;
    exponent 0 holds the subnormals m * 2**-9; S.1111.111 is NaN (there are
    no infinities), so the largest finite value is 1.75 * 2**8 = 448."""
    c = np.asarray(code).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


def e4m3_encode(v):
    """E4M3 code nearest to each value (|v| <= 448), ties to the even code.

    The 127 non-negative finite codes 0x00..0x7E have increasing values, so
    the nearest code is found by search over that table; the sign goes to bit 7
    (so -0.0 and +0.0 both encode as their sign with a zero magnitude)."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.abs(v) > E4M3_MAX) or np.any(~np.isfinite(v)):
        raise ValueError("e4m3_encode takes finite |v| <= 448")
    table = e4m3_value(np.arange(0x7F))
    a = np.abs(v)
    hi = np.clip(np.searchsorted(table, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = a - table[lo]
    d_hi = table[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == table[hi], hi, code)
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def quantize_fp8(x, group=FP8_GROUP):
    """Rows of x [R, d] (d a multiple of group) -> (codes uint8 [R, d],
    scales float32 [R, d / group]).

    Per group of `group` columns, in fp32 as a GPU computes it: amax = max
    |x|; r = 448 / amax, or 0 when amax < 2**-100 (a zero group, or one so
    small that the quotient would overflow fp32: its codes are zeros);
    code = e4m3_encode(clamp(x * r, -448, 448)); scale = amax / 448.  Each
    quotient and product is one fp32 operation, so the codes are exact
    functions of the inputs."""
    x32 = np.asarray(x, dtype=np.float32)
    R, d = x32.shape
    if d % group:
        raise ValueError("d must be a multiple of the group size")
    g = x32.reshape(R, d // group, group)
    amax = np.abs(g).max(axis=2)
    f448 = np.float32(E4M3_MAX)
    big = amax >= np.float32(2.0 ** -100)
    r = np.where(big, f448 / np.where(big, amax, np.float32(1)), np.float32(0))
    r = r.astype(np.float32)
    v = (g * r[:, :, None]).astype(np.float32)
    v = np.clip(v, -f448, f448)
    codes = e4m3_encode(v.astype(np.float64)).reshape(R, d)
    scales = (amax / f448).astype(np.float32)
    return codes, scales


def dequantize_fp8(codes, scales, group=FP8_GROUP):
    """float32 [R, d]: the value of each code times its group's scale (one
    fp32 multiply)."""
    c = np.asarray(codes)
    R, d = c.shape
    val = e4m3_value(c).astype(np.float32).reshape(R, d // group, group)
    s = np.asarray(scales, dtype=np.float32)[:, :, None]
    return (val * s).astype(np.float32).reshape(R, d)


def layer(logits, x, expert_weights, K, W, cap, act, renormalize=False, gate="softmax",
          reroute=False, fp8=False, shared_weights=None):
    """Route (optionally re-routing overflow), dispatch, FFN and combine;
    returns every intermediate.  fp8=True sends both exchanges as fp8: the
    packed rows are quantized (x8, x_scale) and read back as bf16 for the
    FFN; its output rows are quantized (y8, y_scale) and combined from their
    fp8 values.  shared_weights = (wg, wu, wd) makes it a Residual-MoE
    layer: the shared MLP's output on x (y_shared) is added in combine."""
    N, E = np.asarray(logits).shape
    idx, w = route(logits, K, renormalize, gate)
    rerouted = np.zeros(E, dtype=np.int32)
    if reroute:
        idx, w, rerouted = reroute_overflow(logits, idx, cap, gate, renormalize)
    disp = dispatch(idx, E, W, cap)
    x_perm = pack(x, disp["perm_token"])
    res = dict(disp)
    if fp8:
        x8, xs = quantize_fp8(x_perm)
        x_perm = round_storage(dequantize_fp8(x8, xs).astype(np.float64), act)
        res.update(x8=x8, x_scale=xs)
    h, y = grouped_ffn(x_perm, disp["offsets"], expert_weights, act)
    y_in = y
    if fp8:
        y8, ys = quantize_fp8(y)
        y_in = dequantize_fp8(y8, ys).astype(np.float64)
        res.update(y8=y8, y_scale=ys)
    y_shared = None
    if shared_weights is not None:
        y_shared = shared_expert(x, *shared_weights, act)
        res.update(y_shared=y_shared)
    out = combine(y_in, disp["dest"], w, act, shared=y_shared)
    res.update(topk_idx=idx, topk_w=w, x_perm=x_perm, h=h, y_perm=y, out=out,
               rerouted=rerouted)
    return res


def token_outputs(tokens, x_tokens, topk_idx, topk_w, dest, expert_weights, act,
                  shared_weights=None):
    """Outputs of selected tokens only, expert by expert.

    For layers too large to run whole on the CPU: every kept pair (t,k) of a
    selected token runs its expert's FFN on the single row x[t]; the rows are
    independent, so this equals the corresponding rows of the full layer.
    x_tokens[i] is the hidden state of token tokens[i].  shared_weights
    (Residual-MoE): each token's sum starts from the shared MLP's output on
    its row, as in combine.
    Returns (y_rows dict (t,k) -> y [d], out [len(tokens), d]).
    """
    tokens = [int(t) for t in tokens]
    xs = {t: np.asarray(x_tokens[i], dtype=np.float64) for i, t in enumerate(tokens)}
    need = {}
    for t in tokens:
        for k in range(topk_idx.shape[1]):
            if dest[t, k] >= 0:
                need.setdefault(int(topk_idx[t, k]), []).append((t, k))
    y_rows = {}
    for e in sorted(need):
        wg, wu, wd = expert_weights(e)
        pairs = need[e]
        R = np.stack([xs[t] for t, _ in pairs])
        _, y = expert_ffn(R, wg, wu, wd, act)
        for i, tk in enumerate(pairs):
            y_rows[tk] = y[i]
    d = len(next(iter(xs.values())))
    w = np.asarray(topk_w, dtype=np.float32).astype(np.float64)
    out = np.zeros((len(tokens), d), dtype=np.float64)
    if shared_weights is not None:
        out += shared_expert(np.stack([xs[t] for t in tokens]), *shared_weights, act)
    for i, t in enumerate(tokens):
        for k in range(topk_idx.shape[1]):
            if dest[t, k] >= 0:
                out[i] += w[t, k] * y_rows[(t, k)]
    return y_rows, round_storage(out, act)


# --------------------------------------------------------------------------
# virtual multi-source exchange (W source ranks on one GPU)
# --------------------------------------------------------------------------

def shard_bounds(N, W):
    """Token shards of the W virtual source ranks: shard s owns tokens
    [lo[s], lo[s+1]) with lo[s] = floor(s*N/W) (contiguous, nearly equal)."""
    return [(s * N) // W for s in range(W + 1)]


def exchange(topk_idx, dest, E, W):
    """The two local permutations on either side of the all-to-all, for W
    source ranks that each own a contiguous shard of the tokens.

    "MoE 专家并行的 All-to-All 通信瓶颈", section "All-to-All 分发与回收的
    机制": each card packs its tokens by destination card, the all-to-all
    moves them, and each card groups what it received by expert; rank r owns
    experts [r*E/W, (r+1)*E/W).  Built here by walking the layouts in order:

      send buffer   sources s = 0..W-1 one after another; inside a source,
                    experts in order (so destinations in order), inside an
                    expert its kept pairs in token order;
      receive side  destinations r = 0..W-1 one after another; inside r, the
                    chunk of each source s in order, each chunk being source
                    s's send rows for rank r (the all-to-all);
      regrouped     inside r, experts in order, inside an expert the sources
                    in order, inside a source its rows in token order.

    topk_idx [N, K] and dest [N, K] (row of each kept pair in the one-source
    dispatch, -1 when dropped).  Returns a dict: C [W, E] kept pairs per
    (source, expert); D [W, W] pairs per (source, destination rank); and
    three gather maps over rows, each a list of source-row indices:
    send_token (send row -> token), a2a_src (receive row -> send row),
    regroup_src (regrouped row -> receive row); plus send_row [N, K] (send
    row of each kept pair, -1 when dropped).
    """
    idx = np.asarray(topk_idx)
    dest = np.asarray(dest)
    N, K = idx.shape
    per_rank = E // W
    lo = shard_bounds(N, W)
    shard = [0] * N
    for s in range(W):
        for t in range(lo[s], lo[s + 1]):
            shard[t] = s
    # kept pairs by (source, expert), each list in token order
    pairs = [[[] for _ in range(E)] for _ in range(W)]
    for t in range(N):
        for k in range(K):
            if dest[t, k] >= 0:
                pairs[shard[t]][int(idx[t, k])].append((t, k))
    C = np.array([[len(pairs[s][e]) for e in range(E)] for s in range(W)], dtype=np.int64)
    D = np.array([[int(C[s][r * per_rank:(r + 1) * per_rank].sum()) for r in range(W)]
                  for s in range(W)], dtype=np.int64)

    send_token, send_row = [], np.full((N, K), -1, dtype=np.int64)
    send_pos = {}
    for s in range(W):
        for e in range(E):
            for (t, k) in pairs[s][e]:
                send_pos[(t, k)] = len(send_token)
                send_row[t, k] = len(send_token)
                send_token.append(t)
    a2a_src, recv_pos = [], {}
    for r in range(W):
        for s in range(W):
            for e in range(r * per_rank, (r + 1) * per_rank):
                for (t, k) in pairs[s][e]:
                    recv_pos[(t, k)] = len(a2a_src)
                    a2a_src.append(send_pos[(t, k)])
    regroup_src, regroup_pair = [], []
    for r in range(W):
        for e in range(r * per_rank, (r + 1) * per_rank):
            for s in range(W):
                for (t, k) in pairs[s][e]:
                    regroup_src.append(recv_pos[(t, k)])
                    regroup_pair.append((t, k))
    return {
        "C": C.astype(np.int32),
        "D": D.astype(np.int32),
        "send_token": np.array(send_token, dtype=np.int32),
        "send_row": send_row.astype(np.int32),
        "a2a_src": np.array(a2a_src, dtype=np.int32),
        "regroup_src": np.array(regroup_src, dtype=np.int32),
        "regroup_pair": regroup_pair,
    }


def tau_min(D, bandwidth=1.0):
    """Lower bound on the all-to-all time for traffic matrix D (rows sent by
    source i to destination j): the busiest sender's or receiver's volume
    over the per-GPU bandwidth ("MoE Inference Communication", Aurora,
    Theorem 4.2).  Only traffic that leaves a rank counts: the diagonal
    (a rank's pairs for its own experts) moves no data over a link."""
    D = np.asarray(D, dtype=np.float64)
    off = D - np.diag(np.diag(D))
    return max(off.sum(axis=1).max(), off.sum(axis=0).max()) / bandwidth

"""HIP path vs the CPU oracle, element by element, on seeded inputs.

Integer results (topk_idx, demand, counts, offsets, rank_offsets, dest,
perm_token) and the permuted payload x_perm must match bit for bit.  Floating
results must satisfy, per element, |got - ref| <= atol + rtol * |ref| with
  bf16 layers: atol = 2e-2, rtol = 1e-2   (h, y_perm, out)
  fp32 layers: atol = 1e-4, rtol = 1e-4
  gate weights: |got - ref| <= 1e-6.
Small shapes and the full-size layers up to a few TFLOP of oracle FFN run
the whole oracle; the dropless prefill-size layers run the oracle's route and
dispatch in full and its FFN and combine on rows sampled from every row tile.
"""
import numpy as np
import pytest
import torch

from grouped_gemm_route_amd import binding as B
from grouped_gemm_route_amd import synth
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-4)}
W_TOL = 1e-6
DEV = "cuda:0"


def _np(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def _close(name, got, ref, act):
    atol, rtol = TOL[act]
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    assert not bad.any(), (
        f"{name}: {int(bad.sum())} of {bad.size} elements out of tolerance; "
        f"max abs err {err.max():.3e}")


def _cap(cfg):
    if cfg.get("cap") is not None:
        return cfg["cap"]
    return O.capacity(cfg["C"], cfg["N"], cfg["K"], cfg["E"]) if cfg["C"] is not None else -1


def _run_gpu(cfg, inp, cap, packed=False):
    """One layer call; packed=True streams the weights from the layout of
    moe_pack_ffn_weights (bf16 layers)."""
    layer = B.MoeLayer(cfg["N"], cfg["d"], cfg["ffn"], cfg["E"], cfg["K"], cfg["W"], cap,
                       synth.TORCH_DTYPE[cfg["act"]], DEV, cfg.get("renormalize", False))
    if packed:
        pw = B.moe_pack_ffn_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
        layer.forward(inp["logits"], inp["x"], pw)
    else:
        layer.forward(inp["logits"], inp["x"], inp["w_gate"], inp["w_up"], inp["w_down"])
    torch.cuda.synchronize()
    return layer


def _layers(cfg, inp, cap):
    """The plain-weight layer and, for bf16 layers, the packed-weight one,
    one after the other."""
    yield "plain", _run_gpu(cfg, inp, cap)
    if cfg["act"] == "bf16":
        yield "packed", _run_gpu(cfg, inp, cap, packed=True)


def _expert_weights_np(inp):
    cache = {}

    def fn(e):
        if e not in cache:
            cache.clear()
            cache[e] = tuple(_np(inp[k][e]) for k in ("w_gate", "w_up", "w_down"))
        return cache[e]
    return fn


def _check_route_dispatch(cfg, layer, ref, x_dev):
    assert np.array_equal(_np(layer.topk_idx), ref["topk_idx"])
    dw = np.abs(_np(layer.topk_w).astype(np.float64) - ref["topk_w"].astype(np.float64))
    assert dw.max() <= W_TOL, dw.max()
    d = layer.disp
    for k in ("demand", "counts", "offsets", "rank_offsets", "dest"):
        assert np.array_equal(_np(d[k]), ref[k]), k
    M = int(ref["offsets"][-1])
    assert np.array_equal(_np(d["perm_token"])[:M], ref["perm_token"])
    perm = torch.from_numpy(ref["perm_token"].astype(np.int64)).to(DEV)
    assert torch.equal(d["x_perm"][:M], x_dev[perm])          # bitwise row copies
    return M


# ---------------------------------------------------------------------------
# small shapes: whole oracle
# ---------------------------------------------------------------------------

SMALL = {
    "tiny_f32": synth.config("tiny_f32"),
    "ragged_bf16": synth.config("ragged_bf16", N=700, d=256, ffn=320, E=4, K=2, W=2,
                                act="bf16", C=None),
    "ragged_bf16_c0.8": synth.config("ragged_bf16_c0.8", N=700, d=256, ffn=320, E=4, K=2,
                                     W=2, act="bf16", C=0.8),
    "skew_bf16_c1.25": synth.config("skew_bf16_c1.25", N=512, d=128, ffn=192, E=32, K=4,
                                    W=8, act="bf16", bias="zipf", C=1.25),
    "single_token": synth.config("single_token", N=1, d=64, ffn=64, E=8, K=2, W=2,
                                 act="bf16", C=None),
    "k_equals_e": synth.config("k_equals_e", N=37, d=64, ffn=128, E=4, K=4, W=4,
                               act="bf16", C=None),
    "one_expert": synth.config("one_expert", N=50, d=128, ffn=64, E=1, K=1, W=1,
                               act="bf16", C=None),
    "capacity_zero": synth.config("capacity_zero", N=40, d=64, ffn=64, E=8, K=2, W=4,
                                  act="bf16", cap=0),
    "e256_small": synth.config("e256_small", N=64, d=64, ffn=64, E=256, K=8, W=8,
                               act="bf16", C=None),
    "e1024_k16": synth.config("e1024_k16", N=40, d=64, ffn=64, E=1024, K=16, W=8,
                              act="bf16", C=None),
    "f32_nonpow2": synth.config("f32_nonpow2", N=100, d=24, ffn=40, E=6, K=3, W=3,
                                act="f32", C=1.0),
    # fp32 layers whose reductions take two 128-element chunks, the second
    # ragged (gate/up 128 + 72, down 128 + 8), with experts of several
    # 32-row tiles
    "f32_two_chunks": synth.config("f32_two_chunks", N=300, d=200, ffn=136, E=5, K=2, W=5,
                                   act="f32", C=None),
    "renormalized": synth.config("renormalized", N=90, d=64, ffn=64, E=16, K=4, W=4,
                                 act="bf16", C=None, renormalize=True),
    "many_blocks_e8": synth.config("many_blocks_e8", N=1500, d=64, ffn=128, E=8, K=2, W=8,
                                   act="bf16", C=1.1),
    # grids smaller than one round of resident blocks, with reductions long
    # enough to be worth splitting: the grouped GEMMs split tiles along the
    # reduction (here both passes of both kernels: 8 pieces per tile in the
    # packed-weight kernel, 4 and 8 in the row-major one; split8_bf16: 8 in
    # the gate/up pass)
    "split_reduce_bf16": synth.config("split_reduce_bf16", N=48, d=4096, ffn=4096, E=2, K=2,
                                      W=2, act="bf16", C=None),
    "split8_bf16": synth.config("split8_bf16", N=29, d=4096, ffn=512, E=2, K=1, W=2,
                                act="bf16", C=None),
    # the same splits at the tile heights of the full-size layers: 128-row
    # tiles of the packed-weight kernel and 256-row tiles of the row-major one.
    # One expert of 512 rows: every pass splits (packed gate/up 4 pieces, down
    # 8; row-major gate/up 4, down 8); two ragged experts (278 and 234 rows):
    # the down passes split (6 and 5 pieces) with partly empty last tiles; one
    # expert of 600 rows and ffn 2048: the gate/up passes split (6 and 5) with
    # an 88-row last tile.
    "split_full_e1": synth.config("split_full_e1", N=512, d=4096, ffn=4096, E=1, K=1, W=1,
                                  act="bf16", C=None),
    "split_full_ragged_e2": synth.config("split_full_ragged_e2", N=512, d=4096, ffn=4096,
                                         E=2, K=1, W=2, act="bf16", C=None),
    "split_full_tail": synth.config("split_full_tail", N=600, d=4096, ffn=2048, E=1, K=1, W=1,
                                    act="bf16", C=None),
}


def _small_inputs(cfg, logits_override=None):
    inp = synth.make_inputs(cfg, DEV)
    if logits_override is not None:
        inp["logits"] = logits_override.to(DEV)
    return inp


def _check_small(cfg, inp):
    cap = _cap(cfg)
    ref = O.layer(_np(inp["logits"]), _np(inp["x"]), _expert_weights_np(inp), cfg["K"],
                  cfg["W"], cap, cfg["act"], cfg.get("renormalize", False))
    for kind, layer in _layers(cfg, inp, cap):
        print(f"[parity]   {kind} weights", flush=True)
        M = _check_route_dispatch(cfg, layer, ref, inp["x"])
        if M > 0:
            _close(f"{kind} h", _np(layer.h)[:M], ref["h"], cfg["act"])
            _close(f"{kind} y_perm", _np(layer.y_perm)[:M], ref["y_perm"], cfg["act"])
        _close(f"{kind} out", _np(layer.out), ref["out"], cfg["act"])
    return layer, ref


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_layer_matches_oracle(name):
    cfg = SMALL[name]
    print(f"[parity] {name} {cfg}", flush=True)
    layer, ref = _check_small(cfg, _small_inputs(cfg))
    if name == "capacity_zero":
        assert ref["offsets"][-1] == 0 and (_np(layer.out) == 0).all()


def test_tied_logits_match_oracle():
    cfg = synth.config("ties", N=300, d=64, ffn=64, E=16, K=4, W=4, act="bf16", C=1.0)
    g = torch.Generator().manual_seed(5)
    logits = (torch.randint(-2, 3, (cfg["N"], cfg["E"]), generator=g) * 0.5).float()
    logits[::5] = 0.0
    logits[1::7] = -0.0
    _check_small(cfg, _small_inputs(cfg, logits))


def test_unused_rows_are_not_written():
    cfg = SMALL["ragged_bf16_c0.8"]
    inp = _small_inputs(cfg)
    cap = _cap(cfg)
    layer = B.MoeLayer(cfg["N"], cfg["d"], cfg["ffn"], cfg["E"], cfg["K"], cfg["W"], cap,
                       torch.bfloat16, DEV)
    sentinel = torch.tensor(-12345.0, dtype=torch.bfloat16)
    for t in (layer.disp["x_perm"], layer.h, layer.y_perm):
        t.fill_(sentinel)
    layer.disp["perm_token"].fill_(-7)
    layer.forward(inp["logits"], inp["x"], inp["w_gate"], inp["w_up"], inp["w_down"])
    torch.cuda.synchronize()
    M = int(layer.disp["offsets"][-1])
    assert M < cfg["N"] * cfg["K"]
    for t in (layer.disp["x_perm"], layer.h, layer.y_perm):
        assert bool((t[M:] == sentinel).all())
    assert bool((layer.disp["perm_token"][M:] == -7).all())


def test_runs_are_bitwise_deterministic():
    cfg = SMALL["skew_bf16_c1.25"]
    inp = _small_inputs(cfg)
    a = _run_gpu(cfg, inp, _cap(cfg))
    b = _run_gpu(cfg, inp, _cap(cfg))
    M = int(a.disp["offsets"][-1])
    for name in ("topk_idx", "topk_w", "out"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    for name in ("h", "y_perm"):                      # rows >= M are never written
        assert torch.equal(getattr(a, name)[:M], getattr(b, name)[:M]), name
    for k in ("perm_token",):
        assert torch.equal(a.disp[k][:M], b.disp[k][:M]), k
    for k in ("dest", "offsets", "counts", "demand", "rank_offsets"):
        assert torch.equal(a.disp[k], b.disp[k]), k
    assert torch.equal(a.disp["x_perm"][:M], b.disp["x_perm"][:M])


@pytest.mark.parametrize("packed", [False, True])
def test_split_reduction_is_bitwise_deterministic(packed):
    # split tiles are summed in piece order whichever piece finishes last
    cfg = SMALL["split_reduce_bf16"]
    inp = _small_inputs(cfg)
    a = _run_gpu(cfg, inp, _cap(cfg), packed)
    M = int(a.disp["offsets"][-1])
    for _ in range(3):
        b = _run_gpu(cfg, inp, _cap(cfg), packed)
        assert torch.equal(a.h[:M], b.h[:M])
        assert torch.equal(a.y_perm[:M], b.y_perm[:M])
        assert torch.equal(a.out, b.out)


def test_identity_ffn_round_trip_is_bitwise():
    # dispatch then combine with the FFN replaced by the identity and one-hot
    # gate weights gives back x exactly (kept slot 0) or a zero row
    cfg = SMALL["ragged_bf16_c0.8"]
    inp = _small_inputs(cfg)
    layer = B.MoeLayer(cfg["N"], cfg["d"], cfg["ffn"], cfg["E"], cfg["K"], cfg["W"],
                       _cap(cfg), torch.bfloat16, DEV)
    layer.route(inp["logits"])
    layer.dispatch(inp["x"])
    onehot = torch.zeros_like(layer.topk_w)
    onehot[:, 0] = 1.0
    out = B.moe_combine(layer.disp["x_perm"], layer.disp["dest"], onehot)
    torch.cuda.synchronize()
    kept0 = layer.disp["dest"][:, 0] >= 0
    assert torch.equal(out[kept0], inp["x"][kept0])
    assert bool((out[~kept0] == 0).all())


# ---------------------------------------------------------------------------
# full-size layers
# ---------------------------------------------------------------------------

# Whole: every element of h, y_perm and out against the oracle's whole layer
# (the oracle's FFN takes a few seconds per layer in float64 BLAS).
WHOLE = ["dense8", "fine128_zipf_c1.25", "decode256", "prefill256_hot_c1.0"]
# Sampled (dropless prefill sizes, 10-23 TFLOP of oracle FFN): one row drawn
# from every 128-row block of every expert's rows plus every expert's last
# row, so every row tile of 128 rows or more, every expert's ragged last tile
# and every (row tile, column tile) unit -- split ones included -- holds a
# checked row; h and y_perm are compared on those rows, out on their tokens.
SAMPLED = ["prefill256_hot", "prefill256_cal", "prefill256_cal_c1.0"]
SAMPLE_BLOCK = 128


def _close_chunked(name, got_t, ref, act, chunk=4096):
    """_close over row chunks of a device tensor (bounded host memory)."""
    n = ref.shape[0]
    assert got_t.shape[0] >= n, (name, got_t.shape, ref.shape)
    for r0 in range(0, n, chunk):
        r1 = min(n, r0 + chunk)
        _close(f"{name}[{r0}:{r1}]", _np(got_t[r0:r1]), ref[r0:r1], act)


def _full_inputs(name):
    cfg = synth.config(name)
    print(f"[parity] {name} {cfg}", flush=True)
    inp = synth.make_inputs(cfg, DEV)
    cap = _cap(cfg)
    idx, w = O.route(_np(inp["logits"]), cfg["K"])
    ref = O.dispatch(idx, cfg["E"], cfg["W"], cap)
    ref.update(topk_idx=idx, topk_w=w)
    return cfg, inp, cap, ref


@pytest.mark.parametrize("name", WHOLE)
def test_full_size_layer_matches_oracle_whole(name):
    cfg, inp, cap, ref = _full_inputs(name)
    M = int(ref["offsets"][-1])
    x_perm = O.pack(_np(inp["x"]), ref["perm_token"])
    h_ref, y_ref = O.grouped_ffn(x_perm, ref["offsets"], _expert_weights_np(inp), cfg["act"])
    del x_perm
    out_ref = O.combine(y_ref, ref["dest"], ref["topk_w"], cfg["act"])
    print(f"[parity] {name}: oracle layer done, M={M} dropped={ref['dropped']}", flush=True)
    for kind, layer in _layers(cfg, inp, cap):
        assert _check_route_dispatch(cfg, layer, ref, inp["x"]) == M
        print(f"[parity] {name} {kind} weights: comparing h, y_perm, out", flush=True)
        _close_chunked(f"{kind} h", layer.h, h_ref, cfg["act"])
        _close_chunked(f"{kind} y_perm", layer.y_perm, y_ref, cfg["act"])
        _close_chunked(f"{kind} out", layer.out, out_ref, cfg["act"])
        del layer
        torch.cuda.empty_cache()


def _tile_sample_rows(offsets, rng):
    """One random row of every SAMPLE_BLOCK-row block of each expert's rows,
    and each expert's last row."""
    rows = []
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        for r0 in range(a, b, SAMPLE_BLOCK):
            rows.append(int(rng.integers(r0, min(b, r0 + SAMPLE_BLOCK))))
        if b > a:
            rows.append(b - 1)
    return np.unique(np.array(rows, dtype=np.int64))


@pytest.mark.parametrize("name", SAMPLED)
def test_full_size_layer_matches_oracle_sampled(name):
    cfg, inp, cap, ref = _full_inputs(name)
    M = int(ref["offsets"][-1])
    offsets = ref["offsets"]
    rows = _tile_sample_rows(offsets, np.random.default_rng(0))
    # coverage: every non-empty expert's first block, its last (ragged) row
    # tile and every block in between hold a sampled row
    for e in range(cfg["E"]):
        a, b = int(offsets[e]), int(offsets[e + 1])
        for r0 in range(a, b, SAMPLE_BLOCK):
            assert ((rows >= r0) & (rows < min(b, r0 + SAMPLE_BLOCK))).any(), (e, r0)
    toks = np.unique(ref["perm_token"][rows])
    print(f"[parity] {name}: M={M} dropped={ref['dropped']}, {len(rows)} sampled rows, "
          f"{len(toks)} tokens", flush=True)
    x_np = _np(inp["x"][torch.from_numpy(toks).to(DEV)])
    y_rows, out_ref = O.token_outputs(toks, x_np, ref["topk_idx"], ref["topk_w"], ref["dest"],
                                      _expert_weights_np(inp), cfg["act"])
    # h and y_perm of the sampled rows, expert by expert
    weights = _expert_weights_np(inp)
    row_expert = np.searchsorted(offsets, rows, side="right") - 1
    x_rows = _np(inp["x"][torch.from_numpy(ref["perm_token"][rows].astype(np.int64)).to(DEV)])
    h_ref = {}
    for e in np.unique(row_expert):
        sel = np.nonzero(row_expert == e)[0]
        h_e, y_e = O.expert_ffn(x_rows[sel], *weights(int(e)), cfg["act"])
        for i, j in enumerate(sel):
            h_ref[int(rows[j])] = (h_e[i], y_e[i])
    rows_t = torch.from_numpy(rows).to(DEV)
    toks_t = torch.from_numpy(toks.astype(np.int64)).to(DEV)
    for kind, layer in _layers(cfg, inp, cap):
        assert _check_route_dispatch(cfg, layer, ref, inp["x"]) == M
        print(f"[parity] {name} {kind} weights: comparing sampled rows", flush=True)
        h_got = _np(layer.h[rows_t])
        y_got = _np(layer.y_perm[rows_t])
        _close(f"{kind} h", h_got, np.stack([h_ref[int(r)][0] for r in rows]), cfg["act"])
        _close(f"{kind} y_perm", y_got, np.stack([h_ref[int(r)][1] for r in rows]), cfg["act"])
        pair_rows = np.array([int(ref["dest"][t, k]) for (t, k) in y_rows], dtype=np.int64)
        _close(f"{kind} y_perm (pairs of sampled tokens)",
               _np(layer.y_perm[torch.from_numpy(pair_rows).to(DEV)]),
               np.stack(list(y_rows.values())), cfg["act"])
        _close(f"{kind} out", _np(layer.out[toks_t]), out_ref, cfg["act"])
        del layer
        torch.cuda.empty_cache()

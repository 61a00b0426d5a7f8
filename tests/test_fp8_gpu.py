"""FP8 exchange payload on the GPU against the oracle: e4m3 codes and scales
bit for bit (both sides quantize in fp32 with round-to-nearest-even),
dequantized bf16 rows bit for bit, routing outputs bit for bit, and the
combined output within the bf16 tolerance |err| <= 2e-2 + 1e-2 |ref|."""
import numpy as np
import pytest
import torch

from grouped_gemm_route_amd import binding as B
from grouped_gemm_route_amd import synth
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ATOL, RTOL = 2e-2, 1e-2


def _np(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def _rows(R, d, seed):
    """bf16 rows whose 128-column groups span many magnitudes, with zero
    groups, negative zeros and values that land in the subnormal codes."""
    g = torch.Generator().manual_seed(seed)
    g_sign = torch.Generator().manual_seed(seed + 1)
    x = torch.randn(R, d, generator=g)
    mag = 10.0 ** torch.randint(-6, 5, (R, d // 128), generator=g).float()
    x = x * mag.repeat_interleave(128, dim=1)
    x[1, :128] = 0.0
    x[2, 128:256] = -0.0
    x[3, :] = x[3, :] * 1e-3
    x[3, 0] = 50.0                               # most of the group in subnormal codes
    x[4, 256:384] *= 1e-32                       # below 2^-100: zero codes
    if R > 5:
        # a group whose maximum is 448 (scale 1): every value is an exact
        # e4m3 value or the midpoint of two, so rounding ties decide the codes
        t = torch.tensor(O.e4m3_value(np.arange(0x7F)))
        mids = (t[1:] + t[:-1]) / 2
        g = torch.cat([t, mids])[torch.randperm(2 * 0x7F - 1, generator=g)[:127]]
        g = g * torch.where(torch.rand(127, generator=g_sign) < 0.5, -1.0, 1.0)
        x[5, :128] = torch.cat([torch.tensor([448.0]), g])
    return x.to(torch.bfloat16)


def _close(name, got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    assert not bad.any(), f"{name}: {int(bad.sum())} out of tolerance, max err {err.max():.3e}"


@pytest.mark.parametrize("R,d,n", [(37, 512, 37), (64, 4096, 50), (5, 7168, 5), (9, 128, 0)])
def test_quantize_and_dequantize_rows_match_oracle(R, d, n):
    print(f"[fp8] rows R={R} d={d} n={n}", flush=True)
    x = _rows(R, d, R + d).to(DEV)
    n_rows = torch.tensor([n], dtype=torch.int32, device=DEV)
    q = torch.full((R, d), 0xAB, dtype=torch.uint8, device=DEV)
    s = torch.full((R, d // 128), -1.0, dtype=torch.float32, device=DEV)
    B.moe_fp8_quantize_rows(x, n_rows, R, q, s)
    back = torch.full((R, d), 7.0, dtype=torch.bfloat16, device=DEV)
    B.moe_fp8_dequantize_rows(q, s, n_rows, R, back)
    torch.cuda.synchronize()
    rq, rs = O.quantize_fp8(_np(x)[:n])
    assert np.array_equal(_np(q)[:n], rq)
    assert np.array_equal(_np(s)[:n], rs)
    assert (_np(q)[n:] == 0xAB).all() and (_np(s)[n:] == -1.0).all()   # rows >= n untouched
    ref_back = O.round_storage(O.dequantize_fp8(rq, rs).astype(np.float64), "bf16")
    assert np.array_equal(_np(back)[:n], ref_back)
    assert (_np(back)[n:] == 7.0).all()


def test_every_code_and_every_tie():
    # groups whose maximum is 448 (scale 1) holding every finite e4m3 value
    # and every midpoint of neighbours, both signs: each code decision is a
    # table hit or an exact tie; then every code is decoded with scale 1
    t = O.e4m3_value(np.arange(0x7F))
    vals = np.concatenate([t, (t[1:] + t[:-1]) / 2])
    vals = np.concatenate([vals, -vals])
    per = 127
    n_groups = -(-len(vals) // per)
    rows = np.zeros((n_groups, 128), np.float32)
    rows[:, 0] = 448.0
    flat = np.zeros(n_groups * per, np.float32)
    flat[:len(vals)] = vals
    rows[:, 1:] = flat.reshape(n_groups, per)
    x = torch.from_numpy(rows).to(torch.bfloat16)
    assert np.array_equal(x.float().numpy(), rows)              # exact in bf16
    xd = x.to(DEV)
    n = torch.tensor([n_groups], dtype=torch.int32, device=DEV)
    q, s = B.moe_fp8_quantize_rows(xd, n)
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).reshape(2, 128).to(DEV)
    ones = torch.ones(2, 1, dtype=torch.float32, device=DEV)
    back = B.moe_fp8_dequantize_rows(codes, ones, torch.tensor([2], dtype=torch.int32,
                                                               device=DEV))
    torch.cuda.synchronize()
    rq, rs = O.quantize_fp8(rows)
    assert np.array_equal(_np(q), rq) and np.array_equal(_np(s), rs)
    ref = O.e4m3_value(np.arange(256)).reshape(2, 128)
    got = _np(back).astype(np.float64)
    finite = ~np.isnan(ref)
    assert np.array_equal(got[finite], ref[finite])             # each value exact in bf16
    assert np.isnan(got[~finite]).all()


def _fp8_dispatch(cfg, cap):
    inp = synth.make_inputs(cfg, DEV, weights=False)
    idx, w = B.moe_route_topk(inp["logits"], cfg["K"])
    out = B.moe_dispatch_fp8(inp["x"], idx, cfg["E"], cfg["W"], cap)
    torch.cuda.synchronize()
    ri, rw = O.route(_np(inp["logits"]), cfg["K"])
    ref = O.dispatch(ri, cfg["E"], cfg["W"], cap)
    for k in ("demand", "counts", "offsets", "rank_offsets", "dest"):
        assert np.array_equal(_np(out[k]), ref[k]), k
    M = int(ref["offsets"][-1])
    assert np.array_equal(_np(out["perm_token"])[:M], ref["perm_token"])
    return inp, idx, w, out, ref, M


@pytest.mark.parametrize("name,over", [
    ("dense8", {}),
    ("fine128_zipf_c1.25", {}),
    ("small_c0.7", dict(N=300, d=256, ffn=128, E=8, K=2, W=4, act="bf16", C=0.7)),
    ("e256_k8", dict(N=200, d=384, ffn=128, E=256, K=8, W=8, act="bf16", C=None)),
])
def test_dispatch_fp8_matches_oracle(name, over):
    cfg = synth.config(name, **over)
    print(f"[fp8] dispatch {name}", flush=True)
    cap = O.capacity(cfg["C"], cfg["N"], cfg["K"], cfg["E"]) if cfg["C"] is not None else -1
    inp, idx, w, out, ref, M = _fp8_dispatch(cfg, cap)
    # every token's codes once (a token's rows are identical copies)
    tq, ts = O.quantize_fp8(_np(inp["x"]))
    pt = ref["perm_token"].astype(np.int64)
    assert np.array_equal(_np(out["x8"])[:M], tq[pt])
    assert np.array_equal(_np(out["x_scale"])[:M], ts[pt])


def test_combine_fp8_matches_oracle():
    cfg = synth.config("combine_fp8", N=500, d=512, ffn=128, E=8, K=4, W=4, act="bf16", C=0.9)
    cap = O.capacity(cfg["C"], cfg["N"], cfg["K"], cfg["E"])
    inp, idx, w, out, ref, M = _fp8_dispatch(cfg, cap)
    # expert outputs: any bf16 rows; quantize on the GPU, combine from fp8
    y = _rows(M, cfg["d"], 11).to(DEV)
    n_rows = out["offsets"][cfg["E"]:]
    y8, ys = B.moe_fp8_quantize_rows(y, n_rows)
    got = B.moe_combine_fp8(y8, ys, out["dest"], w)
    torch.cuda.synchronize()
    yq, yqs = O.quantize_fp8(_np(y))
    assert np.array_equal(_np(y8), yq) and np.array_equal(_np(ys), yqs)
    ref_out = O.combine(O.dequantize_fp8(yq, yqs).astype(np.float64), ref["dest"], _np(w), "bf16")
    _close("out", _np(got), ref_out)
    dropped = (ref["dest"] < 0).all(1)
    assert dropped.any() and (_np(got)[dropped] == 0).all()


def test_fp8_layer_matches_oracle():
    cfg = synth.config("fp8_layer", N=400, d=256, ffn=192, E=8, K=2, W=4, act="bf16", C=1.0)
    cap = O.capacity(cfg["C"], cfg["N"], cfg["K"], cfg["E"])
    inp = synth.make_inputs(cfg, DEV)
    layer = B.MoeLayer(cfg["N"], cfg["d"], cfg["ffn"], cfg["E"], cfg["K"], cfg["W"], cap,
                       torch.bfloat16, DEV, fp8=True)
    layer.forward(inp["logits"], inp["x"], inp["w_gate"], inp["w_up"], inp["w_down"])
    torch.cuda.synchronize()

    def weights(e):
        return tuple(_np(inp[k][e]) for k in ("w_gate", "w_up", "w_down"))
    ref = O.layer(_np(inp["logits"]), _np(inp["x"]), weights, cfg["K"], cfg["W"], cap, "bf16",
                  fp8=True)
    M = int(ref["offsets"][-1])
    assert np.array_equal(_np(layer.disp["x8"])[:M], ref["x8"])
    assert np.array_equal(_np(layer.disp["x_perm"])[:M], ref["x_perm"])   # dequantized rows
    _close("h", _np(layer.h)[:M], ref["h"])
    _close("y_perm", _np(layer.y_perm)[:M], ref["y_perm"])
    # The combine's fp8 input is the GPU's own y rows, quantized exactly.  It
    # is compared from those codes: y rows that differ from the oracle's by
    # a bf16 rounding can fall on either side of an e4m3 rounding boundary,
    # one code step (1/16 relative) apart, which no bf16 tolerance covers.
    yq, ys = O.quantize_fp8(_np(layer.y_perm)[:M])
    assert np.array_equal(_np(layer.y8)[:M], yq) and np.array_equal(_np(layer.y_scale)[:M], ys)
    ref_out = O.combine(O.dequantize_fp8(yq, ys).astype(np.float64), ref["dest"],
                        ref["topk_w"], "bf16")
    _close("out", _np(layer.out), ref_out)


def test_fp8_full_size_dense_layer():
    cfg = synth.config("dense8")
    print("[fp8] dense8 layer", flush=True)
    inp = synth.make_inputs(cfg, DEV)
    layer = B.MoeLayer(cfg["N"], cfg["d"], cfg["ffn"], cfg["E"], cfg["K"], cfg["W"], -1,
                       torch.bfloat16, DEV, fp8=True)
    layer.forward(inp["logits"], inp["x"], inp["w_gate"], inp["w_up"], inp["w_down"])
    torch.cuda.synchronize()
    M = int(layer.disp["offsets"][-1])
    # sampled tokens: their x8 rows, and the combine of their fp8 y rows
    rng = np.random.default_rng(0)
    toks = np.array(sorted(set([0, cfg["N"] - 1] + rng.choice(cfg["N"], 6, replace=False).tolist())))
    dest = _np(layer.disp["dest"])[toks]
    xq, xs = O.quantize_fp8(_np(inp["x"][torch.from_numpy(toks).to(DEV)]))
    for i, t in enumerate(toks):
        for k in range(cfg["K"]):
            row = int(dest[i, k])
            assert np.array_equal(_np(layer.disp["x8"][row]), xq[i])
            assert np.array_equal(_np(layer.disp["x_scale"][row]), xs[i])
    rows = np.unique(dest[dest >= 0])
    yq, ys = O.quantize_fp8(_np(layer.y_perm[torch.from_numpy(rows).to(DEV)]))
    assert np.array_equal(_np(layer.y8[torch.from_numpy(rows).to(DEV)]), yq)
    # the oracle's combine over the sampled tokens' rows: their fp8 values
    # renumbered 0 .. len(rows) - 1, dest remapped to match
    lut = {int(r): j for j, r in enumerate(rows)}
    dest_s = np.vectorize(lambda r: lut[int(r)] if r >= 0 else -1)(dest).astype(np.int32)
    ref = O.combine(O.dequantize_fp8(yq, ys).astype(np.float64), dest_s,
                    _np(layer.topk_w)[toks], "bf16")
    _close("out", _np(layer.out[torch.from_numpy(toks).to(DEV)]), ref)

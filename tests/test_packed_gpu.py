"""Packed expert weights on the GPU: moe_pack_ffn_weights writes exactly the
layout include/moe_route.h documents (checked byte for byte against a numpy
rearrangement of the same formula), and moe_grouped_ffn_packed matches the
oracle on layers whose tiles split along the reduction, repeatably, with a
workspace shared with moe_grouped_ffn."""
import numpy as np
import pytest
import torch

from grouped_gemm_route_amd import binding as B
from grouped_gemm_route_amd import synth
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ATOL, RTOL = 2e-2, 1e-2


def _u16(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def _expected_packed(w_gate, w_up, w_down):
    """The documented layout: panels of 128 rows; per 16-wide reduction step
    four 1 KB fragments of 32 rows; lane l of fragment i holds the 8 values
    W[row(i, l % 32)][16 s + 8 (l // 32) : + 8]."""
    E, ffn, d = w_gate.shape

    def frag_rows(rows_of_panel, W, K):  # rows_of_panel: [P, 4, 32] (matrix, row) or None: zero
        P = rows_of_panel.shape[0]
        S = K // 16
        out = np.zeros((E, P, S, 4, 64, 8), np.uint16)
        for e in range(E):
            for p in range(P):
                for i in range(4):
                    for l in range(64):
                        r = rows_of_panel[p, i, l % 32]
                        if r is None:
                            continue
                        src, row = r
                        vals = W[src][e, row].reshape(S, 2, 8)[:, l // 32, :]
                        out[e, p, :, i, l, :] = vals
        return out

    P_up = ffn // 64
    rows_up = np.empty((P_up, 4, 32), object)
    for p in range(P_up):
        for i in range(4):
            for r in range(32):
                rows_up[p, i, r] = (0 if i < 2 else 1, p * 64 + (i % 2) * 32 + r)
    up = frag_rows(rows_up, [_u16(w_gate), _u16(w_up)], d)
    P_dn = -(-d // 128)
    rows_dn = np.empty((P_dn, 4, 32), object)
    for p in range(P_dn):
        for i in range(4):
            for r in range(32):
                row = p * 128 + i * 32 + r
                rows_dn[p, i, r] = (0, row) if row < d else None
    dn = frag_rows(rows_dn, [_u16(w_down)], ffn)
    return up, dn


@pytest.mark.parametrize("E,d,ffn", [(2, 128, 64), (3, 320, 192)])
def test_pack_layout_matches_documented_offsets(E, d, ffn):
    print(f"[packed] layout E={E} d={d} ffn={ffn}", flush=True)
    g = torch.Generator().manual_seed(E * 1000 + d)
    ws = [torch.randn(E, ffn, d, generator=g), torch.randn(E, ffn, d, generator=g),
          torch.randn(E, d, ffn, generator=g)]
    wg, wu, wd = (w.to(torch.bfloat16).to(DEV) for w in ws)
    pw = B.moe_pack_ffn_weights(wg, wu, wd)
    torch.cuda.synchronize()
    up, dn = _expected_packed(wg, wu, wd)
    assert pw.up.numel() == up.nbytes == B.moe_packed_ffn_weight_bytes(E, d, ffn, B.MOE_FFN_GATE_UP)
    assert pw.down.numel() == dn.nbytes == B.moe_packed_ffn_weight_bytes(E, d, ffn, B.MOE_FFN_DOWN)
    assert np.array_equal(pw.up.cpu().numpy().view(np.uint16), up.reshape(-1))
    assert np.array_equal(pw.down.cpu().numpy().view(np.uint16), dn.reshape(-1))


def _ffn_case(cfg):
    inp = synth.make_inputs(cfg, DEV)
    layer = B.MoeLayer(cfg["N"], cfg["d"], cfg["ffn"], cfg["E"], cfg["K"], cfg["W"], -1,
                       torch.bfloat16, DEV)
    layer.route(inp["logits"])
    layer.dispatch(inp["x"])
    torch.cuda.synchronize()
    return inp, layer


def _oracle_rows(inp, layer, M):
    off = layer.disp["offsets"].cpu().numpy()
    x = layer.disp["x_perm"][:M].float().cpu().numpy()
    h = np.zeros((M, inp["w_gate"].shape[1]))
    y = np.zeros((M, inp["w_gate"].shape[2]))
    for e in range(len(off) - 1):
        a, b = off[e], off[e + 1]
        if b > a:
            wg, wu, wd = (inp[k][e].float().cpu().numpy() for k in ("w_gate", "w_up", "w_down"))
            h[a:b], y[a:b] = O.expert_ffn(x[a:b], wg, wu, wd, "bf16")
    return h, y


def _close(name, got, ref):
    err = np.abs(got.astype(np.float64) - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    assert not bad.any(), f"{name}: {int(bad.sum())} bad, max err {err.max():.3e}"


@pytest.mark.parametrize("case", [
    # grids below one round of resident blocks with long reductions: tiles
    # split along the reduction (both passes here, the gate/up pass next)
    dict(N=48, d=4096, ffn=4096, E=2, K=2),
    dict(N=29, d=4096, ffn=512, E=2, K=1),
    # 64-row tiles (mean 48 rows per expert) and 32-row tiles (decode-sized)
    dict(N=384, d=256, ffn=320, E=16, K=2),
    dict(N=12, d=512, ffn=256, E=64, K=4),
    # d and ffn not multiples of 128: the last down panel (and, in the
    # row-major kernel, the last column tile) ends past d, the last gate/up
    # column tile holds one panel of features; ragged row tiles
    dict(N=300, d=320, ffn=192, E=4, K=2),
])
def test_packed_ffn_split_layers_match_oracle_and_repeat(case):
    cfg = synth.config("packed_split", W=1, act="bf16", C=None, **case)
    print(f"[packed] {case}", flush=True)
    inp, layer = _ffn_case(cfg)
    pw = B.moe_pack_ffn_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
    M = int(layer.disp["offsets"][-1])
    ws = layer.ffn_ws
    results, plain = [], []
    for rep in range(3):
        # alternate with the plain-weight call on the same workspace: the
        # split counters each call leaves behind must be re-armed
        hp, yp = B.moe_grouped_ffn(layer.disp["x_perm"], layer.disp["offsets"], inp["w_gate"],
                                   inp["w_up"], inp["w_down"], layer.max_rows, workspace=ws)
        torch.cuda.synchronize()
        plain.append((hp[:M].clone(), yp[:M].clone()))
        h, y = B.moe_grouped_ffn_packed(layer.disp["x_perm"], layer.disp["offsets"], pw,
                                        layer.max_rows, workspace=ws)
        torch.cuda.synchronize()
        results.append((h[:M].clone(), y[:M].clone()))
    for h, y in results[1:]:
        assert torch.equal(h, results[0][0]) and torch.equal(y, results[0][1])
    h_ref, y_ref = _oracle_rows(inp, layer, M)
    _close("h", results[0][0].float().cpu().numpy(), h_ref)
    _close("y_perm", results[0][1].float().cpu().numpy(), y_ref)
    _close("h (row-major weights)", plain[0][0].float().cpu().numpy(), h_ref)
    _close("y_perm (row-major weights)", plain[0][1].float().cpu().numpy(), y_ref)

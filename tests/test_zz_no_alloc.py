"""moe_dispatch_noalloc (the dispatch that takes no workspace: its scratch is
the library's fixed per-GPU array) against moe_dispatch with a workspace,
through the C ABI: two calls in a row, the second with a smaller input, every
output bit for bit (the dispatch's results are integers and bit copies)."""
import numpy as np
import pytest
import torch

from grouped_gemm_route_amd import binding as B
from grouped_gemm_route_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

KEYS = ("perm_token", "dest", "demand", "counts", "offsets", "rank_offsets")


def _both(cfg, cap):
    inp = synth.make_inputs(cfg, DEV, weights=False)
    idx, _ = B.moe_route_topk(inp["logits"], cfg["K"])
    ref = B.moe_dispatch(inp["x"], idx, cfg["E"], cfg["W"], cap)
    got = B.moe_dispatch_noalloc(inp["x"], idx, cfg["E"], cfg["W"], cap)
    torch.cuda.synchronize()
    M = int(ref["offsets"][-1])
    for k in KEYS:
        a, b = ref[k], got[k]
        if k == "perm_token":
            a, b = a[:M], b[:M]
        assert torch.equal(a, b), k
    assert torch.equal(ref["x_perm"][:M], got["x_perm"][:M])
    return M


@pytest.mark.parametrize("first,second", [
    # a large call, then a smaller one (the scratch keeps the first call's
    # contents; nothing in it may be relied on as zero)
    (dict(name="prefill256_hot_c1.0"),
     dict(name="na_small", N=300, d=128, ffn=64, E=16, K=4, W=4, act="bf16", C=1.0)),
    (dict(name="dense8"),
     dict(name="na_f32", N=77, d=64, ffn=64, E=8, K=2, W=2, act="f32", C=None)),
    (dict(name="fine128_zipf_c1.25"),
     dict(name="na_one", N=1, d=64, ffn=64, E=8, K=2, W=8, act="bf16", C=None)),
])
def test_noalloc_dispatch_matches_workspace_dispatch(first, second):
    for spec in (first, second):
        name = spec["name"]
        cfg = synth.config(name, **{k: v for k, v in spec.items() if k != "name"})
        cap = (B.moe_capacity(cfg["C"], cfg["N"], cfg["K"], cfg["E"])
               if cfg["C"] is not None else -1)
        print(f"[noalloc] {name} N={cfg['N']} E={cfg['E']} K={cfg['K']} cap={cap}", flush=True)
        M = _both(cfg, cap)
        print(f"[noalloc] {name}: M={M} equal", flush=True)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    x = torch.zeros(300000, 16, dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros(300000, 4, dtype=torch.int32, device=DEV)
    with pytest.raises(B.MoeError) as ei:
        B.moe_dispatch_noalloc(x, idx, 8, 1, -1)
    assert ei.value.status == 2            # MOE_ERR_UNSUPPORTED

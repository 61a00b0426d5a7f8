"""The C-ABI library on a machine without a GPU: it loads, exports every
symbol the header declares, computes capacities exactly, and rejects bad
arguments on the host before any launch.  No call here reaches a kernel."""
import ctypes
import os
import re
import random
from fractions import Fraction
import math

import numpy as np
import pytest

from grouped_gemm_route_amd import binding as B
from oracle import moe_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
           if f.endswith(".h")]

FAKE = ctypes.c_void_p(4096)   # never dereferenced: every case fails its checks first
NUL = ctypes.c_void_p(0)


def declared_functions():
    names = []
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:[\w\*]+\s+)+\**(moe_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    return B.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), f"{n} declared but not exported"
    assert sorted(n for n, _, _ in B.SIGNATURES) == names


def test_version_and_status_strings(lib):
    assert lib.moe_abi_version() == 1
    for s, text in [(0, "MOE_OK"), (1, "MOE_ERR_INVALID_ARG"), (2, "MOE_ERR_UNSUPPORTED"),
                    (3, "MOE_ERR_WORKSPACE"), (4, "MOE_ERR_HIP"), (99, "MOE_ERR_UNKNOWN")]:
        assert lib.moe_status_string(s).decode() == text


def test_capacity_matches_oracle_exactly(lib):
    rnd = random.Random(7)
    cases = [(1.25, 8192, 8, 128), (1.0, 32768, 8, 256), (1.0, 4, 2, 4), (1.1, 10, 1, 1),
             (float(np.nextafter(1.0, 2.0)), 1024, 1, 1), (0.5, 3, 1, 1), (1e-300, 5, 1, 7),
             (1e-300, 0, 1, 7), (3.0, 0, 4, 2), (2.0 ** 40, 1000, 2, 3)]
    for _ in range(2000):
        C = rnd.choice([rnd.uniform(0.01, 4.0), rnd.randint(1, 8) / rnd.choice([1, 2, 4, 8, 3, 10]),
                        math.ldexp(rnd.random(), rnd.randint(-60, 10))])
        if C <= 0:
            continue
        cases.append((C, rnd.randint(0, 1 << 20), rnd.randint(1, 16), rnd.randint(1, 1024)))
    for C, N, K, E in cases:
        assert lib.moe_capacity(C, N, K, E) == O.capacity(C, N, K, E), (C, N, K, E)
    for bad in [(0.0, 1, 1, 1), (-1.0, 1, 1, 1), (float("inf"), 1, 1, 1), (float("nan"), 1, 1, 1),
                (1.0, -1, 1, 1), (1.0, 1, 0, 1), (1.0, 1, 1, 0), (1e300, 1 << 40, 16, 1)]:
        assert lib.moe_capacity(*bad) == -2
    # the bound is the exact rational ceiling, not a float computation
    assert lib.moe_capacity(1.0, 3, 1, 3) == 1
    assert Fraction(0.1) * 30 != 3 and lib.moe_capacity(0.1, 30, 1, 1) == math.ceil(Fraction(0.1) * 30)


def _status(fn, *args):
    return fn(*args)


def test_route_rejects_bad_arguments(lib):
    f = lib.moe_route_topk
    assert f(NUL, 4, 8, 2, 0, FAKE, FAKE, NUL) == 1
    assert f(FAKE, 4, 8, 2, 0, NUL, FAKE, NUL) == 1
    assert f(FAKE, -1, 8, 2, 0, FAKE, FAKE, NUL) == 1
    assert f(FAKE, 4, 8, 0, 0, FAKE, FAKE, NUL) == 1
    assert f(FAKE, 4, 8, 9, 0, FAKE, FAKE, NUL) == 1          # K > E
    assert f(FAKE, 4, 1025, 2, 0, FAKE, FAKE, NUL) == 2       # E limit
    assert f(FAKE, 4, 32, 17, 0, FAKE, FAKE, NUL) == 2        # K limit
    assert "K" in lib.moe_last_error().decode()


def test_gated_route_and_reroute_reject_bad_arguments(lib):
    g = lib.moe_route_topk_gated
    assert g(FAKE, 4, 8, 2, 2, 0, FAKE, FAKE, NUL) == 1        # gate not a moe_gate_t
    assert g(FAKE, 4, 8, 2, -1, 0, FAKE, FAKE, NUL) == 1
    assert g(NUL, 4, 8, 2, 1, 0, FAKE, FAKE, NUL) == 1
    assert g(FAKE, 4, 8, 9, 1, 0, FAKE, FAKE, NUL) == 1        # K > E
    assert g(FAKE, 4, 1025, 2, 1, 0, FAKE, FAKE, NUL) == 2     # E limit

    def rr(**kw):
        a = dict(l=FAKE, N=16, E=8, K=2, gate=0, renorm=0, cap=3, idx=FAKE, w=FAKE,
                 out=FAKE, ws=FAKE, ws_bytes=1 << 30)
        a.update(kw)
        return lib.moe_reroute_overflow(a["l"], a["N"], a["E"], a["K"], a["gate"], a["renorm"],
                                        a["cap"], a["idx"], a["w"], a["out"], a["ws"],
                                        a["ws_bytes"], NUL)
    assert rr(l=NUL) == 1
    assert rr(idx=NUL) == 1
    assert rr(N=0) == 1
    assert rr(K=9) == 1
    assert rr(cap=-2) == 1
    assert rr(gate=7) == 1
    assert rr(E=2048) == 2
    need = lib.moe_reroute_workspace_bytes(16, 8, 2)
    assert need > 0
    assert rr(ws_bytes=need - 1) == 3
    assert rr(ws=NUL) == 3
    assert "workspace" in lib.moe_last_error().decode()


def _dispatch(lib, **kw):
    a = dict(x=FAKE, dtype=1, N=16, d=64, idx=FAKE, E=8, K=2, W=4, cap=-1, x_perm=FAKE,
             perm=FAKE, dest=FAKE, demand=FAKE, counts=FAKE, offsets=FAKE, roff=FAKE,
             ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return lib.moe_dispatch(a["x"], a["dtype"], a["N"], a["d"], a["idx"], a["E"], a["K"],
                            a["W"], a["cap"], a["x_perm"], a["perm"], a["dest"], a["demand"],
                            a["counts"], a["offsets"], a["roff"], a["ws"], a["ws_bytes"], NUL)


def test_dispatch_rejects_bad_arguments(lib):
    assert _dispatch(lib, x=NUL) == 1
    assert _dispatch(lib, dest=NUL) == 1
    assert _dispatch(lib, dtype=5) == 2
    assert _dispatch(lib, N=0) == 1
    assert _dispatch(lib, K=9) == 1
    assert _dispatch(lib, W=3) == 1                 # E % W != 0
    assert _dispatch(lib, W=0) == 1
    assert _dispatch(lib, cap=-2) == 1
    assert _dispatch(lib, d=4) == 1                 # 8 bytes per bf16 row
    assert _dispatch(lib, dtype=0, d=2) == 1        # 8 bytes per fp32 row
    assert _dispatch(lib, E=2048, W=8) == 2
    assert _dispatch(lib, E=32, K=17, W=8) == 2
    assert _dispatch(lib, N=1 << 28, K=8, E=8, W=8) == 1   # N*K >= 2^31
    need = lib.moe_dispatch_workspace_bytes(16, 8, 2)
    assert need > 0
    assert _dispatch(lib, ws_bytes=need - 1) == 3
    assert _dispatch(lib, ws=NUL) == 3
    assert "workspace" in lib.moe_last_error().decode()


def test_fp8_entry_points_reject_bad_arguments(lib):
    def disp(**kw):
        a = dict(x=FAKE, N=16, d=256, idx=FAKE, E=8, K=2, W=4, cap=-1, x8=FAKE, xs=FAKE,
                 perm=FAKE, dest=FAKE, demand=FAKE, counts=FAKE, offsets=FAKE, roff=FAKE,
                 ws=FAKE, ws_bytes=1 << 30)
        a.update(kw)
        return lib.moe_dispatch_fp8(a["x"], a["N"], a["d"], a["idx"], a["E"], a["K"], a["W"],
                                    a["cap"], a["x8"], a["xs"], a["perm"], a["dest"],
                                    a["demand"], a["counts"], a["offsets"], a["roff"], a["ws"],
                                    a["ws_bytes"], NUL)
    assert disp(xs=NUL) == 1
    assert disp(x8=NUL) == 1
    assert disp(d=64) == 1                       # not a multiple of 128
    assert disp(d=200) == 1
    assert disp(K=9) == 1
    assert disp(ws_bytes=1) == 3
    c = lib.moe_combine_fp8
    assert c(FAKE, NUL, 4, 256, 2, FAKE, FAKE, FAKE, NUL) == 1
    assert c(FAKE, FAKE, 4, 96, 2, FAKE, FAKE, FAKE, NUL) == 1
    assert c(FAKE, FAKE, 0, 256, 2, FAKE, FAKE, FAKE, NUL) == 1
    assert c(FAKE, FAKE, 4, 256, 17, FAKE, FAKE, FAKE, NUL) == 2
    q = lib.moe_fp8_quantize_rows
    assert q(FAKE, NUL, 8, 256, FAKE, FAKE, NUL) == 1
    assert q(FAKE, FAKE, -1, 256, FAKE, FAKE, NUL) == 1
    assert q(FAKE, FAKE, 8, 100, FAKE, FAKE, NUL) == 1
    dq = lib.moe_fp8_dequantize_rows
    assert dq(FAKE, FAKE, FAKE, 8, 100, FAKE, NUL) == 1
    assert dq(FAKE, FAKE, FAKE, 1 << 31, 128, FAKE, NUL) == 1
    assert dq(NUL, FAKE, FAKE, 8, 128, FAKE, NUL) == 1
    assert "128" in lib.moe_last_error().decode() or "null" in lib.moe_last_error().decode()


def _ffn(lib, **kw):
    a = dict(x=FAKE, dtype=1, d=128, ffn=128, E=8, off=FAKE, max_rows=64, wg=FAKE, wu=FAKE,
             wd=FAKE, h=FAKE, y=FAKE, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return lib.moe_grouped_ffn(a["x"], a["dtype"], a["d"], a["ffn"], a["E"], a["off"],
                               a["max_rows"], a["wg"], a["wu"], a["wd"], a["h"], a["y"],
                               a["ws"], a["ws_bytes"], NUL)


def test_grouped_ffn_rejects_bad_arguments(lib):
    assert _ffn(lib, wd=NUL) == 1
    assert _ffn(lib, dtype=3) == 2
    assert _ffn(lib, d=0) == 1
    assert _ffn(lib, max_rows=-1) == 1
    assert _ffn(lib, d=96) == 2                     # bf16 needs multiples of 64
    assert _ffn(lib, dtype=0, ffn=12) == 2          # fp32 needs multiples of 8
    assert _ffn(lib, E=1025) == 2
    assert _ffn(lib, max_rows=1 << 31) == 2
    need = lib.moe_grouped_ffn_workspace_bytes(64, 8, 1)
    assert need > 0
    assert _ffn(lib, ws_bytes=need - 1) == 3
    assert _ffn(lib, max_rows=0, ws=NUL) == 0       # nothing to do: no launch


def test_packed_weight_bytes_closed_forms(lib):
    for E, d, ffn in [(1, 64, 64), (8, 4096, 14336), (256, 7168, 2048), (3, 320, 192)]:
        assert lib.moe_packed_ffn_weight_bytes(E, d, ffn, 0) == E * 2 * ffn * d * 2
        assert lib.moe_packed_ffn_weight_bytes(E, d, ffn, 1) == E * (-(-d // 128) * 128) * ffn * 2
    for E, d, ffn, part in [(0, 64, 64, 0), (1, 96, 64, 0), (1, 64, 32, 1), (1, 64, 64, 2)]:
        assert lib.moe_packed_ffn_weight_bytes(E, d, ffn, part) == 0


def test_packed_ffn_entry_points_reject_bad_arguments(lib):
    pack = lib.moe_pack_ffn_weights
    assert pack(FAKE, FAKE, NUL, 8, 128, 128, FAKE, FAKE, NUL) == 1
    assert pack(FAKE, FAKE, FAKE, 0, 128, 128, FAKE, FAKE, NUL) == 1
    assert pack(FAKE, FAKE, FAKE, 1025, 128, 128, FAKE, FAKE, NUL) == 2
    assert pack(FAKE, FAKE, FAKE, 8, 96, 128, FAKE, FAKE, NUL) == 2
    assert pack(FAKE, FAKE, FAKE, 8, 65536, 16384, FAKE, FAKE, NUL) == 2   # > 2 GiB / expert
    assert "2 GiB" in lib.moe_last_error().decode()

    def ffn(**kw):
        a = dict(x=FAKE, d=128, ffn=128, E=8, off=FAKE, max_rows=64, up=FAKE, dn=FAKE, h=FAKE,
                 y=FAKE, ws=FAKE, ws_bytes=1 << 30)
        a.update(kw)
        return lib.moe_grouped_ffn_packed(a["x"], a["d"], a["ffn"], a["E"], a["off"],
                                          a["max_rows"], a["up"], a["dn"], a["h"], a["y"],
                                          a["ws"], a["ws_bytes"], NUL)
    assert ffn(dn=NUL) == 1
    assert ffn(max_rows=-1) == 1
    assert ffn(E=0) == 1
    assert ffn(ffn=96) == 2
    assert ffn(max_rows=1 << 31) == 2
    need = lib.moe_grouped_ffn_workspace_bytes(64, 8, 1)
    assert ffn(ws_bytes=need - 1) == 3
    assert ffn(max_rows=0, ws=NUL) == 0


def test_combine_rejects_bad_arguments(lib):
    f = lib.moe_combine
    assert f(NUL, 1, 4, 64, 2, FAKE, FAKE, FAKE, NUL) == 1
    assert f(FAKE, 2, 4, 64, 2, FAKE, FAKE, FAKE, NUL) == 2
    assert f(FAKE, 1, 0, 64, 2, FAKE, FAKE, FAKE, NUL) == 1
    assert f(FAKE, 1, 4, 4, 2, FAKE, FAKE, FAKE, NUL) == 1
    assert f(FAKE, 1, 4, 64, 17, FAKE, FAKE, FAKE, NUL) == 2


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        B.moe_route_topk(torch.zeros(4, 8), 2)


def test_exchange_plan_rejects_bad_arguments(lib):
    f = lib.moe_exchange_plan
    args = [FAKE] * 4 + [8, 8, 2, 4, 16] + [FAKE] * 7 + [1 << 20, NUL]
    a = list(args); a[0] = NUL
    assert f(*a) == 1                                   # null pointer
    a = list(args); a[7] = 3
    assert f(*a) == 1                                   # E % W != 0
    a = list(args); a[6] = 9
    assert f(*a) == 1                                   # K > E
    a = list(args); a[7] = 128; a[5] = 128
    assert f(*a) == 2                                   # W beyond the limit
    a = list(args); a[16] = 1
    assert f(*a) == 3                                   # workspace too small
    assert lib.moe_exchange_workspace_bytes(8, 4) > 0


def test_rows_permute_rejects_bad_arguments(lib):
    f = lib.moe_rows_permute
    assert f(NUL, FAKE, FAKE, FAKE, 4, 64, 0, NUL) == 1
    assert f(FAKE, ctypes.c_void_p(8192), FAKE, FAKE, 4, 24, 0, NUL) == 1   # row bytes
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 64, 0, NUL) == 1                   # src == dst
    assert f(FAKE, ctypes.c_void_p(8192), FAKE, FAKE, -1, 64, 0, NUL) == 1


def test_combine_entry_points_reject_bad_arguments(lib):
    def comb(fn, **kw):
        a = dict(y=FAKE, dtype=1, N=16, d=64, K=2, dest=FAKE, w=FAKE, shared=FAKE, out=FAKE)
        a.update(kw)
        if fn == "plain":
            return lib.moe_combine(a["y"], a["dtype"], a["N"], a["d"], a["K"], a["dest"],
                                   a["w"], a["out"], NUL)
        return lib.moe_combine_residual(a["y"], a["dtype"], a["N"], a["d"], a["K"], a["dest"],
                                        a["w"], a["shared"], a["out"], NUL)
    for fn in ("plain", "residual"):
        assert comb(fn, out=NUL) == 1
        assert comb(fn, dtype=3) == 2
        assert comb(fn, N=0) == 1
        assert comb(fn, d=4) == 1                   # 8 bytes: not a multiple of 16
        assert comb(fn, K=0) == 1
        assert comb(fn, K=17) == 2
    assert comb("residual", shared=NUL) == 1
    assert "moe_combine_residual" in lib.moe_last_error().decode()


def test_dispatch_noalloc_rejects_on_the_host(lib):
    # every rejection happens before the scratch's device address is looked
    # up, so no GPU is needed
    f = lib.moe_dispatch_noalloc
    ok = dict(x=FAKE, dt=1, N=64, d=64, idx=FAKE, E=8, K=2, W=2, cap=-1)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["dt"], a["N"], a["d"], a["idx"], a["E"], a["K"], a["W"], a["cap"],
                 FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NUL)
    assert call(x=NUL) == 1
    assert call(N=0) == 1
    assert call(W=3) == 1
    assert call(cap=-2) == 1
    assert call(dt=7) == 2
    assert call(E=2048, K=2) == 2
    # scratch: moe_dispatch_workspace_bytes above the fixed 4 MiB array
    limit = 4 << 20
    assert lib.moe_dispatch_workspace_bytes(300000, 8, 4) > limit
    assert call(N=300000, E=8, K=4) == 2
    assert "scratch" in lib.moe_last_error().decode()
    # the largest bench workload fits
    assert lib.moe_dispatch_workspace_bytes(32768, 256, 8) <= limit


def test_router_rejects_bad_arguments(lib):
    f = lib.moe_router_logits
    assert f(NUL, 1, 4, 64, FAKE, 8, FAKE, NUL) == 1
    assert f(FAKE, 1, 0, 64, FAKE, 8, FAKE, NUL) == 1
    assert f(FAKE, 1, 4, 60, FAKE, 8, FAKE, NUL) == 1          # d not a multiple of 8
    assert f(FAKE, 9, 4, 64, FAKE, 8, FAKE, NUL) == 2          # dtype
    assert f(FAKE, 1, 4, 64, FAKE, 1025, FAKE, NUL) == 2       # E limit


def _plan(lib, **kw):
    a = dict(lg=FAKE, N=64, E=8, K=2, gate=0, ren=0, W=2, cap=-1, idx=FAKE, w=FAKE,
             demand=FAKE, counts=FAKE, offsets=FAKE, roff=FAKE, plan=FAKE, plan_bytes=1 << 30)
    a.update(kw)
    return lib.moe_route_plan(a["lg"], a["N"], a["E"], a["K"], a["gate"], a["ren"], a["W"],
                              a["cap"], a["idx"], a["w"], a["demand"], a["counts"],
                              a["offsets"], a["roff"], a["plan"], a["plan_bytes"], NUL)


def test_route_plan_rejects_bad_arguments(lib):
    assert _plan(lib, lg=NUL) == 1
    assert _plan(lib, w=NUL) == 1
    assert _plan(lib, idx=NUL) == 1
    assert _plan(lib, N=0) == 1
    assert _plan(lib, N=-1) == 1
    assert _plan(lib, K=9) == 1
    assert _plan(lib, K=0) == 1
    assert _plan(lib, gate=7) == 1
    assert _plan(lib, offsets=NUL) == 1
    assert _plan(lib, roff=NUL) == 1
    assert _plan(lib, W=3) == 1                  # E % W != 0
    assert _plan(lib, W=0) == 1
    assert _plan(lib, cap=-2) == 1
    assert _plan(lib, E=2048, W=8) == 2
    assert _plan(lib, E=32, K=17, W=8) == 2
    need = lib.moe_route_plan_bytes(64, 8, 2)
    assert need > 0
    assert _plan(lib, plan_bytes=need - 1) == 3
    assert _plan(lib, plan=NUL) == 3
    assert "plan" in lib.moe_last_error().decode()


def test_route_plan_bytes_closed_form(lib):
    # [256-byte counter | block_counts | block_excl | local_rank], each part
    # padded to 256 bytes; blocks of 128 tokens up to 8 experts, else 64
    def up(v):
        return (v + 255) // 256 * 256
    for N, E, K in [(1, 8, 2), (128, 8, 2), (129, 8, 2), (4096, 8, 2), (64, 9, 2), (65, 128, 8),
                    (8192, 128, 8), (32768, 256, 8), (16, 256, 8), (1000, 1024, 16)]:
        T = 128 if E <= 8 else 64
        B = -(-N // T)
        assert lib.moe_route_plan_bytes(N, E, K) == 256 + 2 * up(B * E * 4) + up(N * K * 4)
    assert lib.moe_route_plan_bytes(0, 8, 2) == 0
    assert lib.moe_route_plan_bytes(16, 0, 2) == 0


def _dplan(lib, **kw):
    a = dict(x=FAKE, dtype=1, N=64, d=128, idx=FAKE, E=8, K=2, W=4, cap=-1, plan=FAKE,
             plan_bytes=1 << 30, x_perm=FAKE, x_scale=NUL, perm=FAKE, dest=FAKE, demand=FAKE,
             counts=FAKE, offsets=FAKE, roff=FAKE)
    a.update(kw)
    return lib.moe_dispatch_planned(a["x"], a["dtype"], a["N"], a["d"], a["idx"], a["E"],
                                    a["K"], a["W"], a["cap"], a["plan"], a["plan_bytes"],
                                    a["x_perm"], a["x_scale"], a["perm"], a["dest"],
                                    a["demand"], a["counts"], a["offsets"], a["roff"], NUL)


def test_dispatch_planned_rejects_bad_arguments(lib):
    assert _dplan(lib, x=NUL) == 1
    assert _dplan(lib, offsets=NUL) == 1
    assert _dplan(lib, dest=NUL) == 1
    assert _dplan(lib, roff=NUL) == 1
    assert _dplan(lib, dtype=5) == 2
    assert _dplan(lib, N=0) == 1
    assert _dplan(lib, K=9) == 1
    assert _dplan(lib, W=3) == 1                     # E % W != 0
    assert _dplan(lib, W=0) == 1
    assert _dplan(lib, cap=-2) == 1
    assert _dplan(lib, d=4) == 1                     # 8 bytes per bf16 row
    assert _dplan(lib, dtype=0, d=2) == 1            # 8 bytes per fp32 row
    assert _dplan(lib, x_scale=FAKE, dtype=0) == 1   # fp8 payload from fp32 rows
    assert _dplan(lib, x_scale=FAKE, d=64) == 1      # d not a multiple of 128
    assert _dplan(lib, E=2048, W=8) == 2
    assert _dplan(lib, N=1 << 28, K=8) == 1          # N*K >= 2^31
    assert _dplan(lib, N=1 << 25, E=1024, K=1, W=8) == 2   # count table past 32-bit offsets
    need = lib.moe_route_plan_bytes(64, 8, 2)
    assert _dplan(lib, plan_bytes=need - 1) == 3
    assert _dplan(lib, plan=NUL) == 3

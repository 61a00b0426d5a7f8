"""Python binding of libmoe_route.so (ctypes): argument marshalling only.

Every stage of the layer runs in the library's HIP kernels.  These wrappers
take torch tensors (torch supplies device memory and the current stream),
check dtype, device and contiguity, allocate outputs when none are passed,
and call the C entry point of the same name.  There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_route.so")

MOE_OK = 0
DTYPE_CODE = {torch.float32: 0, torch.bfloat16: 1}
GATE_CODE = {"softmax": 0, "sigmoid": 1}

# (name, restype, argtypes) of every exported function in include/moe_route.h
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
SIGNATURES = [
    ("moe_abi_version", ctypes.c_int, []),
    ("moe_status_string", ctypes.c_char_p, [ctypes.c_int]),
    ("moe_last_error", ctypes.c_char_p, []),
    ("moe_capacity", _I64, [ctypes.c_double, _I64, _I32, _I32]),
    ("moe_route_topk", ctypes.c_int, [_P, _I32, _I32, _I32, _I32, _P, _P, _P]),
    ("moe_route_topk_gated", ctypes.c_int, [_P, _I32, _I32, _I32, _I32, _I32, _P, _P, _P]),
    ("moe_reroute_workspace_bytes", _SZ, [_I32, _I32, _I32]),
    ("moe_reroute_overflow", ctypes.c_int,
     [_P, _I32, _I32, _I32, _I32, _I32, _I64, _P, _P, _P, _P, _SZ, _P]),
    ("moe_dispatch_workspace_bytes", _SZ, [_I32, _I32, _I32]),
    ("moe_dispatch", ctypes.c_int,
     [_P, _I32, _I32, _I32, _P, _I32, _I32, _I32, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    ("moe_dispatch_noalloc", ctypes.c_int,
     [_P, _I32, _I32, _I32, _P, _I32, _I32, _I32, _I64, _P, _P, _P, _P, _P, _P, _P, _P]),
    ("moe_route_plan_bytes", _SZ, [_I32, _I32, _I32]),
    ("moe_route_plan", ctypes.c_int,
     [_P, _I32, _I32, _I32, _I32, _I32, _I32, _I64, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    ("moe_dispatch_planned", ctypes.c_int,
     [_P, _I32, _I32, _I32, _P, _I32, _I32, _I32, _I64, _P, _SZ, _P, _P, _P, _P, _P, _P, _P, _P,
      _P]),
    ("moe_grouped_ffn_workspace_bytes", _SZ, [_I64, _I32, _I32]),
    ("moe_grouped_ffn", ctypes.c_int,
     [_P, _I32, _I32, _I32, _I32, _P, _I64, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    ("moe_packed_ffn_weight_bytes", _SZ, [_I32, _I32, _I32, _I32]),
    ("moe_pack_ffn_weights", ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _P, _P, _P]),
    ("moe_grouped_ffn_packed", ctypes.c_int,
     [_P, _I32, _I32, _I32, _P, _I64, _P, _P, _P, _P, _P, _SZ, _P]),
    ("moe_combine", ctypes.c_int, [_P, _I32, _I32, _I32, _I32, _P, _P, _P, _P]),
    ("moe_combine_residual", ctypes.c_int, [_P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P]),
    ("moe_router_logits", ctypes.c_int, [_P, _I32, _I32, _I32, _P, _I32, _P, _P]),
    ("moe_exchange_workspace_bytes", _SZ, [_I32, _I32]),
    ("moe_exchange_plan", ctypes.c_int,
     [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _I64, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    ("moe_rows_permute", ctypes.c_int, [_P, _P, _P, _P, _I64, _I32, _I32, _P]),
    ("moe_dispatch_fp8", ctypes.c_int,
     [_P, _I32, _I32, _P, _I32, _I32, _I32, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    ("moe_combine_fp8", ctypes.c_int, [_P, _P, _I32, _I32, _I32, _P, _P, _P, _P]),
    ("moe_fp8_quantize_rows", ctypes.c_int, [_P, _P, _I64, _I32, _P, _P, _P]),
    ("moe_fp8_dequantize_rows", ctypes.c_int, [_P, _P, _P, _I64, _I32, _P, _P]),
]

FP8_GROUP = 128  # columns per fp32 scale of the fp8 payload

_lib = None


class MoeError(RuntimeError):
    """A library call returned a non-OK status."""

    def __init__(self, name, status, detail):
        super().__init__(f"{name}: {status_name(status)}: {detail}")
        self.status = status


def load_library(path=None):
    """Load (once) and return the ctypes handle of libmoe_route.so."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} is not built; run `python -m grouped_gemm_route_amd.build` first")
    lib = ctypes.CDLL(p)
    for name, res, args in SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def status_name(status):
    return load_library().moe_status_string(status).decode()


def _check(name, status):
    if status != MOE_OK:
        raise MoeError(name, status, load_library().moe_last_error().decode())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t, name, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")


def _act_code(t, name):
    if t.dtype not in DTYPE_CODE:
        raise ValueError(f"{name}: unsupported dtype {t.dtype}")
    return DTYPE_CODE[t.dtype]


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def moe_abi_version():
    return load_library().moe_abi_version()


def moe_capacity(C, N, K, E):
    """ceil(C*N*K/E) computed exactly by the library (host only)."""
    v = load_library().moe_capacity(float(C), int(N), int(K), int(E))
    if v == -2:
        raise ValueError(f"invalid capacity arguments C={C} N={N} K={K} E={E}")
    return int(v)


def _gate(gate):
    if gate not in GATE_CODE:
        raise ValueError(f"gate must be one of {sorted(GATE_CODE)}")
    return GATE_CODE[gate]


def moe_route_topk(logits, K, renormalize=False, topk_idx=None, topk_w=None, gate="softmax"):
    """Top-K routing: returns (topk_idx int32 [N,K], topk_w fp32 [N,K]).
    gate "softmax" calls moe_route_topk, "sigmoid" moe_route_topk_gated."""
    _need(logits, "logits", torch.float32)
    N, E = logits.shape
    dev = logits.device
    if topk_idx is None:
        topk_idx = torch.empty(N, K, dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty(N, K, dtype=torch.float32, device=dev)
    _need(topk_idx, "topk_idx", torch.int32, dev)
    _need(topk_w, "topk_w", torch.float32, dev)
    if topk_idx.numel() != N * K or topk_w.numel() != N * K:
        raise ValueError("topk_idx/topk_w must hold N*K elements")
    if gate == "softmax":
        _check("moe_route_topk", load_library().moe_route_topk(
            _ptr(logits), N, E, K, int(bool(renormalize)), _ptr(topk_idx), _ptr(topk_w),
            _stream(logits)))
    else:
        _check("moe_route_topk_gated", load_library().moe_route_topk_gated(
            _ptr(logits), N, E, K, _gate(gate), int(bool(renormalize)), _ptr(topk_idx),
            _ptr(topk_w), _stream(logits)))
    return topk_idx, topk_w


def moe_reroute_workspace_bytes(N, E, K):
    return int(load_library().moe_reroute_workspace_bytes(N, E, K))


def moe_reroute_overflow(logits, topk_idx, topk_w, capacity, gate="softmax", renormalize=False,
                         rerouted=None, workspace=None):
    """Re-route capacity overflow to next-best experts, updating topk_idx and
    topk_w in place; returns rerouted int32 [E] (admitted slots per expert)."""
    _need(logits, "logits", torch.float32)
    N, E = logits.shape
    dev = logits.device
    _need(topk_idx, "topk_idx", torch.int32, dev)
    _need(topk_w, "topk_w", torch.float32, dev)
    K = topk_idx.shape[1]
    if tuple(topk_idx.shape) != (N, K) or tuple(topk_w.shape) != (N, K):
        raise ValueError("topk_idx / topk_w must be [N, K]")
    if rerouted is None:
        rerouted = torch.empty(E, dtype=torch.int32, device=dev)
    _need(rerouted, "rerouted", torch.int32, dev)
    if rerouted.numel() < E:
        raise ValueError("rerouted must hold E elements")
    if workspace is None:
        workspace = torch.empty(max(1, moe_reroute_workspace_bytes(N, E, K)),
                                dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", None, dev)
    _check("moe_reroute_overflow", load_library().moe_reroute_overflow(
        _ptr(logits), N, E, K, _gate(gate), int(bool(renormalize)), int(capacity),
        _ptr(topk_idx), _ptr(topk_w), _ptr(rerouted), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(logits)))
    return rerouted


def moe_router_logits(x, w_router, logits=None):
    """Router projection: returns fp32 logits [N, E] = x @ w_router^T."""
    _need(x, "x")
    code = _act_code(x, "x")
    N, d = x.shape
    dev = x.device
    _need(w_router, "w_router", x.dtype, dev)
    E, d2 = w_router.shape
    if d2 != d:
        raise ValueError("w_router must be [E, d]")
    if logits is None:
        logits = torch.empty(N, E, dtype=torch.float32, device=dev)
    _need(logits, "logits", torch.float32, dev)
    if logits.numel() < N * E:
        raise ValueError("logits too small")
    _check("moe_router_logits", load_library().moe_router_logits(
        _ptr(x), code, N, d, _ptr(w_router), E, _ptr(logits), _stream(x)))
    return logits


def moe_dispatch_workspace_bytes(N, E, K):
    return int(load_library().moe_dispatch_workspace_bytes(N, E, K))


DISPATCH_OUTPUTS = ("x_perm", "perm_token", "dest", "demand", "counts", "offsets",
                    "rank_offsets")


def alloc_dispatch_outputs(N, d, E, K, W, dtype, device):
    return {
        "x_perm": torch.empty(N * K, d, dtype=dtype, device=device),
        "perm_token": torch.empty(N * K, dtype=torch.int32, device=device),
        "dest": torch.empty(N, K, dtype=torch.int32, device=device),
        "demand": torch.empty(E, dtype=torch.int32, device=device),
        "counts": torch.empty(E, dtype=torch.int32, device=device),
        "offsets": torch.empty(E + 1, dtype=torch.int32, device=device),
        "rank_offsets": torch.empty(W + 1, dtype=torch.int32, device=device),
        "workspace": torch.empty(max(1, moe_dispatch_workspace_bytes(N, E, K)),
                                 dtype=torch.uint8, device=device),
    }


def moe_dispatch(x, topk_idx, E, W, capacity, out=None):
    """Pack tokens into per-expert rows; returns the dict of outputs."""
    _need(x, "x")
    code = _act_code(x, "x")
    N, d = x.shape
    dev = x.device
    _need(topk_idx, "topk_idx", torch.int32, dev)
    K = topk_idx.shape[1]
    if topk_idx.shape[0] != N:
        raise ValueError("topk_idx must be [N, K]")
    if out is None:
        out = alloc_dispatch_outputs(N, d, E, K, W, x.dtype, dev)
    sizes = {"x_perm": N * K * d, "perm_token": N * K, "dest": N * K, "demand": E,
             "counts": E, "offsets": E + 1, "rank_offsets": W + 1}
    for k in DISPATCH_OUTPUTS:
        _need(out[k], k, x.dtype if k == "x_perm" else torch.int32, dev)
        if out[k].numel() < sizes[k]:
            raise ValueError(f"{k} must hold at least {sizes[k]} elements")
    ws = out["workspace"]
    _need(ws, "workspace", None, dev)
    _check("moe_dispatch", load_library().moe_dispatch(
        _ptr(x), code, N, d, _ptr(topk_idx), E, K, W, int(capacity),
        _ptr(out["x_perm"]), _ptr(out["perm_token"]), _ptr(out["dest"]),
        _ptr(out["demand"]), _ptr(out["counts"]), _ptr(out["offsets"]),
        _ptr(out["rank_offsets"]), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(x)))
    return out


def moe_dispatch_noalloc(x, topk_idx, E, W, capacity, out=None):
    """moe_dispatch through the allocation-free entry point (the library's
    own fixed scratch instead of a workspace); returns the dict of outputs
    (a "workspace" entry, if present, is not used)."""
    _need(x, "x")
    code = _act_code(x, "x")
    N, d = x.shape
    dev = x.device
    _need(topk_idx, "topk_idx", torch.int32, dev)
    K = topk_idx.shape[1]
    if topk_idx.shape[0] != N:
        raise ValueError("topk_idx must be [N, K]")
    if out is None:
        out = alloc_dispatch_outputs(N, d, E, K, W, x.dtype, dev)
    sizes = {"x_perm": N * K * d, "perm_token": N * K, "dest": N * K, "demand": E,
             "counts": E, "offsets": E + 1, "rank_offsets": W + 1}
    for k in DISPATCH_OUTPUTS:
        _need(out[k], k, x.dtype if k == "x_perm" else torch.int32, dev)
        if out[k].numel() < sizes[k]:
            raise ValueError(f"{k} must hold at least {sizes[k]} elements")
    _check("moe_dispatch_noalloc", load_library().moe_dispatch_noalloc(
        _ptr(x), code, N, d, _ptr(topk_idx), E, K, W, int(capacity),
        _ptr(out["x_perm"]), _ptr(out["perm_token"]), _ptr(out["dest"]),
        _ptr(out["demand"]), _ptr(out["counts"]), _ptr(out["offsets"]),
        _ptr(out["rank_offsets"]), _stream(x)))
    return out


def moe_route_plan_bytes(N, E, K):
    return int(load_library().moe_route_plan_bytes(N, E, K))


def alloc_route_plan(N, E, K, device):
    """A plan buffer for moe_route_plan / moe_dispatch_planned, zeroed (its
    arrival counter must start at zero; every call leaves it zero)."""
    return torch.zeros(max(256, moe_route_plan_bytes(N, E, K)), dtype=torch.uint8,
                       device=device)


# MoeLayer's default: planned layers up to this many per-block counts
PLAN_MAX_COUNTS = 65536


def moe_route_plan(logits, K, W, capacity, plan, out=None, renormalize=False, topk_idx=None,
                   topk_w=None, gate="softmax"):
    """Routing that also ranks and counts the tokens per expert, into plan.
    out: a dict holding demand, counts, offsets and rank_offsets (e.g. the
    dispatch outputs the following moe_dispatch_planned gets; allocated when
    None).  Returns (topk_idx, topk_w, out)."""
    _need(logits, "logits", torch.float32)
    N, E = logits.shape
    dev = logits.device
    if topk_idx is None:
        topk_idx = torch.empty(N, K, dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty(N, K, dtype=torch.float32, device=dev)
    _need(topk_idx, "topk_idx", torch.int32, dev)
    _need(topk_w, "topk_w", torch.float32, dev)
    if topk_idx.numel() != N * K or topk_w.numel() != N * K:
        raise ValueError("topk_idx/topk_w must hold N*K elements")
    if out is None:
        out = {"demand": torch.empty(E, dtype=torch.int32, device=dev),
               "counts": torch.empty(E, dtype=torch.int32, device=dev),
               "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
               "rank_offsets": torch.empty(W + 1, dtype=torch.int32, device=dev)}
    sizes = {"demand": E, "counts": E, "offsets": E + 1, "rank_offsets": W + 1}
    for k, n in sizes.items():
        _need(out[k], k, torch.int32, dev)
        if out[k].numel() < n:
            raise ValueError(f"{k} must hold at least {n} elements")
    _need(plan, "plan", None, dev)
    _check("moe_route_plan", load_library().moe_route_plan(
        _ptr(logits), N, E, K, _gate(gate), int(bool(renormalize)), W, int(capacity),
        _ptr(topk_idx), _ptr(topk_w), _ptr(out["demand"]), _ptr(out["counts"]),
        _ptr(out["offsets"]), _ptr(out["rank_offsets"]), _ptr(plan),
        plan.numel() * plan.element_size(), _stream(logits)))
    return topk_idx, topk_w, out


def moe_dispatch_planned(x, topk_idx, E, W, capacity, plan, out=None, fp8=False):
    """moe_dispatch from a plan of moe_route_plan; returns the dict of outputs
    (as moe_dispatch's; fp8=True: as moe_dispatch_fp8's, x8 and x_scale in
    place of x_perm)."""
    _need(x, "x")
    code = _act_code(x, "x")
    N, d = x.shape
    dev = x.device
    _need(topk_idx, "topk_idx", torch.int32, dev)
    K = topk_idx.shape[1]
    if topk_idx.shape[0] != N:
        raise ValueError("topk_idx must be [N, K]")
    if out is None:
        out = (alloc_dispatch_fp8_outputs(N, d, E, K, W, dev) if fp8 else
               alloc_dispatch_outputs(N, d, E, K, W, x.dtype, dev))
    sizes = {"perm_token": N * K, "dest": N * K, "demand": E, "counts": E, "offsets": E + 1,
             "rank_offsets": W + 1}
    for k, n in sizes.items():
        _need(out[k], k, torch.int32, dev)
        if out[k].numel() < n:
            raise ValueError(f"{k} must hold at least {n} elements")
    if fp8:
        rows, scale = out["x8"], out["x_scale"]
        _need(rows, "x8", torch.uint8, dev)
        _need(scale, "x_scale", torch.float32, dev)
        if rows.numel() < N * K * d or scale.numel() < N * K * (d // FP8_GROUP):
            raise ValueError("x8 / x_scale too small")
    else:
        rows, scale = out["x_perm"], None
        _need(rows, "x_perm", x.dtype, dev)
        if rows.numel() < N * K * d:
            raise ValueError(f"x_perm must hold at least {N * K * d} elements")
    _need(plan, "plan", None, dev)
    _check("moe_dispatch_planned", load_library().moe_dispatch_planned(
        _ptr(x), code, N, d, _ptr(topk_idx), E, K, W, int(capacity), _ptr(plan),
        plan.numel() * plan.element_size(), _ptr(rows), None if scale is None else _ptr(scale),
        _ptr(out["perm_token"]), _ptr(out["dest"]), _ptr(out["demand"]), _ptr(out["counts"]),
        _ptr(out["offsets"]), _ptr(out["rank_offsets"]), _stream(x)))
    return out


def alloc_dispatch_fp8_outputs(N, d, E, K, W, device):
    out = alloc_dispatch_outputs(N, 16, E, K, W, torch.bfloat16, device)
    del out["x_perm"]
    out["x8"] = torch.empty(N * K, d, dtype=torch.uint8, device=device)
    out["x_scale"] = torch.empty(N * K, d // FP8_GROUP, dtype=torch.float32, device=device)
    return out


def moe_dispatch_fp8(x, topk_idx, E, W, capacity, out=None):
    """moe_dispatch with an fp8 payload: returns the dict of outputs with x8
    (uint8 e4m3 codes [N*K, d]) and x_scale (fp32 [N*K, d/128]) in place of
    x_perm."""
    _need(x, "x", torch.bfloat16)
    N, d = x.shape
    dev = x.device
    _need(topk_idx, "topk_idx", torch.int32, dev)
    K = topk_idx.shape[1]
    if topk_idx.shape[0] != N:
        raise ValueError("topk_idx must be [N, K]")
    if out is None:
        out = alloc_dispatch_fp8_outputs(N, d, E, K, W, dev)
    sizes = {"perm_token": N * K, "dest": N * K, "demand": E, "counts": E,
             "offsets": E + 1, "rank_offsets": W + 1}
    for k, n in sizes.items():
        _need(out[k], k, torch.int32, dev)
        if out[k].numel() < n:
            raise ValueError(f"{k} must hold at least {n} elements")
    _need(out["x8"], "x8", torch.uint8, dev)
    _need(out["x_scale"], "x_scale", torch.float32, dev)
    if out["x8"].numel() < N * K * d or out["x_scale"].numel() < N * K * (d // FP8_GROUP):
        raise ValueError("x8 / x_scale too small")
    ws = out["workspace"]
    _need(ws, "workspace", None, dev)
    _check("moe_dispatch_fp8", load_library().moe_dispatch_fp8(
        _ptr(x), N, d, _ptr(topk_idx), E, K, W, int(capacity), _ptr(out["x8"]),
        _ptr(out["x_scale"]), _ptr(out["perm_token"]), _ptr(out["dest"]), _ptr(out["demand"]),
        _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["rank_offsets"]), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(x)))
    return out


def moe_combine_fp8(y8, y_scale, dest, topk_w, out=None):
    """Weighted merge of fp8 expert outputs back to token order (bf16 out)."""
    _need(y8, "y8", torch.uint8)
    dev = y8.device
    _need(y_scale, "y_scale", torch.float32, dev)
    _need(dest, "dest", torch.int32, dev)
    _need(topk_w, "topk_w", torch.float32, dev)
    N, K = dest.shape
    d = y8.shape[1]
    if tuple(topk_w.shape) != (N, K):
        raise ValueError("topk_w must match dest [N, K]")
    if out is None:
        out = torch.empty(N, d, dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, dev)
    _check("moe_combine_fp8", load_library().moe_combine_fp8(
        _ptr(y8), _ptr(y_scale), N, d, K, _ptr(dest), _ptr(topk_w), _ptr(out), _stream(y8)))
    return out


def moe_fp8_quantize_rows(src, n_rows, max_rows=None, q=None, scale=None):
    """fp8 codes and scales of rows [0, min(n_rows[0], max_rows)) of a bf16
    [rows, d] tensor; n_rows is a one-element int32 device tensor."""
    _need(src, "src", torch.bfloat16)
    dev = src.device
    _need(n_rows, "n_rows", torch.int32, dev)
    R, d = src.shape
    if max_rows is None:
        max_rows = R
    if max_rows > R:
        raise ValueError("max_rows exceeds src rows")
    if q is None:
        q = torch.empty(R, d, dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty(R, d // FP8_GROUP, dtype=torch.float32, device=dev)
    _need(q, "q", torch.uint8, dev)
    _need(scale, "scale", torch.float32, dev)
    if q.numel() < max_rows * d or scale.numel() < max_rows * (d // FP8_GROUP):
        raise ValueError("q / scale too small")
    _check("moe_fp8_quantize_rows", load_library().moe_fp8_quantize_rows(
        _ptr(src), _ptr(n_rows), int(max_rows), d, _ptr(q), _ptr(scale), _stream(src)))
    return q, scale


def moe_fp8_dequantize_rows(q, scale, n_rows, max_rows=None, dst=None):
    """bf16 rows (code value * scale) of rows [0, min(n_rows[0], max_rows))."""
    _need(q, "q", torch.uint8)
    dev = q.device
    _need(scale, "scale", torch.float32, dev)
    _need(n_rows, "n_rows", torch.int32, dev)
    R, d = q.shape
    if max_rows is None:
        max_rows = R
    if max_rows > R:
        raise ValueError("max_rows exceeds q rows")
    if scale.numel() < max_rows * (d // FP8_GROUP):
        raise ValueError("scale too small")
    if dst is None:
        dst = torch.empty(R, d, dtype=torch.bfloat16, device=dev)
    _need(dst, "dst", torch.bfloat16, dev)
    if dst.numel() < max_rows * d:
        raise ValueError("dst too small")
    _check("moe_fp8_dequantize_rows", load_library().moe_fp8_dequantize_rows(
        _ptr(q), _ptr(scale), _ptr(n_rows), int(max_rows), d, _ptr(dst), _stream(q)))
    return dst


def moe_grouped_ffn_workspace_bytes(max_rows, E, dtype):
    return int(load_library().moe_grouped_ffn_workspace_bytes(max_rows, E, DTYPE_CODE[dtype]))


def moe_grouped_ffn(x_perm, offsets, w_gate, w_up, w_down, max_rows=None, h=None,
                    y_perm=None, workspace=None):
    """Grouped SwiGLU FFN over the packed rows; returns (h, y_perm)."""
    _need(x_perm, "x_perm")
    code = _act_code(x_perm, "x_perm")
    dev = x_perm.device
    d = x_perm.shape[1]
    E, ffn, d2 = w_gate.shape
    if d2 != d or tuple(w_up.shape) != (E, ffn, d) or tuple(w_down.shape) != (E, d, ffn):
        raise ValueError("weights must be w_gate/w_up [E, ffn, d] and w_down [E, d, ffn]")
    for name, t in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _need(t, name, x_perm.dtype, dev)
    _need(offsets, "offsets", torch.int32, dev)
    if offsets.numel() != E + 1:
        raise ValueError("offsets must have E+1 entries")
    if max_rows is None:
        max_rows = x_perm.shape[0]
    if x_perm.shape[0] < max_rows:
        raise ValueError("x_perm must have at least max_rows rows")
    if h is None:
        h = torch.empty(max_rows, ffn, dtype=x_perm.dtype, device=dev)
    if y_perm is None:
        y_perm = torch.empty(max_rows, d, dtype=x_perm.dtype, device=dev)
    _need(h, "h", x_perm.dtype, dev)
    _need(y_perm, "y_perm", x_perm.dtype, dev)
    if h.numel() < max_rows * ffn or y_perm.numel() < max_rows * d:
        raise ValueError("h / y_perm too small for max_rows")
    if workspace is None:
        workspace = torch.empty(max(1, moe_grouped_ffn_workspace_bytes(max_rows, E, x_perm.dtype)),
                                dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", None, dev)
    _check("moe_grouped_ffn", load_library().moe_grouped_ffn(
        _ptr(x_perm), code, d, ffn, E, _ptr(offsets), int(max_rows), _ptr(w_gate),
        _ptr(w_up), _ptr(w_down), _ptr(h), _ptr(y_perm), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(x_perm)))
    return h, y_perm


MOE_FFN_GATE_UP, MOE_FFN_DOWN = 0, 1


def moe_packed_ffn_weight_bytes(E, d, ffn, part):
    return int(load_library().moe_packed_ffn_weight_bytes(E, d, ffn, part))


class PackedFfnWeights:
    """bf16 expert weights packed by moe_pack_ffn_weights (byte tensors up
    and down, for E experts of d x ffn)."""

    def __init__(self, up, down, E, d, ffn):
        self.up, self.down, self.E, self.d, self.ffn = up, down, E, d, ffn


def moe_pack_ffn_weights(w_gate, w_up, w_down):
    """Pack bf16 w_gate/w_up [E, ffn, d] and w_down [E, d, ffn] for
    moe_grouped_ffn_packed (once, at weight-load time)."""
    E, ffn, d = w_gate.shape
    if tuple(w_up.shape) != (E, ffn, d) or tuple(w_down.shape) != (E, d, ffn):
        raise ValueError("weights must be w_gate/w_up [E, ffn, d] and w_down [E, d, ffn]")
    dev = w_gate.device
    for name, t in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _need(t, name, torch.bfloat16, dev)
    nu = moe_packed_ffn_weight_bytes(E, d, ffn, MOE_FFN_GATE_UP)
    nd = moe_packed_ffn_weight_bytes(E, d, ffn, MOE_FFN_DOWN)
    if nu == 0 or nd == 0:
        raise ValueError(f"cannot pack d={d} ffn={ffn}: both must be multiples of 64")
    up = torch.empty(nu, dtype=torch.uint8, device=dev)
    down = torch.empty(nd, dtype=torch.uint8, device=dev)
    _check("moe_pack_ffn_weights", load_library().moe_pack_ffn_weights(
        _ptr(w_gate), _ptr(w_up), _ptr(w_down), E, d, ffn, _ptr(up), _ptr(down),
        _stream(w_gate)))
    return PackedFfnWeights(up, down, E, d, ffn)


def moe_grouped_ffn_packed(x_perm, offsets, packed, max_rows=None, h=None, y_perm=None,
                           workspace=None):
    """moe_grouped_ffn on weights packed by moe_pack_ffn_weights; returns
    (h, y_perm)."""
    _need(x_perm, "x_perm", torch.bfloat16)
    dev = x_perm.device
    E, d, ffn = packed.E, packed.d, packed.ffn
    if x_perm.shape[1] != d:
        raise ValueError("x_perm rows must have d columns")
    _need(packed.up, "packed.up", torch.uint8, dev)
    _need(packed.down, "packed.down", torch.uint8, dev)
    _need(offsets, "offsets", torch.int32, dev)
    if offsets.numel() != E + 1:
        raise ValueError("offsets must have E+1 entries")
    if max_rows is None:
        max_rows = x_perm.shape[0]
    if x_perm.shape[0] < max_rows:
        raise ValueError("x_perm must have at least max_rows rows")
    if h is None:
        h = torch.empty(max_rows, ffn, dtype=x_perm.dtype, device=dev)
    if y_perm is None:
        y_perm = torch.empty(max_rows, d, dtype=x_perm.dtype, device=dev)
    _need(h, "h", x_perm.dtype, dev)
    _need(y_perm, "y_perm", x_perm.dtype, dev)
    if h.numel() < max_rows * ffn or y_perm.numel() < max_rows * d:
        raise ValueError("h / y_perm too small for max_rows")
    if workspace is None:
        workspace = torch.empty(max(1, moe_grouped_ffn_workspace_bytes(max_rows, E, x_perm.dtype)),
                                dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", None, dev)
    _check("moe_grouped_ffn_packed", load_library().moe_grouped_ffn_packed(
        _ptr(x_perm), d, ffn, E, _ptr(offsets), int(max_rows), _ptr(packed.up),
        _ptr(packed.down), _ptr(h), _ptr(y_perm), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(x_perm)))
    return h, y_perm


def moe_combine(y_perm, dest, topk_w, out=None):
    """Weighted merge back to token order; returns out [N, d]."""
    _need(y_perm, "y_perm")
    code = _act_code(y_perm, "y_perm")
    dev = y_perm.device
    _need(dest, "dest", torch.int32, dev)
    _need(topk_w, "topk_w", torch.float32, dev)
    N, K = dest.shape
    d = y_perm.shape[1]
    if tuple(topk_w.shape) != (N, K):
        raise ValueError("topk_w must match dest [N, K]")
    if out is None:
        out = torch.empty(N, d, dtype=y_perm.dtype, device=dev)
    _need(out, "out", y_perm.dtype, dev)
    if out.numel() < N * d:
        raise ValueError("out too small")
    _check("moe_combine", load_library().moe_combine(
        _ptr(y_perm), code, N, d, K, _ptr(dest), _ptr(topk_w), _ptr(out), _stream(y_perm)))
    return out


def moe_combine_residual(y_perm, dest, topk_w, shared, out=None):
    """Residual-MoE combine: out[t] = shared[t] + the weighted sum of the
    token's kept rows; returns out [N, d]."""
    _need(y_perm, "y_perm")
    code = _act_code(y_perm, "y_perm")
    dev = y_perm.device
    _need(dest, "dest", torch.int32, dev)
    _need(topk_w, "topk_w", torch.float32, dev)
    N, K = dest.shape
    d = y_perm.shape[1]
    if tuple(topk_w.shape) != (N, K):
        raise ValueError("topk_w must match dest [N, K]")
    _need(shared, "shared", y_perm.dtype, dev)
    if shared.numel() < N * d or shared.shape[-1] != d:
        raise ValueError("shared must be [N, d]")
    if out is None:
        out = torch.empty(N, d, dtype=y_perm.dtype, device=dev)
    _need(out, "out", y_perm.dtype, dev)
    if out.numel() < N * d:
        raise ValueError("out too small")
    _check("moe_combine_residual", load_library().moe_combine_residual(
        _ptr(y_perm), code, N, d, K, _ptr(dest), _ptr(topk_w), _ptr(shared), _ptr(out),
        _stream(y_perm)))
    return out


def moe_shared_ffn(x, offsets, w_gate, w_up=None, w_down=None, h=None, y=None,
                   workspace=None):
    """The dense MLP of a Residual-MoE layer on every token row of x: the
    grouped FFN with one expert holding rows [0, N).  offsets: device int32
    tensor holding {0, N}; weights [1, ffn_s, d] / [1, d, ffn_s], or w_gate
    alone: PackedFfnWeights of one expert.  Returns (h, y)."""
    if isinstance(w_gate, PackedFfnWeights):
        if w_gate.E != 1:
            raise ValueError("the shared MLP is one expert")
        return moe_grouped_ffn_packed(x, offsets, w_gate, x.shape[0], h, y, workspace)
    if w_gate.shape[0] != 1:
        raise ValueError("the shared MLP is one expert")
    return moe_grouped_ffn(x, offsets, w_gate, w_up, w_down, x.shape[0], h, y, workspace)


def moe_exchange_workspace_bytes(E, W):
    return int(load_library().moe_exchange_workspace_bytes(E, W))


def moe_exchange_plan(topk_idx, disp, E, W, out=None):
    """Plan of the virtual W-source exchange from a dispatch's outputs.

    Returns a dict with src_counts [W, E], traffic [W, W], send_row [N, K]
    and the gather maps send_token, a2a_src, regroup_src [max_rows]."""
    dev = topk_idx.device
    _need(topk_idx, "topk_idx", torch.int32, dev)
    N, K = topk_idx.shape
    max_rows = N * K
    for k in ("dest", "perm_token", "offsets"):
        _need(disp[k], k, torch.int32, dev)
    if out is None:
        out = {
            "src_counts": torch.empty(W, E, dtype=torch.int32, device=dev),
            "traffic": torch.empty(W, W, dtype=torch.int32, device=dev),
            "send_row": torch.empty(N, K, dtype=torch.int32, device=dev),
            "send_token": torch.empty(max_rows, dtype=torch.int32, device=dev),
            "a2a_src": torch.empty(max_rows, dtype=torch.int32, device=dev),
            "regroup_src": torch.empty(max_rows, dtype=torch.int32, device=dev),
            "workspace": torch.empty(max(1, moe_exchange_workspace_bytes(E, W)),
                                     dtype=torch.uint8, device=dev),
        }
    sizes = {"src_counts": W * E, "traffic": W * W, "send_row": N * K, "send_token": max_rows,
             "a2a_src": max_rows, "regroup_src": max_rows}
    for k, n in sizes.items():
        _need(out[k], k, torch.int32, dev)
        if out[k].numel() < n:
            raise ValueError(f"{k} must hold at least {n} elements")
    ws = out["workspace"]
    _need(ws, "workspace", None, dev)
    _check("moe_exchange_plan", load_library().moe_exchange_plan(
        _ptr(topk_idx), _ptr(disp["dest"]), _ptr(disp["perm_token"]), _ptr(disp["offsets"]),
        N, E, K, W, max_rows, _ptr(out["src_counts"]), _ptr(out["traffic"]),
        _ptr(out["send_row"]), _ptr(out["send_token"]), _ptr(out["a2a_src"]),
        _ptr(out["regroup_src"]), _ptr(ws), ws.numel() * ws.element_size(), _stream(topk_idx)))
    return out


def moe_rows_permute(src, dst, row_map, n_rows, scatter=False, max_rows=None):
    """dst[i] = src[map[i]] (gather) or dst[map[i]] = src[i] (scatter) for
    i < min(n_rows[0], max_rows); n_rows is a one-element int32 device tensor."""
    dev = src.device
    _need(src, "src", None, dev)
    _need(dst, "dst", src.dtype, dev)
    _need(row_map, "map", torch.int32, dev)
    _need(n_rows, "n_rows", torch.int32, dev)
    if src.dim() != 2 or dst.dim() != 2 or src.shape[1] != dst.shape[1]:
        raise ValueError("src and dst must be 2-D with the same row length")
    if max_rows is None:
        max_rows = row_map.numel()
    if row_map.numel() < max_rows:
        raise ValueError("map shorter than max_rows")
    row_bytes = src.shape[1] * src.element_size()
    _check("moe_rows_permute", load_library().moe_rows_permute(
        _ptr(src), _ptr(dst), _ptr(row_map), _ptr(n_rows), int(max_rows), row_bytes,
        int(bool(scatter)), _stream(src)))
    return dst


class MoeLayer:
    """The four calls of one layer over preallocated buffers.

    Buffers are sized once for (N, d, ffn, E, K, W, dtype); ``forward`` then
    enqueues route -> dispatch -> grouped FFN -> combine on the current
    stream with no host synchronisation and no allocation.  gate picks the
    router's gate function; reroute=True re-routes capacity overflow to
    next-best experts between route and dispatch.  fp8=True (bf16 layers)
    sends both exchanges as fp8: dispatch packs e4m3 codes, the rows are
    turned back into bf16 for the FFN, its output rows are quantized and
    the combine reads them as fp8.  shared_ffn > 0 makes it a Residual-MoE
    layer with a shared MLP of that width: ``forward(..., shared=...)`` runs
    it on every token and adds its output in the combine.  planned (the
    default without reroute) routes with moe_route_plan, which also ranks
    and counts the tokens per expert, and dispatches with
    moe_dispatch_planned, which needs no counting pass; planned=False
    routes with moe_route_topk and dispatches with moe_dispatch.
    """

    def __init__(self, N, d, ffn, E, K, W, capacity, dtype, device, renormalize=False,
                 gate="softmax", reroute=False, fp8=False, shared_ffn=0, planned=None):
        self.N, self.d, self.ffn_dim, self.E, self.K, self.W = N, d, ffn, E, K, W
        self.capacity = int(capacity)
        self.renormalize = renormalize
        self.gate = gate
        _gate(gate)
        self.reroute = reroute
        if planned is None:
            tokens = 128 if E <= 8 else 64          # moe_route_plan's blocks
            planned = not reroute and -(-N // tokens) * E <= PLAN_MAX_COUNTS
        if planned and reroute:
            raise ValueError("a re-route changes the experts after the plan is made: "
                             "planned=False with reroute=True")
        self.planned = bool(planned)
        self.fp8 = fp8
        if fp8 and (dtype != torch.bfloat16 or d % FP8_GROUP):
            raise ValueError("the fp8 payload needs bf16 rows with d a multiple of 128")
        self.max_rows = N * K
        dev = torch.device(device)
        self.topk_idx = torch.empty(N, K, dtype=torch.int32, device=dev)
        self.topk_w = torch.empty(N, K, dtype=torch.float32, device=dev)
        self.disp = alloc_dispatch_outputs(N, d, E, K, W, dtype, dev)
        self.plan = alloc_route_plan(N, E, K, dev) if self.planned else None
        self.h = torch.empty(self.max_rows, ffn, dtype=dtype, device=dev)
        self.y_perm = torch.empty(self.max_rows, d, dtype=dtype, device=dev)
        self.ffn_ws = torch.empty(max(1, moe_grouped_ffn_workspace_bytes(self.max_rows, E, dtype)),
                                  dtype=torch.uint8, device=dev)
        self.out = torch.empty(N, d, dtype=dtype, device=dev)
        self.rerouted = torch.zeros(E, dtype=torch.int32, device=dev)
        self.reroute_ws = (torch.empty(max(1, moe_reroute_workspace_bytes(N, E, K)),
                                       dtype=torch.uint8, device=dev) if reroute else None)
        self.shared_ffn = int(shared_ffn)
        if self.shared_ffn > 0:
            if fp8:
                raise ValueError("the Residual-MoE combine reads bf16 or fp32 rows")
            self.shared_offsets = torch.tensor([0, N], dtype=torch.int32, device=dev)
            self.h_shared = torch.empty(N, self.shared_ffn, dtype=dtype, device=dev)
            self.y_shared = torch.empty(N, d, dtype=dtype, device=dev)
            self.shared_ws = torch.empty(max(1, moe_grouped_ffn_workspace_bytes(N, 1, dtype)),
                                         dtype=torch.uint8, device=dev)
        if fp8:
            self.disp8 = alloc_dispatch_fp8_outputs(N, d, E, K, W, dev)
            self.disp8["x_perm"] = self.disp["x_perm"]     # receive-side bf16 rows
            self.disp = self.disp8
            self.y8 = torch.empty(self.max_rows, d, dtype=torch.uint8, device=dev)
            self.y_scale = torch.empty(self.max_rows, d // FP8_GROUP, dtype=torch.float32,
                                       device=dev)

    def route(self, logits):
        if self.planned:
            moe_route_plan(logits, self.K, self.W, self.capacity, self.plan, self.disp,
                           self.renormalize, self.topk_idx, self.topk_w, self.gate)
            return self.topk_idx, self.topk_w
        moe_route_topk(logits, self.K, self.renormalize, self.topk_idx, self.topk_w, self.gate)
        if self.reroute:
            moe_reroute_overflow(logits, self.topk_idx, self.topk_w, self.capacity, self.gate,
                                 self.renormalize, self.rerouted, self.reroute_ws)
        return self.topk_idx, self.topk_w

    def dispatch(self, x):
        """(planned layers: after route, which made the plan)"""
        if self.planned:
            moe_dispatch_planned(x, self.topk_idx, self.E, self.W, self.capacity, self.plan,
                                 self.disp, fp8=self.fp8)
            if not self.fp8:
                return self.disp
        elif not self.fp8:
            return moe_dispatch(x, self.topk_idx, self.E, self.W, self.capacity, self.disp)
        else:
            moe_dispatch_fp8(x, self.topk_idx, self.E, self.W, self.capacity, self.disp)
        n_rows = self.disp["offsets"][self.E:]
        moe_fp8_dequantize_rows(self.disp["x8"], self.disp["x_scale"], n_rows, self.max_rows,
                                self.disp["x_perm"])
        return self.disp

    def ffn(self, w_gate, w_up=None, w_down=None):
        """w_gate, w_up, w_down: the weights, or w_gate alone: PackedFfnWeights
        from moe_pack_ffn_weights (bf16 layers)."""
        if isinstance(w_gate, PackedFfnWeights):
            return moe_grouped_ffn_packed(self.disp["x_perm"], self.disp["offsets"], w_gate,
                                          self.max_rows, self.h, self.y_perm, self.ffn_ws)
        return moe_grouped_ffn(self.disp["x_perm"], self.disp["offsets"], w_gate, w_up, w_down,
                               self.max_rows, self.h, self.y_perm, self.ffn_ws)

    def shared(self, x, w_gate, w_up=None, w_down=None):
        """The shared MLP on every token (Residual-MoE layers)."""
        if self.shared_ffn <= 0:
            raise ValueError("layer built without a shared MLP (shared_ffn=0)")
        return moe_shared_ffn(x, self.shared_offsets, w_gate, w_up, w_down, self.h_shared,
                              self.y_shared, self.shared_ws)

    def combine(self, residual=False):
        if residual:
            return moe_combine_residual(self.y_perm, self.disp["dest"], self.topk_w,
                                        self.y_shared, self.out)
        if not self.fp8:
            return moe_combine(self.y_perm, self.disp["dest"], self.topk_w, self.out)
        n_rows = self.disp["offsets"][self.E:]
        moe_fp8_quantize_rows(self.y_perm, n_rows, self.max_rows, self.y8, self.y_scale)
        return moe_combine_fp8(self.y8, self.y_scale, self.disp["dest"], self.topk_w, self.out)

    def capture(self, logits, x, w_gate, w_up=None, w_down=None, shared=None, warmup=2):
        """Record ``forward`` on these buffers as one HIP graph and return it
        (a torch.cuda.CUDAGraph).  ``graph.replay()`` then enqueues route ->
        dispatch -> grouped FFN -> combine as one graph launch, reading
        whatever the buffers hold at replay time: decode-sized layers, whose
        step is a handful of short kernels, lose the per-call launch costs.
        Nothing is allocated inside the captured calls (every buffer and
        workspace belongs to the layer), and no library call records a
        memset.  The input buffers, weights and the layer must stay alive,
        at the same addresses, for as long as the graph is replayed.  A few
        eager calls run first (``warmup``) so that one-time set-up (kernel
        attributes, device properties) happens outside the capture."""
        dev = self.topk_idx.device
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            for _ in range(warmup):
                self.forward(logits, x, w_gate, w_up, w_down, shared)
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize(dev)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.forward(logits, x, w_gate, w_up, w_down, shared)
        return graph

    def forward(self, logits, x, w_gate, w_up=None, w_down=None, shared=None):
        """shared (Residual-MoE layers): the shared MLP's weights as a tuple
        (w_gate, w_up, w_down) of one expert, or PackedFfnWeights of one."""
        self.route(logits)
        self.dispatch(x)
        self.ffn(w_gate, w_up, w_down)
        if shared is None:
            return self.combine()
        if isinstance(shared, PackedFfnWeights):
            self.shared(x, shared)
        else:
            self.shared(x, *shared)
        return self.combine(residual=True)

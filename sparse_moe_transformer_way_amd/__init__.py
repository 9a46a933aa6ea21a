"""Mixtral sparse mixture-of-experts feed-forward layer on MI355X (gfx950).

Thin Python binding over the C ABI of libmoe_mi355x.so (declared in
include/moe.h).  Every function has the name of the C entry point it calls and
does argument marshalling only: torch supplies device memory and the current
HIP stream, the library's HIP kernels do all of the layer's work.  Outputs that
are not passed in are allocated with torch.empty on the inputs' device.

    desc = make_desc(d_model=4096, d_ffn=14336, dtype=torch.bfloat16)
    y, idx, gate, counts = moe_layer_forward(desc, x, w_gate, w1, w3, w2)
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from ._lib import (  # noqa: F401
    LIB_PATH, MOE_BF16, MOE_FP8_E4M3, MOE_NOALLOC_SCRATCH_BYTES, MOE_ERR_HIP, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED,
    MOE_ERR_WORKSPACE_TOO_SMALL, MOE_F32, MOE_OK, LayerDesc, MoeError, SIGNATURES, lib,
)

__all__ = [
    "make_desc", "moe_version", "moe_default_tile_m", "moe_max_permuted_rows", "moe_workspace_size",
    "moe_router_topk", "moe_permute", "moe_expert_gate_up", "moe_expert_down", "moe_grouped_swiglu",
    "moe_combine", "moe_rmsnorm", "moe_layer_forward", "moe_layer_forward_timed", "moe_layer_forward_noalloc", "moe_block_workspace_size",
    "moe_block_forward", "moe_quantize_fp8", "moe_expert_gate_up_fp8", "moe_expert_down_fp8",
    "moe_layer_forward_fp8", "moe_backward_workspace_size", "moe_layer_backward", "LayerDesc", "MoeError",
]

_DT = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}


def make_desc(d_model: int, d_ffn: int, n_experts: int = 8, top_k: int = 2,
              dtype: torch.dtype = torch.bfloat16,
              weight_dtype: Optional[torch.dtype] = None) -> LayerDesc:
    """Layer descriptor.  weight_dtype defaults to dtype; torch.float8_e4m3fn
    selects FP8 expert weights (bf16 activations, the *_fp8 calls)."""
    if dtype not in _DT:
        raise TypeError(f"unsupported dtype {dtype}")
    code = _DT[dtype]
    if weight_dtype is None or weight_dtype == dtype:
        wcode = code
    elif weight_dtype == torch.float8_e4m3fn:
        wcode = MOE_FP8_E4M3
    else:
        raise TypeError(f"unsupported weight dtype {weight_dtype}")
    return LayerDesc(d_model, d_ffn, n_experts, top_k, code, wcode)


def _act_dtype(desc: LayerDesc) -> torch.dtype:
    return torch.bfloat16 if desc.act_dtype == MOE_BF16 else torch.float32


def _validate(fn: str, *specs) -> list:
    """Check every tensor argument of one call, then return their device
    pointers (None for an absent optional one).

    Each spec is (name, tensor, shape, dtype, optional).  The C ABI receives
    raw pointers and cannot see sizes, so a tensor smaller than the call reads
    or writes would be accessed out of bounds on the device; every shape is
    therefore checked against the descriptor, T and P_max here, and all shapes
    and dtypes are checked before any device check.  Raises ValueError
    (shape, contiguity, device) or TypeError (dtype) before any library call."""
    for name, t, shape, dtype, optional in specs:
        if t is None:
            if not optional:
                raise ValueError(f"{fn}: {name} is required")
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{fn}: {name} must be a torch.Tensor, got {type(t).__name__}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{fn}: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{fn}: {name} must be {dtype}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{fn}: {name} must be contiguous")
    dev = None
    for name, t, _, _, _ in specs:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{fn}: {name} must be a device tensor, got {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{fn}: {name} is on {t.device}, the other tensors on {dev}")
    return [None if t is None else t.data_ptr() for _, t, _, _, _ in specs]


def _rows(fn: str, desc: LayerDesc, T: int, tile_m: int) -> int:
    """P_max of the permuted layout (raises on an invalid descriptor, T or tile)."""
    P = lib.moe_max_permuted_rows(desc, T, tile_m)
    if P < 0:
        raise MoeError(fn, MOE_ERR_INVALID_ARGUMENT)
    return P


def _workspace(fn: str, workspace, need: int, dev):
    if workspace is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if workspace.dim() != 1:
        raise ValueError(f"{fn}: workspace must be a 1-D uint8 tensor")
    return workspace


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status)


def moe_version() -> int:
    return lib.moe_version()


def moe_default_tile_m(desc: LayerDesc, T: int) -> int:
    return lib.moe_default_tile_m(desc, T)


def moe_max_permuted_rows(desc: LayerDesc, T: int, tile_m: int = 0) -> int:
    return lib.moe_max_permuted_rows(desc, T, tile_m)


def moe_workspace_size(desc: LayerDesc, T: int, tile_m: int = 0) -> int:
    return lib.moe_workspace_size(desc, T, tile_m)


def moe_block_workspace_size(desc: LayerDesc, T: int) -> int:
    return lib.moe_block_workspace_size(desc, T)


def moe_router_topk(desc, x, w_gate, topk_idx=None, topk_gate=None, logits_out=None, stream=None):
    """Router logits, Top-K and gates.  Returns (topk_idx [T,K] int32, topk_gate [T,K] fp32)."""
    fn = "moe_router_topk"
    T = x.shape[0]
    d, n, K = desc.d_model, desc.n_experts, desc.top_k
    dev = x.device
    if topk_idx is None:
        topk_idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    if topk_gate is None:
        topk_gate = torch.empty((T, K), dtype=torch.float32, device=dev)
    p = _validate(fn, ("x", x, (T, d), _act_dtype(desc), False),
                  ("w_gate", w_gate, (d, n), torch.float32, False),
                  ("topk_idx", topk_idx, (T, K), torch.int32, False),
                  ("topk_gate", topk_gate, (T, K), torch.float32, False),
                  ("logits_out", logits_out, (T, n), torch.float32, True))
    _check(fn, lib.moe_router_topk(desc, T, *p, _stream(stream)))
    return topk_idx, topk_gate


def moe_permute(desc, topk_idx, tile_m, counts=None, offsets=None, row_src=None, row_of=None,
                stream=None):
    """Group assignments by expert.  Returns (counts, offsets, row_src, row_of)."""
    fn = "moe_permute"
    T = topk_idx.shape[0]
    dev = topk_idx.device
    P = _rows(fn, desc, T, tile_m)
    n, K = desc.n_experts, desc.top_k
    counts = torch.empty(n, dtype=torch.int32, device=dev) if counts is None else counts
    offsets = torch.empty(n + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    row_src = torch.empty(P, dtype=torch.int32, device=dev) if row_src is None else row_src
    row_of = torch.empty((T, K), dtype=torch.int32, device=dev) if row_of is None else row_of
    p = _validate(fn, ("topk_idx", topk_idx, (T, K), torch.int32, False),
                  ("counts", counts, (n,), torch.int32, False),
                  ("offsets", offsets, (n + 1,), torch.int32, False),
                  ("row_src", row_src, (P,), torch.int32, False),
                  ("row_of", row_of, (T, K), torch.int32, False))
    _check(fn, lib.moe_permute(desc, T, tile_m, *p, _stream(stream)))
    return counts, offsets, row_src, row_of


def _grouped_specs(desc, T, P, x=None, row_src=None, counts=None, offsets=None, w1=None, w3=None,
                   h=None, w2=None, y_perm=None, gate_up=True, down=True):
    """Argument specs of the grouped expert calls (bf16 or fp32 weights)."""
    dt = _act_dtype(desc)
    d, F, n = desc.d_model, desc.d_ffn, desc.n_experts
    specs = []
    if gate_up:
        specs += [("x", x, (T, d), dt, False), ("row_src", row_src, (P,), torch.int32, False)]
    specs += [("counts", counts, (n,), torch.int32, False), ("offsets", offsets, (n + 1,), torch.int32, False)]
    if gate_up:
        specs += [("w1", w1, (n, F, d), dt, False), ("w3", w3, (n, F, d), dt, False)]
    if down:
        specs += [("w2", w2, (n, d, F), dt, False)]
    specs += [("h", h, (P, F), dt, False)]
    if down:
        specs += [("y_perm", y_perm, (P, d), torch.float32, False)]
    return specs


def moe_expert_gate_up(desc, T, tile_m, x, row_src, counts, offsets, w1, w3, h=None, stream=None):
    """h = SiLU(w1 . x) * (w3 . x) over the grouped rows.  Returns h [P_max, F]."""
    fn = "moe_expert_gate_up"
    P = _rows(fn, desc, T, tile_m)
    if h is None:
        h = torch.empty((P, desc.d_ffn), dtype=_act_dtype(desc), device=x.device)
    xp, rp, cp, op, w1p, w3p, hp = _validate(fn, *_grouped_specs(
        desc, T, P, x=x, row_src=row_src, counts=counts, offsets=offsets, w1=w1, w3=w3, h=h, down=False))
    _check(fn, lib.moe_expert_gate_up(desc, T, tile_m, xp, rp, cp, op, w1p, w3p, hp, _stream(stream)))
    return h


def moe_expert_down(desc, T, tile_m, h, counts, offsets, w2, y_perm=None, stream=None):
    """y_perm = w2 . h over the grouped rows.  Returns y_perm [P_max, d] fp32."""
    fn = "moe_expert_down"
    P = _rows(fn, desc, T, tile_m)
    if y_perm is None:
        y_perm = torch.empty((P, desc.d_model), dtype=torch.float32, device=h.device)
    cp, op, w2p, hp, yp = _validate(fn, *_grouped_specs(
        desc, T, P, counts=counts, offsets=offsets, h=h, w2=w2, y_perm=y_perm, gate_up=False))
    _check(fn, lib.moe_expert_down(desc, T, tile_m, hp, cp, op, w2p, yp, _stream(stream)))
    return y_perm


def moe_grouped_swiglu(desc, T, tile_m, x, row_src, counts, offsets, w1, w3, w2, h=None,
                       y_perm=None, stream=None):
    """Both expert projections.  Returns (h, y_perm)."""
    fn = "moe_grouped_swiglu"
    P = _rows(fn, desc, T, tile_m)
    if h is None:
        h = torch.empty((P, desc.d_ffn), dtype=_act_dtype(desc), device=x.device)
    if y_perm is None:
        y_perm = torch.empty((P, desc.d_model), dtype=torch.float32, device=x.device)
    xp, rp, cp, op, w1p, w3p, w2p, hp, yp = _validate(fn, *_grouped_specs(
        desc, T, P, x=x, row_src=row_src, counts=counts, offsets=offsets, w1=w1, w3=w3, h=h, w2=w2,
        y_perm=y_perm))
    _check(fn, lib.moe_grouped_swiglu(desc, T, tile_m, xp, rp, cp, op, w1p, w3p, w2p, hp, yp,
                                      _stream(stream)))
    return h, y_perm


def moe_combine(desc, y_perm, row_of, topk_gate, residual=None, y=None, stream=None):
    """y = sum_s gate[:, s] * y_perm[row_of[:, s]] (+ residual).  Returns y [T, d].

    row_of must be moe_permute's output for the layout y_perm was computed in
    (every entry below y_perm's row count, or negative)."""
    fn = "moe_combine"
    T = row_of.shape[0]
    dt = _act_dtype(desc)
    d, K = desc.d_model, desc.top_k
    if y is None:
        y = torch.empty((T, d), dtype=dt, device=y_perm.device)
    if y_perm.dim() != 2 or y_perm.shape[0] < T * K:
        raise ValueError(f"{fn}: y_perm has shape {tuple(y_perm.shape)}, expected [>= {T * K}, {d}]")
    p = _validate(fn, ("y_perm", y_perm, (y_perm.shape[0], d), torch.float32, False),
                  ("row_of", row_of, (T, K), torch.int32, False),
                  ("topk_gate", topk_gate, (T, K), torch.float32, False),
                  ("residual", residual, (T, d), dt, True),
                  ("y", y, (T, d), dt, False))
    _check(fn, lib.moe_combine(desc, T, *p, _stream(stream)))
    return y


def moe_rmsnorm(h, eps: float = 1e-5, x_out=None, stream=None):
    """x = h / sqrt(mean(h^2) + eps) per row.  Returns x [T, d]."""
    fn = "moe_rmsnorm"
    if h.dim() != 2:
        raise ValueError(f"{fn}: h must be 2-D [T, d], got shape {tuple(h.shape)}")
    T, d = h.shape
    if h.dtype not in _DT:
        raise TypeError(f"unsupported dtype {h.dtype}")
    if x_out is None:
        x_out = torch.empty_like(h)
    hp, xp = _validate(fn, ("h", h, (T, d), h.dtype, False), ("x_out", x_out, (T, d), h.dtype, False))
    _check(fn, lib.moe_rmsnorm(T, d, _DT[h.dtype], hp, eps, xp, _stream(stream)))
    return x_out


def _layer_specs(desc, T, x, w_gate, w1, w3, w2, residual, y, topk_idx_out, topk_gate_out, counts_out,
                 wdt=None, scales=None):
    dt = _act_dtype(desc)
    wdt = dt if wdt is None else wdt
    d, F, n, K = desc.d_model, desc.d_ffn, desc.n_experts, desc.top_k
    specs = [("x", x, (T, d), dt, False), ("w_gate", w_gate, (d, n), torch.float32, False)]
    s1, s3, s2 = scales if scales is not None else (None, None, None)
    specs.append(("w1", w1, (n, F, d), wdt, False))
    if scales is not None:
        specs.append(("s1", s1, (n, F), torch.float32, False))
    specs.append(("w3", w3, (n, F, d), wdt, False))
    if scales is not None:
        specs.append(("s3", s3, (n, F), torch.float32, False))
    specs.append(("w2", w2, (n, d, F), wdt, False))
    if scales is not None:
        specs.append(("s2", s2, (n, d), torch.float32, False))
    specs += [("residual", residual, (T, d), dt, True), ("y", y, (T, d), dt, False),
              ("topk_idx_out", topk_idx_out, (T, K), torch.int32, False),
              ("topk_gate_out", topk_gate_out, (T, K), torch.float32, False),
              ("counts_out", counts_out, (n,), torch.int32, False)]
    return specs


def moe_layer_forward(desc, x, w_gate, w1, w3, w2, residual=None, y=None, topk_idx_out=None,
                      topk_gate_out=None, counts_out=None, workspace=None, stream=None):
    """The whole layer.  Returns (y, topk_idx, topk_gate, counts).

    ``workspace`` may be a preallocated 1-D uint8 device tensor of at least
    moe_workspace_size(desc, T) bytes (256-byte aligned); otherwise one is allocated.
    """
    fn = "moe_layer_forward"
    T = x.shape[0]
    dt = _act_dtype(desc)
    dev = x.device
    n, K = desc.n_experts, desc.top_k
    if y is None:
        y = torch.empty((T, desc.d_model), dtype=dt, device=dev)
    if topk_idx_out is None:
        topk_idx_out = torch.empty((T, K), dtype=torch.int32, device=dev)
    if topk_gate_out is None:
        topk_gate_out = torch.empty((T, K), dtype=torch.float32, device=dev)
    if counts_out is None:
        counts_out = torch.empty(n, dtype=torch.int32, device=dev)
    workspace = _workspace(fn, workspace, lib.moe_workspace_size(desc, T, 0), dev)
    p = _validate(fn, *_layer_specs(desc, T, x, w_gate, w1, w3, w2, residual, y, topk_idx_out,
                                    topk_gate_out, counts_out),
                  ("workspace", workspace, (workspace.numel(),), torch.uint8, False))
    _check(fn, lib.moe_layer_forward(desc, T, *p, workspace.numel(), _stream(stream)))
    return y, topk_idx_out, topk_gate_out, counts_out


def moe_layer_forward_timed(desc, x, w_gate, w1, w3, w2, events, residual=None, y=None, topk_idx_out=None,
                            topk_gate_out=None, counts_out=None, workspace=None, stream=None):
    """moe_layer_forward with six torch.cuda.Event objects (timing enabled, each
    recorded at least once so that it exists) recorded on the stream before the
    router and after each of the five stages.  Returns (y, topk_idx, topk_gate, counts)."""
    fn = "moe_layer_forward_timed"
    if len(events) != 6:
        raise ValueError(f"{fn}: expected 6 events, got {len(events)}")
    handles = [e.cuda_event for e in events]
    if not all(handles):
        raise ValueError(f"{fn}: every event must have been recorded once (created) before the call")
    T = x.shape[0]
    dt = _act_dtype(desc)
    dev = x.device
    n, K = desc.n_experts, desc.top_k
    if y is None:
        y = torch.empty((T, desc.d_model), dtype=dt, device=dev)
    if topk_idx_out is None:
        topk_idx_out = torch.empty((T, K), dtype=torch.int32, device=dev)
    if topk_gate_out is None:
        topk_gate_out = torch.empty((T, K), dtype=torch.float32, device=dev)
    if counts_out is None:
        counts_out = torch.empty(n, dtype=torch.int32, device=dev)
    workspace = _workspace(fn, workspace, lib.moe_workspace_size(desc, T, 0), dev)
    p = _validate(fn, *_layer_specs(desc, T, x, w_gate, w1, w3, w2, residual, y, topk_idx_out,
                                    topk_gate_out, counts_out),
                  ("workspace", workspace, (workspace.numel(),), torch.uint8, False))
    arr = (ctypes.c_void_p * 6)(*handles)
    _check(fn, lib.moe_layer_forward_timed(desc, T, *p, workspace.numel(), arr, _stream(stream)))
    return y, topk_idx_out, topk_gate_out, counts_out


def moe_layer_forward_noalloc(desc, x, w_gate, w1, w3, w2, residual=None, y=None, topk_idx_out=None,
                              topk_gate_out=None, counts_out=None, stream=None):
    """The whole layer with the library's per-GPU scratch instead of a workspace
    (the C call allocates nothing; outputs not passed in are allocated here).
    Calls that overlap on one GPU race on that scratch.  Returns
    (y, topk_idx, topk_gate, counts)."""
    fn = "moe_layer_forward_noalloc"
    T = x.shape[0]
    dt = _act_dtype(desc)
    dev = x.device
    n, K = desc.n_experts, desc.top_k
    if y is None:
        y = torch.empty((T, desc.d_model), dtype=dt, device=dev)
    if topk_idx_out is None:
        topk_idx_out = torch.empty((T, K), dtype=torch.int32, device=dev)
    if topk_gate_out is None:
        topk_gate_out = torch.empty((T, K), dtype=torch.float32, device=dev)
    if counts_out is None:
        counts_out = torch.empty(n, dtype=torch.int32, device=dev)
    p = _validate(fn, *_layer_specs(desc, T, x, w_gate, w1, w3, w2, residual, y, topk_idx_out,
                                    topk_gate_out, counts_out))
    _check(fn, lib.moe_layer_forward_noalloc(desc, T, *p, _stream(stream)))
    return y, topk_idx_out, topk_gate_out, counts_out


def moe_block_forward(desc, h, w_gate, w1, w3, w2, eps: float = 1e-5, h_out=None,
                      topk_idx_out=None, counts_out=None, workspace=None, stream=None):
    """h_out = h + MoE(RMSNorm(h)).  Returns (h_out, topk_idx, counts)."""
    fn = "moe_block_forward"
    T = h.shape[0]
    dt = _act_dtype(desc)
    dev = h.device
    d, F, n, K = desc.d_model, desc.d_ffn, desc.n_experts, desc.top_k
    if h_out is None:
        h_out = torch.empty_like(h)
    if topk_idx_out is None:
        topk_idx_out = torch.empty((T, K), dtype=torch.int32, device=dev)
    if counts_out is None:
        counts_out = torch.empty(n, dtype=torch.int32, device=dev)
    workspace = _workspace(fn, workspace, lib.moe_block_workspace_size(desc, T), dev)
    hp, wgp, w1p, w3p, w2p, hop, ip, cp, wsp = _validate(
        fn, ("h", h, (T, d), dt, False), ("w_gate", w_gate, (d, n), torch.float32, False),
        ("w1", w1, (n, F, d), dt, False), ("w3", w3, (n, F, d), dt, False), ("w2", w2, (n, d, F), dt, False),
        ("h_out", h_out, (T, d), dt, False), ("topk_idx_out", topk_idx_out, (T, K), torch.int32, False),
        ("counts_out", counts_out, (n,), torch.int32, False),
        ("workspace", workspace, (workspace.numel(),), torch.uint8, False))
    _check(fn, lib.moe_block_forward(desc, T, hp, eps, wgp, w1p, w3p, w2p, hop, ip, cp, wsp, workspace.numel(),
                                     _stream(stream)))
    return h_out, topk_idx_out, counts_out


# ---------------------------------------------------------------------------
# FP8 (E4M3) expert weights: uint8 code tensors plus fp32 per-row scales
# ---------------------------------------------------------------------------

def moe_quantize_fp8(w, q=None, scale=None, stream=None):
    """Per-row E4M3 quantization of a bf16 tensor [..., cols].
    Returns (q uint8 of w's shape, scale fp32 [...])."""
    fn = "moe_quantize_fp8"
    if w.dim() < 1:
        raise ValueError(f"{fn}: w must have at least one dimension")
    cols = w.shape[-1]
    rows = w.numel() // cols if cols else 0
    if q is None:
        q = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    if scale is None:
        scale = torch.empty(w.shape[:-1], dtype=torch.float32, device=w.device)
    p = _validate(fn, ("w", w, tuple(w.shape), torch.bfloat16, False),
                  ("q", q, tuple(w.shape), torch.uint8, False),
                  ("scale", scale, tuple(w.shape[:-1]), torch.float32, False))
    _check(fn, lib.moe_quantize_fp8(rows, cols, *p, _stream(stream)))
    return q, scale


def moe_expert_gate_up_fp8(desc, T, x, row_src, counts, offsets, w1, s1, w3, s3, h=None, stream=None):
    """h = SiLU(s1 * (q1 . x)) * (s3 * (q3 . x)) over the grouped rows (tile_m 16).
    Returns h [P_max, F] bf16."""
    fn = "moe_expert_gate_up_fp8"
    d, F, n = desc.d_model, desc.d_ffn, desc.n_experts
    P = _rows(fn, desc, T, 16)
    if h is None:
        h = torch.empty((P, F), dtype=torch.bfloat16, device=x.device)
    u8, f32 = torch.uint8, torch.float32
    p = _validate(fn, ("x", x, (T, d), torch.bfloat16, False), ("row_src", row_src, (P,), torch.int32, False),
                  ("counts", counts, (n,), torch.int32, False), ("offsets", offsets, (n + 1,), torch.int32, False),
                  ("w1", w1, (n, F, d), u8, False), ("s1", s1, (n, F), f32, False),
                  ("w3", w3, (n, F, d), u8, False), ("s3", s3, (n, F), f32, False),
                  ("h", h, (P, F), torch.bfloat16, False))
    _check(fn, lib.moe_expert_gate_up_fp8(desc, T, *p, _stream(stream)))
    return h


def moe_expert_down_fp8(desc, T, h, counts, offsets, w2, s2, y_perm=None, stream=None):
    """y_perm = s2 * (q2 . h) over the grouped rows (tile_m 16).  Returns y_perm [P_max, d] fp32."""
    fn = "moe_expert_down_fp8"
    d, F, n = desc.d_model, desc.d_ffn, desc.n_experts
    P = _rows(fn, desc, T, 16)
    if y_perm is None:
        y_perm = torch.empty((P, d), dtype=torch.float32, device=h.device)
    p = _validate(fn, ("h", h, (P, F), torch.bfloat16, False), ("counts", counts, (n,), torch.int32, False),
                  ("offsets", offsets, (n + 1,), torch.int32, False),
                  ("w2", w2, (n, d, F), torch.uint8, False), ("s2", s2, (n, d), torch.float32, False),
                  ("y_perm", y_perm, (P, d), torch.float32, False))
    _check(fn, lib.moe_expert_down_fp8(desc, T, *p, _stream(stream)))
    return y_perm


def moe_layer_forward_fp8(desc, x, w_gate, w1, s1, w3, s3, w2, s2, residual=None, y=None,
                          topk_idx_out=None, topk_gate_out=None, counts_out=None, workspace=None,
                          stream=None):
    """The whole layer with FP8 expert weights.  Returns (y, topk_idx, topk_gate, counts)."""
    fn = "moe_layer_forward_fp8"
    T = x.shape[0]
    dev = x.device
    n, K = desc.n_experts, desc.top_k
    bf = torch.bfloat16
    if y is None:
        y = torch.empty((T, desc.d_model), dtype=bf, device=dev)
    if topk_idx_out is None:
        topk_idx_out = torch.empty((T, K), dtype=torch.int32, device=dev)
    if topk_gate_out is None:
        topk_gate_out = torch.empty((T, K), dtype=torch.float32, device=dev)
    if counts_out is None:
        counts_out = torch.empty(n, dtype=torch.int32, device=dev)
    workspace = _workspace(fn, workspace, lib.moe_workspace_size(desc, T, 0), dev)
    p = _validate(fn, *_layer_specs(desc, T, x, w_gate, w1, w3, w2, residual, y, topk_idx_out, topk_gate_out,
                                    counts_out, wdt=torch.uint8, scales=(s1, s3, s2)),
                  ("workspace", workspace, (workspace.numel(),), torch.uint8, False))
    _check(fn, lib.moe_layer_forward_fp8(desc, T, *p, workspace.numel(), _stream(stream)))
    return y, topk_idx_out, topk_gate_out, counts_out


# ---------------------------------------------------------------------------
# Backward pass
# ---------------------------------------------------------------------------

def moe_backward_workspace_size(desc, T: int) -> int:
    return lib.moe_backward_workspace_size(desc, T)


def moe_layer_backward(desc, x, w_gate, w1, w3, w2, dy, dx=None, dw_gate=None, dw1=None, dw3=None, dw2=None,
                       workspace=None, stream=None):
    """Gradients of sum(dy * y) for the bf16 layer.
    Returns (dx bf16 [T, d], dw_gate fp32 [d, n], dw1, dw3 fp32 [n, F, d], dw2 fp32 [n, d, F])."""
    fn = "moe_layer_backward"
    T = x.shape[0]
    dev = x.device
    n, d, F = desc.n_experts, desc.d_model, desc.d_ffn
    bf, f32 = torch.bfloat16, torch.float32
    if dx is None:
        dx = torch.empty((T, d), dtype=bf, device=dev)
    if dw_gate is None:
        dw_gate = torch.empty((d, n), dtype=f32, device=dev)
    if dw1 is None:
        dw1 = torch.empty((n, F, d), dtype=f32, device=dev)
    if dw3 is None:
        dw3 = torch.empty((n, F, d), dtype=f32, device=dev)
    if dw2 is None:
        dw2 = torch.empty((n, d, F), dtype=f32, device=dev)
    workspace = _workspace(fn, workspace, lib.moe_backward_workspace_size(desc, T), dev)
    p = _validate(fn, ("x", x, (T, d), bf, False), ("w_gate", w_gate, (d, n), f32, False),
                  ("w1", w1, (n, F, d), bf, False), ("w3", w3, (n, F, d), bf, False),
                  ("w2", w2, (n, d, F), bf, False), ("dy", dy, (T, d), bf, False), ("dx", dx, (T, d), bf, False),
                  ("dw_gate", dw_gate, (d, n), f32, False), ("dw1", dw1, (n, F, d), f32, False),
                  ("dw3", dw3, (n, F, d), f32, False), ("dw2", dw2, (n, d, F), f32, False),
                  ("workspace", workspace, (workspace.numel(),), torch.uint8, False))
    _check(fn, lib.moe_layer_backward(desc, T, *p, workspace.numel(), _stream(stream)))
    return dx, dw_gate, dw1, dw3, dw2

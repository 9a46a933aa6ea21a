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

from typing import Optional

import torch

from ._lib import (  # noqa: F401
    LIB_PATH, MOE_BF16, MOE_FP8_E4M3, MOE_ERR_HIP, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED,
    MOE_ERR_WORKSPACE_TOO_SMALL, MOE_F32, MOE_OK, LayerDesc, MoeError, SIGNATURES, lib,
)

__all__ = [
    "make_desc", "moe_version", "moe_default_tile_m", "moe_max_permuted_rows", "moe_workspace_size",
    "moe_router_topk", "moe_permute", "moe_expert_gate_up", "moe_expert_down", "moe_grouped_swiglu",
    "moe_combine", "moe_rmsnorm", "moe_layer_forward", "moe_block_workspace_size",
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


def _ptr(t: Optional[torch.Tensor], dtype: Optional[torch.dtype] = None, name: str = "") -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a device tensor, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    return t.data_ptr()


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
    T = x.shape[0]
    dev = x.device
    if topk_idx is None:
        topk_idx = torch.empty((T, desc.top_k), dtype=torch.int32, device=dev)
    if topk_gate is None:
        topk_gate = torch.empty((T, desc.top_k), dtype=torch.float32, device=dev)
    _check("moe_router_topk", lib.moe_router_topk(
        desc, T, _ptr(x, _act_dtype(desc), "x"), _ptr(w_gate, torch.float32, "w_gate"),
        _ptr(topk_idx, torch.int32, "topk_idx"), _ptr(topk_gate, torch.float32, "topk_gate"),
        _ptr(logits_out, torch.float32, "logits_out"), _stream(stream)))
    return topk_idx, topk_gate


def moe_permute(desc, topk_idx, tile_m, counts=None, offsets=None, row_src=None, row_of=None,
                stream=None):
    """Group assignments by expert.  Returns (counts, offsets, row_src, row_of)."""
    T = topk_idx.shape[0]
    dev = topk_idx.device
    P = lib.moe_max_permuted_rows(desc, T, tile_m)
    if P < 0:
        raise MoeError("moe_max_permuted_rows", MOE_ERR_INVALID_ARGUMENT)
    n, K = desc.n_experts, desc.top_k
    counts = torch.empty(n, dtype=torch.int32, device=dev) if counts is None else counts
    offsets = torch.empty(n + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    row_src = torch.empty(P, dtype=torch.int32, device=dev) if row_src is None else row_src
    row_of = torch.empty((T, K), dtype=torch.int32, device=dev) if row_of is None else row_of
    _check("moe_permute", lib.moe_permute(
        desc, T, tile_m, _ptr(topk_idx, torch.int32, "topk_idx"), _ptr(counts, torch.int32, "counts"),
        _ptr(offsets, torch.int32, "offsets"), _ptr(row_src, torch.int32, "row_src"),
        _ptr(row_of, torch.int32, "row_of"), _stream(stream)))
    return counts, offsets, row_src, row_of


def moe_expert_gate_up(desc, T, tile_m, x, row_src, counts, offsets, w1, w3, h=None, stream=None):
    """h = SiLU(w1 . x) * (w3 . x) over the grouped rows.  Returns h [P_max, F]."""
    dt = _act_dtype(desc)
    if h is None:
        h = torch.empty((row_src.shape[0], desc.d_ffn), dtype=dt, device=x.device)
    _check("moe_expert_gate_up", lib.moe_expert_gate_up(
        desc, T, tile_m, _ptr(x, dt, "x"), _ptr(row_src, torch.int32, "row_src"),
        _ptr(counts, torch.int32, "counts"), _ptr(offsets, torch.int32, "offsets"),
        _ptr(w1, dt, "w1"), _ptr(w3, dt, "w3"), _ptr(h, dt, "h"), _stream(stream)))
    return h


def moe_expert_down(desc, T, tile_m, h, counts, offsets, w2, y_perm=None, stream=None):
    """y_perm = w2 . h over the grouped rows.  Returns y_perm [P_max, d] fp32."""
    dt = _act_dtype(desc)
    if y_perm is None:
        y_perm = torch.empty((h.shape[0], desc.d_model), dtype=torch.float32, device=h.device)
    _check("moe_expert_down", lib.moe_expert_down(
        desc, T, tile_m, _ptr(h, dt, "h"), _ptr(counts, torch.int32, "counts"),
        _ptr(offsets, torch.int32, "offsets"), _ptr(w2, dt, "w2"),
        _ptr(y_perm, torch.float32, "y_perm"), _stream(stream)))
    return y_perm


def moe_grouped_swiglu(desc, T, tile_m, x, row_src, counts, offsets, w1, w3, w2, h=None,
                       y_perm=None, stream=None):
    """Both expert projections.  Returns (h, y_perm)."""
    dt = _act_dtype(desc)
    P = row_src.shape[0]
    if h is None:
        h = torch.empty((P, desc.d_ffn), dtype=dt, device=x.device)
    if y_perm is None:
        y_perm = torch.empty((P, desc.d_model), dtype=torch.float32, device=x.device)
    _check("moe_grouped_swiglu", lib.moe_grouped_swiglu(
        desc, T, tile_m, _ptr(x, dt, "x"), _ptr(row_src, torch.int32, "row_src"),
        _ptr(counts, torch.int32, "counts"), _ptr(offsets, torch.int32, "offsets"),
        _ptr(w1, dt, "w1"), _ptr(w3, dt, "w3"), _ptr(w2, dt, "w2"), _ptr(h, dt, "h"),
        _ptr(y_perm, torch.float32, "y_perm"), _stream(stream)))
    return h, y_perm


def moe_combine(desc, y_perm, row_of, topk_gate, residual=None, y=None, stream=None):
    """y = sum_s gate[:, s] * y_perm[row_of[:, s]] (+ residual).  Returns y [T, d]."""
    T = row_of.shape[0]
    dt = _act_dtype(desc)
    if y is None:
        y = torch.empty((T, desc.d_model), dtype=dt, device=y_perm.device)
    _check("moe_combine", lib.moe_combine(
        desc, T, _ptr(y_perm, torch.float32, "y_perm"), _ptr(row_of, torch.int32, "row_of"),
        _ptr(topk_gate, torch.float32, "topk_gate"), _ptr(residual, dt, "residual"),
        _ptr(y, dt, "y"), _stream(stream)))
    return y


def moe_rmsnorm(h, eps: float = 1e-5, x_out=None, stream=None):
    """x = h / sqrt(mean(h^2) + eps) per row.  Returns x [T, d]."""
    T, d = h.shape
    if h.dtype not in _DT:
        raise TypeError(f"unsupported dtype {h.dtype}")
    if x_out is None:
        x_out = torch.empty_like(h)
    _check("moe_rmsnorm", lib.moe_rmsnorm(T, d, _DT[h.dtype], _ptr(h, h.dtype, "h"), eps,
                                          _ptr(x_out, h.dtype, "x_out"), _stream(stream)))
    return x_out


def moe_layer_forward(desc, x, w_gate, w1, w3, w2, residual=None, y=None, topk_idx_out=None,
                      topk_gate_out=None, counts_out=None, workspace=None, stream=None):
    """The whole layer.  Returns (y, topk_idx, topk_gate, counts).

    ``workspace`` may be a preallocated uint8 device tensor of at least
    moe_workspace_size(desc, T) bytes (256-byte aligned); otherwise one is allocated.
    """
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
    need = lib.moe_workspace_size(desc, T, 0)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check("moe_layer_forward", lib.moe_layer_forward(
        desc, T, _ptr(x, dt, "x"), _ptr(w_gate, torch.float32, "w_gate"), _ptr(w1, dt, "w1"),
        _ptr(w3, dt, "w3"), _ptr(w2, dt, "w2"), _ptr(residual, dt, "residual"), _ptr(y, dt, "y"),
        _ptr(topk_idx_out, torch.int32, "topk_idx_out"),
        _ptr(topk_gate_out, torch.float32, "topk_gate_out"),
        _ptr(counts_out, torch.int32, "counts_out"), _ptr(workspace, torch.uint8, "workspace"),
        workspace.numel(), _stream(stream)))
    return y, topk_idx_out, topk_gate_out, counts_out


def moe_block_forward(desc, h, w_gate, w1, w3, w2, eps: float = 1e-5, h_out=None,
                      topk_idx_out=None, counts_out=None, workspace=None, stream=None):
    """h_out = h + MoE(RMSNorm(h)).  Returns (h_out, topk_idx, counts)."""
    T = h.shape[0]
    dt = _act_dtype(desc)
    dev = h.device
    if h_out is None:
        h_out = torch.empty_like(h)
    if topk_idx_out is None:
        topk_idx_out = torch.empty((T, desc.top_k), dtype=torch.int32, device=dev)
    if counts_out is None:
        counts_out = torch.empty(desc.n_experts, dtype=torch.int32, device=dev)
    need = lib.moe_block_workspace_size(desc, T)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check("moe_block_forward", lib.moe_block_forward(
        desc, T, _ptr(h, dt, "h"), eps, _ptr(w_gate, torch.float32, "w_gate"), _ptr(w1, dt, "w1"),
        _ptr(w3, dt, "w3"), _ptr(w2, dt, "w2"), _ptr(h_out, dt, "h_out"),
        _ptr(topk_idx_out, torch.int32, "topk_idx_out"), _ptr(counts_out, torch.int32, "counts_out"),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))
    return h_out, topk_idx_out, counts_out


# ---------------------------------------------------------------------------
# FP8 (E4M3) expert weights: uint8 code tensors plus fp32 per-row scales
# ---------------------------------------------------------------------------

def moe_quantize_fp8(w, q=None, scale=None, stream=None):
    """Per-row E4M3 quantization of a bf16 tensor [..., cols].
    Returns (q uint8 of w's shape, scale fp32 [...])."""
    cols = w.shape[-1]
    rows = w.numel() // cols if cols else 0
    if q is None:
        q = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    if scale is None:
        scale = torch.empty(w.shape[:-1], dtype=torch.float32, device=w.device)
    _check("moe_quantize_fp8", lib.moe_quantize_fp8(
        rows, cols, _ptr(w, torch.bfloat16, "w"), _ptr(q, torch.uint8, "q"),
        _ptr(scale, torch.float32, "scale"), _stream(stream)))
    return q, scale


def moe_expert_gate_up_fp8(desc, T, x, row_src, counts, offsets, w1, s1, w3, s3, h=None, stream=None):
    """h = SiLU(s1 * (q1 . x)) * (s3 * (q3 . x)) over the grouped rows (tile_m 16).
    Returns h [P_max, F] bf16."""
    if h is None:
        h = torch.empty((row_src.shape[0], desc.d_ffn), dtype=torch.bfloat16, device=x.device)
    _check("moe_expert_gate_up_fp8", lib.moe_expert_gate_up_fp8(
        desc, T, _ptr(x, torch.bfloat16, "x"), _ptr(row_src, torch.int32, "row_src"),
        _ptr(counts, torch.int32, "counts"), _ptr(offsets, torch.int32, "offsets"),
        _ptr(w1, torch.uint8, "w1"), _ptr(s1, torch.float32, "s1"), _ptr(w3, torch.uint8, "w3"),
        _ptr(s3, torch.float32, "s3"), _ptr(h, torch.bfloat16, "h"), _stream(stream)))
    return h


def moe_expert_down_fp8(desc, T, h, counts, offsets, w2, s2, y_perm=None, stream=None):
    """y_perm = s2 * (q2 . h) over the grouped rows (tile_m 16).  Returns y_perm [P_max, d] fp32."""
    if y_perm is None:
        y_perm = torch.empty((h.shape[0], desc.d_model), dtype=torch.float32, device=h.device)
    _check("moe_expert_down_fp8", lib.moe_expert_down_fp8(
        desc, T, _ptr(h, torch.bfloat16, "h"), _ptr(counts, torch.int32, "counts"),
        _ptr(offsets, torch.int32, "offsets"), _ptr(w2, torch.uint8, "w2"), _ptr(s2, torch.float32, "s2"),
        _ptr(y_perm, torch.float32, "y_perm"), _stream(stream)))
    return y_perm


def moe_layer_forward_fp8(desc, x, w_gate, w1, s1, w3, s3, w2, s2, residual=None, y=None,
                          topk_idx_out=None, topk_gate_out=None, counts_out=None, workspace=None,
                          stream=None):
    """The whole layer with FP8 expert weights.  Returns (y, topk_idx, topk_gate, counts)."""
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
    need = lib.moe_workspace_size(desc, T, 0)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check("moe_layer_forward_fp8", lib.moe_layer_forward_fp8(
        desc, T, _ptr(x, bf, "x"), _ptr(w_gate, torch.float32, "w_gate"), _ptr(w1, torch.uint8, "w1"),
        _ptr(s1, torch.float32, "s1"), _ptr(w3, torch.uint8, "w3"), _ptr(s3, torch.float32, "s3"),
        _ptr(w2, torch.uint8, "w2"), _ptr(s2, torch.float32, "s2"), _ptr(residual, bf, "residual"),
        _ptr(y, bf, "y"), _ptr(topk_idx_out, torch.int32, "topk_idx_out"),
        _ptr(topk_gate_out, torch.float32, "topk_gate_out"), _ptr(counts_out, torch.int32, "counts_out"),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))
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
    need = lib.moe_backward_workspace_size(desc, T)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check("moe_layer_backward", lib.moe_layer_backward(
        desc, T, _ptr(x, bf, "x"), _ptr(w_gate, f32, "w_gate"), _ptr(w1, bf, "w1"), _ptr(w3, bf, "w3"),
        _ptr(w2, bf, "w2"), _ptr(dy, bf, "dy"), _ptr(dx, bf, "dx"), _ptr(dw_gate, f32, "dw_gate"),
        _ptr(dw1, f32, "dw1"), _ptr(dw3, f32, "dw3"), _ptr(dw2, f32, "dw2"),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))
    return dx, dw_gate, dw1, dw3, dw2

"""Host-side checks of the C-ABI library: it loads, exports every entry point
include/moe.h declares, and rejects bad arguments before enqueuing anything
(no compute call is made here)."""
import ctypes
import os
import re

import pytest

import sparse_moe_transformer_way_amd as moe
from sparse_moe_transformer_way_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    with open(os.path.join(ROOT, "include", "moe.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_header_and_library_agree():
    declared = header_functions()
    assert len(declared) >= 15
    assert set(declared) == set(_lib.SIGNATURES)
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_layer_entry_points_present():
    for name in ("moe_router_topk", "moe_permute", "moe_grouped_swiglu", "moe_combine",
                 "moe_layer_forward"):
        assert name in header_functions()


def test_status_strings_and_version():
    lib = _lib.lib
    for code, name in [(0, b"MOE_OK"), (1, b"MOE_ERR_INVALID_ARGUMENT"), (2, b"MOE_ERR_UNSUPPORTED"),
                       (3, b"MOE_ERR_WORKSPACE_TOO_SMALL"), (4, b"MOE_ERR_HIP"), (99, b"MOE_ERR_UNKNOWN")]:
        assert lib.moe_status_string(code) == name
    assert moe.moe_version() == 10000


def D(**kw):
    base = dict(d_model=4096, d_ffn=14336, n_experts=8, top_k=2, act_dtype=1, weight_dtype=1)
    base.update(kw)
    return _lib.LayerDesc(**base)


def test_sizes():
    d = D()
    assert moe.moe_default_tile_m(d, 32) == 16
    assert moe.moe_default_tile_m(d, 65) == 256
    assert moe.moe_default_tile_m(D(act_dtype=0, weight_dtype=0, d_model=128, d_ffn=256), 4096) == 16
    assert moe.moe_max_permuted_rows(d, 4096, 256) == 8192 + 8 * 255
    assert moe.moe_max_permuted_rows(d, 32, 0) == 64 + 8 * 15
    assert moe.moe_max_permuted_rows(d, 32, 100) == -1
    # tile 256 reaches x rows through 32-bit byte offsets: T * d * 2 (plus
    # one row of k offsets) must stay below 4 GiB
    T_big = (1 << 32) // (4096 * 2) - 1
    assert moe.moe_default_tile_m(d, T_big - 1) == 256
    assert moe.moe_default_tile_m(d, T_big) == 16
    assert moe.moe_max_permuted_rows(d, T_big, 256) == -1
    assert moe.moe_max_permuted_rows(d, T_big, 16) == 2 * T_big + 8 * 15
    ws = moe.moe_workspace_size(d, 4096, 0)
    P = 8192 + 8 * 255
    assert ws >= P * 14336 * 2 + P * 4096 * 4
    # 1 <= K <= n, n <= 16, K <= 4
    assert moe.moe_workspace_size(D(n_experts=17), 10, 0) == 0
    assert moe.moe_workspace_size(D(n_experts=16, top_k=5), 10, 0) == 0
    assert moe.moe_workspace_size(D(n_experts=3, top_k=4), 10, 0) == 0
    for n, K in [(16, 4), (4, 1), (1, 1), (5, 3)]:
        assert moe.moe_workspace_size(D(n_experts=n, top_k=K), 10, 0) > 0
        assert moe.moe_max_permuted_rows(D(n_experts=n, top_k=K), 10, 16) == 10 * K + n * 15
    assert moe.moe_block_workspace_size(d, 100) > moe.moe_workspace_size(d, 100, 0)


FAKE = 0x100000  # 16-byte-aligned non-null pointer value; never dereferenced


@pytest.mark.parametrize("desc,T,expect", [
    (None, 4, 1),
    (D(n_experts=17), 4, 2),
    (D(top_k=5), 4, 2),
    (D(top_k=9), 4, 1),
    (D(top_k=0), 4, 1),
    (D(act_dtype=0), 4, 2),
    (D(act_dtype=7), 4, 1),
    (D(d_model=100), 4, 1),
    (D(d_model=1024 + 8), 4, 2),   # bf16 needs d % 512
    (D(d_ffn=0), 4, 1),
    (D(), -1, 1),
])
def test_router_validation(desc, T, expect):
    lib = _lib.lib
    p = ctypes.byref(desc) if desc is not None else None
    assert lib.moe_router_topk(p, T, FAKE, FAKE, FAKE, FAKE, None, None) == expect


def test_null_and_alignment_rejections():
    lib = _lib.lib
    d = ctypes.byref(D())
    assert lib.moe_router_topk(d, 4, None, FAKE, FAKE, FAKE, None, None) == 1
    assert lib.moe_router_topk(d, 4, FAKE + 2, FAKE, FAKE, FAKE, None, None) == 1
    assert lib.moe_router_topk(d, 0, None, None, None, None, None, None) == 0  # T == 0 no-op
    assert lib.moe_permute(d, 4, 17, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.moe_permute(d, 4, 16, None, FAKE, FAKE, FAKE, FAKE, None) == 1
    f32 = ctypes.byref(D(act_dtype=0, weight_dtype=0, d_model=128, d_ffn=256))
    assert lib.moe_permute(f32, 4, 256, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert lib.moe_expert_gate_up(d, 4, 16, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None) == 1
    assert lib.moe_expert_down(d, 4, 16, FAKE, FAKE, FAKE, FAKE, None, None) == 1
    assert lib.moe_grouped_swiglu(d, 4, 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None) == 1
    assert lib.moe_combine(d, 4, FAKE, FAKE, FAKE, None, None, None) == 1
    assert lib.moe_rmsnorm(4, 12, 1, FAKE, 1e-5, FAKE, None) == 1
    assert lib.moe_rmsnorm(4, 16, 1, FAKE, -1.0, FAKE, None) == 1
    assert lib.moe_rmsnorm(4, 16, 1, FAKE, 1e-5, FAKE, None) == 1  # x_out aliases h
    assert lib.moe_rmsnorm(0, 16, 1, None, 1e-5, None, None) == 0


def test_layer_forward_workspace_checks():
    lib = _lib.lib
    d = D()
    need = moe.moe_workspace_size(d, 64, 0)
    args = [ctypes.byref(d), 64, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE + 4096, None, None, None]
    assert lib.moe_layer_forward(*args, FAKE, need - 1, None) == 3
    assert lib.moe_layer_forward(*args, FAKE + 16, need, None) == 1   # workspace not 256-aligned
    assert lib.moe_layer_forward(*args, None, need, None) == 1
    same = [ctypes.byref(d), 64, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, None]
    assert lib.moe_layer_forward(*same, FAKE, need, None) == 1        # y aliases x
    assert lib.moe_block_forward(ctypes.byref(d), 64, FAKE, 1e-5, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 None, None, FAKE, 10, None) == 3


def test_timed_and_noalloc_argument_checks():
    """moe_layer_forward_timed needs six event handles; moe_layer_forward_noalloc
    refuses a T whose workspace exceeds its scratch, before touching a device."""
    lib = _lib.lib
    d = ctypes.byref(D())
    args = [d, 32, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE + 4096, None, None, None]
    need = moe.moe_workspace_size(D(), 32, 0)
    ev = (ctypes.c_void_p * 6)(*([FAKE] * 5 + [None]))
    assert lib.moe_layer_forward_timed(*args, FAKE, need, None, None) == 1
    assert lib.moe_layer_forward_timed(*args, FAKE, need, ev, None) == 1
    f8 = ctypes.byref(D(weight_dtype=2))
    assert lib.moe_layer_forward_timed(f8, 32, *args[2:], FAKE, need, ev, None) == 1
    big = [d, 65, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE + 4096, None, None, None, None]
    assert moe.moe_workspace_size(D(), 65, 0) > moe.MOE_NOALLOC_SCRATCH_BYTES >= moe.moe_workspace_size(D(), 64, 0)
    assert lib.moe_layer_forward_noalloc(*big) == 3
    assert lib.moe_layer_forward_noalloc(d, 0, *([None] * 11)) == 0
    assert lib.moe_layer_forward_noalloc(d, 8, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, None,
                                         None) == 1  # y aliases x
    assert lib.moe_layer_forward_noalloc(f8, 8, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE + 4096, None, None, None,
                                         None) == 1


def test_binding_requires_device_tensors():
    import torch
    d = moe.make_desc(4096, 14336)
    with pytest.raises(ValueError, match="device tensor"):
        moe.moe_router_topk(d, torch.zeros(2, 4096, dtype=torch.bfloat16),
                            torch.zeros(4096, 8))


def _binding_calls(bad):
    """Each binding called with CPU tensors of the right shapes, except for the
    one argument named ``bad``, which gets one row too few (or the wrong dtype
    when bad ends in ':dtype').  d = 512, F = 1024, n = 8, K = 2, T = 40."""
    import torch
    bf, f32, i32, u8 = torch.bfloat16, torch.float32, torch.int32, torch.uint8
    d, F, n, K, T = 512, 1024, 8, 2, 40
    desc = moe.make_desc(d, F)
    P16 = moe.moe_max_permuted_rows(desc, T, 16)

    def t(name, shape, dt):
        if bad == name:
            shape = (shape[0] - 1,) + tuple(shape[1:]) if shape and shape[0] > 0 else (1,)
        if bad == name + ":dtype":
            dt = f32 if dt != f32 else bf
        return torch.zeros(shape, dtype=dt)

    return {
        "moe_router_topk": lambda: moe.moe_router_topk(
            desc, torch.zeros(T, d, dtype=bf), t("w_gate", (d, n), f32), t("topk_idx", (T, K), i32),
            t("topk_gate", (T, K), f32), t("logits_out", (T, n), f32)),
        "moe_permute": lambda: moe.moe_permute(
            desc, torch.zeros(T, K, dtype=i32), 16, t("counts", (n,), i32), t("offsets", (n + 1,), i32),
            t("row_src", (P16,), i32), t("row_of", (T, K), i32)),
        "moe_expert_gate_up": lambda: moe.moe_expert_gate_up(
            desc, T, 16, t("x", (T, d), bf), t("row_src", (P16,), i32), t("counts", (n,), i32),
            t("offsets", (n + 1,), i32), t("w1", (n, F, d), bf), t("w3", (n, F, d), bf), t("h", (P16, F), bf)),
        "moe_expert_down": lambda: moe.moe_expert_down(
            desc, T, 16, t("h", (P16, F), bf), t("counts", (n,), i32), t("offsets", (n + 1,), i32),
            t("w2", (n, d, F), bf), t("y_perm", (P16, d), f32)),
        "moe_grouped_swiglu": lambda: moe.moe_grouped_swiglu(
            desc, T, 16, t("x", (T, d), bf), t("row_src", (P16,), i32), t("counts", (n,), i32),
            t("offsets", (n + 1,), i32), t("w1", (n, F, d), bf), t("w3", (n, F, d), bf), t("w2", (n, d, F), bf),
            t("h", (P16, F), bf), t("y_perm", (P16, d), f32)),
        "moe_combine": lambda: moe.moe_combine(
            desc, t("y_perm", (P16, d), f32), torch.zeros(T, K, dtype=i32), t("topk_gate", (T, K), f32),
            t("residual", (T, d), bf), t("y", (T, d), bf)),
        "moe_layer_forward": lambda: moe.moe_layer_forward(
            desc, torch.zeros(T, d, dtype=bf), t("w_gate", (d, n), f32), t("w1", (n, F, d), bf),
            t("w3", (n, F, d), bf), t("w2", (n, d, F), bf), t("residual", (T, d), bf), t("y", (T, d), bf),
            t("topk_idx_out", (T, K), i32), t("topk_gate_out", (T, K), f32), t("counts_out", (n,), i32),
            workspace=torch.zeros(moe.moe_workspace_size(desc, T, 0), dtype=u8)),
        "moe_block_forward": lambda: moe.moe_block_forward(
            desc, torch.zeros(T, d, dtype=bf), t("w_gate", (d, n), f32), t("w1", (n, F, d), bf),
            t("w3", (n, F, d), bf), t("w2", (n, d, F), bf), h_out=t("h_out", (T, d), bf),
            topk_idx_out=t("topk_idx_out", (T, K), i32), counts_out=t("counts_out", (n,), i32),
            workspace=torch.zeros(16, dtype=u8)),
        "moe_layer_backward": lambda: moe.moe_layer_backward(
            desc, torch.zeros(T, d, dtype=bf), t("w_gate", (d, n), f32), t("w1", (n, F, d), bf),
            t("w3", (n, F, d), bf), t("w2", (n, d, F), bf), t("dy", (T, d), bf), t("dx", (T, d), bf),
            t("dw_gate", (d, n), f32), t("dw1", (n, F, d), f32), t("dw3", (n, F, d), f32),
            t("dw2", (n, d, F), f32), workspace=torch.zeros(16, dtype=u8)),
    }


BAD_ARGS = [("moe_router_topk", "w_gate"), ("moe_router_topk", "topk_gate"), ("moe_router_topk", "logits_out"),
            ("moe_permute", "row_src"), ("moe_permute", "offsets"), ("moe_permute", "row_of"),
            ("moe_expert_gate_up", "x"), ("moe_expert_gate_up", "h"), ("moe_expert_gate_up", "w3"),
            ("moe_expert_gate_up", "row_src"), ("moe_expert_down", "y_perm"), ("moe_expert_down", "w2"),
            ("moe_grouped_swiglu", "w1"), ("moe_grouped_swiglu", "y_perm"), ("moe_combine", "y"),
            ("moe_combine", "residual"), ("moe_combine", "topk_gate"), ("moe_layer_forward", "w2"),
            ("moe_layer_forward", "y"), ("moe_layer_forward", "counts_out"), ("moe_block_forward", "h_out"),
            ("moe_block_forward", "w1"), ("moe_layer_backward", "dw2"), ("moe_layer_backward", "dy")]


@pytest.mark.parametrize("fn,bad", BAD_ARGS)
def test_binding_checks_shapes_before_any_call(fn, bad):
    """A tensor smaller than the call would touch is refused by the binding
    (the C ABI sees raw pointers only), before any device check."""
    with pytest.raises(ValueError, match=f"{bad} has shape"):
        _binding_calls(bad)[fn]()


@pytest.mark.parametrize("fn,bad", [("moe_router_topk", "w_gate:dtype"), ("moe_expert_gate_up", "w1:dtype"),
                                    ("moe_layer_forward", "topk_idx_out:dtype")])
def test_binding_checks_dtypes(fn, bad):
    with pytest.raises(TypeError):
        _binding_calls(bad)[fn]()


@pytest.mark.parametrize("fn", ["moe_router_topk", "moe_permute", "moe_expert_gate_up", "moe_expert_down",
                                "moe_grouped_swiglu", "moe_combine", "moe_layer_forward", "moe_block_forward",
                                "moe_layer_backward"])
def test_binding_well_shaped_host_tensors_still_refused(fn):
    with pytest.raises(ValueError, match="device tensor"):
        _binding_calls(None)[fn]()


def test_fp8_descriptor_rules():
    """FP8 expert weights: bf16 activations, d and F multiples of 1024, tile 16
    only; the bf16 expert calls and the FP8 calls each reject the other's
    descriptor before any launch."""
    f8 = D(weight_dtype=2)
    assert moe.moe_default_tile_m(f8, 1000) == 16
    assert moe.moe_workspace_size(f8, 100, 256) == 0
    assert moe.moe_workspace_size(f8, 100, 0) == moe.moe_workspace_size(D(), 100, 16) > 0
    assert moe.moe_workspace_size(D(weight_dtype=2, d_model=1536), 10, 0) == 0
    assert moe.moe_workspace_size(D(weight_dtype=2, act_dtype=0), 10, 0) == 0
    assert moe.moe_workspace_size(D(weight_dtype=3), 10, 0) == 0
    lib = _lib.lib
    p8, pb = ctypes.byref(f8), ctypes.byref(D())
    assert lib.moe_expert_gate_up(p8, 4, 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.moe_expert_down(p8, 4, 16, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.moe_grouped_swiglu(p8, 4, 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.moe_layer_forward(p8, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE + 4096, None, None, None,
                                 FAKE, 1 << 30, None) == 1
    assert lib.moe_expert_gate_up_fp8(pb, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.moe_expert_down_fp8(pb, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.moe_layer_forward_fp8(pb, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE + 4096,
                                     None, None, None, FAKE, 1 << 30, None) == 1
    assert lib.moe_expert_down_fp8(p8, 4, FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == 1      # no scales
    assert lib.moe_expert_gate_up_fp8(p8, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 4, FAKE, FAKE, FAKE,
                                      None) == 1                                              # misaligned s1
    assert lib.moe_layer_forward_fp8(p8, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, FAKE + 4096,
                                     None, None, None, FAKE, 1 << 30, None) == 1              # no s3
    assert lib.moe_expert_gate_up_fp8(p8, 0, None, None, None, None, None, None, None, None, None, None) == 0


def test_quantize_fp8_argument_checks():
    lib = _lib.lib
    assert lib.moe_quantize_fp8(10, 12, FAKE, FAKE, FAKE, None) == 1        # cols % 8
    assert lib.moe_quantize_fp8(-1, 16, FAKE, FAKE, FAKE, None) == 1
    assert lib.moe_quantize_fp8(1 << 31, 16, FAKE, FAKE, FAKE, None) == 1
    assert lib.moe_quantize_fp8(10, 16, FAKE + 4, FAKE, FAKE, None) == 1    # w alignment
    assert lib.moe_quantize_fp8(10, 16, FAKE, FAKE + 4, FAKE, None) == 1    # q alignment
    assert lib.moe_quantize_fp8(10, 16, FAKE, FAKE, None, None) == 1
    assert lib.moe_quantize_fp8(0, 16, None, None, None, None) == 0


def test_backward_descriptor_rules():
    """The backward pass takes bf16 layers only; argument checks come before
    any launch."""
    assert moe.moe_backward_workspace_size(D(), 4096) > 0
    assert moe.moe_backward_workspace_size(D(act_dtype=0, weight_dtype=0, d_model=512, d_ffn=512), 64) == 0
    assert moe.moe_backward_workspace_size(D(weight_dtype=2), 64) == 0
    assert moe.moe_backward_workspace_size(D(), -1) == 0
    assert moe.moe_backward_workspace_size(D(), 16384) > 0       # the skewed prefill size
    assert moe.moe_backward_workspace_size(D(), 80000) == 0     # one expert's rows of da past 4 GiB
    lib = _lib.lib
    f32 = ctypes.byref(D(act_dtype=0, weight_dtype=0, d_model=512, d_ffn=512))
    args = [FAKE] * 11
    assert lib.moe_layer_backward(f32, 4, *args, FAKE, 1 << 30, None) == 2
    pb = ctypes.byref(D())
    assert lib.moe_layer_backward(pb, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                                  FAKE, 1 << 40, None) == 1          # no dw_gate
    assert lib.moe_layer_backward(pb, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  FAKE, 1 << 40, None) == 1          # dx aliases x
    assert lib.moe_layer_backward(pb, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 4096, FAKE, FAKE, FAKE,
                                  FAKE, FAKE + 16, 1 << 40, None) == 1  # workspace not 256-aligned
    assert lib.moe_layer_backward(pb, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 4096, FAKE, FAKE, FAKE,
                                  FAKE, FAKE, 10, None) == 3         # workspace too small
    assert lib.moe_layer_backward(pb, -1, *args, FAKE, 1 << 30, None) == 1


def test_bench_refuses_more_than_one_gpu():
    """The benchmark measures one GPU: --gpus above 1 exits with a message and a
    non-zero status before touching a device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "no multi-GPU path" in r.stderr

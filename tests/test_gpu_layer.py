"""Whole-layer parity (moe_layer_forward / moe_block_forward) with the CPU oracle:
small shapes element by element, the full-size workloads on every token's
routing and on a seeded sample of output rows."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
import sparse_moe_transformer_way_amd as moe
from moe_testutil import (TOL_BF16, TOL_F32, assert_routing_equal, margin_filtered,
                          per_token_rel_err, sample_rows)

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    yield
    torch.cuda.synchronize()


def run_layer(inp, residual=None):
    desc = moe.make_desc(inp.d, inp.F, dtype=DT[inp.dtype])
    x, wg, w1, w3, w2 = (t.cuda() for t in (inp.x, inp.wg, inp.w1, inp.w3, inp.w2))
    y, idx, gate, counts = moe.moe_layer_forward(desc, x, wg, w1, w3, w2,
                                                 residual=None if residual is None else residual.cuda())
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), idx.cpu().numpy(), gate.cpu().numpy(), counts.cpu().numpy()


def check_full(inp, tol):
    xn, wgn, w1n, w3n, w2n = inp.numpy_f32()
    ref = oracle.moe_layer(xn, wgn, w1n, w3n, w2n)
    y, idx, gate, counts = run_layer(inp)
    assert_routing_equal(idx, gate, ref, xn, wgn)
    np.testing.assert_array_equal(counts, ref["counts"])
    err = per_token_rel_err(y, ref["y"])
    assert err.max() <= tol, f"max per-token rel err {err.max():.3e}"
    return err.max()


@pytest.mark.parametrize("dtype,T,d,F", [
    ("f32", 64, 128, 256),      # the tiny fp32 workload's shape, other seed
    ("f32", 1, 128, 256),
    ("f32", 333, 64, 48),
    ("bf16", 32, 1024, 2048),   # decode kernels (T <= 64)
    ("bf16", 1, 512, 512),
    ("bf16", 64, 512, 1024),
    ("bf16", 65, 512, 1024),    # first T on the tiled kernels, few rows per expert
    ("bf16", 1000, 512, 1024),  # tiled kernels, ~250 rows per expert
    ("bf16", 2500, 1024, 512),
    ("bf16", 1150, 512, 1024),  # short expert tails past full 256-row tiles
    ("bf16", 2100, 1024, 512),
])
def test_layer_small(dtype, T, d, F):
    init = "fanin" if dtype == "f32" else "mixtral"
    inp = margin_filtered(mi.make_layer(T, d, F, dtype=dtype, init=init, seed=T + d, workload=300))
    check_full(inp, TOL_F32 if dtype == "f32" else TOL_BF16)


def test_tiny_workload():
    """The tiny fp32 workload exactly as specified (T=64, d=128, F=256, seed 0)."""
    check_full(margin_filtered(mi.make_workload(0)), TOL_F32)


@pytest.mark.parametrize("T", [40, 700])
def test_layer_single_expert_dominant(T):
    """Every token's top expert is 3 (bias trick on channel 0); the second
    expert varies.  Exercises one very long segment."""
    d, F = 512, 1024
    inp = mi.make_layer(T, d, F, skew=True, seed=T, workload=301)  # x[:, 0] == 1, kept by redraws
    inp.wg[0, :] = 0.0
    inp.wg[0, 3] = 20.0
    inp = margin_filtered(inp)
    xn, wgn = inp.x.float().numpy(), inp.wg.numpy()
    assert (oracle.gating(xn, wgn)[1][:, 0] == 3).all()
    check_full(inp, TOL_BF16)


def test_layer_forward_residual_and_T0():
    T, d, F = 100, 512, 512
    inp = margin_filtered(mi.make_layer(T, d, F, seed=1, workload=302))
    res = torch.randn(T, d).to(torch.bfloat16)
    xn, wgn, w1n, w3n, w2n = inp.numpy_f32()
    ref = oracle.moe_layer(xn, wgn, w1n, w3n, w2n)["y"] + res.float().numpy()
    y, *_ = run_layer(inp, residual=res)
    assert per_token_rel_err(y, ref).max() <= TOL_BF16
    desc = moe.make_desc(d, F)
    e = torch.empty(0, d, dtype=torch.bfloat16, device="cuda")
    out = moe.moe_layer_forward(desc, e, inp.wg.cuda(), inp.w1.cuda(), inp.w3.cuda(), inp.w2.cuda())
    assert out[0].shape == (0, d)


@pytest.mark.parametrize("T", [48, 600])
def test_block_forward(T):
    """h + MoE(RMSNorm(h)) against the oracle's block with bf16 storage."""
    d, F = 512, 1024
    inp = mi.make_layer(T, d, F, init="stack", seed=T, workload=303)
    # margin on the normalised input the layer will see
    for _ in range(50):
        xn = oracle.round_bf16(oracle.rmsnorm(inp.x.float().numpy()))
        bad = np.nonzero(oracle.routing_margin(xn, inp.wg.numpy()) < 1e-3)[0]
        if bad.size == 0:
            break
        inp = mi.redraw_rows(inp, bad)
    desc = moe.make_desc(d, F)
    h = inp.x.cuda()
    h_out, idx, counts = moe.moe_block_forward(desc, h, inp.wg.cuda(), inp.w1.cuda(), inp.w3.cuda(),
                                               inp.w2.cuda(), eps=1e-5)
    torch.cuda.synchronize()
    h_ref, out = oracle.moe_block(inp.x.float().numpy(), inp.wg.numpy(), inp.w1.float().numpy(),
                                  inp.w3.float().numpy(), inp.w2.float().numpy())
    np.testing.assert_array_equal(np.sort(idx.cpu().numpy(), 1), np.sort(out["idx"], 1))
    np.testing.assert_array_equal(counts.cpu().numpy(), out["counts"])
    # compare the MoE contribution (h_out - h) per token; bf16 storage of h_out
    # adds at most half an ulp of |h| per element
    got = h_out.float().cpu().numpy() - inp.x.float().numpy()
    exp = out["y"]
    slack = np.abs(inp.x.float().numpy()).max(axis=1) * 2 ** -8
    err = np.abs(got - exp).max(axis=1)
    assert (err <= TOL_BF16 * np.abs(exp).max(axis=1) + slack).all()


# ---------------------------------------------------------------------------
# Full-size workloads: routing of every token, outputs on sampled rows
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("wl,n_rows", [(1, 32), (2, 192), (3, 192)])
def test_workload_full_size(wl, n_rows):
    inp = margin_filtered(mi.make_workload(wl))
    T = inp.T
    desc = moe.make_desc(inp.d, inp.F)
    x, wg, w1, w3, w2 = (t.cuda() for t in (inp.x, inp.wg, inp.w1, inp.w3, inp.w2))
    y, idx, gate, counts = moe.moe_layer_forward(desc, x, wg, w1, w3, w2)
    torch.cuda.synchronize()
    y, idx, gate, counts = (t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()
                            for t in (y, idx, gate, counts))
    del x, w1, w3, w2
    xn = inp.x.float().numpy()
    wgn = inp.wg.numpy()
    G, ridx, _ = oracle.gating(xn, wgn)
    ref_r = dict(idx=ridx, gates=G[np.arange(T)[:, None], ridx],
                 counts=np.bincount(ridx.ravel(), minlength=8).astype(np.int32))
    assert_routing_equal(idx, gate, ref_r, xn, wgn)
    np.testing.assert_array_equal(counts, ref_r["counts"])
    rows = sample_rows(T, ridx, n_rows, seed=wl)
    w1n, w3n, w2n = inp.w1.float().numpy(), inp.w3.float().numpy(), inp.w2.float().numpy()
    ref = oracle.moe_layer(xn[rows], wgn, w1n, w3n, w2n)
    np.testing.assert_array_equal(ref["idx"], ridx[rows])
    err = per_token_rel_err(y[rows], ref["y"])
    print(f"workload {wl}: counts {counts.tolist()} max per-token rel err {err.max():.3e}")
    assert err.max() <= TOL_BF16
    if wl == 3:
        share = counts[:2].sum() / counts.sum()
        assert 0.5 < share < 0.8, share

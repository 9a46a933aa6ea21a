"""Parity of each C-ABI entry point with the CPU oracle at sizes the oracle
finishes in seconds (several tiles, ragged tails, degenerate cases)."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
import sparse_moe_transformer_way_amd as moe
from moe_testutil import (GATE_TOL, TOL_BF16, TOL_F32, assert_routing_equal, margin_filtered,
                          per_token_rel_err)

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    yield
    torch.cuda.synchronize()


def layer(T, d, F, dtype, seed=0, workload=200):
    init = "fanin" if dtype == "f32" else "mixtral"
    return margin_filtered(mi.make_layer(T, d, F, dtype=dtype, init=init, seed=seed, workload=workload))


# ---------------------------------------------------------------------------
# Router
# ---------------------------------------------------------------------------

# T <= 256 runs one token per block, larger T eight: 256 and 257 straddle the switch.
# With one token per block a lane takes two 8-channel chunks per pass: d = 4096
# fills both, 1536 only the first, 4608 a full pass and then a half-empty one.
@pytest.mark.parametrize("dtype,T,d", [("f32", 64, 128), ("bf16", 37, 512), ("bf16", 1, 4096),
                                       ("bf16", 32, 4096), ("bf16", 19, 1536), ("bf16", 32, 4608),
                                       ("f32", 5, 4608), ("bf16", 256, 512), ("bf16", 257, 512),
                                       ("bf16", 1000, 512), ("f32", 17, 8)])
def test_router(dtype, T, d):
    inp = layer(T, d, 512, dtype, seed=T)
    x, wg = inp.x.cuda(), inp.wg.cuda()
    desc = moe.make_desc(d, 512, dtype=DT[dtype])
    logits = torch.empty((T, 8), dtype=torch.float32, device="cuda")
    idx, gate = moe.moe_router_topk(desc, x, wg, logits_out=logits)
    torch.cuda.synchronize()
    xn, wgn = inp.x.float().numpy(), inp.wg.numpy()
    G, ridx, rlog = oracle.gating(xn, wgn)
    ref = dict(idx=ridx, gates=G[np.arange(T)[:, None], ridx], logits=rlog,
               counts=np.bincount(ridx.ravel(), minlength=8))
    np.testing.assert_allclose(logits.cpu().numpy(), ref["logits"], rtol=0,
                               atol=1e-5 * max(1.0, np.abs(ref["logits"]).max()))
    assert_routing_equal(idx.cpu().numpy(), gate.cpu().numpy(), ref, xn, wgn)


def test_router_all_ties():
    """W_g = 0: every logit ties, so experts (0, 1) with gates exactly (0.5, 0.5)."""
    T, d = 50, 512
    x = torch.randn(T, d).to(torch.bfloat16).cuda()
    wg = torch.zeros(d, 8, device="cuda")
    idx, gate = moe.moe_router_topk(moe.make_desc(d, 512), x, wg)
    assert (idx.cpu().numpy() == np.array([0, 1])).all()
    assert (gate.cpu().numpy() == 0.5).all()


def test_router_partial_ties():
    """Logits with exact ties at the 2nd/3rd place: lower index wins."""
    T, d = 8, 8
    x = torch.eye(8, dtype=torch.float32)[:T].cuda()
    wg_np = np.array([[3, 1, 1, 0, 0, 0, 0, 0],
                      [0, 0, 2, 2, 2, 0, 0, 0],
                      [1, 1, 1, 1, 1, 1, 1, 1],
                      [0, 0, 0, 0, 0, 0, 5, 5],
                      [-1, -1, -1, -1, -1, -1, -1, 0],
                      [0, 4, 0, 4, 0, 4, 0, 0],
                      [7, 0, 0, 0, 0, 0, 0, 7],
                      [0, 0, 0, 0, 0, 0, 0, 0]], np.float32)
    idx, gate = moe.moe_router_topk(moe.make_desc(8, 8, dtype=torch.float32), x,
                                    torch.from_numpy(wg_np).cuda())
    G, ridx, _ = oracle.gating(np.eye(8, dtype=np.float32), wg_np)
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    np.testing.assert_allclose(gate.cpu().numpy(), G[np.arange(8)[:, None], ridx], rtol=0, atol=1e-7)


# ---------------------------------------------------------------------------
# Permute
# ---------------------------------------------------------------------------

def _random_idx(T, seed, skew=False):
    rng = np.random.default_rng(seed)
    if T == 0:
        return np.zeros((0, 2), np.int32)
    if skew:
        return np.tile(np.array([[1, 0]], np.int32), (T, 1))
    return np.stack([rng.permutation(8)[:2] for _ in range(T)]).astype(np.int32).reshape(T, 2)


# 2000, 6000, 16000 and 17000 tokens: each thread of the one-block kernel holds
# up to 8 or up to 32 assignments in registers, or (above 32768) reads them twice.
@pytest.mark.parametrize("T,tile_m,skew", [(0, 16, False), (1, 16, False), (31, 16, False),
                                           (6000, 256, False), (16000, 256, True), (17000, 256, False),
                                           (32, 16, False), (32, 256, False), (32, 16, True),
                                           (33, 16, False), (37, 16, False),
                                           (300, 256, False), (2000, 256, False),
                                           (5000, 16, False), (16384, 256, False),
                                           (999, 256, True), (64, 16, True)])
def test_permute(T, tile_m, skew):
    desc = moe.make_desc(4096, 14336)
    idx = _random_idx(T, T + tile_m, skew)
    idx_d = torch.from_numpy(idx).cuda() if T > 0 else torch.empty((0, 2), dtype=torch.int32, device="cuda")
    counts, offsets, row_src, row_of = moe.moe_permute(desc, idx_d, tile_m)
    torch.cuda.synchronize()
    ref = oracle.group_by_expert(idx, 8, tile_m)
    np.testing.assert_array_equal(counts.cpu().numpy(), ref["counts"])
    np.testing.assert_array_equal(offsets.cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(row_src.cpu().numpy(), ref["row_src"])
    np.testing.assert_array_equal(row_of.cpu().numpy(), ref["row_of"])


@pytest.mark.parametrize("T", [100, 20])
def test_permute_ignores_out_of_range_experts(T):
    idx = _random_idx(T, 5)
    idx[3, 1] = -1
    idx[T // 2, 0] = 8
    idx[T - 1, 1] = 1 << 20
    counts, offsets, row_src, row_of = moe.moe_permute(moe.make_desc(4096, 14336),
                                                       torch.from_numpy(idx).cuda(), 16)
    flat = idx.ravel()
    valid = (flat >= 0) & (flat < 8)
    exp_counts = np.bincount(flat[valid], minlength=8)
    np.testing.assert_array_equal(counts.cpu().numpy(), exp_counts)
    ro = row_of.cpu().numpy().ravel()
    assert (ro[~valid] == -1).all()
    rs = row_src.cpu().numpy()
    np.testing.assert_array_equal(rs[ro[valid]], np.nonzero(valid)[0])
    assert (rs >= -1).all() and ((rs >= 0).sum() == valid.sum())


# ---------------------------------------------------------------------------
# Grouped expert projections
# ---------------------------------------------------------------------------

# tile 256 with T = 1150 and 2100 leaves most experts a remainder of at most
# 128 rows past their full tiles (which the layer may give to the
# weight-streaming kernels; the standalone entry points run them as tiles)
CASES = [("f32", 64, 128, 256, 16), ("f32", 5, 64, 40, 16), ("bf16", 40, 512, 1024, 16),
         ("bf16", 3, 1024, 512, 16), ("bf16", 1500, 512, 1024, 256), ("bf16", 150, 1024, 512, 256),
         ("bf16", 1150, 512, 1024, 256), ("bf16", 2100, 1024, 512, 256),
         ("bf16", 200, 512, 512, 16), ("bf16", 600, 512, 512, 16)]


@pytest.mark.parametrize("dtype,T,d,F,tile_m", CASES)
def test_grouped_swiglu(dtype, T, d, F, tile_m):
    inp = layer(T, d, F, dtype, seed=d + F + T)
    xn, wgn, w1n, w3n, w2n = inp.numpy_f32()
    ref = oracle.moe_layer(xn, wgn, w1n, w3n, w2n)
    grp = oracle.group_by_expert(ref["idx"], 8, tile_m)
    h_ref, yp_ref = oracle.expert_rows(xn, grp["row_src"], grp["offsets"], w1n, w3n, w2n)
    desc = moe.make_desc(d, F, dtype=DT[dtype])
    x, wg, w1, w3, w2 = (t.cuda() for t in (inp.x, inp.wg, inp.w1, inp.w3, inp.w2))
    row_src = torch.from_numpy(grp["row_src"]).cuda()
    counts = torch.from_numpy(grp["counts"]).cuda()
    offsets = torch.from_numpy(grp["offsets"]).cuda()
    h, yp = moe.moe_grouped_swiglu(desc, T, tile_m, x, row_src, counts, offsets, w1, w3, w2)
    torch.cuda.synchronize()
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    real = grp["row_src"] >= 0
    pad = ~real
    pad[grp["offsets"][8]:] = False  # rows past the last segment are never written
    hg = h.float().cpu().numpy()
    ypg = yp.cpu().numpy()
    assert per_token_rel_err(hg[real], h_ref[real]).max() <= tol
    assert per_token_rel_err(ypg[real], yp_ref[real]).max() <= tol
    assert (hg[pad] == 0).all()

    # down projection alone, fed the oracle's h in the layer dtype
    h_in = torch.from_numpy(h_ref).to(DT[dtype]).cuda()
    yp2 = moe.moe_expert_down(desc, T, tile_m, h_in, counts, offsets, w2)
    torch.cuda.synchronize()
    h_in_np = h_in.float().cpu().numpy()
    yp2_np = yp2.cpu().numpy()
    for e in range(8):
        rows = np.arange(grp["offsets"][e], grp["offsets"][e] + grp["counts"][e])
        if rows.size:
            exp = h_in_np[rows] @ w2n[e].T
            assert per_token_rel_err(yp2_np[rows], exp).max() <= (1e-5 if dtype == "f32" else 1e-4)


# Per-expert row counts on both sides of the tiled kernels' tile shapes: an
# expert's last 256-row tile runs as a 64-row tile up to 64 real rows, as a
# 128-row tile up to 128, and as a full tile above (64, 65, 128, 129 alone and
# past one full tile).  The assignments are placed directly, not routed.
NARROW_COUNTS = [64, 65, 128, 129, 320, 321, 384, 385]


@pytest.mark.parametrize("counts_target", [NARROW_COUNTS, NARROW_COUNTS[::-1], [1, 2, 63, 127, 255, 257, 0, 130]])
def test_grouped_swiglu_tile_shape_boundaries(counts_target):
    d, F = 512, 1024
    flat = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts_target)])
    rng = np.random.default_rng(len(flat))
    flat = flat[rng.permutation(flat.size)]
    if flat.size % 2:
        flat = np.concatenate([flat, np.array([-1], np.int32)])  # one assignment to no expert
    idx = flat.reshape(-1, 2)
    T = idx.shape[0]
    inp = mi.make_layer(T, d, F, seed=T, workload=204)
    xn, _, w1n, w3n, w2n = inp.numpy_f32()
    valid = idx >= 0
    grp = oracle.group_by_expert(np.where(valid, idx, 8), 9, 256)  # the -1 goes to a ninth, dropped expert
    P = moe.moe_max_permuted_rows(moe.make_desc(d, F), T, 256)
    offsets = grp["offsets"][:9]
    row_src = np.full(P, -1, np.int32)
    row_src[:offsets[8]] = grp["row_src"][:offsets[8]]
    counts = grp["counts"][:8]
    np.testing.assert_array_equal(counts, counts_target)
    h_ref, yp_ref = oracle.expert_rows(xn, row_src, offsets, w1n, w3n, w2n)
    desc = moe.make_desc(d, F)
    h, yp = moe.moe_grouped_swiglu(desc, T, 256, inp.x.cuda(), torch.from_numpy(row_src).cuda(),
                                   torch.from_numpy(counts).cuda(), torch.from_numpy(offsets).cuda(),
                                   inp.w1.cuda(), inp.w3.cuda(), inp.w2.cuda())
    torch.cuda.synchronize()
    real = row_src >= 0
    pad = ~real
    pad[offsets[8]:] = False
    hg = h.float().cpu().numpy()
    assert per_token_rel_err(hg[real], h_ref[real]).max() <= TOL_BF16
    assert per_token_rel_err(yp.cpu().numpy()[real], yp_ref[real]).max() <= TOL_BF16
    assert (hg[pad] == 0).all()


def test_grouped_swiglu_empty_and_full_experts():
    """All tokens on experts 2 and 5, six experts with no rows."""
    T, d, F = 300, 512, 1024
    inp = mi.make_layer(T, d, F, seed=9, workload=201)
    xn, _, w1n, w3n, w2n = inp.numpy_f32()
    idx = np.tile(np.array([[5, 2]], np.int32), (T, 1))
    for tile_m in (16, 256):
        grp = oracle.group_by_expert(idx, 8, tile_m)
        h_ref, yp_ref = oracle.expert_rows(xn, grp["row_src"], grp["offsets"], w1n, w3n, w2n)
        desc = moe.make_desc(d, F)
        h, yp = moe.moe_grouped_swiglu(desc, T, tile_m, inp.x.cuda(), torch.from_numpy(grp["row_src"]).cuda(),
                                       torch.from_numpy(grp["counts"]).cuda(),
                                       torch.from_numpy(grp["offsets"]).cuda(), inp.w1.cuda(),
                                       inp.w3.cuda(), inp.w2.cuda())
        real = grp["row_src"] >= 0
        assert per_token_rel_err(yp.cpu().numpy()[real], yp_ref[real]).max() <= TOL_BF16
        assert per_token_rel_err(h.float().cpu().numpy()[real], h_ref[real]).max() <= TOL_BF16


# ---------------------------------------------------------------------------
# Combine and RMSNorm
# ---------------------------------------------------------------------------

# d = 4608: one full pass of four column groups per thread, then a remainder;
# `drop`: some slots have no row (an assignment to no expert).
@pytest.mark.parametrize("dtype,T,d,residual,drop", [("f32", 64, 128, False, False), ("bf16", 333, 4096, False, False),
                                                     ("bf16", 333, 512, True, False), ("f32", 7, 64, True, False),
                                                     ("bf16", 97, 4608, True, True), ("f32", 40, 4608, False, True)])
def test_combine(dtype, T, d, residual, drop):
    rng = np.random.default_rng(T + d)
    idx = _random_idx(T, T)
    grp = oracle.group_by_expert(idx, 8, 16)
    row_of = grp["row_of"].copy()
    if drop:
        row_of[rng.random(row_of.shape) < 0.2] = -1
        row_of[0] = -1  # one token with no expert at all
    P = len(grp["row_src"])
    yp = rng.standard_normal((P, d)).astype(np.float32)
    g0 = rng.uniform(0.5, 1.0, T).astype(np.float32)
    gates = np.stack([g0, (1 - g0)], axis=1).astype(np.float32)
    res = torch.randn(T, d).to(DT[dtype]) if residual else None
    desc = moe.make_desc(d, 512, dtype=DT[dtype])
    y = moe.moe_combine(desc, torch.from_numpy(yp).cuda(), torch.from_numpy(row_of).cuda(),
                        torch.from_numpy(gates).cuda(), residual=None if res is None else res.cuda())
    ref = oracle.combine(yp, row_of, gates, None if res is None else res.float().numpy())
    got = y.float().cpu().numpy()
    if dtype == "bf16":
        ref = oracle.round_bf16(ref)
        np.testing.assert_allclose(got, ref, rtol=2 ** -7, atol=1e-6)
    else:
        np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("dtype,T,d", [("bf16", 100, 4096), ("f32", 9, 128), ("bf16", 1, 512)])
def test_rmsnorm(dtype, T, d):
    h = (torch.randn(T, d) * 3).to(DT[dtype])
    x = moe.moe_rmsnorm(h.cuda(), eps=1e-5)
    ref = oracle.rmsnorm(h.float().numpy(), 1e-5)
    got = x.float().cpu().numpy()
    if dtype == "bf16":
        np.testing.assert_allclose(got, oracle.round_bf16(ref), rtol=2 ** -7, atol=0)
    else:
        np.testing.assert_allclose(got, ref, rtol=2e-6, atol=0)


def test_gate_tolerance_constant():
    assert GATE_TOL == 1e-5

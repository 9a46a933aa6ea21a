"""Parity with the CPU oracle for expert counts n != 8 and top-K != 2.

Mixtral routes each token to 2 of 8 experts; the gating equation itself is
written for any K <= n (Mixtral of Experts, paper-graph-ui page, section 3.4,
TopK equation), and the library accepts 1 <= K <= min(n, 4), n <= 16.  Every
entry point is checked here at such shapes: the router (vector W_g path at
n = 8 and 16, scalar path otherwise), the permute, the grouped projections on
both tile sizes, the K-slot combine and the whole layer."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
import sparse_moe_transformer_way_amd as moe
from moe_testutil import (TOL_BF16, TOL_F32, assert_routing_equal, margin_filtered,
                          per_token_rel_err)

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    yield
    torch.cuda.synchronize()


def layer(T, d, F, n, K, dtype, seed, workload=400):
    init = "fanin" if dtype == "f32" else "mixtral"
    return margin_filtered(mi.make_layer(T, d, F, n=n, K=K, dtype=dtype, init=init, seed=seed,
                                         workload=workload))


def ref_routing(inp):
    xn, wgn = inp.x.float().numpy(), inp.wg.numpy()
    G, ridx, rlog = oracle.gating(xn, wgn, inp.K)
    return dict(idx=ridx, gates=G[np.arange(inp.T)[:, None], ridx], logits=rlog,
                counts=np.bincount(ridx.ravel(), minlength=inp.n)), xn, wgn


@pytest.mark.parametrize("n,K,dtype,T,d", [
    (4, 1, "bf16", 37, 512), (8, 1, "bf16", 300, 512), (8, 3, "bf16", 257, 512),
    (8, 4, "f32", 64, 128), (16, 2, "bf16", 1, 4096), (16, 4, "bf16", 1000, 512),
    (5, 3, "f32", 17, 64), (12, 4, "bf16", 300, 512), (1, 1, "f32", 10, 64),
    (16, 3, "bf16", 256, 512), (3, 3, "bf16", 40, 512)])
def test_router_general(n, K, dtype, T, d):
    inp = layer(T, d, 512, n, K, dtype, seed=T + 16 * n + K)
    desc = moe.make_desc(d, 512, n, K, dtype=DT[dtype])
    logits = torch.empty((T, n), dtype=torch.float32, device="cuda")
    idx, gate = moe.moe_router_topk(desc, inp.x.cuda(), inp.wg.cuda(), logits_out=logits)
    torch.cuda.synchronize()
    ref, xn, wgn = ref_routing(inp)
    np.testing.assert_allclose(logits.cpu().numpy(), ref["logits"], rtol=0,
                               atol=1e-5 * max(1.0, np.abs(ref["logits"]).max()))
    assert_routing_equal(idx.cpu().numpy(), gate.cpu().numpy(), ref, xn, wgn)
    if K == 1:
        assert (gate.cpu().numpy() == 1.0).all()


def test_router_general_ties():
    """W_g = 0 with n = 16, K = 4: all logits tie, so experts 0..3 in index
    order, each with gate exactly 1/4."""
    T, d = 20, 512
    x = torch.randn(T, d).to(torch.bfloat16).cuda()
    wg = torch.zeros(d, 16, device="cuda")
    idx, gate = moe.moe_router_topk(moe.make_desc(d, 512, 16, 4), x, wg)
    assert (idx.cpu().numpy() == np.arange(4)).all()
    assert (gate.cpu().numpy() == 0.25).all()


def _random_idx(T, n, K, seed):
    rng = np.random.default_rng(seed)
    if T == 0:
        return np.zeros((0, K), np.int32)
    return np.stack([rng.permutation(n)[:K] for _ in range(T)]).astype(np.int32).reshape(T, K)


@pytest.mark.parametrize("n,K,T,tile_m", [(16, 4, 1000, 256), (16, 4, 37, 16), (16, 4, 16, 16),
                                          (13, 3, 21, 16), (3, 1, 64, 16), (3, 1, 500, 16),
                                          (5, 3, 2000, 256), (12, 4, 16384, 256), (9, 2, 0, 16),
                                          (1, 1, 300, 256)])
def test_permute_general(n, K, T, tile_m):
    desc = moe.make_desc(4096, 14336, n, K)
    idx = _random_idx(T, n, K, T + n + K)
    idx_d = torch.from_numpy(idx).cuda() if T > 0 else torch.empty((0, K), dtype=torch.int32, device="cuda")
    counts, offsets, row_src, row_of = moe.moe_permute(desc, idx_d, tile_m)
    torch.cuda.synchronize()
    ref = oracle.group_by_expert(idx, n, tile_m)
    np.testing.assert_array_equal(counts.cpu().numpy(), ref["counts"])
    np.testing.assert_array_equal(offsets.cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(row_src.cpu().numpy(), ref["row_src"])
    np.testing.assert_array_equal(row_of.cpu().numpy(), ref["row_of"])


def test_permute_general_ignores_experts_past_n():
    """n = 5: indices 5..15 fit the kernel's 8 expert slots but are not experts."""
    T, n, K = 200, 5, 3
    idx = _random_idx(T, n, K, 11)
    idx[7, 2] = 5
    idx[8, 0] = 7
    idx[150, 1] = 15
    counts, offsets, row_src, row_of = moe.moe_permute(moe.make_desc(4096, 14336, n, K),
                                                       torch.from_numpy(idx).cuda(), 16)
    flat = idx.ravel()
    valid = flat < n
    np.testing.assert_array_equal(counts.cpu().numpy(), np.bincount(flat[valid], minlength=n))
    assert offsets.shape == (n + 1,)
    ro = row_of.cpu().numpy().ravel()
    assert (ro[~valid] == -1).all()
    rs = row_src.cpu().numpy()
    np.testing.assert_array_equal(rs[ro[valid]], np.nonzero(valid)[0])
    assert (rs >= -1).all() and ((rs >= 0).sum() == valid.sum())


@pytest.mark.parametrize("n,K,dtype,T,d,F,tile_m", [
    (4, 1, "bf16", 40, 512, 1024, 16), (16, 4, "bf16", 300, 512, 512, 256),
    (6, 3, "f32", 50, 128, 64, 16), (16, 2, "bf16", 60, 1024, 512, 16),
    (12, 3, "bf16", 700, 512, 1024, 256), (3, 1, "bf16", 900, 1024, 512, 256)])
def test_grouped_swiglu_general(n, K, dtype, T, d, F, tile_m):
    inp = layer(T, d, F, n, K, dtype, seed=T + d + F + n)
    xn, wgn, w1n, w3n, w2n = inp.numpy_f32()
    idx = oracle.gating(xn, wgn, K)[1]
    grp = oracle.group_by_expert(idx, n, tile_m)
    h_ref, yp_ref = oracle.expert_rows(xn, grp["row_src"], grp["offsets"], w1n, w3n, w2n, K=K)
    desc = moe.make_desc(d, F, n, K, dtype=DT[dtype])
    h, yp = moe.moe_grouped_swiglu(desc, T, tile_m, inp.x.cuda(), torch.from_numpy(grp["row_src"]).cuda(),
                                   torch.from_numpy(grp["counts"]).cuda(),
                                   torch.from_numpy(grp["offsets"]).cuda(), inp.w1.cuda(), inp.w3.cuda(),
                                   inp.w2.cuda())
    torch.cuda.synchronize()
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    real = grp["row_src"] >= 0
    pad = ~real
    pad[grp["offsets"][n]:] = False  # rows past the last segment are never written
    hg = h.float().cpu().numpy()
    assert per_token_rel_err(hg[real], h_ref[real]).max() <= tol
    assert per_token_rel_err(yp.cpu().numpy()[real], yp_ref[real]).max() <= tol
    assert (hg[pad] == 0).all()


@pytest.mark.parametrize("K,dtype,T,d,residual", [(1, "bf16", 100, 4096, False), (3, "f32", 64, 128, True),
                                                  (4, "bf16", 333, 512, True), (4, "f32", 7, 64, False)])
def test_combine_general(K, dtype, T, d, residual):
    n = 16
    rng = np.random.default_rng(T + d + K)
    idx = _random_idx(T, n, K, T)
    grp = oracle.group_by_expert(idx, n, 16)
    P = len(grp["row_src"])
    yp = rng.standard_normal((P, d)).astype(np.float32)
    g = rng.uniform(0.1, 1.0, (T, K))
    gates = (g / g.sum(axis=1, keepdims=True)).astype(np.float32)
    res = torch.randn(T, d).to(DT[dtype]) if residual else None
    desc = moe.make_desc(d, 512, n, K, dtype=DT[dtype])
    y = moe.moe_combine(desc, torch.from_numpy(yp).cuda(), torch.from_numpy(grp["row_of"]).cuda(),
                        torch.from_numpy(gates).cuda(), residual=None if res is None else res.cuda())
    ref = oracle.combine(yp, grp["row_of"], gates, None if res is None else res.float().numpy())
    got = y.float().cpu().numpy()
    if dtype == "bf16":
        np.testing.assert_allclose(got, oracle.round_bf16(ref), rtol=2 ** -7, atol=1e-6)
    else:
        np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("n,K,dtype,T,d,F", [
    (4, 1, "bf16", 32, 512, 1024),     # decode kernels
    (16, 4, "bf16", 48, 512, 512),
    (16, 4, "bf16", 600, 512, 1024),   # tiled kernels
    (6, 3, "f32", 64, 128, 256),
    (8, 3, "bf16", 1000, 512, 1024),
    (12, 2, "bf16", 300, 1024, 512),
    (1, 1, "bf16", 100, 512, 512),
    (8, 1, "bf16", 2000, 512, 512),
])
def test_layer_general(n, K, dtype, T, d, F):
    inp = layer(T, d, F, n, K, dtype, seed=T + n + K, workload=401)
    xn, wgn, w1n, w3n, w2n = inp.numpy_f32()
    ref = oracle.moe_layer(xn, wgn, w1n, w3n, w2n, K=K)
    desc = moe.make_desc(d, F, n, K, dtype=DT[dtype])
    y, idx, gate, counts = moe.moe_layer_forward(desc, inp.x.cuda(), inp.wg.cuda(), inp.w1.cuda(),
                                                 inp.w3.cuda(), inp.w2.cuda())
    torch.cuda.synchronize()
    assert_routing_equal(idx.cpu().numpy(), gate.cpu().numpy(), ref, xn, wgn)
    np.testing.assert_array_equal(counts.cpu().numpy(), ref["counts"])
    err = per_token_rel_err(y.float().cpu().numpy(), ref["y"])
    assert err.max() <= (TOL_F32 if dtype == "f32" else TOL_BF16), f"max per-token rel err {err.max():.3e}"

"""The 32-layer MoE FFN stack (attention omitted): T=8192, d=4096, F=14336,
independent seeded weights per layer (~90 GB resident), each block
h <- h + MoE(RMSNorm(h)).

* Per layer, on generator inputs: moe_block_forward against the oracle's block
  (routing of all 8192 tokens bit-exact, outputs on sampled rows).
* Free-running: all 32 blocks chained on the GPU; sampled tokens are followed
  through the oracle's 32 blocks (tokens are independent when attention is
  omitted) and compared layer by layer.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
import sparse_moe_transformer_way_amd as moe
from moe_testutil import MARGIN, TOL_BF16, per_token_rel_err

pytestmark = pytest.mark.gpu

WL = mi.WORKLOADS[4]
T, D, F, L = WL["T"], WL["d"], WL["F"], WL["layers"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def host_f32(t):
    return t.float().cpu().numpy()


def normed_bf16(h):
    return oracle.round_bf16(oracle.rmsnorm(h))


@pytest.mark.parametrize("layer", [0, 7, 15, 23, 31])
def test_stack_layer_parity(layer):
    wg, w1, w3, w2 = mi.stack_layer_weights(layer, D, F, device="cuda")
    wg_h = wg.cpu()
    # h0 with every token's margin >= 1e-3 under this layer's router
    inp = mi.LayerInputs(x=mi.stack_input(T, D), wg=wg_h, w1=None, w3=None, w2=None, T=T, d=D, F=F,
                         n=8, K=2, dtype="bf16", key=(0, 4, layer), init="stack")
    for _ in range(50):
        bad = np.nonzero(oracle.routing_margin(normed_bf16(host_f32(inp.x)), wg_h.numpy()) < MARGIN)[0]
        if bad.size == 0:
            break
        inp = mi.redraw_rows(inp, bad)
    h = inp.x.cuda()
    desc = moe.make_desc(D, F)
    h_out, idx, counts = moe.moe_block_forward(desc, h, wg, w1, w3, w2, eps=1e-5)
    torch.cuda.synchronize()
    hn = host_f32(inp.x)
    xn = normed_bf16(hn)
    G, ridx, _ = oracle.gating(xn, wg_h.numpy())
    np.testing.assert_array_equal(np.sort(idx.cpu().numpy(), 1), np.sort(ridx, 1))
    np.testing.assert_array_equal(counts.cpu().numpy(), np.bincount(ridx.ravel(), minlength=8))
    rng = np.random.default_rng(layer)
    rows = np.sort(rng.choice(T, size=48, replace=False))
    w1n, w3n, w2n = host_f32(w1), host_f32(w3), host_f32(w2)
    _, out = oracle.moe_block(hn[rows], wg_h.numpy(), w1n, w3n, w2n)
    got = host_f32(h_out)[rows] - hn[rows]
    err = per_token_rel_err(got, out["y"])
    # bf16 storage of h_out adds at most half an ulp of |h| per element
    slack = np.abs(hn[rows]).max(axis=1) * 2.0 ** -8 / np.abs(out["y"]).max(axis=1)
    assert (err <= TOL_BF16 + slack).all(), err.max()


def test_stack_free_running():
    desc = moe.make_desc(D, F)
    layers = [mi.stack_layer_weights(l, D, F, device="cuda") for l in range(L)]
    h0 = mi.stack_input(T, D)
    h = h0.cuda()
    ws = torch.empty(moe.moe_block_workspace_size(desc, T), dtype=torch.uint8, device="cuda")
    idx_all = torch.empty((L, T, 2), dtype=torch.int32, device="cuda")
    cnt_all = torch.empty((L, 8), dtype=torch.int32, device="cuda")
    for l, (wg, w1, w3, w2) in enumerate(layers):
        moe.moe_block_forward(desc, h, wg, w1, w3, w2, eps=1e-5, h_out=h, topk_idx_out=idx_all[l],
                              counts_out=cnt_all[l], workspace=ws)
    torch.cuda.synchronize()
    h_gpu = host_f32(h)
    idx_gpu = idx_all.cpu().numpy()
    assert np.isfinite(h_gpu).all()
    assert (cnt_all.cpu().numpy().sum(axis=1) == 2 * T).all()

    # Follow a sample of tokens through the oracle's 32 blocks.  The GPU's and
    # the oracle's residual streams are rounded to bf16 independently after
    # every block, so they drift apart; a token's routing may therefore first
    # diverge only at a layer where the oracle's 2nd-vs-3rd logit gap is within
    # that drift.  Tokens that never diverge must match at the end.
    DRIFT_BOUND = 0.25
    rng = np.random.default_rng(7)
    cand = np.sort(rng.choice(T, size=256, replace=False))
    hs = host_f32(h0)[cand]
    alive = np.ones(cand.size, bool)
    first_gap = []
    for l, (wg, w1, w3, w2) in enumerate(layers):
        wgn = wg.cpu().numpy()
        gap = oracle.routing_margin(normed_bf16(hs), wgn)
        hs, out = oracle.moe_block(hs, wgn, host_f32(w1), host_f32(w3), host_f32(w2))
        same = (np.sort(idx_gpu[l][cand], 1) == np.sort(out["idx"], 1)).all(axis=1)
        diverged = alive & ~same
        first_gap += gap[diverged].tolist()
        alive &= same
    print(f"stack: {alive.sum()} of {cand.size} sampled tokens keep the oracle's routing through "
          f"{L} layers; first-divergence gaps {np.round(first_gap, 4).tolist()}")
    assert all(g < DRIFT_BOUND for g in first_gap)
    # most tokens meet a close call somewhere in 32 layers; enough must remain
    assert alive.sum() >= cand.size // 8
    err = per_token_rel_err(h_gpu[cand[alive]], hs[alive])
    print(f"stack: max per-token rel err of h_32 over those tokens {err.max():.3e}")
    # Not the single-layer tolerance: 32 chained blocks whose residual streams
    # are rounded to bf16 independently on each side (the GPU also rounds the
    # SwiGLU intermediate once per layer) compound to ~6e-2 (measured); each
    # layer on its own meets 2e-2 in test_stack_layer_parity.
    assert err.max() <= 1e-1

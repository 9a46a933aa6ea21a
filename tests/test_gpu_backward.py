"""Backward pass (moe_layer_backward) against the float64 CPU oracle: every
gradient element by element at small shapes (several tiles, ragged expert
segments, other K and n, empty experts, T = 0), and the prefill-shaped layer
(T=4096, d=4096, F=14336) on sampled tokens and weight rows."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
import sparse_moe_transformer_way_amd as moe
from moe_testutil import TOL_BF16, margin_filtered

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    yield
    torch.cuda.synchronize()


def row_rel_err(got, ref):
    """Per-row max-norm relative error; rows whose reference is all zero must be zero."""
    got = np.asarray(got, np.float64).reshape(-1, np.shape(ref)[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, np.shape(ref)[-1])
    den = np.abs(ref).max(axis=1)
    num = np.abs(got - ref).max(axis=1)
    assert (num[den == 0] == 0).all()
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), 0.0)


def _dy(T, d, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(T, d, generator=g).to(torch.bfloat16)


def run_backward(inp, dy):
    desc = moe.make_desc(inp.d, inp.F, inp.n, inp.K)
    outs = moe.moe_layer_backward(desc, inp.x.cuda(), inp.wg.cuda(), inp.w1.cuda(), inp.w3.cuda(), inp.w2.cuda(),
                                  dy.cuda())
    torch.cuda.synchronize()
    return [o.float().cpu().numpy() for o in outs]


@pytest.mark.parametrize("T,d,F,n,K", [
    (64, 512, 512, 8, 2), (300, 512, 1024, 8, 2), (1000, 1024, 512, 8, 2), (1, 512, 512, 8, 2),
    (200, 512, 512, 4, 1), (150, 512, 512, 16, 4), (500, 512, 512, 8, 3),
])
def test_backward_small(T, d, F, n, K):
    inp = margin_filtered(mi.make_layer(T, d, F, n=n, K=K, seed=T + d, workload=700))
    dy = _dy(T, d, T + F)
    dx, dwg, dw1, dw3, dw2 = run_backward(inp, dy)
    xn, wgn, w1n, w3n, w2n = inp.numpy_f32()
    ref = oracle.moe_layer_backward(xn, wgn, w1n, w3n, w2n, dy.float().numpy(), K=K)
    assert row_rel_err(dx, ref["dx"]).max() <= TOL_BF16
    assert row_rel_err(dwg.T, ref["dwg"].T).max() <= TOL_BF16
    for name, got in (("dw1", dw1), ("dw3", dw3), ("dw2", dw2)):
        err = row_rel_err(got, ref[name])
        assert err.max() <= TOL_BF16, f"{name}: max row rel err {err.max():.3e}"


def test_backward_empty_experts_and_T0():
    """All tokens on experts 3 and 6: the other experts' weight gradients are
    exactly zero; T = 0 writes zero weight gradients."""
    T, d, F = 300, 512, 512
    inp = mi.make_layer(T, d, F, skew=True, seed=3, workload=701)
    inp.wg[0, :] = 0.0
    inp.wg[0, 3] = 20.0
    inp.wg[0, 6] = 19.0
    inp = margin_filtered(inp)
    idx = oracle.gating(inp.x.float().numpy(), inp.wg.numpy())[1]
    assert set(np.unique(idx)) == {3, 6}
    dy = _dy(T, d, 5)
    dx, dwg, dw1, dw3, dw2 = run_backward(inp, dy)
    xn, wgn, w1n, w3n, w2n = inp.numpy_f32()
    ref = oracle.moe_layer_backward(xn, wgn, w1n, w3n, w2n, dy.float().numpy())
    for e in (0, 1, 2, 4, 5, 7):
        assert (dw1[e] == 0).all() and (dw3[e] == 0).all() and (dw2[e] == 0).all()
    for name, got in (("dx", dx), ("dw1", dw1), ("dw3", dw3), ("dw2", dw2)):
        assert row_rel_err(got, ref[name]).max() <= TOL_BF16, name
    desc = moe.make_desc(d, F)
    e = torch.empty(0, d, dtype=torch.bfloat16, device="cuda")
    outs = [torch.full(s, 7.0, device="cuda") for s in ((d, 8), (8, F, d), (8, F, d), (8, d, F))]
    moe.moe_layer_backward(desc, e, inp.wg.cuda(), inp.w1.cuda(), inp.w3.cuda(), inp.w2.cuda(), e,
                           dw_gate=outs[0], dw1=outs[1], dw3=outs[2], dw2=outs[3])
    torch.cuda.synchronize()
    assert all((o == 0).all().item() for o in outs)


class _Experts:
    """Index e -> expert e's weights as float32 numpy (the oracle helpers read
    one expert at a time; a whole bf16 stack upcast at once would not fit)."""

    def __init__(self, t):
        self.t = t

    def __getitem__(self, e):
        return self.t[int(e)].float().numpy()


def test_backward_prefill_workload_sampled():
    """The prefill-shaped layer (T=4096, d=4096, F=14336, 8 experts, top-2) in
    the configuration the bench times: dx of 48 sampled tokens (router term
    included) and rows of dw1, dw3, dw2 of two experts, against the oracle's
    per-token and per-expert-row evaluations.  dW_g is checked element by
    element at the small shapes above."""
    inp = margin_filtered(mi.make_workload(2))
    T, d, F = inp.T, inp.d, inp.F
    dy = _dy(T, d, 11)
    dx, dwg, dw1, dw3, dw2 = run_backward(inp, dy)
    assert np.isfinite(dwg).all()
    x, wg, dyn = inp.x.float().numpy(), inp.wg.numpy(), dy.float().numpy()
    w1, w3, w2 = _Experts(inp.w1), _Experts(inp.w3), _Experts(inp.w2)
    rng = np.random.default_rng(0)
    tok = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 46, replace=False)]))
    r = oracle.backward_token_rows(x, wg, w1, w3, w2, dyn, tok)
    err = row_rel_err(dx[tok], r["dx"])
    assert err.max() <= TOL_BF16, f"dx: {err.max():.3e}"
    for e in (0, 5):
        f_rows = np.sort(rng.choice(F, 6, replace=False))
        j_rows = np.sort(rng.choice(d, 6, replace=False))
        rows = oracle.backward_expert_rows(x, wg, w1, w3, w2, dyn, e, f_rows, j_rows)
        assert rows["count"] > 0
        for name, got in (("dw1", dw1[e][f_rows]), ("dw3", dw3[e][f_rows]), ("dw2", dw2[e][j_rows])):
            err = row_rel_err(got, rows[name])
            assert err.max() <= TOL_BF16, f"expert {e} {name}: {err.max():.3e}"


def test_backward_skewed_workload_sampled():
    """The skewed prefill layer (T=16384, two experts take about 65% of the
    assignments; the per-row buffers pass 2 GiB): dx of 32 sampled tokens and
    rows of dw1, dw3, dw2 of two lightly loaded experts."""
    inp = margin_filtered(mi.make_workload(3))
    T, d, F = inp.T, inp.d, inp.F
    dy = _dy(T, d, 13)
    dx, dwg, dw1, dw3, dw2 = run_backward(inp, dy)
    assert np.isfinite(dwg).all() and np.isfinite(dw1[0]).all()
    x, wg, dyn = inp.x.float().numpy(), inp.wg.numpy(), dy.float().numpy()
    w1, w3, w2 = _Experts(inp.w1), _Experts(inp.w3), _Experts(inp.w2)
    rng = np.random.default_rng(1)
    tok = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 30, replace=False)]))
    r = oracle.backward_token_rows(x, wg, w1, w3, w2, dyn, tok)
    err = row_rel_err(dx[tok], r["dx"])
    assert err.max() <= TOL_BF16, f"dx: {err.max():.3e}"
    for e in (3, 6):
        f_rows = np.sort(rng.choice(F, 4, replace=False))
        j_rows = np.sort(rng.choice(d, 4, replace=False))
        rows = oracle.backward_expert_rows(x, wg, w1, w3, w2, dyn, e, f_rows, j_rows)
        assert 0 < rows["count"] < 4000
        for name, got in (("dw1", dw1[e][f_rows]), ("dw3", dw3[e][f_rows]), ("dw2", dw2[e][j_rows])):
            err = row_rel_err(got, rows[name])
            assert err.max() <= TOL_BF16, f"expert {e} {name}: {err.max():.3e}"

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
    desc = moe.make_desc(inp.d, inp.F, inp.n, inp.K, dtype=DT[inp.dtype])
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
    ("bf16", 1150, 512, 1024),  # short expert tails (the tiled kernel keeps them at d = 512)
    ("bf16", 2100, 1024, 512),
])
def test_layer_small(dtype, T, d, F):
    init = "fanin" if dtype == "f32" else "mixtral"
    inp = margin_filtered(mi.make_layer(T, d, F, dtype=dtype, init=init, seed=T + d, workload=300))
    check_full(inp, TOL_F32 if dtype == "f32" else TOL_BF16)


TAIL_ROWS = 128  # the longest tail past an expert's full 256-row tiles that the streaming pass takes


def down_plan(counts, d, F, T, K=2, n=8):
    """The down projection's plan that the library takes on the device: the
    largest K split allowed (2 when the worst-case tiles fill fewer than four
    rounds of 256 workgroups), then for each split whether the experts' short
    tails go to the streaming pass (when that lowers the number of rounds):
    tails of up to TAIL_ROWS rows past their full 256-row tiles while
    n_tail * d / 256 <= 80, else of up to TAIL_ROWS / 2; and the split whose
    rounds x K per tile is smallest (no split on a tie).  Returns (K parts,
    longest tail streamed, 0 for none)."""
    P = T * K + n * 255
    n_tt, n_wt = -(-P // 256), d // 256
    ks_max = 2 if (n_tt * n_wt < 4 * 256 and (F // 2) % 256 == 0) else 1
    without = sum(-(-c // 256) for c in counts)
    n_long = sum(1 for c in counts if 0 < c % 256 <= TAIL_ROWS)
    tmax = TAIL_ROWS if n_long * n_wt <= 80 else TAIL_ROWS // 2
    with_tail = sum(c // 256 if 0 < c % 256 <= tmax else -(-c // 256) for c in counts)
    best = None
    for ks in range(1, ks_max + 1):
        r_with = -(-with_tail * n_wt * ks // 256)
        r_without = -(-without * n_wt * ks // 256)
        tail = tmax if r_with < r_without else 0
        r = min(r_with, r_without)
        if best is None or r * best[0] < best[2] * ks:
            best = (ks, tail, r)
    return best[0], best[1]


# d = 4096 with a small F at T = 1150: every expert gets 255-316 rows, so the
# down projection cuts K in two and hands the tails (under 64 rows) to the
# streaming pass.  With F = 1536 the tail pass runs in one K part (its rows have
# no second partial); with F = 2048 it cuts K in two into the tail buffer.
@pytest.mark.parametrize("F,seed", [(1536, 1), (2048, 0)])
def test_layer_down_tail_pass(F, seed):
    T, d = 1150, 4096
    inp = margin_filtered(mi.make_layer(T, d, F, seed=seed, workload=305))
    counts = np.bincount(oracle.gating(inp.x.float().numpy(), inp.wg.numpy())[1].ravel(), minlength=8)
    ks, tail = down_plan(counts.tolist(), d, F, T)
    assert ks == 2 and tail, (counts, ks, tail)
    err = check_full(inp, TOL_BF16)
    print(f"down tail pass, F={F}: counts {counts.tolist()}, max per-token rel err {err:.3e}")


def routed_layer(counts, d, F, seed):
    """A seeded layer whose routing is set by construction: token t's two
    experts are the t-th and (t+T)-th entries of the expert ids listed counts[e]
    times each (distinct, as every count is under T), marked by x[t, a] = 1.0
    and x[t, b] = 0.9 on top of small noise, with W_g[e, e] = 10 (other entries
    small).  The two chosen logits lead the others by about 8, so the routing
    and its order are exact; the gates are softmax(10, 9).  n = len(counts)."""
    n = len(counts)
    T = sum(counts) // 2
    inp = mi.make_layer(T, d, F, n=n, seed=seed, workload=306 if n == 8 else 307)
    ids = np.repeat(np.arange(n), counts)
    a, b = ids[:T], ids[T:]
    x = inp.x.float() * 0.1
    x[np.arange(T), a] = 1.0
    x[np.arange(T), b] = 0.9
    wg = inp.wg.clone()
    wg[np.arange(n), np.arange(n)] = 10.0
    inp.x, inp.wg = x.to(inp.x.dtype), wg
    return inp


# Tails of 65-128 rows: experts 0-2 get 100, 90 and 70 rows past two full
# tiles, the others exactly two tiles.  Streaming the three tails saves a round
# (16 x 16 full tiles against 19 x 16), the pass takes them in 5-7 token blocks
# of 16 rows in one pass over the weights, and with F = 2048 in two K parts.
@pytest.mark.parametrize("F", [1536, 2048])
def test_layer_down_long_tails(F):
    counts = [612, 602, 582] + [512] * 5
    d = 4096
    inp = routed_layer(counts, d, F, seed=F)
    T = inp.x.shape[0]
    got = np.bincount(oracle.gating(inp.x.float().numpy(), inp.wg.numpy())[1].ravel(), minlength=8)
    np.testing.assert_array_equal(got, counts)
    assert down_plan(counts, d, F, T) == (1, TAIL_ROWS)
    err = check_full(inp, TOL_BF16)
    print(f"down long tails, F={F}: counts {counts}, max per-token rel err {err:.3e}")


# Sixteen experts with the tiled kernels' full tiles, the tail pass and the K
# split: every expert lane of the device-side tile deal, the down projection's
# plan and the combine's expert search is a real segment.  Three experts get
# 70-100-row tails past two full tiles, which the pass takes (35 x 16 tiles
# against 32 x 16: three rounds against two); one expert's 144-row tail is too
# long for the pass, and 17 x 16 tiles in halves of K fill three rounds of half
# the length against two full ones, so the plan cuts K in two.
@pytest.mark.parametrize("counts,F,plan", [
    ([612, 602, 582] + [512] * 13, 1536, (1, TAIL_ROWS)),
    ([400] + [256] * 15, 2048, (2, 0)),
])
def test_layer_16_experts_tails_and_split(counts, F, plan):
    d = 4096
    inp = routed_layer(counts, d, F, seed=F + len(counts))
    T = inp.x.shape[0]
    got = np.bincount(oracle.gating(inp.x.float().numpy(), inp.wg.numpy())[1].ravel(), minlength=16)
    np.testing.assert_array_equal(got, counts)
    assert down_plan(counts, d, F, T, n=16) == plan
    err = check_full(inp, TOL_BF16)
    print(f"16 experts, plan {plan}: max per-token rel err {err:.3e}")


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
    # plus tokens whose assignment lands in an expert's short tail (at most
    # TAIL_ROWS rows past its full 256-row tiles): the down projection may
    # compute those rows in its streaming pass, in two K halves that the
    # combine adds
    grp = oracle.group_by_expert(ridx, 8, 256)
    tails = []
    for e in range(8):
        c, off = int(grp["counts"][e]), int(grp["offsets"][e])
        if 0 < c % 256 <= TAIL_ROWS:
            tails += (grp["row_src"][off + c - c % 256: off + c] // 2).tolist()
    tail_tokens = np.unique(np.array(tails, np.int64))
    tail_tokens = np.random.default_rng(wl).permutation(tail_tokens)[:48]
    rows = np.union1d(rows, tail_tokens)
    w1n, w3n, w2n = inp.w1.float().numpy(), inp.w3.float().numpy(), inp.w2.float().numpy()
    ref = oracle.moe_layer(xn[rows], wgn, w1n, w3n, w2n)
    np.testing.assert_array_equal(ref["idx"], ridx[rows])
    err = per_token_rel_err(y[rows], ref["y"])
    print(f"workload {wl}: counts {counts.tolist()}, {rows.size} rows ({tail_tokens.size} with a tail row), "
          f"max per-token rel err {err.max():.3e}")
    assert err.max() <= TOL_BF16
    if wl == 3:
        share = counts[:2].sum() / counts.sum()
        assert 0.5 < share < 0.8, share


@pytest.mark.parametrize("T,d,F", [(32, 1024, 2048), (1150, 4096, 2048)])
def test_layer_forward_timed_matches_layer(T, d, F):
    """moe_layer_forward_timed runs the layer's own launch sequence: the same
    outputs bit for bit, and its six events in stream order."""
    inp = mi.make_layer(T, d, F, seed=5, workload=306)
    desc = moe.make_desc(d, F)
    x, wg, w1, w3, w2 = (t.cuda() for t in (inp.x, inp.wg, inp.w1, inp.w3, inp.w2))
    ref = moe.moe_layer_forward(desc, x, wg, w1, w3, w2)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for e in ev:
        e.record(stream)
    got = moe.moe_layer_forward_timed(desc, x, wg, w1, w3, w2, ev)
    torch.cuda.synchronize()
    for r, g in zip(ref, got):
        assert torch.equal(r.cpu(), g.cpu())
    stages = [ev[i].elapsed_time(ev[i + 1]) for i in range(5)]
    assert all(s >= 0 for s in stages), stages
    assert stages[2] > 0 and stages[3] > 0  # the two expert projections

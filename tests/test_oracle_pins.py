"""Pins of the CPU oracle against facts the pages and the mathematics fix.

None of these re-derive the oracle's own formula: each one checks a value the
pages print, a closed form worked out by hand, a brute-force enumeration, an
invariant, or a special case that reduces to something simpler.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sig(z):
    return 1.0 / (1.0 + math.exp(-z))


# ---------------------------------------------------------------------------
# Hand-worked example: n=8, K=2, d=2, F=3, two tokens.
# Logit rows are the rows of W_g because x is one-hot.
#   token 0 = e_0: l = [0, 3, 1, 2, -1, 0.5, 2.5, -2] -> experts (1, 6),
#            gates (sigma(0.5), 1 - sigma(0.5))
#   token 1 = e_1: l = [2, -1, 0, 0, 0, 1, 1, -3] -> experts (0, 5) (5 beats 6 on
#            the tie by lower index), gates (sigma(1), 1 - sigma(1))
# Expert weights of experts 0, 1, 5, 6 are small integers picked so that every
# pre-activation is 0, +-1, +-2 or 5; the other experts get large weights that
# would show up in y if a masked expert leaked in.
# ---------------------------------------------------------------------------

def hand_example():
    n, d, F = 8, 2, 3
    x = np.array([[1, 0], [0, 1]], np.float32)
    wg = np.array([[0, 3, 1, 2, -1, 0.5, 2.5, -2],
                   [2, -1, 0, 0, 0, 1, 1, -3]], np.float32)
    w1 = np.full((n, F, d), 7.0, np.float32)
    w3 = np.full((n, F, d), -9.0, np.float32)
    w2 = np.full((n, d, F), 11.0, np.float32)
    # expert 1 (token 0): w1.x = [1, 0, -1], w3.x = [2, 5, 1]
    w1[1] = [[1, 0], [0, 1], [-1, 0]]
    w3[1] = [[2, 0], [5, 0], [1, 1]]
    w2[1] = [[1, 1, 1], [0, 0, 2]]
    # expert 6 (token 0): w1.x = [0, 2, 0], w3.x = [0, 1, 0]
    w1[6] = [[0, 0], [2, 0], [0, 0]]
    w3[6] = [[0, 0], [1, 0], [0, 0]]
    w2[6] = [[0, 1, 0], [0, -1, 0]]
    # expert 0 (token 1): w1.x = [1, -2, 0], w3.x = [3, 1, 0]
    w1[0] = [[0, 1], [0, -2], [0, 0]]
    w3[0] = [[0, 3], [0, 1], [7, 0]]
    w2[0] = [[1, 0, 0], [1, 1, 5]]
    # expert 5 (token 1): w1.x = [0, 0, 1], w3.x = [0, 0, -4]
    w1[5] = [[0, 0], [0, 0], [0, 1]]
    w3[5] = [[0, 0], [0, 0], [0, -4]]
    w2[5] = [[0, 0, 1], [0, 0, 0]]
    return x, wg, w1, w3, w2


def hand_expected():
    silu = lambda z: z * sig(z)  # noqa: E731
    # token 0: h1 = silu([1,0,-1]) * [2,5,1] = [2 silu(1), 0, silu(-1)]
    #          E1 = [h1_0 + h1_1 + h1_2, 2 h1_2]
    #          h6 = [0, silu(2) * 1, 0]; E6 = [silu(2), -silu(2)]
    E1 = [2 * silu(1) + silu(-1), 2 * silu(-1)]
    E6 = [silu(2), -silu(2)]
    g = sig(0.5)
    y0 = [g * E1[j] + (1 - g) * E6[j] for j in range(2)]
    # token 1: h0 = silu([1,-2,0]) * [3,1,0] = [3 silu(1), silu(-2), 0]
    #          E0 = [h0_0, h0_0 + h0_1 + 5 h0_2]
    #          h5 = [0, 0, silu(1) * -4]; E5 = [-4 silu(1), 0]
    E0 = [3 * silu(1), 3 * silu(1) + silu(-2)]
    E5 = [-4 * silu(1), 0.0]
    g = sig(1.0)
    y1 = [g * E0[j] + (1 - g) * E5[j] for j in range(2)]
    return dict(idx=[[1, 6], [0, 5]], gates=[[sig(0.5), 1 - sig(0.5)], [sig(1.0), 1 - sig(1.0)]],
                y=[y0, y1], counts=[1, 1, 0, 0, 0, 1, 1, 0])


def test_hand_worked_example():
    out = oracle.moe_layer(*hand_example(), K=2)
    exp = hand_expected()
    np.testing.assert_array_equal(out["idx"], exp["idx"])
    np.testing.assert_array_equal(out["counts"], exp["counts"])
    np.testing.assert_allclose(out["gates"], exp["gates"], rtol=1e-6, atol=0)
    np.testing.assert_allclose(out["y"], exp["y"], rtol=2e-6, atol=1e-6)


def test_hand_example_sparse_path_matches():
    """The reference layouts (group -> expert rows -> combine) give the same y."""
    x, wg, w1, w3, w2 = hand_example()
    for tile_m in (1, 4):
        out = oracle.moe_layer(x, wg, w1, w3, w2, K=2)
        grp = oracle.group_by_expert(out["idx"], 8, tile_m)
        _, y_perm = oracle.expert_rows(x, grp["row_src"], grp["offsets"], w1, w3, w2, K=2)
        y = oracle.combine(y_perm, grp["row_of"], out["gates"])
        np.testing.assert_allclose(y, hand_expected()["y"], rtol=2e-6, atol=1e-6)


def test_silu_closed_forms():
    z = np.array([0.0, 1.0, -1.0, 2.0, 30.0, -30.0, -200.0], np.float32)
    got = oracle.silu(z)
    exp = [0.0, sig(1), -sig(-1) * 1, 2 * sig(2), 30.0, -30.0 * sig(-30.0), 0.0]
    np.testing.assert_allclose(got, exp, rtol=1e-6, atol=1e-30)
    assert got[0] == 0.0
    assert abs(got[1] - 0.7310585786300049) < 1e-7


def test_routing_margin_hand():
    x, wg, *_ = hand_example()
    np.testing.assert_array_equal(oracle.routing_margin(x, wg), [0.5, 0.0])
    np.testing.assert_array_equal(oracle.top_gap(x, wg), [0.5, 1.0])
    np.testing.assert_array_equal(oracle.slot_order_gap(x, wg, 2), [0.5, 1.0])
    assert np.isinf(oracle.slot_order_gap(x, wg, 1)).all()


# ---------------------------------------------------------------------------
# Top-2 by brute force
# ---------------------------------------------------------------------------

def _key_beats(l, i, j):
    """Expert i is ordered before expert j: larger logit, or equal and lower index."""
    return l[i] > l[j] or (l[i] == l[j] and i < j)


@pytest.mark.parametrize("n,K", [(8, 2), (4, 1), (8, 3), (8, 4), (16, 2), (16, 4), (5, 5)])
@pytest.mark.parametrize("grid", [None, 1.0, 0.25])
def test_topk_brute_force(n, K, grid):
    """Every K-subset is tried: exactly one beats all unselected experts under
    the (logit desc, index asc) key, and the oracle returns it in key order."""
    rng = np.random.default_rng(123 + 16 * n + K)
    logits = rng.standard_normal((150, n)).astype(np.float32)
    if grid is not None:  # coarse grid -> many exact ties
        logits = (np.round(logits / grid) * grid).astype(np.float32)
    idx = oracle.topk_indices(logits, K)
    for t in range(logits.shape[0]):
        l = logits[t]
        winners = [sub for sub in itertools.combinations(range(n), K)
                   if all(_key_beats(l, a, b) for a in sub for b in range(n) if b not in sub)]
        assert len(winners) == 1
        assert set(idx[t]) == set(winners[0])
        for s in range(K - 1):
            assert _key_beats(l, idx[t, s], idx[t, s + 1])


def test_top1_gate_is_one():
    """K = 1: the softmax over one surviving logit is exactly 1."""
    inp = mi.make_layer(64, 32, 16, n=6, K=1, dtype="f32", init="fanin", seed=8, workload=103)
    x, wg, *_ = inp.numpy_f32()
    G, idx, l = oracle.gating(x, wg, K=1)
    rows = np.arange(64)
    assert (G[rows, idx[:, 0]] == 1.0).all() and ((G != 0).sum(axis=1) == 1).all()
    np.testing.assert_array_equal(idx[:, 0], np.argmax(l, axis=1))


def test_topk_all_experts_is_plain_softmax():
    """K = n: TopK masks nothing, so G is the textbook softmax of the logits."""
    from scipy.special import softmax as sp_softmax
    inp = mi.make_layer(50, 32, 16, n=5, K=5, dtype="f32", init="fanin", seed=9, workload=104)
    x, wg, *_ = inp.numpy_f32()
    G, _, l = oracle.gating(x, wg, K=5)
    np.testing.assert_allclose(G, sp_softmax(np.asarray(l, np.float64), axis=1), rtol=2e-6, atol=1e-7)


def test_top2_scale_invariance():
    inp = mi.make_layer(64, 32, 16, dtype="f32", init="fanin", seed=3, workload=101)
    x, wg, *_ = inp.numpy_f32()
    idx = oracle.gating(x, wg)[1]
    for s in (2.0, 0.5, 1024.0):
        np.testing.assert_array_equal(oracle.gating(x, wg * np.float32(s))[1], idx)


# ---------------------------------------------------------------------------
# Gate invariants
# ---------------------------------------------------------------------------

def test_gate_invariants():
    inp = mi.make_layer(256, 64, 32, dtype="f32", init="fanin", seed=5, workload=102)
    x, wg, *_ = inp.numpy_f32()
    G, idx, _ = oracle.gating(x, wg)
    assert ((G != 0).sum(axis=1) == 2).all()
    assert (G >= 0).all()
    np.testing.assert_allclose(G.sum(axis=1), 1.0, rtol=0, atol=2.0 ** -22)
    rows = np.arange(G.shape[0])
    assert (G[rows, idx[:, 0]] >= 0.5).all() and (G[rows, idx[:, 1]] <= 0.5).all()


def test_zero_router_tie():
    x = np.random.default_rng(0).standard_normal((5, 16)).astype(np.float32)
    wg = np.zeros((16, 8), np.float32)
    G, idx, _ = oracle.gating(x, wg)
    np.testing.assert_array_equal(idx, np.tile([0, 1], (5, 1)))
    np.testing.assert_array_equal(G[:, :2], 0.5)
    np.testing.assert_array_equal(G[:, 2:], 0.0)


# ---------------------------------------------------------------------------
# Layer special cases
# ---------------------------------------------------------------------------

def _small(seed, T=24, d=32, F=48):
    inp = mi.make_layer(T, d, F, dtype="f32", init="fanin", seed=seed, workload=103)
    return inp.numpy_f32()


@pytest.mark.parametrize("a", [0, 3, 7])
def test_single_expert_dominance_bitwise(a):
    x, wg, w1, w3, w2 = _small(7)
    x = x.copy()
    wg = wg.copy()
    x[:, 0] = 1.0
    wg[0, a] = 1e4  # l_a - l_b >= ~1e4: exp(l_b - l_a) underflows to exactly 0
    out = oracle.moe_layer(x, wg, w1, w3, w2)
    assert (out["idx"][:, 0] == a).all()
    assert (out["gates"][:, 0] == 1.0).all() and (out["gates"][:, 1] == 0.0).all()
    Ea = oracle.swiglu_expert(x, w1[a], w3[a], w2[a])
    assert np.array_equal(out["y"], Ea)


def test_identical_experts():
    x, wg, w1, w3, w2 = _small(8)
    w1 = np.repeat(w1[:1], 8, axis=0)
    w3 = np.repeat(w3[:1], 8, axis=0)
    w2 = np.repeat(w2[:1], 8, axis=0)
    out = oracle.moe_layer(x, wg, w1, w3, w2)
    E = oracle.swiglu_expert(x, w1[0], w3[0], w2[0])
    np.testing.assert_allclose(out["y"], E, rtol=1e-5, atol=1e-6 * np.abs(E).max())


def test_token_permutation_equivariance():
    x, wg, w1, w3, w2 = _small(9)
    perm = np.random.default_rng(1).permutation(x.shape[0])
    a = oracle.moe_layer(x, wg, w1, w3, w2)
    b = oracle.moe_layer(x[perm], wg, w1, w3, w2)
    np.testing.assert_array_equal(b["idx"], a["idx"][perm])
    np.testing.assert_allclose(b["y"], a["y"][perm], rtol=1e-5, atol=1e-6)


def test_expert_relabelling_invariance():
    x, wg, w1, w3, w2 = _small(10)
    p = np.array([5, 2, 7, 0, 3, 6, 1, 4])  # new expert j is old expert p[j]
    a = oracle.moe_layer(x, wg, w1, w3, w2)
    b = oracle.moe_layer(x, wg[:, p], w1[p], w3[p], w2[p])
    assert oracle.routing_margin(x, wg).min() > 0 and oracle.top_gap(x, wg).min() > 0
    np.testing.assert_array_equal(p[b["idx"]], a["idx"])
    np.testing.assert_array_equal(b["counts"], a["counts"][p])
    np.testing.assert_allclose(b["y"], a["y"], rtol=1e-5, atol=1e-6)


def test_fp64_loop_bound():
    """fp32 oracle within 1e-5 (per-token relative) of a float64 evaluation
    written as explicit loops over the selected experts."""
    x, wg, w1, w3, w2 = _small(11, T=6, d=8, F=12)
    out = oracle.moe_layer(x, wg, w1, w3, w2)
    x64, w1_, w3_, w2_ = (a.astype(np.float64) for a in (x, w1, w3, w2))
    for t in range(x.shape[0]):
        l = [sum(float(x[t, k]) * float(wg[k, e]) for k in range(8)) for e in range(8)]
        order = sorted(range(8), key=lambda e: (-l[e], e))[:2]
        m = max(l[e] for e in order)
        z = sum(math.exp(l[e] - m) for e in order)
        y = [0.0] * 8
        for e in order:
            g = math.exp(l[e] - m) / z
            h = []
            for f in range(12):
                a = sum(x64[t, k] * w1_[e, f, k] for k in range(8))
                b = sum(x64[t, k] * w3_[e, f, k] for k in range(8))
                h.append(a / (1 + math.exp(-a)) * b)
            for j in range(8):
                y[j] += g * sum(w2_[e, j, f] * h[f] for f in range(12))
        err = np.abs(out["y"][t] - np.array(y)).max() / np.abs(y).max()
        assert err < 1e-5
        assert sorted(order) == sorted(out["idx"][t].tolist())


# ---------------------------------------------------------------------------
# Reference layouts
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,K", [(8, 2), (16, 4), (3, 1), (6, 3)])
@pytest.mark.parametrize("tile_m", [1, 16, 128])
def test_group_by_expert_properties(tile_m, n, K):
    rng = np.random.default_rng(tile_m + 100 * n + K)
    T = 300
    idx = np.stack([rng.permutation(n)[:K] for _ in range(T)]).astype(np.int32)
    g = oracle.group_by_expert(idx, n, tile_m)
    counts, offsets, row_src, row_of = g["counts"], g["offsets"], g["row_src"], g["row_of"]
    assert counts.sum() == T * K
    np.testing.assert_array_equal(counts, np.bincount(idx.ravel(), minlength=n))
    assert offsets[0] == 0 and (np.diff(offsets) % tile_m == 0).all()
    assert (np.diff(offsets) >= counts).all() and (np.diff(offsets) < counts + tile_m).all()
    assert len(row_src) == T * K + n * (tile_m - 1)
    for e in range(n):
        seg = row_src[offsets[e]:offsets[e + 1]]
        real = seg[:counts[e]]
        assert (seg[counts[e]:] == -1).all()
        assert (np.diff(real) > 0).all()
        assert (idx.ravel()[real] == e).all()
    assert (row_src[offsets[n]:] == -1).all()
    flat_of = row_of.ravel()
    np.testing.assert_array_equal(row_src[flat_of], np.arange(T * K))


def test_sparse_path_equals_dense():
    x, wg, w1, w3, w2 = _small(12, T=40)
    out = oracle.moe_layer(x, wg, w1, w3, w2)
    g = oracle.group_by_expert(out["idx"], 8, 16)
    _, y_perm = oracle.expert_rows(x, g["row_src"], g["offsets"], w1, w3, w2)
    y = oracle.combine(y_perm, g["row_of"], out["gates"])
    np.testing.assert_allclose(y, out["y"], rtol=1e-5, atol=1e-6)


def test_combine_dropped_slots_brute_force():
    """A slot whose permuted row is negative adds nothing (an assignment to no
    expert is dropped by the grouping); a token with every slot dropped keeps
    only its residual.  Element-by-element loops on a tiny case."""
    rng = np.random.default_rng(3)
    T, K, d, P = 5, 2, 3, 7
    y_perm = rng.standard_normal((P, d)).astype(np.float32)
    row_of = np.array([[0, 1], [-1, 2], [3, -1], [-1, -1], [6, 5]], np.int32)
    gates = rng.uniform(0.1, 1.0, (T, K)).astype(np.float32)
    res = rng.standard_normal((T, d)).astype(np.float32)
    got = oracle.combine(y_perm, row_of, gates, res)
    for t in range(T):
        for j in range(d):
            acc = 0.0
            for s in range(K):
                if row_of[t, s] >= 0:
                    acc += float(gates[t, s]) * float(y_perm[row_of[t, s], j])
            assert abs(got[t, j] - (acc + float(res[t, j]))) <= 1e-5 * (1.0 + abs(acc))
    np.testing.assert_array_equal(got[3], res[3])


@pytest.mark.parametrize("n,K", [(6, 3), (16, 4), (4, 1)])
def test_sparse_path_equals_dense_general_k(n, K):
    """Grouped rows + slot-order combine reproduce the dense per-token sum for
    other expert counts and K (token of assignment a is a // K)."""
    inp = mi.make_layer(40, 32, 24, n=n, K=K, dtype="f32", init="fanin", seed=n + K, workload=105)
    x, wg, w1, w3, w2 = inp.numpy_f32()
    out = oracle.moe_layer(x, wg, w1, w3, w2, K=K)
    assert out["idx"].shape == (40, K)
    g = oracle.group_by_expert(out["idx"], n, 16)
    _, y_perm = oracle.expert_rows(x, g["row_src"], g["offsets"], w1, w3, w2, K=K)
    y = oracle.combine(y_perm, g["row_of"], out["gates"])
    np.testing.assert_allclose(y, out["y"], rtol=1e-5, atol=1e-6)


# ---------------------------------------------------------------------------
# RMSNorm, bf16 rounding
# ---------------------------------------------------------------------------

def test_rmsnorm_closed_form():
    h = np.array([[3.0, 4.0], [-2.0, -2.0], [0.0, 0.0]], np.float32)
    x = oracle.rmsnorm(h, eps=1e-5)
    np.testing.assert_allclose(x[0], np.array([3, 4]) / math.sqrt(12.5 + 1e-5), rtol=1e-6)
    np.testing.assert_allclose(x[1], -2 / math.sqrt(4 + 1e-5), rtol=1e-6)
    np.testing.assert_array_equal(x[2], 0.0)
    big = np.random.default_rng(0).standard_normal((4, 4096)).astype(np.float32) * 7
    np.testing.assert_allclose((oracle.rmsnorm(big) ** 2).mean(axis=1), 1.0, rtol=1e-5)


def test_round_bf16():
    v = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8 + 2 ** -20), 3.0e-39], np.float32)
    np.testing.assert_array_equal(oracle.round_bf16(v)[:4], [1.0, 1.0, 1 + 2 ** -6, -(1 + 2 ** -7)])
    r = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 100
    ref = torch.from_numpy(r).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(oracle.round_bf16(r), ref)


def test_moe_block_residual():
    x, wg, w1, w3, w2 = _small(13)
    h_next, out = oracle.moe_block(x, wg, w1, w3, w2, bf16_storage=False)
    xn = oracle.rmsnorm(x)
    ref = oracle.moe_layer(xn, wg, w1, w3, w2)["y"]
    np.testing.assert_allclose(h_next - x, ref, rtol=1e-4, atol=1e-5)


def _bf16(v):
    """Round float64 values to bf16 with torch's cast (an implementation
    independent of the oracle's), returned as float64."""
    return torch.tensor(np.asarray(v, np.float64), dtype=torch.float64).to(torch.float32) \
        .to(torch.bfloat16).double().numpy()


def test_moe_block_bf16_storage_hand_placed():
    """Where the stack's bf16 storage rounds: the normalised x is rounded to bf16
    after the norm (it is the stored input of the layer), and the block output
    h + y is rounded once after the residual add.  Identical identity experts
    and an all-zero router (gates exactly 1/2, 1/2) make y = SiLU(x) * x, which
    is written out here in float64 from the closed form sigma(z) = 1/(1+e^-z)."""
    d = n = 4
    eye = np.eye(d, dtype=np.float32)
    w = np.stack([eye] * n)
    wg = np.zeros((d, n), np.float32)
    h = np.array([[3.0, 4.0, 0.5, -1.25], [-2.0, 0.375, 1.5, 2.75], [0.125, -7.0, 6.5, 1.0]], np.float32)
    assert (_bf16(h) == h).all()
    h64 = h.astype(np.float64)
    x_exact = h64 / np.sqrt((h64 ** 2).mean(axis=1, keepdims=True) + 1e-5)
    x_hand = _bf16(x_exact)

    def e(x):
        return x * x / (1.0 + np.exp(-x))

    want = _bf16(h64 + e(x_hand))
    # the case tells the placements apart: no rounding of x, no rounding of the
    # output, and rounding y before the residual add all give other values
    assert (x_hand != x_exact).any()
    assert (_bf16(h64 + e(x_exact)) != want).any()
    assert (h64 + e(x_hand) != want).any()
    assert (h64 + _bf16(e(x_hand)) != want).any() or (_bf16(h64 + _bf16(e(x_hand))) != want).any()
    # no value sits near a bf16 rounding boundary, so fp32 evaluation order cannot flip it
    v = h64 + e(x_hand)
    ulp = 2.0 ** (np.floor(np.log2(np.abs(v))) - 7)
    frac = np.abs(v / ulp - np.round(v / ulp))
    assert (np.abs(frac - 0.5) > 1e-3).all()

    h_next, out = oracle.moe_block(h, wg, w, w, w, K=2, bf16_storage=True)
    np.testing.assert_array_equal(out["x"], x_hand)
    np.testing.assert_array_equal(out["gates"], 0.5)
    np.testing.assert_array_equal(h_next, want)
    # without bf16 storage the same block keeps fp32 values
    h32, out32 = oracle.moe_block(h, wg, w, w, w, K=2, bf16_storage=False)
    np.testing.assert_allclose(out32["x"], x_exact, rtol=1e-6)
    np.testing.assert_allclose(h32, h64 + e(x_exact), rtol=1e-6)


# ---------------------------------------------------------------------------
# The pages' printed parameter counts
# ---------------------------------------------------------------------------

def test_parameter_counts_golden():
    with open(os.path.join(GOLDEN, "mixtral_param_counts.json")) as f:
        g = json.load(f)
    for wl in mi.WORKLOADS[1:]:
        d, F, n = wl["d"], wl["F"], wl["n"]
        assert (d, F, n, wl["K"]) == (g["dims"]["d_model"], g["dims"]["d_ffn"],
                                      g["dims"]["n_experts"], g["dims"]["top_k"])
        small = mi.make_layer(2, 16, 24, n=n, dtype="bf16", seed=0, workload=104)
        # shapes follow [n, F, d] / [n, d, F] / [d, n] whatever the sizes
        assert small.w1.shape == (n, 24, 16) and small.w3.shape == (n, 24, 16)
        assert small.w2.shape == (n, 16, 24) and small.wg.shape == (16, n)
        per_expert = F * d + F * d + d * F
        per_layer = n * per_expert
        L = g["dims"]["n_layers"]
        assert round(per_expert / 1e6, 2) == g["printed"]["per_expert_millions"]
        assert round(per_layer / 1e9, 3) == g["printed"]["per_layer_billions"]
        assert round(L * per_layer / 1e9, 1) == g["printed"]["all_layers_billions"]
        assert round(L * d * n / 1e6, 2) == g["printed"]["router_all_layers_millions"]
    assert mi.WORKLOADS[4]["layers"] == g["dims"]["n_layers"]


def test_tiny_workload_runs_fast():
    inp = mi.make_workload(0)
    out = oracle.moe_layer(*inp.numpy_f32())
    assert out["y"].shape == (64, 128) and out["counts"].sum() == 128


# ---------------------------------------------------------------------------
# FP8 (OCP E4M3) expert weights
# ---------------------------------------------------------------------------

def test_e4m3_decode_all_codes_vs_torch():
    """Every code against torch's float8_e4m3fn (a library decoder)."""
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert ((got == ref) | (np.isnan(got) & np.isnan(ref))).all()
    assert np.isnan(got).sum() == 2  # 0x7F and 0xFF


def test_e4m3_hand_values():
    d = oracle.e4m3_decode(np.array([0x38, 0x3C, 0x7E, 0x01, 0x07, 0x08, 0x80, 0x00, 0xB8, 0x7F], np.uint8))
    np.testing.assert_array_equal(d[:8], [1.0, 1.5, 448.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 0.0, 0.0])
    assert np.signbit(d[6]) and not np.signbit(d[7])
    assert d[8] == -1.0 and np.isnan(d[9])


def test_e4m3_encode_vs_torch_in_range():
    """Inside +-448 the oracle's rounding equals torch's round-to-nearest-even
    cast, on random values over many binades and on every exact midpoint
    between neighbouring codes (ties go to the even mantissa)."""
    rng = np.random.default_rng(7)
    v = (rng.standard_normal(50000) * rng.choice([1e-3, 0.05, 1.0, 100.0], 50000)).astype(np.float32)
    v = np.clip(v, -448, 448).astype(np.float32)
    vals = np.unique(oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8)))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    assert (mids.astype(np.float64) == (vals[:-1] + vals[1:]) / 2).all()  # exact in fp32
    for a in (v, mids, -mids):
        ref = torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        np.testing.assert_array_equal(oracle.e4m3_encode_rne(a), ref)
    # a tie between 1.0 (M=0) and 1.125 (M=1) goes to 1.0; between 1.125 and 1.25 to 1.25
    np.testing.assert_array_equal(oracle.e4m3_encode_rne(np.array([1.0625, 1.1875], np.float32)), [0x38, 0x3A])


def test_e4m3_saturation():
    got = oracle.e4m3_encode_rne(np.array([448, 449, 500, 1e30, -1e30, -460], np.float32))
    np.testing.assert_array_equal(got, [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE])


def test_quantize_rows_bounds():
    """Round trip within half a quantum of w / scale; every non-zero row
    reaches the code of +-448; an all-zero row gets scale 1 and code 0."""
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((3, 40, 96)) * 0.02).astype(np.float32)
    w[1, 5] = 0.0
    q, s = oracle.quantize_rows_fp8(w)
    assert q.shape == w.shape and s.shape == (3, 40) and s.dtype == np.float32
    assert s[1, 5] == 1.0 and (q[1, 5] == 0).all()
    v = (w / s[..., None]).astype(np.float64)
    dq = oracle.e4m3_decode(q)
    a = np.abs(v)
    half_quantum = np.where(a >= 2.0 ** -6, np.ldexp(1.0, np.frexp(a)[1] - 1 - 4), 2.0 ** -10)
    assert (np.abs(dq - v) <= half_quantum).all()
    nz = np.abs(w).max(axis=-1) > 0
    assert ((np.abs(dq).max(axis=-1) == 448.0) == nz).all()


def test_fp8_layer_equals_plain_layer_on_representable_weights():
    """Weights that are E4M3 values times a power of two, with a row maximum of
    448 times that power, quantize without error (scale exact, codes exact), so
    the FP8 layer must equal the plain layer bit for bit."""
    rng = np.random.default_rng(11)
    T, d, F, n = 24, 32, 48, 8
    pos = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))

    def draw(shape, m):
        w = (rng.choice(pos, size=shape) * rng.choice([-1.0, 1.0], size=shape))
        w[..., 0] = 448.0  # the row maximum
        return (w * 2.0 ** -m).astype(np.float32)

    w1, w3, w2 = draw((n, F, d), 12), draw((n, F, d), 11), draw((n, d, F), 13)
    x = rng.standard_normal((T, d)).astype(np.float32)
    wg = (rng.standard_normal((d, n)) * 0.3).astype(np.float32)
    (q1, s1), (q3, s3), (q2, s2) = (oracle.quantize_rows_fp8(w) for w in (w1, w3, w2))
    assert (s1 == np.float32(2.0 ** -12)).all() and (s2 == np.float32(2.0 ** -13)).all()
    got = oracle.moe_layer_fp8(x, wg, q1, s1, q3, s3, q2, s2)["y"]
    ref = oracle.moe_layer(x, wg, w1, w3, w2)["y"]
    np.testing.assert_array_equal(got, ref)


def test_fp8_error_against_plain_layer():
    """What FP8 weights do to the layer (a property of the format, not parity):
    E4M3 rounding leaves a relative error of about 2^-3 / sqrt(12) / 1.4 ~ 2.6%
    rms per weight, and three chained matrices about sqrt(3) times that ~ 4.5%
    rms per output; the per-token max-norm error stays below 0.10."""
    inp = mi.make_layer(64, 512, 1024, seed=1, workload=600)
    xn, wgn, w1, w3, w2 = inp.numpy_f32()
    ref = oracle.moe_layer(xn, wgn, w1, w3, w2)
    qs = [oracle.quantize_rows_fp8(w) for w in (w1, w3, w2)]
    got = oracle.moe_layer_fp8(xn, wgn, *qs[0], *qs[1], *qs[2])
    np.testing.assert_array_equal(got["idx"], ref["idx"])  # the router is not quantized
    err = np.abs(got["y"] - ref["y"]).max(axis=1) / np.abs(ref["y"]).max(axis=1)
    rms = np.sqrt(((got["y"] - ref["y"]) ** 2).mean(axis=1) / (ref["y"] ** 2).mean(axis=1))
    assert err.max() < 0.10
    assert 0.03 < np.median(rms) < 0.06


# ---------------------------------------------------------------------------
# Backward pass
# ---------------------------------------------------------------------------

def _bwd_case(seed, T=12, d=16, F=24, n=8, K=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((d, n)) * 0.5
    w1 = rng.standard_normal((n, F, d)) / np.sqrt(d)
    w3 = rng.standard_normal((n, F, d)) / np.sqrt(d)
    w2 = rng.standard_normal((n, d, F)) / np.sqrt(F)
    dy = rng.standard_normal((T, d))
    return x, wg, w1, w3, w2, dy


@pytest.mark.parametrize("n,K", [(8, 2), (8, 1), (6, 3), (4, 4)])
def test_backward_vs_torch_autograd(n, K):
    """Every gradient against torch autograd on a float64 dense formulation
    (the TopK selection is taken from the forward oracle and held fixed, as
    it is piecewise constant)."""
    x, wg, w1, w3, w2, dy = _bwd_case(20 + n + K, n=n, K=K)
    g = oracle.moe_layer_backward(x, wg, w1, w3, w2, dy, K=K)
    tx, twg, tw1, tw3, tw2 = (torch.tensor(a, dtype=torch.float64, requires_grad=True)
                              for a in (x, wg, w1, w3, w2))
    logits = tx @ twg
    mask = torch.zeros_like(logits, dtype=torch.bool)
    mask[torch.arange(x.shape[0])[:, None], torch.from_numpy(g["idx"].astype(np.int64))] = True
    G = torch.softmax(logits.masked_fill(~mask, float("-inf")), dim=1)
    y = 0
    for i in range(n):
        a1 = tx @ tw1[i].T
        hh = torch.nn.functional.silu(a1) * (tx @ tw3[i].T)
        y = y + G[:, i:i + 1] * (hh @ tw2[i].T)
    (y * torch.from_numpy(dy)).sum().backward()
    for name, t in (("dx", tx), ("dwg", twg), ("dw1", tw1), ("dw3", tw3), ("dw2", tw2)):
        np.testing.assert_allclose(g[name], t.grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=name)


def test_backward_vs_finite_differences():
    """Central differences of the float64 forward at random coordinates of
    every input (routing margins checked so that no step changes the
    selection)."""
    x, wg, w1, w3, w2, dy = _bwd_case(31, T=6, d=8, F=10, n=6, K=2)
    g = oracle.moe_layer_backward(x, wg, w1, w3, w2, dy, K=2)
    s = -np.sort(-(x @ wg), axis=1)
    assert (s[:, 1] - s[:, 2]).min() > 1e-3
    rng = np.random.default_rng(5)
    args = [x, wg, w1, w3, w2]
    names = ["dx", "dwg", "dw1", "dw3", "dw2"]
    eps = 1e-6
    for ai, name in enumerate(names):
        for _ in range(6):
            pos = tuple(rng.integers(0, m) for m in args[ai].shape)
            lo = [a.copy() for a in args]
            hi = [a.copy() for a in args]
            lo[ai][pos] -= eps
            hi[ai][pos] += eps
            f_hi = (oracle.forward64(*hi, K=2)["y"] * dy).sum()
            f_lo = (oracle.forward64(*lo, K=2)["y"] * dy).sum()
            fd = (f_hi - f_lo) / (2 * eps)
            assert abs(fd - g[name][pos]) <= 1e-6 * max(1.0, abs(fd)), (name, pos, fd, g[name][pos])


def test_backward_top1_closed_form():
    """K = 1: the gate is exactly 1, so the router gets no gradient and the
    layer's gradients are those of the selected expert alone."""
    x, wg, w1, w3, w2, dy = _bwd_case(41, n=5, K=1)
    g = oracle.moe_layer_backward(x, wg, w1, w3, w2, dy, K=1)
    assert (g["dwg"] == 0).all()
    for t in range(x.shape[0]):
        e = g["idx"][t, 0]
        a1, a3 = w1[e] @ x[t], w3[e] @ x[t]
        s = 1 / (1 + np.exp(-a1))
        dh = w2[e].T @ dy[t]
        dx = w1[e].T @ (dh * a3 * s * (1 + a1 * (1 - s))) + w3[e].T @ (dh * a1 * s)
        np.testing.assert_allclose(g["dx"][t], dx, rtol=1e-12, atol=1e-12)
    for e in range(5):
        sel = g["idx"][:, 0] == e
        h = (x[sel] @ w1[e].T) * (1 / (1 + np.exp(-(x[sel] @ w1[e].T)))) * (x[sel] @ w3[e].T)
        np.testing.assert_allclose(g["dw2"][e], dy[sel].T @ h, rtol=1e-12, atol=1e-12)


def test_backward_sampled_helpers_match_dense():
    """The per-token and per-expert-row backward helpers (used on full-size
    layers) agree with the dense backward oracle."""
    x, wg, w1, w3, w2, dy = _bwd_case(51, T=20, d=16, F=24, n=6, K=2)
    g = oracle.moe_layer_backward(x, wg, w1, w3, w2, dy, K=2)
    tok = np.array([0, 3, 7, 19])
    r = oracle.backward_token_rows(x, wg, w1, w3, w2, dy, tok, K=2)
    np.testing.assert_allclose(r["dx"], g["dx"][tok], rtol=1e-12, atol=1e-12)
    for e in range(6):
        rows = oracle.backward_expert_rows(x, wg, w1, w3, w2, dy, e, [0, 5, 23], [1, 15], K=2)
        np.testing.assert_allclose(rows["dw1"], g["dw1"][e][[0, 5, 23]], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(rows["dw3"], g["dw3"][e][[0, 5, 23]], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(rows["dw2"], g["dw2"][e][[1, 15]], rtol=1e-12, atol=1e-12)

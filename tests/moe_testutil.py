"""Shared helpers of the parity tests: margin-filtered inputs, device upload and
the comparison rules (routing bit-exact, outputs by per-token relative error)."""
from __future__ import annotations

import numpy as np
import torch

import moe_inputs as mi
import oracle

MARGIN = 1e-3          # minimum gap between the 2nd and 3rd logit of every token
TOL_BF16 = 2e-2        # max per-token relative error, bf16 layers
TOL_F32 = 1e-4         # max per-token relative error, fp32 layers
GATE_TOL = 1e-5


def margin_filtered(inp: mi.LayerInputs, margin: float = MARGIN, max_rounds: int = 50) -> mi.LayerInputs:
    """Redraw token rows until every token's 2nd-vs-3rd logit gap is >= margin
    (gap computed by the oracle in float64 from the exact input values)."""
    for _ in range(max_rounds):
        x = inp.x.float().numpy()
        bad = np.nonzero(oracle.routing_margin(x, inp.wg.numpy(), inp.K) < margin)[0]
        if bad.size == 0:
            return inp
        inp = mi.redraw_rows(inp, bad)
    raise RuntimeError("margin filter did not converge")


def to_device(inp: mi.LayerInputs, device="cuda"):
    return (inp.x.to(device), inp.wg.to(device), inp.w1.to(device), inp.w3.to(device),
            inp.w2.to(device))


def per_token_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """max_j |got - ref| / max_j |ref| for each row (rows of ref that are all zero
    use an absolute error)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(got - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def assert_routing_equal(idx_gpu, gate_gpu, ref: dict, x, wg, K=2, gate_tol=GATE_TOL):
    """Bit-exact routing: per token the selected expert set, the slot order where
    every gap between neighbouring selected logits is >= MARGIN, and the
    per-expert counts; gates matched by expert id within gate_tol."""
    idx_gpu = np.asarray(idx_gpu)
    gate_gpu = np.asarray(gate_gpu)
    ridx = ref["idx"]
    assert idx_gpu.shape == ridx.shape
    np.testing.assert_array_equal(np.sort(idx_gpu, axis=1), np.sort(ridx, axis=1))
    sure = oracle.slot_order_gap(x, wg, ridx.shape[1]) >= MARGIN
    np.testing.assert_array_equal(idx_gpu[sure], ridx[sure])
    n = wg.shape[1]
    np.testing.assert_array_equal(np.bincount(idx_gpu.ravel(), minlength=n), ref["counts"])
    # gates matched by expert id
    T = idx_gpu.shape[0]
    Gg = np.zeros((T, n))
    Gg[np.arange(T)[:, None], idx_gpu] = gate_gpu
    Gr = np.zeros((T, n))
    Gr[np.arange(T)[:, None], ridx] = ref["gates"]
    assert np.abs(Gg - Gr).max() <= gate_tol


def sample_rows(T: int, idx: np.ndarray, n_rows: int, seed: int = 0, must_cover: int = 8) -> np.ndarray:
    """A seeded sample of token rows that covers every expert at least
    ``must_cover`` times where possible (first and last tokens included)."""
    rng = np.random.default_rng(seed)
    chosen = {0, T - 1}
    for e in range(int(idx.max()) + 1):
        cand = np.nonzero((idx == e).any(axis=1))[0]
        if cand.size:
            chosen.update(rng.choice(cand, size=min(must_cover, cand.size), replace=False).tolist())
    rest = rng.permutation(T)
    for t in rest:
        if len(chosen) >= n_rows:
            break
        chosen.add(int(t))
    return np.array(sorted(chosen), dtype=np.int64)

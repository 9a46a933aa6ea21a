"""CPU oracle of the Mixtral sparse mixture-of-experts feed-forward layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports, links or calls this
module; it exists so that the tests, the package's smoke check and the bench's
CPU-baseline leg can check the HIP path against a plain, slow, obviously correct
evaluation of the layer.  It shares no code with the HIP path.

Sources (cited by page and section; the pages are web summaries of
"Mixtral of Experts", arXiv 2401.04088):
  [P1] paper-graph-ui.vercel.app/p/moe/2401.04088-Mixtral-of-Experts,
       section 3.4 "Detailed, Sentence-Based Technical Breakdown":
       "MoE Layer Formulation" (gating equation G(x) = Softmax(TopK(x.W_g)),
       TopK equation, output equation y = sum_i G(x)_i E_i(x)),
       "Expert Network Structure (SwiGLU)" (SwiGLU equation, SiLU(z) = z.sigma(z)),
       "Top-K Gating Mechanism and Routing" (no router bias; the three
       mechanical steps of top-2), "Architectural Inheritance from Mistral 7B"
       (pre-norm RMSNorm), section 3.2 (residual add after the MoE block).
  [P3] xyznot.com/paper/2401.04088, "Method (with the key equations)":
       G(x) := Softmax(TopK(x.W_g)), TopK over the top-K coordinates of l = x.W_g,
       y = sum_{i=0}^{n-1} G(x)_i SwiGLU_i(x).

Precision: float32 throughout (the dense formula is evaluated in fp32, as the
layer's specification asks); bf16 inputs are upcast exactly before they arrive.

Readings where the pages are silent (each also listed in the design notes):
  * weight names: w1 = gate projection (gets SiLU), w3 = up projection (linear),
    w2 = down projection.  [P1]'s SwiGLU equation names the same three matrices
    W_{1,i} (SiLU), W_{2,i} (linear), W_{3,i} (down); only the labels differ.
  * TopK ties: the order key is (logit descending, expert index ascending), so
    the lower expert index wins a tie; slot 0 holds the larger logit.
  * RMSNorm: x = h / sqrt(mean(h^2) + eps) with eps = 1e-5 and unit gain (the
    pages name RMSNorm but give neither).

Pins (tests/test_oracle_pins.py): brute-force top-2 enumeration, gate
invariants and the all-zero-router tie case, a hand-worked example with closed-
form values, single-expert dominance (bitwise), identical experts, token
permutation and expert relabelling, an fp64 evaluation bound, the pages'
parameter counts.  Functions without a pin: none.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


# --------------------------------------------------------------------------
# Router: logits, TopK, softmax  ([P1] "MoE Layer Formulation"; [P3] Method)
# --------------------------------------------------------------------------

def router_logits(x: np.ndarray, wg: np.ndarray) -> np.ndarray:
    """l = x . W_g, one row of n logits per token, fp32.  No bias term
    ([P1] "Top-K Gating Mechanism and Routing": the router is a linear map and
    no bias is mentioned)."""
    return np.asarray(x, F32) @ np.asarray(wg, F32)


def topk_indices(logits: np.ndarray, K: int) -> np.ndarray:
    """Indices of the K largest logits of each row, largest first.

    A stable sort on -l keeps equal logits in index order, i.e. the order key is
    (logit descending, index ascending): the lower index wins ties."""
    order = np.argsort(-logits, axis=1, kind="stable")
    return order[:, :K].astype(np.int32)


def topk_mask(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """(TopK(l))_i = l_i for the selected coordinates, -inf elsewhere."""
    masked = np.full(logits.shape, -np.inf, dtype=F32)
    rows = np.arange(logits.shape[0])[:, None]
    masked[rows, idx] = logits[rows, idx]
    return masked


def softmax(v: np.ndarray) -> np.ndarray:
    """Row softmax; exp(-inf) = 0, so masked coordinates get weight exactly 0."""
    m = np.max(v, axis=1, keepdims=True)
    e = np.exp(v - m)
    return (e / np.sum(e, axis=1, keepdims=True)).astype(F32)


def gating(x: np.ndarray, wg: np.ndarray, K: int = 2):
    """G(x) = Softmax(TopK(x . W_g)).

    Returns (G [T,n] fp32 with exactly K non-zeros per row, idx [T,K] int32 in
    slot order, logits [T,n])."""
    logits = router_logits(x, wg)
    idx = topk_indices(logits, K)
    G = softmax(topk_mask(logits, idx))
    return G, idx, logits


# --------------------------------------------------------------------------
# Experts  ([P1] "Expert Network Structure (SwiGLU)")
# --------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigma(z), sigma(z) = 1 / (1 + exp(-z))."""
    z = np.asarray(z, F32)
    with np.errstate(over="ignore"):
        return (z * (F32(1.0) / (F32(1.0) + np.exp(-z)))).astype(F32)


def swiglu_expert(x: np.ndarray, w1: np.ndarray, w3: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """E(x) = w2 . (SiLU(w1 . x) * (w3 . x)) for a batch of row vectors x [T,d].

    w1, w3: [F, d]; w2: [d, F] (rows are output features)."""
    a = np.asarray(x, F32) @ np.asarray(w1, F32).T
    b = np.asarray(x, F32) @ np.asarray(w3, F32).T
    return (silu(a) * b) @ np.asarray(w2, F32).T


# --------------------------------------------------------------------------
# The layer  ([P1] output equation; [P3] y = sum_i G(x)_i SwiGLU_i(x))
# --------------------------------------------------------------------------

def moe_layer(x, wg, w1, w3, w2, K: int = 2) -> dict:
    """Dense evaluation of y = sum_{i=0}^{n-1} G(x)_i E_i(x).

    Every expert is evaluated on every token and multiplied by its gate, zero
    gates included; the sum runs in expert-index order.  Returns a dict with y
    [T,d] fp32, idx [T,K], gates [T,K] (gate of idx[:, s]), counts [n], G, logits.
    """
    x = np.asarray(x, F32)
    n = wg.shape[1]
    G, idx, logits = gating(x, wg, K)
    y = np.zeros((x.shape[0], w2.shape[1]), dtype=F32)
    for i in range(n):
        y += G[:, i:i + 1] * swiglu_expert(x, w1[i], w3[i], w2[i])
    rows = np.arange(x.shape[0])[:, None]
    counts = np.bincount(idx.reshape(-1), minlength=n).astype(np.int32)
    return dict(y=y, idx=idx, gates=G[rows, idx].astype(F32), counts=counts, G=G,
                logits=logits)


def rmsnorm(h: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    """x = h / sqrt(mean(h^2) + eps), unit gain ([P1] "Architectural
    Inheritance from Mistral 7B": pre-norm RMSNorm before the MoE block)."""
    h = np.asarray(h, F32)
    return (h / np.sqrt(np.mean(h * h, axis=1, keepdims=True) + F32(eps))).astype(F32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even), returned as fp32.
    Models the bf16 storage of activations between layers of the stack."""
    u = np.ascontiguousarray(a, F32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(F32).reshape(np.shape(a))


def moe_block(h, wg, w1, w3, w2, K: int = 2, eps: float = 1e-5, bf16_storage: bool = True):
    """One decoder MoE block with the attention omitted: h + MoE(RMSNorm(h))
    ([P1] section 3.2: the MoE output is added to the residual stream).
    With ``bf16_storage`` the normalised x and the block output are rounded to
    bf16, as they are stored in bf16 between steps.  Returns (h_next, layer dict)."""
    x = rmsnorm(h, eps)
    if bf16_storage:
        x = round_bf16(x)
    out = moe_layer(x, wg, w1, w3, w2, K)
    h_next = np.asarray(h, F32) + out["y"]
    if bf16_storage:
        h_next = round_bf16(h_next)
    out["x"] = x
    return h_next, out


# --------------------------------------------------------------------------
# Reference layouts for the library's intermediate calls (plain definitions)
# --------------------------------------------------------------------------

def max_permuted_rows(T: int, K: int, n: int, tile_m: int) -> int:
    """Worst-case padded row count: every expert segment padded up to tile_m."""
    return T * K + n * (tile_m - 1)


def group_by_expert(idx: np.ndarray, n: int, tile_m: int) -> dict:
    """Dropless grouping of the T*K (token, slot) assignments by expert.

    Assignment a = t*K + s goes to expert idx[t, s].  Segments are laid out in
    expert order; inside a segment assignments keep ascending a (a stable
    sort); each segment's length is rounded up to a multiple of tile_m and the
    padding rows hold -1.  Returns counts [n], offsets [n+1], row_src [P_max]
    (assignment of each permuted row or -1) and row_of [T,K] (permuted row of
    each assignment)."""
    T, K = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=n).astype(np.int32)
    padded = ((counts + tile_m - 1) // tile_m) * tile_m
    offsets = np.zeros(n + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(padded)
    P_max = max_permuted_rows(T, K, n, tile_m)
    row_src = np.full(P_max, -1, dtype=np.int32)
    row_of = np.full(T * K, -1, dtype=np.int32)
    order = np.argsort(flat, kind="stable")
    start = 0
    for e in range(n):
        members = order[start:start + counts[e]]
        start += counts[e]
        pos = offsets[e] + np.arange(counts[e])
        row_src[pos] = members
        row_of[members] = pos
    return dict(counts=counts, offsets=offsets, row_src=row_src, row_of=row_of.reshape(T, K))


def expert_rows(x, row_src, offsets, w1, w3, w2, K: int = 2):
    """The grouped expert computation on permuted rows: for permuted row p of
    expert e's segment holding assignment a (token a // K), h[p] = SiLU(w1[e].x)
    * (w3[e].x) and y_perm[p] = w2[e].h[p].  Padding rows are zero.
    Returns (h [P,F], y_perm [P,d]) in fp32."""
    x = np.asarray(x, F32)
    n = len(offsets) - 1
    P = len(row_src)
    F = w1.shape[1]
    d = w2.shape[1]
    h = np.zeros((P, F), dtype=F32)
    y_perm = np.zeros((P, d), dtype=F32)
    for e in range(n):
        p = np.arange(offsets[e], offsets[e + 1])
        p = p[row_src[p] >= 0]
        if p.size == 0:
            continue
        xe = x[row_src[p] // K]
        a = xe @ np.asarray(w1[e], F32).T
        b = xe @ np.asarray(w3[e], F32).T
        h[p] = silu(a) * b
        y_perm[p] = h[p] @ np.asarray(w2[e], F32).T
    return h, y_perm


def combine(y_perm, row_of, gates, residual=None):
    """y[t] = sum_s gates[t,s] * y_perm[row_of[t,s]] (+ residual[t]), fp32,
    slots summed in slot order.  A slot whose row is negative (an assignment
    to no expert, dropped by the grouping) adds nothing."""
    T, K = row_of.shape
    y = np.zeros((T, y_perm.shape[1]), dtype=F32)
    yp = np.asarray(y_perm, F32)
    for s in range(K):
        r = np.asarray(row_of[:, s])
        keep = r >= 0
        term = np.asarray(gates[:, s:s + 1], F32) * yp[np.where(keep, r, 0)]
        y += np.where(keep[:, None], term, F32(0))
    if residual is not None:
        y += np.asarray(residual, F32)
    return y


# --------------------------------------------------------------------------
# Input margins (used by callers to keep routing decisions well separated)
# --------------------------------------------------------------------------

def routing_margin(x, wg, K: int = 2) -> np.ndarray:
    """Per token, l_(K) - l_(K+1): the gap between the K-th and (K+1)-th largest
    logit, computed in float64 from the exact input values; +inf when K = n
    (every expert is selected, so there is no decision to separate)."""
    l = np.asarray(x, np.float64) @ np.asarray(wg, np.float64)
    s = -np.sort(-l, axis=1)
    if K >= l.shape[1]:
        return np.full(l.shape[0], np.inf)
    return s[:, K - 1] - s[:, K]


def top_gap(x, wg) -> np.ndarray:
    """Per token, l_(1) - l_(2) in float64 (decides the slot order only)."""
    l = np.asarray(x, np.float64) @ np.asarray(wg, np.float64)
    s = -np.sort(-l, axis=1)
    return s[:, 0] - s[:, 1]


def slot_order_gap(x, wg, K: int = 2) -> np.ndarray:
    """Per token, the smallest gap l_(s) - l_(s+1), s = 1..K-1, between
    neighbouring selected logits in float64: where it is large enough the slot
    order of the K selected experts is fixed.  +inf for K = 1."""
    l = np.asarray(x, np.float64) @ np.asarray(wg, np.float64)
    s = -np.sort(-l, axis=1)
    if K < 2:
        return np.full(l.shape[0], np.inf)
    return (s[:, :K - 1] - s[:, 1:K]).min(axis=1)

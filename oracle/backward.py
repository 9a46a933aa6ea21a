"""CPU oracle of the backward pass of the Mixtral sparse-MoE feed-forward layer.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the library never
imports, links or calls it, and it shares no code with the HIP path.

The layer (paper-graph-ui page, section 3.4: gating equation
G(x) = Softmax(TopK(x . W_g)), output equation y = sum_i G(x)_i E_i(x), SwiGLU
equation E_i(x) = w2_i . (SiLU(w1_i . x) * (w3_i . x))) is differentiated by
the chain rule, densely over all n experts, in float64.  For one token x with
upstream gradient dy:

  E_i      = w2_i h_i,  h_i = SiLU(a1_i) * a3_i,  a1_i = w1_i x,  a3_i = w3_i x
  dG_i     = dy . E_i
  dl_i     = G_i (dG_i - sum_j G_j dG_j)         softmax over the survivors; a
                                                 masked logit has G_i = 0, so it
                                                 gets no gradient (TopK is a
                                                 selection, flat almost everywhere)
  dW_g    += x (x) dl,       dx += W_g dl
  dE_i     = G_i dy
  dw2_i   += dE_i (x) h_i,   dh_i = w2_i^T dE_i
  da3_i    = dh_i * SiLU(a1_i)
  da1_i    = dh_i * a3_i * SiLU'(a1_i),  SiLU'(z) = s(z) (1 + z (1 - s(z))), s = sigmoid
  dw1_i   += da1_i (x) x,    dw3_i += da3_i (x) x
  dx      += w1_i^T da1_i + w3_i^T da3_i

Experts with G_i = 0 contribute exactly zero.  The routing itself (which K
experts) is the forward oracle's: order key (logit descending, index
ascending).

Pins (tests/test_oracle_pins.py): torch autograd on a float64 dense
formulation, central finite differences of a float64 forward, and the closed
form of a single selected expert (K = 1, where dl = 0 and G = 1).
"""
from __future__ import annotations

import numpy as np

from .moe_oracle import topk_indices

F64 = np.float64


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def forward64(x, wg, w1, w3, w2, K: int = 2) -> dict:
    """The layer in float64, densely (every expert on every token, times its
    gate), with the intermediates the backward pass uses."""
    x, wg, w1, w3, w2 = (np.asarray(a, F64) for a in (x, wg, w1, w3, w2))
    T = x.shape[0]
    n = wg.shape[1]
    logits = x @ wg
    idx = topk_indices(logits, K)
    rows = np.arange(T)[:, None]
    masked = np.full_like(logits, -np.inf)
    masked[rows, idx] = logits[rows, idx]
    e = np.exp(masked - masked.max(axis=1, keepdims=True))
    G = e / e.sum(axis=1, keepdims=True)
    a1 = np.einsum("td,nfd->ntf", x, w1)
    a3 = np.einsum("td,nfd->ntf", x, w3)
    h = a1 * _sigmoid(a1) * a3
    E = np.einsum("ntf,njf->ntj", h, w2)
    y = np.einsum("tn,ntj->tj", G, E)
    return dict(y=y, G=G, idx=idx, logits=logits, a1=a1, a3=a3, h=h, E=E, n=n)


def moe_layer_backward(x, wg, w1, w3, w2, dy, K: int = 2) -> dict:
    """Gradients of sum(dy * y) with respect to x, W_g, w1, w3, w2 (float64).

    Returns dict(dx [T,d], dwg [d,n], dw1 [n,F,d], dw3 [n,F,d], dw2 [n,d,F],
    idx [T,K], G [T,n])."""
    fw = forward64(x, wg, w1, w3, w2, K)
    x, wg, w1, w3, w2, dy = (np.asarray(a, F64) for a in (x, wg, w1, w3, w2, dy))
    G, a1, a3, h, E = fw["G"], fw["a1"], fw["a3"], fw["h"], fw["E"]
    # router
    dG = np.einsum("tj,ntj->tn", dy, E)
    dl = G * (dG - (G * dG).sum(axis=1, keepdims=True))
    dwg = x.T @ dl
    dx = dl @ wg.T
    # experts
    dE = G.T[:, :, None] * dy[None, :, :]                    # [n, T, d]
    dw2 = np.einsum("ntj,ntf->njf", dE, h)
    dh = np.einsum("ntj,njf->ntf", dE, w2)
    s = _sigmoid(a1)
    da3 = dh * a1 * s
    da1 = dh * a3 * s * (1.0 + a1 * (1.0 - s))
    dw1 = np.einsum("ntf,td->nfd", da1, x)
    dw3 = np.einsum("ntf,td->nfd", da3, x)
    dx = dx + np.einsum("ntf,nfd->td", da1, w1) + np.einsum("ntf,nfd->td", da3, w3)
    return dict(dx=dx, dwg=dwg, dw1=dw1, dw3=dw3, dw2=dw2, idx=fw["idx"], G=G)


def _route64(x, wg, K):
    logits = np.asarray(x, F64) @ np.asarray(wg, F64)
    idx = topk_indices(logits, K)
    rows = np.arange(logits.shape[0])[:, None]
    masked = np.full_like(logits, -np.inf)
    masked[rows, idx] = logits[rows, idx]
    e = np.exp(masked - masked.max(axis=1, keepdims=True))
    return idx, e / e.sum(axis=1, keepdims=True)


def backward_token_rows(x, wg, w1, w3, w2, dy, tokens, K: int = 2) -> dict:
    """dx and dl (router logit gradients) of the given tokens only, each token
    from its K selected experts (the experts with G = 0 contribute nothing),
    float64.  The same formulas as moe_layer_backward, for large layers."""
    tokens = np.asarray(tokens)
    xs = np.asarray(x, F64)[tokens]
    dys = np.asarray(dy, F64)[tokens]
    wg = np.asarray(wg, F64)
    idx, G = _route64(xs, wg, K)
    n = wg.shape[1]
    dG = np.zeros_like(G)
    cache = {}
    for e in np.unique(idx):
        S = np.nonzero((idx == e).any(axis=1))[0]
        w1e, w3e, w2e = (np.asarray(w[e], F64) for w in (w1, w3, w2))
        a1 = xs[S] @ w1e.T
        a3 = xs[S] @ w3e.T
        h = a1 * _sigmoid(a1) * a3
        dG[S, e] = (dys[S] * (h @ w2e.T)).sum(axis=1)
        cache[e] = (S, w1e, w3e, w2e, a1, a3)
    dl = G * (dG - (G * dG).sum(axis=1, keepdims=True))
    dx = dl @ wg.T
    for e, (S, w1e, w3e, w2e, a1, a3) in cache.items():
        dh = (G[S, e][:, None] * dys[S]) @ w2e
        s = _sigmoid(a1)
        dx[S] += (dh * a3 * s * (1.0 + a1 * (1.0 - s))) @ w1e + (dh * a1 * s) @ w3e
    return dict(dx=dx, dl=dl, idx=idx, G=G, n=n)


def backward_expert_rows(x, wg, w1, w3, w2, dy, e: int, f_rows, j_rows, K: int = 2) -> dict:
    """Rows f_rows of dw1[e] and dw3[e] and rows j_rows of dw2[e], float64,
    summed over every token routed to expert e."""
    x64 = np.asarray(x, F64)
    idx, G = _route64(x64, wg, K)
    S = np.nonzero((idx == e).any(axis=1))[0]
    xs, dys, gs = x64[S], np.asarray(dy, F64)[S], G[S, e]
    w1e, w3e, w2e = (np.asarray(w[e], F64) for w in (w1, w3, w2))
    a1 = xs @ w1e.T
    a3 = xs @ w3e.T
    h = a1 * _sigmoid(a1) * a3
    dw2 = (gs[:, None] * dys[:, j_rows]).T @ h
    f_rows = np.asarray(f_rows)
    dh = gs[:, None] * (dys @ w2e[:, f_rows])
    a1f, a3f = a1[:, f_rows], a3[:, f_rows]
    s = _sigmoid(a1f)
    dw1 = (dh * a3f * s * (1.0 + a1f * (1.0 - s))).T @ xs
    dw3 = (dh * a1f * s).T @ xs
    return dict(dw1=dw1, dw3=dw3, dw2=dw2, count=S.size)

"""Seeded synthetic inputs for the sparse mixture-of-experts feed-forward layer.

This module only draws random tensors.  It is shared by the tests, the bench and
the oracle's callers, and it holds none of the layer's arithmetic (no router
logits, no top-k, no SwiGLU, no combine): every number it produces is a seeded
random draw, a fixed constant, or the row scaling that a workload's input recipe
names.

Workloads (the five shapes of the Mixtral MoE block, "Mixtral of Experts",
paper-graph-ui page, section 3.4 "MoE Layer Formulation" / "Expert Network
Structure": d = 4096, ffn = 14336, n = 8 experts, top-2):

  0  tiny fp32      T=64,    d=128,  F=256    x~N(0,1), W_g,w1,w3~N(0,1/d), w2~N(0,1/F)
  1  decode bf16    T=32,    d=4096, F=14336  W_g fp32 std 0.02, experts bf16 std 0.02,
                                              x = rows of N(0,1) scaled to unit RMS, bf16
  2  prefill bf16   T=4096   (as 1)
  3  skewed bf16    T=16384  (as 1) + input channel 0 held at 1.0 and
                                       W_g[0,:] = [1.5*s, 1.5*s, 0, ...], s = 0.02*sqrt(d)
  4  stack bf16     T=8192, 32 layers, h0 ~ N(0,1) bf16, independent weights per layer

Variance convention: N(0, 1/d) is a variance (std 1/sqrt(d)); "std 0.02" is a
standard deviation.

Streams: every tensor has its own PCG64 stream keyed by
SeedSequence([seed, workload, layer, tensor_id, chunk]); large tensors are drawn
in fixed 4 Mi-element chunks so that the values do not depend on how many
threads draw them.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np
import torch

# tensor ids inside a (seed, workload, layer) key
X_ID, WG_ID, W1_ID, W3_ID, W2_ID, H0_ID, REDRAW_ID = 0, 1, 2, 3, 4, 5, 6

_CHUNK = 1 << 22
RMS_EPS = 1e-5  # epsilon of the unit-RMS input recipe

WORKLOADS = [
    dict(name="tiny_fp32", T=64, d=128, F=256, n=8, K=2, dtype="f32", init="fanin",
         skew=False, layers=1),
    dict(name="decode_bf16", T=32, d=4096, F=14336, n=8, K=2, dtype="bf16", init="mixtral",
         skew=False, layers=1),
    dict(name="prefill_bf16", T=4096, d=4096, F=14336, n=8, K=2, dtype="bf16",
         init="mixtral", skew=False, layers=1),
    dict(name="skewed_prefill_bf16", T=16384, d=4096, F=14336, n=8, K=2, dtype="bf16",
         init="mixtral", skew=True, layers=1),
    dict(name="stack32_bf16", T=8192, d=4096, F=14336, n=8, K=2, dtype="bf16",
         init="stack", skew=False, layers=32),
]


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _normal(shape, key, std: float, out_dtype: torch.dtype) -> torch.Tensor:
    """N(0, std^2) draws, rounded once to ``out_dtype`` (round-to-nearest-even)."""
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=out_dtype)
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def work(c: int) -> None:
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key) + [c])))
        tmp = g.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            tmp *= np.float32(std)
        out[lo:hi].copy_(torch.from_numpy(tmp))

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out.reshape(shape)


def _unit_rms_rows(h: torch.Tensor) -> torch.Tensor:
    """Input recipe of the bf16 single-layer workloads: each fp32 row divided by
    sqrt(mean(row^2) + 1e-5), in float64, then rounded to fp32."""
    h64 = h.double()
    return (h64 / torch.sqrt(h64.pow(2).mean(dim=1, keepdim=True) + RMS_EPS)).float()


@dataclass
class LayerInputs:
    """One MoE layer's inputs as CPU torch tensors.

    x  [T, d]      act dtype (fp32 or bf16)
    wg [d, n]      fp32 router matrix (no bias)
    w1 [n, F, d]   gate projection (gets SiLU), weight dtype
    w3 [n, F, d]   up projection (linear), weight dtype
    w2 [n, d, F]   down projection, weight dtype
    """
    x: torch.Tensor
    wg: torch.Tensor
    w1: torch.Tensor
    w3: torch.Tensor
    w2: torch.Tensor
    T: int
    d: int
    F: int
    n: int
    K: int
    dtype: str
    key: tuple = ()
    init: str = "mixtral"
    skew: bool = False
    redraws: int = 0
    meta: dict = field(default_factory=dict)

    def numpy_f32(self):
        """Exact fp32 copies (bf16 -> fp32 is exact) for the CPU oracle."""
        return (self.x.float().numpy(), self.wg.float().numpy(), self.w1.float().numpy(),
                self.w3.float().numpy(), self.w2.float().numpy())


def _draw_x(T, d, key, init, skew, tdtype):
    if init == "fanin":
        return _normal((T, d), key, 1.0, torch.float32)
    if init == "stack":
        return _normal((T, d), key, 1.0, tdtype)
    x = _unit_rms_rows(_normal((T, d), key, 1.0, torch.float32))
    if skew:
        x[:, 0] = 1.0
    return x.to(tdtype)


def make_layer(T: int, d: int, F: int, n: int = 8, K: int = 2, dtype: str = "bf16",
               init: str = "mixtral", skew: bool = False, seed: int = 0,
               workload: int = 100, layer: int = 0) -> LayerInputs:
    """Seeded inputs of one layer at an arbitrary shape.

    ``workload`` is only a stream id: the five named workloads use 0..4, ad-hoc
    test shapes use other ids so that their streams never coincide.
    """
    tdtype = torch.float32 if dtype == "f32" else torch.bfloat16
    base = (seed, workload, layer)
    x = _draw_x(T, d, base + (X_ID,), init, skew, tdtype)
    if init == "fanin":
        wg = _normal((d, n), base + (WG_ID,), 1.0 / math.sqrt(d), torch.float32)
        w1 = _normal((n, F, d), base + (W1_ID,), 1.0 / math.sqrt(d), tdtype)
        w3 = _normal((n, F, d), base + (W3_ID,), 1.0 / math.sqrt(d), tdtype)
        w2 = _normal((n, d, F), base + (W2_ID,), 1.0 / math.sqrt(F), tdtype)
    else:
        wg = _normal((d, n), base + (WG_ID,), 0.02, torch.float32)
        w1 = _normal((n, F, d), base + (W1_ID,), 0.02, tdtype)
        w3 = _normal((n, F, d), base + (W3_ID,), 0.02, tdtype)
        w2 = _normal((n, d, F), base + (W2_ID,), 0.02, tdtype)
    if skew:
        s = 0.02 * math.sqrt(d)
        wg[0, :] = 0.0
        wg[0, 0] = 1.5 * s
        wg[0, 1] = 1.5 * s
    return LayerInputs(x=x, wg=wg, w1=w1, w3=w3, w2=w2, T=T, d=d, F=F, n=n, K=K,
                       dtype=dtype, key=base, init=init, skew=skew)


def make_workload(i: int, seed: int = 0, layer: int = 0, T: Optional[int] = None) -> LayerInputs:
    """Inputs of named workload ``i`` (0..4).  For the 32-layer stack, ``layer``
    selects that layer's weights (host-drawn) and ``x`` is the stack input h0
    whatever ``layer`` is.  ``T`` may shrink the token count (the
    first ``T`` rows are then a prefix of the full draw only up to the chunking,
    so treat it as its own input)."""
    w = WORKLOADS[i]
    TT = w["T"] if T is None else T
    li = make_layer(TT, w["d"], w["F"], w["n"], w["K"], w["dtype"], w["init"], w["skew"],
                    seed=seed, workload=i, layer=layer)
    if w["init"] == "stack":
        li.x = stack_input(TT, w["d"], seed=seed, workload=i)
    li.meta["workload"] = w["name"]
    return li


def redraw_rows(inp: LayerInputs, rows: np.ndarray) -> LayerInputs:
    """Replace the given token rows of x with fresh draws of the same recipe,
    from a stream keyed by how many redraws came before.  Callers loop this
    until whatever row filter they apply passes."""
    rows = np.asarray(rows, dtype=np.int64)
    if rows.size == 0:
        return inp
    tdtype = inp.x.dtype
    key = inp.key + (REDRAW_ID, inp.redraws)
    fresh = _draw_x(rows.size, inp.d, key, inp.init, inp.skew, tdtype)
    x = inp.x.clone()
    x[torch.from_numpy(rows)] = fresh
    return replace(inp, x=x, redraws=inp.redraws + 1)


def stack_input(T: int, d: int, seed: int = 0, workload: int = 4) -> torch.Tensor:
    """h0 of the layer stack: N(0,1) rounded to bf16."""
    return _draw_x(T, d, (seed, workload, 0, H0_ID), "stack", False, torch.bfloat16)


def stack_layer_weights(layer: int, d: int, F: int, n: int = 8, seed: int = 0,
                        workload: int = 4, device: str = "cpu"):
    """Weights of one stack layer generated directly in device memory with
    torch's seeded generator on that device (the stack holds ~90 GB, too much to
    draw on the host).  Returns (wg fp32 [d,n], w1, w3 [n,F,d], w2 [n,d,F] bf16).
    The same (seed, layer, device type) always gives the same tensors; a host
    copy for checking is made by copying these tensors back."""
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence([seed, workload, layer]).generate_state(1)[0]))
    wg = torch.empty((d, n), dtype=torch.float32, device=device).normal_(0.0, 0.02, generator=g)
    out = []
    for shape in ((n, F, d), (n, F, d), (n, d, F)):
        t = torch.empty(shape, dtype=torch.bfloat16, device=device)
        # draw in fp32 slabs and round once, so that bf16 values are RNE of the fp32 draw
        flat = t.view(-1)
        step = 1 << 26
        for lo in range(0, flat.numel(), step):
            hi = min(flat.numel(), lo + step)
            flat[lo:hi].copy_(torch.empty(hi - lo, dtype=torch.float32, device=device)
                              .normal_(0.0, 0.02, generator=g))
        out.append(t)
    return (wg, *out)

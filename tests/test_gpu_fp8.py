"""FP8 (OCP E4M3) expert weights against the CPU oracle: the quantizer bit for
bit, the FP8 expert projections and the FP8 layer element by element at small
shapes, and the decode workload at full size."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
import sparse_moe_transformer_way_amd as moe
from moe_testutil import TOL_BF16, assert_routing_equal, margin_filtered, per_token_rel_err

pytestmark = pytest.mark.gpu

F8 = torch.float8_e4m3fn


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    yield
    torch.cuda.synchronize()


def _bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)


def _exact_rows(rows, cols, rng):
    """Rows with maximum 448 (scale exactly 1, so w / scale = w): every
    midpoint between neighbouring E4M3 values (ties), subnormal-range values
    and random bf16 values, with random signs."""
    vals = np.unique(oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8)))
    mids = (vals[:-1] + vals[1:]) / 2
    pool = np.concatenate([vals, mids, rng.uniform(0, 2.0 ** -6, 64), rng.uniform(0, 448, 256)])
    w = rng.choice(pool, size=(rows, cols)) * rng.choice([-1.0, 1.0], size=(rows, cols))
    w[:, 0] = 448.0
    return w


@pytest.mark.parametrize("rows,cols,kind", [(64, 512, "normal"), (200, 1024, "wide"), (96, 256, "exact"),
                                            (33, 4096, "normal"), (8, 14336, "wide"), (50, 64, "zero_rows")])
def test_quantize_fp8_bit_exact(rows, cols, kind):
    rng = np.random.default_rng(rows + cols)
    if kind == "normal":
        w = rng.standard_normal((rows, cols)) * 0.02
    elif kind == "wide":
        w = rng.standard_normal((rows, cols)) * 10.0 ** rng.uniform(-8, 3, (rows, 1))
    elif kind == "exact":
        w = _exact_rows(rows, cols, rng)
    else:
        w = rng.standard_normal((rows, cols))
        w[::3] = 0.0
    wb = _bf16(w)
    q, s = moe.moe_quantize_fp8(wb.cuda())
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_rows_fp8(wb.float().numpy())
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)


def _quantized(inp):
    """GPU-quantized weights (checked bit for bit against the oracle's) and the
    oracle's dequantized copies."""
    gpu, deq = [], []
    for w in (inp.w1, inp.w3, inp.w2):
        q, s = moe.moe_quantize_fp8(w.cuda())
        q_ref, s_ref = oracle.quantize_rows_fp8(w.float().numpy())
        np.testing.assert_array_equal(q.cpu().numpy(), q_ref)
        np.testing.assert_array_equal(s.cpu().numpy(), s_ref)
        gpu += [q, s]
        deq.append(oracle.dequantize_rows_fp8(q_ref, s_ref))
    return gpu, deq


@pytest.mark.parametrize("n,K,T,d,F", [(8, 2, 40, 1024, 1024), (8, 2, 1, 2048, 1024), (8, 2, 200, 1024, 2048),
                                       (4, 1, 64, 1024, 1024), (16, 4, 30, 1024, 1024)])
def test_expert_projections_fp8(n, K, T, d, F):
    inp = margin_filtered(mi.make_layer(T, d, F, n=n, K=K, seed=T + d, workload=500))
    (q1, s1, q3, s3, q2, s2), (w1d, w3d, w2d) = _quantized(inp)
    xn, wgn = inp.x.float().numpy(), inp.wg.numpy()
    grp = oracle.group_by_expert(oracle.gating(xn, wgn, K)[1], n, 16)
    h_ref, yp_ref = oracle.expert_rows(xn, grp["row_src"], grp["offsets"], w1d, w3d, w2d, K=K)
    desc = moe.make_desc(d, F, n, K, weight_dtype=F8)
    row_src, counts, offsets = (torch.from_numpy(grp[k]).cuda() for k in ("row_src", "counts", "offsets"))
    h = moe.moe_expert_gate_up_fp8(desc, T, inp.x.cuda(), row_src, counts, offsets, q1, s1, q3, s3)
    yp = moe.moe_expert_down_fp8(desc, T, h, counts, offsets, q2, s2)
    torch.cuda.synchronize()
    real = grp["row_src"] >= 0
    pad = ~real
    pad[grp["offsets"][n]:] = False
    hg = h.float().cpu().numpy()
    assert per_token_rel_err(hg[real], h_ref[real]).max() <= TOL_BF16
    assert (hg[pad] == 0).all()
    assert per_token_rel_err(yp.cpu().numpy()[real], yp_ref[real]).max() <= TOL_BF16


@pytest.mark.parametrize("n,K,T,d,F", [(8, 2, 32, 1024, 2048), (8, 2, 100, 2048, 1024), (8, 3, 16, 1024, 1024),
                                       (8, 2, 1, 1024, 1024)])
def test_layer_fp8(n, K, T, d, F):
    inp = margin_filtered(mi.make_layer(T, d, F, n=n, K=K, seed=T + F, workload=501))
    (q1, s1, q3, s3, q2, s2), (w1d, w3d, w2d) = _quantized(inp)
    xn, wgn = inp.x.float().numpy(), inp.wg.numpy()
    ref = oracle.moe_layer(xn, wgn, w1d, w3d, w2d, K=K)
    res = torch.randn(T, d).to(torch.bfloat16)
    desc = moe.make_desc(d, F, n, K, weight_dtype=F8)
    y, idx, gate, counts = moe.moe_layer_forward_fp8(desc, inp.x.cuda(), inp.wg.cuda(), q1, s1, q3, s3, q2, s2,
                                                     residual=res.cuda())
    torch.cuda.synchronize()
    assert_routing_equal(idx.cpu().numpy(), gate.cpu().numpy(), ref, xn, wgn)
    np.testing.assert_array_equal(counts.cpu().numpy(), ref["counts"])
    err = per_token_rel_err(y.float().cpu().numpy() - res.float().numpy(), ref["y"])
    # the bf16 rounding of y + residual adds up to half an ulp of |y + residual|
    slack = np.abs(y.float().cpu().numpy()).max(axis=1) * 2.0 ** -8 / np.abs(ref["y"]).max(axis=1)
    assert (err <= TOL_BF16 + slack).all(), f"max per-token rel err {err.max():.3e}"


def test_decode_workload_fp8_full_size():
    """The decode workload (T=32, d=4096, F=14336, 8 experts, top-2) with FP8
    weights, in the launch configuration the bench times: every code and scale
    against the oracle's quantizer, every token's routing and output against
    the oracle's dense layer on its own dequantized weights (one expert at a
    time, in expert order, as the dense formula sums)."""
    inp = margin_filtered(mi.make_workload(1))
    T, d, F, n = inp.T, inp.d, inp.F, inp.n
    xn, wgn = inp.x.float().numpy(), inp.wg.numpy()
    G, ridx, _ = oracle.gating(xn, wgn, 2)
    y_ref = np.zeros((T, d), np.float32)
    gpu = []
    for w in (inp.w1, inp.w3, inp.w2):
        q, s = moe.moe_quantize_fp8(w.cuda())
        gpu.append((q, s))
    qc = [(q.cpu().numpy(), s.cpu().numpy()) for q, s in gpu]
    for e in range(n):
        deq = []
        for (qg, sg), w in zip(qc, (inp.w1, inp.w3, inp.w2)):
            q_ref, s_ref = oracle.quantize_rows_fp8(w[e].float().numpy())
            np.testing.assert_array_equal(qg[e], q_ref)
            np.testing.assert_array_equal(sg[e], s_ref)
            deq.append(oracle.dequantize_rows_fp8(q_ref, s_ref))
        y_ref += G[:, e:e + 1] * oracle.swiglu_expert(xn, *deq)
    desc = moe.make_desc(d, F, n, 2, weight_dtype=F8)
    (q1, s1), (q3, s3), (q2, s2) = gpu
    y, idx, gate, counts = moe.moe_layer_forward_fp8(desc, inp.x.cuda(), inp.wg.cuda(), q1, s1, q3, s3, q2, s2)
    torch.cuda.synchronize()
    ref = dict(idx=ridx, gates=G[np.arange(T)[:, None], ridx], counts=np.bincount(ridx.ravel(), minlength=n))
    assert_routing_equal(idx.cpu().numpy(), gate.cpu().numpy(), ref, xn, wgn)
    err = per_token_rel_err(y.float().cpu().numpy(), y_ref)
    assert err.max() <= TOL_BF16, f"max per-token rel err {err.max():.3e}"

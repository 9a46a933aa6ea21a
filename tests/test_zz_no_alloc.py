"""moe_layer_forward_noalloc, the entry point for callers that cannot allocate
(graph capture, serving loops): its output equals moe_layer_forward's on the
same inputs, call after call, whatever the previous call left in the shared
per-GPU scratch."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import sparse_moe_transformer_way_amd as moe

pytestmark = pytest.mark.gpu

D, F = 4096, 14336


@pytest.fixture(scope="module")
def weights():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    wg, w1, w3, w2 = mi.stack_layer_weights(0, D, F, seed=11, workload=900, device="cuda")
    yield wg, w1, w3, w2
    torch.cuda.synchronize()


def both(desc, x, wg, w1, w3, w2, residual=None):
    ref = moe.moe_layer_forward(desc, x, wg, w1, w3, w2, residual=residual)
    got = moe.moe_layer_forward_noalloc(desc, x, wg, w1, w3, w2, residual=residual)
    torch.cuda.synchronize()
    return [t.cpu() for t in ref], [t.cpu() for t in got]


def assert_same(ref, got):
    # the same kernels on the same inputs: routing, gates, counts and y agree bit for bit
    for r, g in zip(ref, got):
        assert r.dtype == g.dtype and r.shape == g.shape
        assert torch.equal(r, g)


def test_noalloc_matches_layer_forward_twice(weights):
    wg, w1, w3, w2 = weights
    desc = moe.make_desc(D, F)
    # the largest decode batch the scratch holds at the Mixtral shape, then a smaller one
    assert moe.moe_workspace_size(desc, 64, 0) <= moe.MOE_NOALLOC_SCRATCH_BYTES
    for T, seed in ((64, 1), (5, 2)):
        gen = torch.Generator(device="cuda").manual_seed(seed)
        x = torch.randn((T, D), generator=gen, device="cuda").to(torch.bfloat16)
        ref, got = both(desc, x, wg, w1, w3, w2)
        assert_same(ref, got)
        assert ref[0].float().abs().max() > 0
        assert int(ref[3].sum()) == 2 * T


def test_noalloc_residual_small_shape():
    desc = moe.make_desc(512, 1024)
    inp = mi.make_layer(150, 512, 1024, seed=4, workload=901)  # tile-256 kernels, scratch under the limit
    assert 0 < moe.moe_workspace_size(desc, 150, 0) <= moe.MOE_NOALLOC_SCRATCH_BYTES
    x, wg, w1, w3, w2 = (t.cuda() for t in (inp.x, inp.wg, inp.w1, inp.w3, inp.w2))
    res = torch.randn(150, 512).to(torch.bfloat16).cuda()
    ref, got = both(desc, x, wg, w1, w3, w2, residual=res)
    assert_same(ref, got)


def test_noalloc_rejects_beyond_scratch(weights):
    wg, w1, w3, w2 = weights
    desc = moe.make_desc(D, F)
    assert moe.moe_workspace_size(desc, 65, 0) > moe.MOE_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((65, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError, match="WORKSPACE_TOO_SMALL"):
        moe.moe_layer_forward_noalloc(desc, x, wg, w1, w3, w2)

"""The allocation-free entry point (sparse_gemv_threshold_noalloc) against
sparse_gemv_threshold, through the C ABI: two calls in a row on the fixed
scratch, the second smaller, each equal to the workspace entry point's
output bit for bit and to the oracle within tolerance; a shape too large
for the scratch is refused before any launch."""

import numpy as np
import pytest
import torch

import sparse_input_gemv_amd as sa
import synthetic as syn
from oracle import gemv, sparsify

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _close(y, ref):
    y = y.detach().cpu().numpy().astype(np.float64)
    err = y - ref
    assert np.linalg.norm(err) / np.linalg.norm(ref) <= 2e-3
    assert np.max(np.abs(err)) <= 1e-2


def test_noalloc_matches_the_workspace_entry_point():
    cases = [(4096, 11008, 1, "laplace", 0.69873046875),   # the down projection
             (1024, 2048, 1, "gaussian", 0.6745)]         # then a smaller call
    for d_out, d_in, batch, dist, t in cases:
        wt = syn.weight_t(d_out, d_in, d_in + 3)
        x = syn.activation((d_in,), dist, d_out)
        wt_g, x_g = _dev(wt), _dev(x)
        y = torch.full((d_out,), float("nan"), dtype=torch.float16, device=DEV)
        sa.sparse_gemv_threshold_noalloc(wt_g, x_g, t, y)
        ref = sa.sparse_gemv_threshold(wt_g, x_g, t)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), (d_out, d_in)
        keep = sparsify.threshold_sparsify(x, t)[0]
        _close(y, gemv.masked_gemv(wt, x, keep))


def test_noalloc_batch_two_and_back():
    """Batch 2 (also one launch, in the same scratch), then batch 1 again:
    the hand-off counters left by each call are zero for the next."""
    d_out, d_in = 4096, 11008
    wt_g = _dev(syn.weight_t(d_out, d_in, 61))
    xb = _dev(syn.laplace_f16((2, d_in), 1.0, 62))
    yb = torch.empty((2, d_out), dtype=torch.float16, device=DEV)
    sa.sparse_gemv_threshold_noalloc(wt_g, xb, 0.69, yb)
    assert torch.equal(yb, sa.sparse_gemv_threshold(wt_g, xb, 0.69))
    ref1 = sa.sparse_gemv_threshold(wt_g, xb[1], 0.69)  # batch 1 sums in another order
    y1 = torch.empty((d_out,), dtype=torch.float16, device=DEV)
    for _ in range(3):
        sa.sparse_gemv_threshold_noalloc(wt_g, xb[1], 0.69, y1)
        assert torch.equal(y1, ref1)


def test_noalloc_refuses_oversized_shapes():
    wt_g = torch.empty((4096, 22016), dtype=torch.float16, device=DEV)
    x_g = torch.zeros((4096,), dtype=torch.float16, device=DEV)
    y = torch.empty((22016,), dtype=torch.float16, device=DEV)
    with pytest.raises(sa.SparseActError) as e:
        sa.sparse_gemv_threshold_noalloc(wt_g, x_g, 0.5, y)
    assert e.value.status == 2  # SA_ERR_UNSUPPORTED
    assert "scratch" in str(e.value)

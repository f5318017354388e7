"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Masks, indices, counts and calibrated thresholds must match bit for bit;
outputs must satisfy relative L2 error <= 2e-3 and max abs error <= 1e-2
against the oracle's fp64 result.  Inputs come from ``synthetic`` with the
shapes and distributions of the workloads (Llama-2-7B / Llama-3-8B layers).
"""

import numpy as np
import pytest
import torch

import sparse_input_gemv_amd as sa
import synthetic as syn
from oracle import calibrate, correct, gemv, rana, sparsify, swiglu

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REL_L2 = 2e-3
MAX_ABS = 1e-2


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    return t if isinstance(t, np.ndarray) else t.detach().cpu().numpy()


def words(t):
    return host(t).view(np.uint32)


def assert_close(y_gpu, ref):
    y = host(y_gpu).astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert y.shape == ref.shape
    err = y - ref
    nrm = np.linalg.norm(ref)
    rel = np.linalg.norm(err) / (nrm if nrm > 0 else 1.0)
    mx = float(np.max(np.abs(err))) if err.size else 0.0
    assert rel <= REL_L2 and mx <= MAX_ABS, f"rel_l2={rel:.3e} max_abs={mx:.3e}"


def check_lists(mask_g, idx_g, val_g, nnz_g, x, keep):
    """Bit-exact comparison of a sparsifier's outputs with the oracle mask."""
    x2 = np.atleast_2d(x)
    keep2 = np.atleast_2d(keep)
    nnz = host(nnz_g)
    idx = np.atleast_2d(host(idx_g))
    val = np.atleast_2d(host(val_g))
    if mask_g is not None:
        assert np.array_equal(np.atleast_2d(words(mask_g)), sparsify.pack_mask(keep2))
    for r in range(x2.shape[0]):
        ref_idx = np.flatnonzero(keep2[r])
        assert nnz[r] == len(ref_idx)
        assert np.array_equal(idx[r, :nnz[r]], ref_idx)
        assert np.array_equal(val[r, :nnz[r]].view(np.uint16), x2[r][ref_idx].view(np.uint16))


# ---------------------------------------------------------------------------
# threshold sparsifier + sparse GEMV: single 1024 x 1024 layer, seeds 0..9
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(10))
def test_single_layer_1024(seed):
    wt = syn.weight_t(1024, 1024, 1000)
    x = syn.gaussian_f16((1024,), 1.0, seed)
    t = float(calibrate.magnitude_threshold(x, 0.5))  # 50th percentile of |x|
    keep, idx, val, nnz = sparsify.threshold_sparsify(x, t)
    y_ref = gemv.sparse_gemv(wt, idx, val)

    wt_g, x_g = dev(wt), dev(x)
    m_g, i_g, v_g, n_g = sa.act_sparsify_threshold(x_g, t)
    check_lists(m_g, i_g, v_g, n_g, x, keep)
    assert_close(sa.sparse_gemv(wt_g, i_g, v_g, n_g), y_ref)
    assert_close(sa.sparse_gemv_threshold(wt_g, x_g, t), y_ref)
    assert_close(sa.masked_gemv(wt_g, x_g, m_g), y_ref)
    # the GPU calibration of the same percentile gives the same fp32 threshold
    assert float(host(sa.act_calibrate_threshold(x_g, 0.5))[0]) == t


# rows up to 4096 run 512 threads of 8 entries, longer ones 1024 threads of 16
@pytest.mark.parametrize("d", [1, 31, 32, 33, 100, 1000, 4095, 4096, 4097, 11008, 14336, 16385,
                               40000])
def test_threshold_ragged_and_edges(d):
    rng = np.random.default_rng(d)
    X = syn.laplace_f16((3, d), 1.0, d)
    X[0, ::7] = 0
    X[1, ::5] = np.float16(-0.0)
    t = float(np.float32(0.6931))
    X[2, ::3] = np.float16(t)  # ties at t are kept (>=)
    for tt in (t, 0.0, 1e4):
        keep = sparsify.threshold_sparsify(X, tt)[0]
        check_lists(*sa.act_sparsify_threshold(dev(X), tt), X, keep)
    # a row start that is not 16-byte aligned takes the scalar path
    big = np.concatenate([np.zeros(1, np.float16), X.reshape(-1)])
    xg = dev(big)[1:].view(3, d)
    keep = sparsify.threshold_sparsify(X, t)[0]
    check_lists(*sa.act_sparsify_threshold(xg, t), X, keep)
    assert rng is not None


# ---------------------------------------------------------------------------
# Llama-2-7B decoder layer at batch 1: fused threshold + GEMV per projection
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["q", "o", "gate", "down"])
@pytest.mark.parametrize("sparsity", [0.4, 0.5, 0.6])
def test_llama2_layer_projection(name, sparsity):
    d_out, d_in, inp = syn.LLAMA2_7B[name]
    _, dist = syn.LLAMA2_7B_INPUTS[inp]
    wt = syn.weight_t(d_out, d_in, syn.weight_seed(name))
    x = syn.activation((d_in,), dist, 0)
    samples = syn.calibration_samples(inp)
    t = float(calibrate.magnitude_threshold(samples, sparsity))
    keep, idx, val, nnz = sparsify.threshold_sparsify(x, t)
    y_ref = gemv.sparse_gemv(wt, idx, val)

    wt_g, x_g = dev(wt), dev(x)
    t_g = float(host(sa.act_calibrate_threshold(dev(samples), sparsity))[0])
    assert t_g == t
    assert_close(sa.sparse_gemv_threshold(wt_g, x_g, t), y_ref)
    m_g, i_g, v_g, n_g = sa.act_sparsify_threshold(x_g, t)
    check_lists(m_g, i_g, v_g, n_g, x, keep)
    assert_close(sa.sparse_gemv(wt_g, i_g, v_g, n_g), y_ref)


@pytest.mark.parametrize("name", ["qkv", "gateup"])
@pytest.mark.parametrize("sparsity", [0.5, 0.6])
def test_fused_projection(name, sparsity):
    """One sparsified block input through the members' weights side by side
    (q|k|v 4096 -> 12288, gate|up 4096 -> 22016) in one call: the oracle's
    result, and each member's block within tolerance of its own call."""
    members, inp = syn.LLAMA2_7B_FUSED[name]
    _, dist = syn.LLAMA2_7B_INPUTS[inp]
    wt = syn.fused_weight_t(name)
    x = syn.activation((wt.shape[0],), dist, 1)
    t = float(calibrate.magnitude_threshold(syn.calibration_samples(inp), sparsity))
    keep, idx, val, nnz = sparsify.threshold_sparsify(x, t)
    y_ref = gemv.sparse_gemv(wt, idx, val)
    wt_g, x_g = dev(wt), dev(x)
    y = sa.sparse_gemv_threshold(wt_g, x_g, t)
    assert_close(y, y_ref)
    m_g, i_g, v_g, n_g = sa.act_sparsify_threshold(x_g, t)
    assert_close(sa.sparse_gemv(wt_g, i_g, v_g, n_g), y_ref)
    o = 0
    for m in members:
        d_out = syn.LLAMA2_7B[m][0]
        part = sa.sparse_gemv_threshold(wt_g[:, o:o + d_out].contiguous(), x_g, t)
        assert_close(y[o:o + d_out], y_ref[o:o + d_out])
        assert_close(part, y_ref[o:o + d_out])
        o += d_out


def test_dense_gemv_matches_oracle():
    for (d_out, d_in) in [(4096, 11008), (11008, 4096), (1024, 1024), (72, 130)]:
        wt = syn.weight_t(d_out, d_in, 5)
        x = syn.gaussian_f16((2, d_in), 1.0, 6)
        y = sa.dense_gemv(dev(wt), dev(x))
        assert_close(y, np.stack([gemv.dense_gemv(wt, x[b]) for b in range(2)]))


@pytest.mark.parametrize("d_out,d_in", [(11008, 4096), (22016, 4096), (11008, 2048),
                                         (1032, 3000)])
def test_padded_tile_plans(d_out, d_in):
    """Batch 1 with a tile count that is not a multiple of 8: the grid pads
    it (padding workgroups exit at once) and keeps the partials in L2.  The
    result matches the oracle and the written-through form bit for bit."""
    plan = sa.gemv_plan("threshold", d_out, d_in, 1)
    assert plan["handoff"] == 3 and plan["grid_o"] % 8 != 0
    wt = syn.weight_t(d_out, d_in, d_out + d_in)
    x = syn.laplace_f16((d_in,), 1.0, 3)
    t = 0.7
    keep = sparsify.threshold_sparsify(x, t)[0]
    wt_g, x_g = dev(wt), dev(x)
    y_t = sa.sparse_gemv_threshold(wt_g, x_g, t)
    y_d = sa.dense_gemv(wt_g, x_g)
    assert_close(y_t, gemv.masked_gemv(wt, x, keep))
    assert_close(y_d, gemv.dense_gemv(wt, x))
    try:
        sa.set_gemv_tuning(-1, 0, 2)
        assert torch.equal(sa.sparse_gemv_threshold(wt_g, x_g, t), y_t)
        assert torch.equal(sa.dense_gemv(wt_g, x_g), y_d)
    finally:
        sa.set_gemv_tuning(-1, 0, 0)


def test_threshold_zero_reproduces_dense():
    wt = syn.weight_t(4096, 4096, 7)
    x = syn.gaussian_f16((4096,), 1.0, 8)
    x[::11] = 0
    y_sparse = sa.sparse_gemv_threshold(dev(wt), dev(x), 0.0)
    ref = gemv.dense_gemv(wt, x)
    assert_close(y_sparse, ref)
    # the dense kernel also multiplies the zero entries, so its rows are split
    # differently across lanes: same result up to fp32 summation order
    assert_close(sa.dense_gemv(dev(wt), dev(x)), ref)


def test_empty_and_full_lists():
    wt = syn.weight_t(512, 300, 9)
    x = syn.gaussian_f16((300,), 1.0, 10)
    wt_g, x_g = dev(wt), dev(x)
    y = sa.sparse_gemv_threshold(wt_g, x_g, 1e4)  # nothing survives
    assert torch.count_nonzero(y).item() == 0
    m, i, v, n = sa.act_sparsify_threshold(x_g, 1e4)
    assert host(n)[0] == 0
    assert torch.count_nonzero(sa.sparse_gemv(wt_g, i, v, n)).item() == 0
    m, i, v, n = sa.act_sparsify_topk(x_g, 300)  # everything survives
    assert_close(sa.sparse_gemv(wt_g, i, v, n), gemv.dense_gemv(wt, x))


def test_ragged_output_tiles():
    """d_out not a multiple of any tile width, d_in spanning a ragged slice."""
    for d_out, d_in in [(8, 5), (136, 777), (1032, 3000), (4104, 11009)]:
        wt = syn.weight_t(d_out, d_in, 11)
        x = syn.laplace_f16((3, d_in), 1.0, 12)
        t = 0.69
        keep = sparsify.threshold_sparsify(x, t)[0]
        ref = gemv.batched_masked_gemv(wt, x, keep)
        assert_close(sa.sparse_gemv_threshold(dev(wt), dev(x), t), ref)


@pytest.mark.parametrize("d_out,d_in", [(1024, 4096), (512, 4096), (264, 4096), (2048, 2048),
                                         (4096, 1024), (1000, 1000), (4096, 512), (200, 3000)])
@pytest.mark.parametrize("batch", [1, 2])
def test_small_weight_shapes(d_out, d_in, batch):
    """Weights up to 8 MB, where the automatic choice picks full-K (wide,
    short-K shapes) or one-workgroup-per-CU split-K with narrow tiles."""
    wt = syn.weight_t(d_out, d_in, 13)
    x = syn.gaussian_f16((batch, d_in), 1.0, 14)
    t = 0.6745
    keep = sparsify.threshold_sparsify(x, t)[0]
    wt_g, x_g = dev(wt), dev(x)
    assert_close(sa.sparse_gemv_threshold(wt_g, x_g, t), gemv.batched_masked_gemv(wt, x, keep))
    assert_close(sa.dense_gemv(wt_g, x_g), np.stack([gemv.dense_gemv(wt, x[b]) for b in range(batch)]))
    m_g = sa.act_sparsify_threshold(x_g, t)[0]
    assert_close(sa.masked_gemv(wt_g, x_g, m_g), gemv.batched_masked_gemv(wt, x, keep))
    if batch == 1:
        _, i_g, v_g, n_g = sa.act_sparsify_threshold(x_g[0], t)
        assert_close(sa.sparse_gemv(wt_g, i_g, v_g, n_g), gemv.batched_masked_gemv(wt, x, keep)[0])


def test_deterministic_and_stream():
    d_out, d_in, _ = syn.LLAMA2_7B["down"]
    wt = dev(syn.weight_t(d_out, d_in, 13))
    x = dev(syn.laplace_f16((d_in,), 1.0, 14))
    y1 = sa.sparse_gemv_threshold(wt, x, 0.69)
    # calls sharing the per-device workspace must be ordered: the side stream
    # waits for the default one, and vice versa afterwards
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        y2 = sa.sparse_gemv_threshold(wt, x, 0.69)
        m, i, v, n = sa.act_sparsify_threshold(x, 0.69)
        y3 = sa.sparse_gemv(wt, i, v, n)
    torch.cuda.current_stream().wait_stream(s)
    s.synchronize()
    assert torch.equal(y1, y2)
    m2, i2, v2, n2 = sa.act_sparsify_threshold(x, 0.69)
    torch.cuda.synchronize()
    assert torch.equal(m, m2) and torch.equal(n, n2)
    nn = int(host(n)[0])
    assert torch.equal(i[:nn], i2[:nn])
    assert_close(y3, host(y1).astype(np.float64))


@pytest.mark.parametrize("tiling", range(11))
def test_every_tiling_headline(tiling):
    d_out, d_in, _ = syn.LLAMA2_7B["down"]
    wt = syn.weight_t(d_out, d_in, syn.weight_seed("down"))
    x = syn.laplace_f16((d_in,), 1.0, 3)
    t = 0.69
    keep, idx, val, nnz = sparsify.threshold_sparsify(x, t)
    ref = gemv.sparse_gemv(wt, idx, val)
    wt_g, x_g = dev(wt), dev(x)
    try:
        for target in (0, 256, 4096):
            sa.set_gemv_tuning(tiling, target, 0)
            assert_close(sa.sparse_gemv_threshold(wt_g, x_g, t), ref)
            m, i, v, n = sa.act_sparsify_threshold(x_g, t)
            assert_close(sa.sparse_gemv(wt_g, i, v, n), ref)
            assert_close(sa.dense_gemv(wt_g, x_g), gemv.dense_gemv(wt, x))
    finally:
        sa.set_gemv_tuning(-1, 0, 0)


# ---------------------------------------------------------------------------
# Top-K (Q-Sparse) + batched union GEMV
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d", [4096, 11008])
@pytest.mark.parametrize("pct", [60, 50, 40])
@pytest.mark.parametrize("batch", [1, 2, 4, 8])
def test_topk_and_union_gemv(d, pct, batch):
    k = syn.topk_k(pct, d)
    X = syn.laplace_f16((batch, d), 1.0, 100 + batch)
    keep, idx, val, nnz = sparsify.topk_sparsify(X, k)
    d_out = 11008 if d == 4096 else 4096
    wt = syn.weight_t(d_out, d, 20 + d)
    ref = gemv.batched_masked_gemv(wt, X, keep)

    X_g, wt_g = dev(X), dev(wt)
    m_g, i_g, v_g, n_g = sa.act_sparsify_topk(X_g, k)
    check_lists(m_g, i_g, v_g, n_g, X, keep)
    assert np.all(host(n_g) == k)
    assert_close(sa.sparse_gemv(wt_g, i_g, v_g, n_g), ref)
    assert_close(sa.masked_gemv(wt_g, X_g, m_g), ref)


# rows up to 4096 take the two-pass radix select (512 threads of 8
# entries), longer ones the 2^15-bin select
@pytest.mark.parametrize("d", [1, 5, 33, 64, 100, 1000, 4095, 4096, 4097, 16384, 16385, 30000])
def test_topk_edges_and_ties(d):
    rng = np.random.default_rng(d)
    pool = np.array([0.0, -0.0, 0.5, -0.5, 1.0, -1.0, 2.0, 0.25], dtype=np.float16)
    X = np.stack([pool[rng.integers(0, len(pool), size=d)], syn.laplace_f16((d,), 1.0, d)])
    for k in sorted({0, 1, d // 3, d // 2, d - 1, d} - {-1}):
        if k < 0:
            continue
        keep = sparsify.topk_sparsify(X, k)[0]
        check_lists(*sa.act_sparsify_topk(dev(X), k), X, keep)


def oracle_cutoff(x, keep):
    """The (tau, i*) pair an oracle Top-K mask implies: tau the smallest kept
    magnitude key (fp16 bits without the sign), i* the last kept index with
    that key; (32768, -1) when nothing is kept."""
    key = np.atleast_2d(x).view(np.uint16).astype(np.int64) & 0x7FFF
    out = []
    for r in range(key.shape[0]):
        kept = np.flatnonzero(np.atleast_2d(keep)[r])
        if kept.size == 0:
            out.append((32768, -1))
            continue
        tau = int(key[r, kept].min())
        out.append((tau, int(kept[key[r, kept] == tau].max())))
    return np.array(out, dtype=np.int32)


@pytest.mark.parametrize("d", [1, 5, 33, 64, 100, 1000, 4095, 4096, 4097, 11008, 16384, 16385,
                               30000, 65536])
def test_topk_cutoff_bit_exact(d):
    rng = np.random.default_rng(d + 7)
    pool = np.array([0.0, -0.0, 0.5, -0.5, 1.0, -1.0, 2.0, 0.25], dtype=np.float16)
    X = np.stack([pool[rng.integers(0, len(pool), size=d)], syn.laplace_f16((d,), 1.0, d),
                  np.zeros(d, np.float16)])
    for k in sorted({0, 1, d // 3, d // 2, d - 1, d} - {-1}):
        keep = sparsify.topk_sparsify(X, k)[0]
        cut = host(sa.act_topk_cutoff(dev(X), k))
        assert np.array_equal(cut, oracle_cutoff(X, keep)), (d, k)
        # the pair reproduces the mask it came from
        key = X.view(np.uint16).astype(np.int64) & 0x7FFF
        i = np.arange(d)[None, :]
        rule = (key > cut[:, :1]) | ((key == cut[:, :1]) & (i <= cut[:, 1:]))
        assert np.array_equal(rule, keep)


@pytest.mark.parametrize("d", [4096, 11008])
@pytest.mark.parametrize("pct", [60, 50, 40])
@pytest.mark.parametrize("batch", [1, 2, 4, 8])
def test_sparse_gemv_topk(d, pct, batch):
    k = syn.topk_k(pct, d)
    X = syn.laplace_f16((batch, d), 1.0, 300 + batch)
    keep = sparsify.topk_sparsify(X, k)[0]
    d_out = 11008 if d == 4096 else 4096
    wt = syn.weight_t(d_out, d, 40 + d)
    y = sa.sparse_gemv_topk(dev(wt), dev(X), k)
    assert_close(y, gemv.batched_masked_gemv(wt, X, keep))


@pytest.mark.parametrize("d_out,d_in,batch", [(8, 1, 1), (104, 300, 3), (1024, 1024, 1),
                                              (4096, 1000, 2), (336, 5000, 8)])
def test_sparse_gemv_topk_edges(d_out, d_in, batch):
    rng = np.random.default_rng(d_in)
    pool = np.array([0.0, -0.0, 0.5, -0.5, 1.0, -1.0], dtype=np.float16)
    X = pool[rng.integers(0, len(pool), size=(batch, d_in))]  # heavy ties
    wt = syn.weight_t(d_out, d_in, 5)
    wt_g, X_g = dev(wt), dev(X)
    for k in sorted({0, 1, d_in // 2, d_in}):
        keep = sparsify.topk_sparsify(X, k)[0]
        y = sa.sparse_gemv_topk(wt_g, X_g, k)
        assert_close(y, gemv.batched_masked_gemv(wt, X, keep))
        if k == 0:
            assert not np.any(host(y).view(np.uint16) & 0x7FFF)


@pytest.mark.parametrize("d_out,d_in,batch", [(11008, 4096, 1), (4096, 4096, 1), (4096, 1024, 1),
                                              (1024, 1024, 1), (8, 1, 1), (520, 4095, 1),
                                              (264, 2055, 1), (4096, 4097, 1), (4096, 11008, 1),
                                              (1032, 12288, 1), (264, 12289, 1), (1024, 1000, 2)])
def test_sparse_gemv_topk_one_launch_matches_two(d_out, d_in, batch):
    """Where every GEMV workgroup selects the cutoff itself (batch 1, the
    row fits a workgroup), the output equals the two-launch form's (the
    select kernel, then the GEMV) bit for bit wherever both run the same
    GEMV plan, on Laplace rows and on rows of heavy ties, for k from 0 to
    d_in; both equal the oracle everywhere."""
    rng = np.random.default_rng(d_in + batch)
    pool = np.array([0.0, -0.0, 0.25, -0.25, 0.5, -0.5, 1.0, -1.0], dtype=np.float16)
    wt = syn.weight_t(d_out, d_in, 6)
    wt_g = dev(wt)
    for X in (syn.laplace_f16((batch, d_in), 1.0, 500 + d_in),
              pool[rng.integers(0, len(pool), size=(batch, d_in))]):
        X_g = dev(X)
        for k in sorted({min(k, d_in) for k in (0, 1, 2, d_in // 3, d_in // 2, d_in - 1, d_in)}):
            y1 = sa.sparse_gemv_topk(wt_g, X_g, k).clone()
            p1 = sa.gemv_plan("topk", d_out, d_in, batch)
            try:
                sa.set_gemv_test_hooks(2)
                y2 = sa.sparse_gemv_topk(wt_g, X_g, k)
                p2 = sa.gemv_plan("topk", d_out, d_in, batch)
            finally:
                sa.set_gemv_test_hooks(0)
            if p1 == p2:
                assert torch.equal(y1, y2), (k,)
            keep = sparsify.topk_sparsify(X, k)[0]
            ref = gemv.batched_masked_gemv(wt, X, keep)
            assert_close(y1, ref)
            assert_close(y2, ref)


# ---------------------------------------------------------------------------
# calibration
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("inp", ["attn_in", "o_in", "mlp_in", "down_in"])
def test_calibration_bit_exact(inp):
    smp = syn.calibration_samples(inp)
    g = dev(smp)
    for s in (0.0, 0.1, 0.4, 0.5, 0.6, 0.7, 0.99, 1.0):
        t_ref = calibrate.magnitude_threshold(smp, s)
        t_gpu = host(sa.act_calibrate_threshold(g, s))[0]
        assert np.float32(t_gpu).view(np.uint32) == np.float32(t_ref).view(np.uint32), (s,)


def test_calibration_small_n():
    # up to 16384 samples are held in registers; more are read in every pass
    for n in (1, 2, 3, 7, 1025, 16383, 16384, 16385, 40000):
        smp = syn.laplace_f16((n,), 1.0, n)
        for s in (0.0, 0.3, 0.5, 1.0):
            t_ref = calibrate.magnitude_threshold(smp, s)
            assert host(sa.act_calibrate_threshold(dev(smp), s))[0] == t_ref


# ---------------------------------------------------------------------------
# N:M sparsifier
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (8, 16), (16, 32), (1, 4), (3, 4), (8, 8),
                                 (5, 16), (31, 32), (32, 32)])
def test_nm_small(n, m):
    X = syn.gaussian_f16((64, 1024), 1.0, n * 100 + m)
    X[3, :] = np.float16(0.5)  # all ties
    X[4, ::2] = np.float16(-0.0)
    keep, vals = sparsify.nm_sparsify(X, n, m)
    mask_g, val_g = sa.act_sparsify_nm(dev(X), n, m)
    assert np.array_equal(words(mask_g), sparsify.pack_mask(keep))
    assert np.array_equal(host(val_g).view(np.uint16), vals.view(np.uint16))


@pytest.mark.parametrize("n,m", [(8, 16), (16, 32), (1, 32), (31, 32), (5, 16)])
@pytest.mark.parametrize("T,d", [(1, 32), (3, 96), (5, 160), (7, 2080), (33, 544)])
def test_nm_ragged_group_counts(n, m, T, d):
    """Group counts that leave a workgroup's last pair of groups half empty
    (an odd number of 32-groups) or a short last block."""
    X = syn.gaussian_f16((T, d), 1.0, T * d + m)
    keep, vals = sparsify.nm_sparsify(X, n, m)
    mask_g, val_g = sa.act_sparsify_nm(dev(X), n, m)
    assert np.array_equal(np.atleast_2d(words(mask_g)), sparsify.pack_mask(keep))
    assert np.array_equal(np.atleast_2d(host(val_g)).view(np.uint16), vals.view(np.uint16))


@pytest.mark.parametrize("n,m", [(8, 16), (5, 16), (16, 32), (3, 32)])
def test_nm_multi_block(n, m):
    """8192 x 4096: more blocks of groups than the grid has workgroups, so
    each workgroup walks several blocks with its two register sets taking
    turns.  Rows sampled across the whole array are checked against the
    oracle (every row's groups are independent)."""
    T, d = 8192, 4096
    X = syn.gaussian_f16((T, d), 1.0, 77 + m)
    X[5000, :] = np.float16(1.0)  # a row of ties
    mask_g, val_g = sa.act_sparsify_nm(dev(X), n, m)
    rows = np.unique(np.concatenate([np.arange(0, T, 97), [T - 1, 5000]]))
    keep, vals = sparsify.nm_sparsify(X[rows], n, m)
    assert np.array_equal(words(mask_g)[rows], sparsify.pack_mask(keep))
    assert np.array_equal(host(val_g)[rows].view(np.uint16), vals.view(np.uint16))


@pytest.mark.parametrize("n,m", [(1, 16), (3, 16), (8, 16), (15, 16), (1, 32), (7, 32),
                                 (16, 32), (31, 32), (2, 8), (3, 4)])
def test_nm_heavy_ties(n, m):
    """Few distinct magnitudes, both signs of zero and infinities: the
    cutoff among equal magnitudes (lower index first) decides most groups,
    across the lanes that share a group."""
    rng = np.random.default_rng(n * 1000 + m)
    choices = np.array([0.0, -0.0, 0.5, -0.5, 1.0, -1.0, np.inf, -np.inf], dtype=np.float16)
    X = choices[rng.integers(0, 8, size=(96, 1024))]
    X[5, :] = np.float16(-0.0)
    X[6, :] = np.float16(2.0)
    keep, vals = sparsify.nm_sparsify(X, n, m)
    mask_g, val_g = sa.act_sparsify_nm(dev(X), n, m)
    assert np.array_equal(words(mask_g), sparsify.pack_mask(keep))
    assert np.array_equal(host(val_g).view(np.uint16), vals.view(np.uint16))


@pytest.mark.parametrize("shape", [(4096, 1024), (2048, 4096)])
@pytest.mark.parametrize("n,m", [(2, 4), (8, 16), (16, 32)])
def test_nm_full_shapes(shape, n, m):
    X = syn.gaussian_f16(shape, 1.0, 7)
    keep, vals = sparsify.nm_sparsify(X, n, m)
    mask_g, val_g = sa.act_sparsify_nm(dev(X), n, m)
    w = words(mask_g)
    assert np.array_equal(w, sparsify.pack_mask(keep))
    assert np.array_equal(host(val_g).view(np.uint16), vals.view(np.uint16))


# ---------------------------------------------------------------------------
# masked SwiGLU down projection (CATS / RaNA), Llama-3-8B MLP shape
# ---------------------------------------------------------------------------

def test_col_norms():
    wdt = syn.weight_t(4096, 14336, 30)
    ref = swiglu.column_norms(wdt)
    got = host(sa.weight_col_norms(dev(wdt)))
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=0)


@pytest.mark.parametrize("mode", ["cats", "rana"])
@pytest.mark.parametrize("rate", [0.5, 0.7])
def test_masked_swiglu_down(mode, rate):
    d_model, d_ff = syn.LLAMA3_8B_MLP["d_model"], syn.LLAMA3_8B_MLP["d_ff"]
    g, u = syn.swiglu_gate_up(d_ff, d_model, 0)
    wdt = syn.weight_t(d_model, d_ff, 31)
    cn = swiglu.column_norms(wdt)
    sc = swiglu.scores(g, u, mode, cn)
    t = swiglu.threshold_for_mask_rate(sc, rate)
    keep, y_ref = swiglu.masked_swiglu_down(g, u, wdt, t, mode, cn)

    wdt_g = dev(wdt)
    cn_g = sa.weight_col_norms(wdt_g) if mode == "rana" else None
    y, mask, nnz = sa.masked_swiglu_down(dev(g), dev(u), wdt_g, t, mode, cn_g)
    got = sparsify.unpack_mask(words(mask), d_ff)
    # the decision is taken in fp64 on both sides; entries whose score lies
    # within 1e-12 of t could differ by the last ulp of exp -- none expected
    ambiguous = np.abs(sc - t) <= 1e-12 * t
    assert ambiguous.sum() == 0
    assert np.array_equal(got, keep)
    assert host(nnz)[0] == keep.sum()
    assert abs(1 - keep.mean() - rate) < 0.01
    assert_close(y, y_ref)


@pytest.mark.parametrize("d_model,d_ff", [(1024, 4096), (4096, 1024), (512, 3000), (264, 14336),
                                           (2048, 2048), (4096, 6000)])
@pytest.mark.parametrize("mode", ["cats", "rana"])
def test_masked_swiglu_shapes(d_model, d_ff, mode):
    """Full-K, one-pass split-K (slices of whole 64-entry words, a ragged
    last one) and small-weight plans of the masked SwiGLU down projection;
    the mask is bit-exact, kept count and output as the oracle."""
    g, u = syn.swiglu_gate_up(d_ff, d_model, 5)
    wdt = syn.weight_t(d_model, d_ff, 33)
    cn = swiglu.column_norms(wdt)
    sc = swiglu.scores(g, u, mode, cn)
    t = swiglu.threshold_for_mask_rate(sc, 0.6)
    keep, y_ref = swiglu.masked_swiglu_down(g, u, wdt, t, mode, cn)
    wdt_g = dev(wdt)
    cn_g = sa.weight_col_norms(wdt_g) if mode == "rana" else None
    y, mask, nnz = sa.masked_swiglu_down(dev(g), dev(u), wdt_g, t, mode, cn_g)
    assert (np.abs(sc - t) <= 1e-12 * t).sum() == 0
    assert np.array_equal(sparsify.unpack_mask(words(mask), d_ff), keep)
    assert host(nnz)[0] == keep.sum()
    assert_close(y, y_ref)


def test_masked_swiglu_t0_dense():
    g, u = syn.swiglu_gate_up(1000, 256, 3)
    wdt = syn.weight_t(256, 1000, 32)
    keep, y_ref = swiglu.masked_swiglu_down(g, u, wdt, 0.0, "cats")
    y, mask, nnz = sa.masked_swiglu_down(dev(g), dev(u), dev(wdt), 0.0, "cats")
    assert host(nnz)[0] == 1000
    assert_close(y, y_ref)


@pytest.mark.parametrize("handoff,skew", [(1, 0), (2, 0), (3, 0), (3, 1)])
def test_split_k_handoff_is_deterministic(handoff, skew):
    """Many back-to-back split-K calls on rotating weights: every result must
    equal the first one bit for bit (the cross-workgroup hand-off is exact),
    also when the L2 form's placement check is made to fail (the last
    workgroup of each tile then recomputes the other slices)."""
    d_out, d_in, _ = syn.LLAMA2_7B["down"]
    wt0 = syn.weight_t(d_out, d_in, 15)
    x = dev(syn.laplace_f16((d_in,), 1.0, 16))
    wts = [dev(wt0), dev(np.ascontiguousarray(wt0[::-1]))]
    try:
        sa.set_gemv_test_hooks(skew)
        for tiling, target in [(-1, 0), (0, 4096), (6, 1024), (2, 2048), (8, 0), (10, 0)]:
            sa.set_gemv_tuning(tiling, target, handoff)
            ref = [sa.sparse_gemv_threshold(w, x, 0.69).clone() for w in wts]
            outs = [sa.sparse_gemv_threshold(wts[i % 2], x, 0.69) for i in range(200)]
            torch.cuda.synchronize()
            for i, y in enumerate(outs):
                assert torch.equal(y, ref[i % 2]), (tiling, target, i)
    finally:
        sa.set_gemv_test_hooks(0)
        sa.set_gemv_tuning(-1, 0, 0)


def _every_gemv_entry(wt, x1, xb, lists1, listsb, swiglu_in, t):
    """One output of every split-K entry point (batch 1 and batched)."""
    mb, ib, vb, nb = listsb
    _, i1, v1, n1 = lists1
    g, u, wdt, cn = swiglu_in
    outs = [sa.sparse_gemv_threshold(wt, x1, t), sa.sparse_gemv_threshold(wt, xb, t),
            sa.dense_gemv(wt, x1), sa.dense_gemv(wt, xb), sa.masked_gemv(wt, xb, mb),
            sa.sparse_gemv(wt, i1, v1, n1), sa.sparse_gemv(wt, ib, vb, nb)]
    for mode, c in (("cats", None), ("rana", cn)):
        y, m, n = sa.masked_swiglu_down(g, u, wdt, 0.02 if mode == "cats" else 0.01, mode, c)
        outs += [y, m, n]
    return outs


@pytest.mark.parametrize("tiling", [-1, 0, 1, 2, 3, 4, 5, 6, 7])
def test_one_launch_handoff_matches_two_launches(tiling):
    """The in-launch hand-off (last workgroup per output tile sums the
    partials) must give the same bits as the second-launch reduction, for
    every entry point, batch, ragged output tile and change of size between
    calls (its counters must come back to zero)."""
    shapes = [(4096, 11008, 5), (1032, 3000, 512), (136, 700, 64), (4096, 11008, 2048)]
    data = []
    for d_out, d_in, target in shapes:
        wt = dev(syn.weight_t(d_out, d_in, d_in + 7))
        x1 = dev(syn.laplace_f16((d_in,), 1.0, d_out))
        xb = dev(syn.laplace_f16((4, d_in), 1.0, d_out + 1))
        g, u = syn.swiglu_gate_up(d_in, d_out, 5)
        wdt = wt
        swiglu_in = (dev(g), dev(u), wdt, sa.weight_col_norms(wdt))
        data.append((target, wt, x1, xb, sa.act_sparsify_threshold(x1, 0.7),
                     sa.act_sparsify_threshold(xb, 0.7), swiglu_in))
    try:
        res = {}
        for handoff, skew in ((1, 0), (2, 0), (3, 0), (3, 1)):
            sa.set_gemv_test_hooks(skew)
            for k, (target, wt, x1, xb, l1, lb, sw) in enumerate(data):
                sa.set_gemv_tuning(tiling, target, handoff)
                res[(handoff, skew), k] = [o.clone() for o in _every_gemv_entry(
                    wt, x1, xb, l1, lb, sw, 0.7)]
        torch.cuda.synchronize()
        for k in range(len(data)):
            for h in ((2, 0), (3, 0), (3, 1)):
                for j, (a, b) in enumerate(zip(res[(1, 0), k], res[h, k])):
                    assert torch.equal(a, b), (tiling, shapes[k], h, j)
    finally:
        sa.set_gemv_test_hooks(0)
        sa.set_gemv_tuning(-1, 0, 0)


# ---------------------------------------------------------------------------
# weight-aware selection, static shift (S-PTS), variance correction (VAR)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("nm", [(0, 0), (2, 4), (4, 8), (8, 16), (16, 32)])
@pytest.mark.parametrize("d,rows", [(64, 1), (1024, 3), (4096, 2), (11008, 1), (40000, 2)])
@pytest.mark.parametrize("shifted,weighted", [(False, False), (True, False), (True, True)])
def test_scored_sparsify(d, rows, nm, shifted, weighted):
    n, m = nm
    X = syn.laplace_f16((rows, d), 1.0, d + rows + m)
    X[0, ::11] = np.float16(0.5)  # ties
    mu = syn.gaussian_f16((d,), 0.25, d) if shifted else None
    cn = correct.column_norms(syn.weight_t(16, d, 3)) if weighted else None
    t = 0.7 if not weighted else 0.7 * float(np.median(cn))
    g = sa.act_sparsify_scored(dev(X), t=t, n=n, m=m, mu=None if mu is None else dev(mu),
                               colnorm=None if cn is None else torch.from_numpy(cn).to(DEV))
    mask_g, idx_g, val_g, nnz_g, alpha_g = g
    XS = np.stack([correct.shift(X[r], mu) for r in range(rows)])
    keep = np.stack([correct.threshold_keep(XS[r], cn, t) if m == 0 else
                     correct.nm_keep(XS[r], cn, n, m) for r in range(rows)])
    check_lists(mask_g, idx_g, val_g, nnz_g, XS, keep)
    alpha = host(alpha_g)
    for r in range(rows):
        assert alpha[r] == pytest.approx(correct.var_alpha(XS[r], keep[r]), rel=2e-6)


@pytest.mark.parametrize("d,nm", [(48, (8, 16)), (1000, (2, 4)), (1000, (4, 8)), (4112, (8, 16)),
                                  (72, (1, 4)), (40, (3, 8)), (8256, (31, 32)), (96, (16, 32))])
def test_scored_sparsify_ragged_rows(d, nm):
    """N:M by score over workgroups of 64 groups: rows whose last mask word
    is partly past the row (d not a multiple of 32), rows ending inside a
    workgroup, every n; lists, masks and alpha against the oracle."""
    n, m = nm
    rows = 3
    X = syn.laplace_f16((rows, d), 1.0, 7 * d + m)
    X[1, ::3] = np.float16(-0.0)
    mu = syn.gaussian_f16((d,), 0.25, d + 1)
    cn = correct.column_norms(syn.weight_t(16, d, 5))
    mask_g, idx_g, val_g, nnz_g, alpha_g = sa.act_sparsify_scored(
        dev(X), t=0.0, n=n, m=m, mu=dev(mu), colnorm=torch.from_numpy(cn).to(DEV))
    XS = np.stack([correct.shift(X[r], mu) for r in range(rows)])
    keep = np.stack([correct.nm_keep(XS[r], cn, n, m) for r in range(rows)])
    check_lists(mask_g, idx_g, val_g, nnz_g, XS, keep)
    alpha = host(alpha_g)
    for r in range(rows):
        assert alpha[r] == pytest.approx(correct.var_alpha(XS[r], keep[r]), rel=2e-6)
    # without the mask output: the same lists and alpha
    g2 = sa.act_sparsify_scored(dev(X), t=0.0, n=n, m=m, mu=dev(mu),
                                colnorm=torch.from_numpy(cn).to(DEV), with_mask=False)
    assert g2[0] is None
    for a, b in zip(g2[1:], (idx_g, val_g, nnz_g, alpha_g)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("d", [4096, 4112, 5000, 4127, 16400, 65536])
def test_scored_threshold_two_pass(d):
    """Rows long enough for the two-pass threshold kind (decisions over
    1024-entry chunks, then the list): last mask words cut at 8, 16 and 31
    entries, a list longer than one pass, the longest row; with and without
    the mask output."""
    rows = 3
    X = syn.laplace_f16((rows, d), 1.0, 5 * d + 1)
    X[2, ::5] = np.float16(0.0)
    mu = syn.gaussian_f16((d,), 0.25, d + 2)
    cn = correct.column_norms(syn.weight_t(16, d, 6))
    XS = np.stack([correct.shift(X[r], mu) for r in range(rows)])
    sc = np.sort(correct.scores(XS[0], cn))
    t = float(0.5 * (sc[d // 2 - 1] + sc[d // 2]))
    args = dict(t=t, n=0, m=0, mu=dev(mu), colnorm=torch.from_numpy(cn).to(DEV))
    mask_g, idx_g, val_g, nnz_g, alpha_g = sa.act_sparsify_scored(dev(X), **args)
    keep = np.stack([correct.threshold_keep(XS[r], cn, t) for r in range(rows)])
    check_lists(mask_g, idx_g, val_g, nnz_g, XS, keep)
    alpha = host(alpha_g)
    for r in range(rows):
        assert alpha[r] == pytest.approx(correct.var_alpha(XS[r], keep[r]), rel=2e-6)
    g2 = sa.act_sparsify_scored(dev(X), with_mask=False, **args)
    assert g2[0] is None
    for a, b in zip(g2[1:], (idx_g, val_g, nnz_g, alpha_g)):
        n_ = host(nnz_g)
        if a.dim() == 2 and a.shape == b.shape and a.dtype != torch.float32:
            for r in range(rows):
                assert torch.equal(a[r, :int(n_[r])], b[r, :int(n_[r])])
        else:
            assert torch.equal(a, b)


def test_scored_sparsify_many_rows():
    """More rows than a grid's y dimension holds (70000 > 65535): rows run
    along x.  Sampled rows against the oracle."""
    rows, d, n, m = 70000, 64, 2, 4
    X = syn.laplace_f16((rows, d), 1.0, 91)
    mask_g, idx_g, val_g, nnz_g, alpha_g = sa.act_sparsify_scored(dev(X), t=0.0, n=n, m=m)
    sample = np.unique(np.concatenate([np.arange(0, rows, 997), [65535, 65536, rows - 1]]))
    XS = X[sample]
    keep = np.stack([correct.nm_keep(XS[i], None, n, m) for i in range(len(sample))])
    check_lists(mask_g[sample], idx_g[sample], val_g[sample], nnz_g[sample], XS, keep)
    alpha = host(alpha_g)[sample]
    for i in range(len(sample)):
        assert alpha[i] == pytest.approx(correct.var_alpha(XS[i], keep[i]), rel=2e-6)


@pytest.mark.parametrize("kind", ["threshold", "8:16"])
@pytest.mark.parametrize("d_out,d_in", [(4096, 11008), (264, 1024), (11008, 4096)])
def test_corrected_gemv(d_out, d_in, kind):
    """The whole corrected step against the oracle: shift, weight-aware
    selection, the sparse GEMV scaled by alpha plus the bias W mu."""
    wt = syn.weight_t(d_out, d_in, d_out + d_in)
    x = syn.laplace_f16((d_in,), 1.0, 12)
    mu = syn.gaussian_f16((d_in,), 0.25, 13)
    wt_g = dev(wt)
    cn_g = sa.weight_col_norms(wt_g)
    cn = host(cn_g)
    np.testing.assert_allclose(cn, correct.column_norms(wt), rtol=1e-12)
    xs = correct.shift(x, mu)
    if kind == "threshold":
        sc = np.sort(correct.scores(xs, cn))
        t = float(0.5 * (sc[d_in // 2 - 1] + sc[d_in // 2]))
        n, m = 0, 0
        keep_fn = lambda v, c: correct.threshold_keep(v, c, t)  # noqa: E731
    else:
        t, n, m = 0.0, 8, 16
        keep_fn = lambda v, c: correct.nm_keep(v, c, 8, 16)  # noqa: E731
    mask_g, idx_g, val_g, nnz_g, alpha_g = sa.act_sparsify_scored(
        dev(x), t=t, n=n, m=m, mu=dev(mu), colnorm=cn_g)
    bias_g = sa.dense_gemv(wt_g, dev(mu))
    y = sa.sparse_gemv_corrected(wt_g, idx_g, val_g, nnz_g, alpha=alpha_g, bias=bias_g)
    _, keep, alpha, y_ref = correct.corrected_gemv(wt, x, mu, cn, keep_fn, var=True)
    check_lists(mask_g, idx_g, val_g, nnz_g, xs, keep)
    assert_close(y, y_ref)
    # without the corrections the same call is the plain list GEMV
    y0 = sa.sparse_gemv_corrected(wt_g, idx_g, val_g, nnz_g)
    assert torch.equal(y0, sa.sparse_gemv(wt_g, idx_g, val_g, nnz_g))


@pytest.mark.parametrize("d_out,d_in", [(4096, 11008), (264, 1024), (11008, 4096), (72, 40000)])
@pytest.mark.parametrize("shifted,weighted,var,biased", [(True, True, True, True),
                                                        (False, True, False, False),
                                                        (True, False, True, False),
                                                        (False, False, False, True)])
def test_scored_fused(d_out, d_in, shifted, weighted, var, biased):
    """sparse_gemv_scored (one launch) against the oracle, with the one- and
    two-launch hand-offs giving identical bits."""
    wt = syn.weight_t(d_out, d_in, d_out + 7 * d_in)
    x = syn.laplace_f16((d_in,), 1.0, 21)
    mu = syn.gaussian_f16((d_in,), 0.25, 22) if shifted else None
    wt_g = dev(wt)
    cn_g = sa.weight_col_norms(wt_g) if weighted else None
    cn = host(cn_g) if weighted else None
    xs = correct.shift(x, mu)
    sc = np.sort(correct.scores(xs, cn))
    t = float(0.5 * (sc[d_in // 2 - 1] + sc[d_in // 2]))
    bias_g = sa.dense_gemv(wt_g, dev(mu if mu is not None else x)) if biased else None
    # the oracle's alpha * W s (its own W mu left out), plus the bias passed
    _, keep, alpha, y_ref = correct.corrected_gemv(
        wt, x, None if mu is None else mu, cn, lambda v, c: correct.threshold_keep(v, c, t),
        var=var)
    if mu is not None:
        y_ref = y_ref - gemv.dense_gemv(wt, mu)
    if biased:
        y_ref = y_ref + host(bias_g).astype(np.float64)
    mu_g = dev(mu) if mu is not None else None
    out = {}
    try:
        for handoff in (2, 1, 3):
            sa.set_gemv_tuning(-1, 0, handoff)
            out[handoff] = sa.sparse_gemv_scored(wt_g, dev(x), t, mu=mu_g, colnorm=cn_g, var=var,
                                                 bias=bias_g).clone()
    finally:
        sa.set_gemv_tuning(-1, 0, 0)
    assert torch.equal(out[1], out[2]) and torch.equal(out[1], out[3])
    assert_close(out[2], y_ref)


@pytest.mark.parametrize("d_out,d_in,n,m", [(4096, 11008, 8, 16), (4096, 11008, 16, 32),
                                           (264, 1024, 2, 4), (11008, 4096, 4, 8),
                                           (72, 40000, 8, 16), (136, 1000, 4, 8),
                                           (200, 96, 1, 32), (64, 4104, 3, 8)])
@pytest.mark.parametrize("shifted,weighted,var,biased", [(True, True, True, True),
                                                        (False, True, False, False),
                                                        (True, False, True, False)])
def test_scored_nm_fused(d_out, d_in, n, m, shifted, weighted, var, biased):
    """sparse_gemv_scored_nm (one launch) against the oracle's corrected GEMV
    with n of every m kept by score; the one- and two-launch hand-offs give
    identical bits; the list path (act_sparsify_scored, then
    sparse_gemv_corrected) agrees within the tolerance."""
    wt = syn.weight_t(d_out, d_in, d_out + 3 * d_in + m)
    x = syn.laplace_f16((d_in,), 1.0, 31 + n)
    x[::13] = np.float16(0.25)  # ties inside groups
    mu = syn.gaussian_f16((d_in,), 0.25, 32) if shifted else None
    wt_g = dev(wt)
    cn_g = sa.weight_col_norms(wt_g) if weighted else None
    cn = host(cn_g) if weighted else None
    bias_g = sa.dense_gemv(wt_g, dev(mu if mu is not None else x)) if biased else None
    _, keep, alpha, y_ref = correct.corrected_gemv(
        wt, x, mu, cn, lambda v, c: correct.nm_keep(v, c, n, m), var=var)
    if mu is not None:
        y_ref = y_ref - gemv.dense_gemv(wt, mu)
    if biased:
        y_ref = y_ref + host(bias_g).astype(np.float64)
    mu_g = dev(mu) if mu is not None else None
    out = {}
    try:
        for handoff in (2, 1, 3):
            sa.set_gemv_tuning(-1, 0, handoff)
            out[handoff] = sa.sparse_gemv_scored_nm(wt_g, dev(x), n, m, mu=mu_g, colnorm=cn_g,
                                                    var=var, bias=bias_g).clone()
    finally:
        sa.set_gemv_tuning(-1, 0, 0)
    assert torch.equal(out[1], out[2]) and torch.equal(out[1], out[3])
    assert_close(out[2], y_ref)
    # the two-step list path: same kept set (bit-exact lists), same output within tolerance
    mask_g, idx_g, val_g, nnz_g, alpha_g = sa.act_sparsify_scored(
        dev(x).reshape(1, -1), t=0.0, n=n, m=m, mu=mu_g, colnorm=cn_g)
    assert np.array_equal(host(idx_g)[0, :int(host(nnz_g)[0])], np.flatnonzero(keep))
    y2 = sa.sparse_gemv_corrected(wt_g, idx_g, val_g, nnz_g, alpha=alpha_g if var else None,
                                  bias=bias_g)
    assert_close(out[2], host(y2).reshape(-1).astype(np.float64))


@pytest.mark.gpu
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (3, 8), (8, 16), (5, 16), (16, 32), (11, 32)])
def test_scored_nm_near_ties(n, m):
    """The one-launch N:M GEMV ranks scores in fp32 when that decides them,
    else in fp64.  Groups whose fp64 scores differ below fp32's resolution,
    exact ties, and zeros sit in some 64-entry blocks, plain random groups in
    the others.  With the identity as the weight, y is x on the kept entries
    and 0 elsewhere, so the kept set is compared bit for bit with the oracle's
    N:M rule."""
    d = 4096
    rng = np.random.default_rng(1000 + 37 * m + n)
    x = syn.laplace_f16((d,), 1.0, 500 + n + m)
    cn = rng.uniform(0.5, 2.0, d)
    for blk in range(0, d, 64):
        kind = (blk // 64) % 4
        if kind == 0:
            continue  # random scores: decided in fp32
        for g in range(blk, blk + 64, m):
            if kind == 1:  # equal x, fp64 norms 2^-40 apart: one fp32 key
                x[g:g + m] = np.float16(0.5)
                cn[g:g + m] = 1.0 + rng.permutation(m) * 2.0 ** -40
            elif kind == 2:  # exact ties: the lower index wins
                x[g:g + m] = np.float16(-0.75)
                cn[g:g + m] = 1.25
            else:  # some zeros among random entries
                x[g:g + m:3] = np.float16(0)
    wt = np.eye(d, dtype=np.float16)
    keep = correct.nm_keep(x, cn, n, m)
    y = sa.sparse_gemv_scored_nm(dev(wt), dev(x), n, m, colnorm=dev(cn), var=False)
    expect = np.where(keep, x, np.float16(0))
    assert np.array_equal(host(y).view(np.uint16), expect.view(np.uint16))
    # near-tie groups are not decided by position alone
    kind1 = np.zeros(d, dtype=bool)
    for blk in range(64, d, 256):
        kind1[blk:blk + 64] = True
    first_n = np.zeros(d, dtype=bool)
    for g in range(0, d, m):
        first_n[g:g + n] = True
    assert not np.array_equal(keep[kind1], first_n[kind1])


# ---------------------------------------------------------------------------
# RaNA linear-layer rank adapter A (m ⊙ B x), m_i = v_i^2 >= t
# ---------------------------------------------------------------------------

def oracle_v16(bt, X):
    """The oracle's fp16 v = B x, one row per token (fp64 sums, rounded once)."""
    return np.stack([rana.adapter_v(bt, X[b]).astype(np.float16) for b in range(len(X))])


def fp16_order(a):
    """fp16 values as integers in their numeric order, adjacent values one
    apart (+0 and -0 both 0)."""
    b = np.asarray(a, dtype=np.float16).view(np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def gap_threshold(v16, rate):
    """A threshold between two adjacent squares of the oracle's |v| such that
    a value one fp16 ulp away from any oracle v stays on the same side: an
    implementation whose v is within one ulp of the oracle's (fp32 instead of
    fp64 sums, rounded to fp16) then takes exactly the oracle's decisions.
    Searched outward from the split that masks `rate` of the entries; rate 0
    gives t = 0 (keep all), rate 1 a t above every reachable square."""
    a = np.sort(np.abs(np.asarray(v16, dtype=np.float16).ravel()))
    if rate <= 0.0:
        return 0.0
    up = np.nextafter(a, np.float16(np.inf)).astype(np.float64)
    if rate >= 1.0:
        return float(np.float32(4.0 * up[-1] ** 2 + 1.0))
    dn = np.nextafter(a, np.float16(0)).astype(np.float64)
    k0 = int(rate * len(a))
    for k in sorted(range(1, len(a)), key=lambda k: (abs(k - k0), k)):
        lo, hi = up[k - 1] ** 2, dn[k] ** 2
        t = float(np.float32(0.5 * (lo + hi)))
        if lo < t < hi:
            return t
    raise AssertionError("no gap between the oracle's squares")


def gpu_adapter_mask(bt, X, t):
    """The mask the kernel applies, read out exactly: with A = I the second
    GEMV returns m ⊙ v with every kept entry unchanged (one product by 1.0)
    and every dropped entry 0, so the kept set is where y is nonzero (t > 0:
    a kept entry has v^2 >= t > 0)."""
    r = bt.shape[1]
    eye = np.eye(r, dtype=np.float16)
    v_g, y_g = sa.rana_adapter_gemv(dev(bt.T), dev(eye), dev(X), t)
    v, y = host(v_g).reshape(len(X), r), host(y_g).reshape(len(X), r)
    keep = y != 0
    assert np.array_equal(y[keep].view(np.uint16), v[keep].view(np.uint16))
    return keep, v


def check_adapter(bt, at, X, t, v_g, y_g):
    """The whole chain against the oracle's own: its fp16 v (the GPU's within
    one ulp, so t in a gap of the oracle's squares decides alike), its mask
    (the kernel's mask, read out through A = I, bit for bit) and its y over
    the kept columns of A (within tolerance).  No GPU value enters the
    oracle."""
    v_g, y_g = host(v_g).reshape(len(X), -1), host(y_g).reshape(len(X), -1)
    v16 = oracle_v16(bt, X)
    keep_ref = v16.astype(np.float64) ** 2 >= t
    # fp32 sums against fp64 sums, each rounded once to fp16: at most one ulp
    # apart wherever |v| is well above the sums' absolute error (near zero
    # the fp32 error can span several of the tiny ulps there); every split
    # gap_threshold picks lies far above that
    big = np.abs(v16.astype(np.float64)) >= 2.0 ** -4
    assert np.all(np.abs(fp16_order(v_g) - fp16_order(v16))[big] <= 1)
    assert t == 0.0 or np.sqrt(t) >= 2.0 ** -3
    if t > 0:
        keep_g, v_probe = gpu_adapter_mask(bt, X, t)
        assert np.array_equal(v_probe.view(np.uint16), v_g.view(np.uint16))
        assert np.array_equal(keep_g, keep_ref)
    for b in range(len(X)):
        v, v16b, keep, y_ref = rana.rank_adapter(bt, at, X[b], t)
        assert np.array_equal(v16b.view(np.uint16), v16[b].view(np.uint16))
        assert np.array_equal(keep, keep_ref[b])
        assert_close(v_g[b], v)
        assert_close(y_g[b], y_ref)
    return keep_ref


@pytest.mark.parametrize("batch", [1, 2, 3, 8])
@pytest.mark.parametrize("r,d_in,d_out", [(136, 130, 72), (1024, 512, 264), (8, 33, 2056)])
def test_rana_adapter_small(r, d_in, d_out, batch):
    bt, at = syn.rank_adapter_weights(d_out, d_in, r, r + d_in, std=0.1)
    X = syn.gaussian_f16((batch, d_in), 1.0, batch + d_out)
    v16 = oracle_v16(bt, X)
    for rate in (0.0, 0.3, 0.5, 0.8, 1.0):
        t = gap_threshold(v16, rate)
        v_g, y_g = sa.rana_adapter_gemv(dev(bt.T), dev(at), dev(X), t)
        check_adapter(bt, at, X, t, v_g, y_g)


def test_rana_adapter_exact_square_threshold():
    """B = A = I (r = d_in = d_out = 64): v = x, y = m ⊙ x.  At t = 0.25 the
    entries +-0.5 are kept and their fp16 neighbours below 0.5 are not."""
    eye = np.eye(64, dtype=np.float16)
    below = np.nextafter(np.float16(0.5), np.float16(0))
    x = np.tile(np.array([0.5, -0.5, below, -below, 0.0, 2.0, -0.25, 0.75], np.float16), 8)
    v_g, y_g = sa.rana_adapter_gemv(dev(eye), dev(eye), dev(x), 0.25)
    assert np.array_equal(host(v_g), x)
    assert np.array_equal(host(y_g), np.where(x.astype(np.float64) ** 2 >= 0.25, x, 0))


@pytest.mark.parametrize("rate", [0.5, 0.7])
def test_rana_adapter_llama_gate(rate):
    """The gate projection (11008 x 4096) as a rank-2048 adapter at 50% and
    70% mask rates, batch 1: t from the oracle's own squares (a gap near the
    rate), the kernel's mask equal to the oracle's, y against the oracle's
    end-to-end chain."""
    bt, at = syn.rank_adapter_weights(11008, 4096, 2048, 3000)
    x = syn.activation((4096,), "gaussian", 7)[None]
    t = gap_threshold(oracle_v16(bt, x), rate)
    v_g, y_g = sa.rana_adapter_gemv(dev(bt.T), dev(at), dev(x), t)
    keep = check_adapter(bt, at, x, t, v_g, y_g)
    assert abs(int(keep.sum()) - round((1 - rate) * 2048)) <= 64


# ---------------------------------------------------------------------------
# batched N:M matmul and the dense MFMA GEMM
# ---------------------------------------------------------------------------

from oracle import spmm  # noqa: E402


# (tile rows, engine, pipelined stages): automatic, then each engine at each
# tile height, then deeper pipelines, then the 256 x 256 engine at each of
# its stage counts
GEMM_CHOICES = [(0, 0, 0), (128, 1, 0), (256, 1, 0), (128, 2, 0), (256, 2, 0), (128, 2, 4),
                (256, 2, 5), (128, 2, 6), (0, 3, 0), (256, 3, 3), (0, 3, 4), (0, 3, 6)]
STAGES = [3, 4, 5, 6]


@pytest.mark.parametrize("choice", GEMM_CHOICES)
@pytest.mark.parametrize("T,d_in,d_out", [(64, 1024, 1024), (130, 96, 136), (1, 32, 8),
                                          (257, 4096, 264), (600, 256, 1032)])
def test_dense_gemm_small(T, d_in, d_out, choice):
    X = syn.gaussian_f16((T, d_in), 1.0, T)
    wt = syn.weight_t(d_out, d_in, d_in)
    try:
        sa.set_gemm_tuning(*choice)
        Y = sa.dense_gemm(dev(X), dev(wt))
    finally:
        sa.set_gemm_tuning(0, 0, 0)
    assert_close(Y, X.astype(np.float64) @ wt.astype(np.float64))


@pytest.mark.parametrize("stages", STAGES)
@pytest.mark.parametrize("tile_rows", [128, 256])
@pytest.mark.parametrize("T,d_in,d_out", [(64, 32, 128), (256, 64, 128), (40, 96, 136),
                                          (300, 128, 136), (300, 160, 264), (17, 192, 8),
                                          (129, 224, 72), (513, 256, 264), (256, 320, 128),
                                          (70, 448, 1000), (260, 1088, 392), (33, 352, 64),
                                          (64, 384, 136), (96, 416, 64), (31, 480, 200)])
def test_dense_gemm_k_pipeline_lengths(T, d_in, d_out, tile_rows, stages):
    """K a multiple of 32 takes the pipelined dense engine (K steps of 32):
    1 to 15 and 34 K steps cover, for every stage count, runs shorter than
    the prefetch distance, the steady loop and every tail length, with
    ragged rows/columns."""
    X = syn.gaussian_f16((T, d_in), 1.0, T + d_in)
    wt = syn.weight_t(d_out, d_in, d_out)
    try:
        sa.set_gemm_tuning(tile_rows, 2, stages)
        Y = sa.dense_gemm(dev(X), dev(wt))
    finally:
        sa.set_gemm_tuning(0, 0, 0)
    assert_close(Y, X.astype(np.float64) @ wt.astype(np.float64))


@pytest.mark.parametrize("stages", [3, 4, 5])
@pytest.mark.parametrize("T,d_in,d_out", [(64, 32, 128), (256, 64, 256), (40, 96, 136),
                                          (300, 128, 520), (17, 192, 8), (129, 224, 72),
                                          (513, 256, 264), (257, 320, 768), (70, 448, 1000),
                                          (33, 352, 64), (96, 416, 264), (31, 480, 200),
                                          (260, 1088, 392)])
def test_dense_gemm_wide_k_pipeline_lengths(T, d_in, d_out, stages):
    """The 256 x 256 engine (engine 3): 1 to 15 and 34 K steps at each of its
    stage counts, ragged rows and columns (partial row and column tiles,
    columns past the last 256 clamped), against the oracle and bit-equal to
    the 256 x 128 engine."""
    X = syn.gaussian_f16((T, d_in), 1.0, 2 * T + d_in)
    wt = syn.weight_t(d_out, d_in, d_out + 5)
    X_g, wt_g = dev(X), dev(wt)
    try:
        sa.set_gemm_tuning(0, 3, stages)
        Y = sa.dense_gemm(X_g, wt_g).clone()
        sa.set_gemm_tuning(256, 2, 0)
        Yn = sa.dense_gemm(X_g, wt_g)
    finally:
        sa.set_gemm_tuning(0, 0, 0)
    assert_close(Y, X.astype(np.float64) @ wt.astype(np.float64))
    assert torch.equal(Y, Yn)


@pytest.mark.parametrize("T,d_in,d_out", [(2048, 4096, 13312), (4096, 1024, 4096)])
def test_dense_gemm_wide_full_shapes(T, d_in, d_out):
    """Shapes where the automatic choice takes the 256 x 256 engine (2048 x
    13312: 416 tiles on 256 CUs; 4096 x 4096: one tile per CU): every output
    row against the oracle, bits equal to the 256 x 128 engine, and the
    8:16 two-pass product (expanded copy on the same engine) likewise."""
    X = syn.gaussian_f16((T, d_in), 1.0, 9)
    wt = syn.weight_t(d_out, d_in, 43)
    X_g, wt_g = dev(X), dev(wt)
    Y = sa.dense_gemm(X_g, wt_g).clone()
    mask_g, val_g = sa.act_sparsify_nm(X_g, 8, 16)
    Ys = sa.nm_act_spmm(val_g, mask_g, 8, 16, wt_g).clone()
    try:
        sa.set_gemm_tuning(256, 2, 0)
        Yn = sa.dense_gemm(X_g, wt_g)
        Ysn = sa.nm_act_spmm(val_g, mask_g, 8, 16, wt_g)
    finally:
        sa.set_gemm_tuning(0, 0, 0)
    assert torch.equal(Y, Yn)
    assert torch.equal(Ys, Ysn)
    assert_close(Y, spmm.masked_matmul(X, np.ones(X.shape, dtype=bool), wt))
    keep, _ = sparsify.nm_sparsify(X, 8, 16)
    assert_close(Ys, spmm.masked_matmul(X, keep, wt))


@pytest.mark.parametrize("stages", STAGES)
@pytest.mark.parametrize("tile_rows", [128, 256])
@pytest.mark.parametrize("T,d_in,d_out", [(64, 64, 128), (40, 192, 136), (300, 320, 264),
                                          (129, 448, 72), (70, 576, 200), (256, 704, 128),
                                          (33, 832, 64), (100, 960, 136), (17, 2176, 8)])
def test_nm24_k_pipeline_lengths(T, d_in, d_out, tile_rows, stages):
    """2:4 steps K by 64: 1, 3, 5, 7, 9, 11, 13, 15 and 34 K steps at every
    stage count (at 256-row tiles, stage counts past what LDS holds run the
    most that fit)."""
    X = syn.gaussian_f16((T, d_in), 1.0, 3 * T + d_in)
    wt = syn.weight_t(d_out, d_in, d_out + 1)
    keep, _ = sparsify.nm_sparsify(X, 2, 4)
    ref = spmm.nm_spmm(X, keep, wt)
    mask_g, val_g = sa.act_sparsify_nm(dev(X), 2, 4)
    try:
        sa.set_gemm_tuning(tile_rows, 2, stages)
        Y = sa.nm_act_spmm(val_g, mask_g, 2, 4, dev(wt))
    finally:
        sa.set_gemm_tuning(0, 0, 0)
    assert_close(Y, ref)


@pytest.mark.parametrize("T,d_in,d_out", [(1, 64, 8), (300, 128, 264), (257, 192, 520),
                                          (40, 256, 136), (513, 320, 256), (64, 384, 1000),
                                          (100, 448, 72), (256, 512, 512), (33, 704, 264),
                                          (70, 2176, 256)])
def test_nm24_wide_engine(T, d_in, d_out):
    """2:4 on the 256 x 256-tile engine (engine 3): K steps of 64 from 1 to
    34 (the tail alone, one rolled round and more), ragged rows and columns.
    Against the oracle, and bit for bit against the 128 x 128-tile engine
    (same sparse MFMA sequence per output block)."""
    X = syn.gaussian_f16((T, d_in), 1.0, 11 * T + d_in)
    X[0, :] = np.float16(0.5)  # ties
    wt = syn.weight_t(d_out, d_in, d_out + 7)
    keep, _ = sparsify.nm_sparsify(X, 2, 4)
    mask_g, val_g = sa.act_sparsify_nm(dev(X), 2, 4)
    wt_g = dev(wt)
    try:
        sa.set_gemm_tuning(0, 3, 0)
        assert sa.gemm_plan("nm", T, d_in, d_out, 2, 4)["engine"] == "wide"
        Yw = sa.nm_act_spmm(val_g, mask_g, 2, 4, wt_g).clone()
        sa.set_gemm_tuning(128, 2, 0)
        Yn = sa.nm_act_spmm(val_g, mask_g, 2, 4, wt_g).clone()
    finally:
        sa.set_gemm_tuning(0, 0, 0)
    assert torch.equal(Yw, Yn)
    assert_close(Yw, spmm.nm_spmm(X, keep, wt))


@pytest.mark.parametrize("choice", GEMM_CHOICES)
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (8, 16), (16, 32), (1, 4), (3, 4), (5, 16),
                                 (32, 32)])
@pytest.mark.parametrize("T,d_in,d_out", [(64, 1024, 512), (100, 96, 136), (300, 128, 264)])
def test_nm_spmm_small(n, m, T, d_in, d_out, choice):
    if d_in % m:
        pytest.skip("d_in not a multiple of m")
    X = syn.gaussian_f16((T, d_in), 1.0, n * 7 + m)
    wt = syn.weight_t(d_out, d_in, 40 + m)
    keep, vals = sparsify.nm_sparsify(X, n, m)
    ref = spmm.nm_spmm(X, keep, wt)
    mask_g, val_g = sa.act_sparsify_nm(dev(X), n, m)
    try:
        sa.set_gemm_tuning(*choice)
        Y = sa.nm_act_spmm(val_g, mask_g, n, m, dev(wt))
    finally:
        sa.set_gemm_tuning(0, 0, 0)
    assert_close(Y, ref)
    # each token's row is that token's masked GEMV
    r = 3
    assert_close(sa.masked_gemv(dev(wt), dev(X[r]), mask_g[r]), ref[r])


@pytest.mark.parametrize("T,d_in,d_out", [(256, 64, 128), (300, 192, 136), (513, 320, 264),
                                          (70, 1088, 1000), (1024, 1024, 1024)])
def test_gemm_engines_agree(T, d_in, d_out):
    """The pipelined engine (default when K is a multiple of its step: 32
    dense, 64 for 2:4) and the staged-register engine, each at both tile
    heights, issue the same MFMA sequence per output block: dense and 2:4
    results must be identical."""
    X = syn.gaussian_f16((T, d_in), 1.0, T * 7 + d_in)
    X_g, wt_g = dev(X), dev(syn.weight_t(d_out, d_in, d_out + 3))
    mask_g, val_g = sa.act_sparsify_nm(X_g, 2, 4)
    out = {}
    try:
        for choice in GEMM_CHOICES:
            sa.set_gemm_tuning(*choice)
            out[choice] = (sa.dense_gemm(X_g, wt_g).clone(),
                           sa.nm_act_spmm(val_g, mask_g, 2, 4, wt_g).clone())
    finally:
        sa.set_gemm_tuning(0, 0, 0)
    for choice in GEMM_CHOICES[1:]:
        assert torch.equal(out[GEMM_CHOICES[0]][0], out[choice][0]), ("dense", choice)
        assert torch.equal(out[GEMM_CHOICES[0]][1], out[choice][1]), ("2:4", choice)


@pytest.mark.parametrize("n,m", [(8, 16), (16, 32), (4, 8), (1, 4), (3, 4), (5, 16), (7, 32),
                                 (32, 32)])
@pytest.mark.parametrize("T,d_in,d_out", [(256, 64, 128), (300, 192, 136), (70, 1088, 1000)])
def test_nm_spmm_two_pass_matches_single_pass(T, d_in, d_out, n, m):
    """With a workspace, N:M patterns other than 2:4 are expanded to a dense
    copy and run on the dense engine; without one, they are scattered into
    LDS tiles in one pass.  The MFMA sequence is the same: identical bits,
    and both match the oracle."""
    X = syn.gaussian_f16((T, d_in), 1.0, T + n * 31 + m)
    X[1, :] = np.float16(0.25)  # ties
    wt = syn.weight_t(d_out, d_in, d_out + m)
    X_g, wt_g = dev(X), dev(wt)
    mask_g, val_g = sa.act_sparsify_nm(X_g, n, m)
    y2 = sa.nm_act_spmm(val_g, mask_g, n, m, wt_g)
    y1 = sa.nm_act_spmm(val_g, mask_g, n, m, wt_g, use_workspace=False)
    assert torch.equal(y1, y2)
    keep = sparsify.nm_sparsify(X, n, m)[0]
    assert_close(y2, spmm.nm_spmm(X, keep, wt))


@pytest.mark.parametrize("T,d_in,d_out", [(4096, 1024, 1024), (2048, 4096, 11008)])
@pytest.mark.parametrize("n,m", [(2, 4), (8, 16), (16, 32)])
def test_nm_spmm_full_shapes(T, d_in, d_out, n, m):
    """The benchmarked launches at full size: every mask row bit-exact and
    every output row (so every row and column tile of the matmul's grid)
    against the oracle's fp64 masked matmul; the dense GEMM likewise."""
    X = syn.gaussian_f16((T, d_in), 1.0, 5)
    wt = syn.weight_t(d_out, d_in, 41)
    X_g, wt_g = dev(X), dev(wt)
    mask_g, val_g = sa.act_sparsify_nm(X_g, n, m)
    Y = sa.nm_act_spmm(val_g, mask_g, n, m, wt_g)
    Yd = sa.dense_gemm(X_g, wt_g)
    keep, vals = sparsify.nm_sparsify(X, n, m)
    assert np.array_equal(words(mask_g), sparsify.pack_mask(keep))
    assert np.array_equal(host(val_g).view(np.uint16), vals.view(np.uint16))
    assert_close(Y, spmm.masked_matmul(X, keep, wt))
    assert_close(Yd, spmm.masked_matmul(X, np.ones(X.shape, dtype=bool), wt))


# ---------------------------------------------------------------------------
# tile-shared N:M: sparsifier and matmul
# ---------------------------------------------------------------------------

SHARED_PATTERNS = [(2, 4), (1, 4), (3, 4), (4, 8), (2, 8), (7, 8), (8, 16), (4, 16), (5, 16),
                   (16, 32), (8, 32), (32, 32)]


def shared_whole_tile(d_in, n, m, tt):
    """Conditions of the whole-tile gather (one pattern per row tile)."""
    return (tt % 128 == 0 and 32 % n == 0 and d_in % m == 0 and d_in <= 32768
            and (d_in // m * n) % 32 == 0)


def shared_per_block(d_in, n, m, tt):
    """Conditions of the per-32-row-block gather."""
    return tt % 32 == 0 and 32 % n == 0 and m in (2 * n, 4 * n) and d_in % (32 * m // n) == 0


@pytest.mark.parametrize("n,m", SHARED_PATTERNS)
@pytest.mark.parametrize("T,d,tt", [(1, 32, 32), (70, 1056, 32), (33, 64, 1), (100, 2048, 7),
                                    (300, 1024, 64), (257, 96, 256), (64, 3072, 32)])
def test_nm_shared_sparsify(T, d, tt, n, m):
    """Masks and values bit-exact: ragged last tiles, partial column chunks,
    one-row tiles and the largest tile."""
    X = syn.gaussian_f16((T, d), 1.0, T * 13 + d + tt)
    _, tile_keep, vals = sparsify.nm_shared_sparsify(X, n, m, tt)
    mask_g, val_g = sa.act_sparsify_nm_shared(dev(X), n, m, tt)
    assert np.array_equal(words(mask_g), sparsify.pack_mask(tile_keep))
    assert np.array_equal(host(val_g).view(np.uint16), vals.view(np.uint16))


@pytest.mark.parametrize("n,m", [(2, 4), (3, 8), (8, 16), (16, 32), (5, 32)])
def test_nm_shared_sparsify_ties(n, m):
    """Few distinct magnitudes (tied tile sums decide most groups), a tile
    of equal magnitudes (the first n of each group) and signed zeros."""
    rng = np.random.default_rng(n * 100 + m)
    pool = np.array([0.0, -0.0, 0.5, -0.5, 1.0, -1.0, 2.0], dtype=np.float16)
    X = pool[rng.integers(0, len(pool), size=(100, 1024))]
    X[32:64] = np.float16(-0.25)
    X[64:96] = np.float16(-0.0)
    _, tile_keep, vals = sparsify.nm_shared_sparsify(X, n, m, 32)
    mask_g, val_g = sa.act_sparsify_nm_shared(dev(X), n, m, 32)
    assert np.array_equal(words(mask_g), sparsify.pack_mask(tile_keep))
    assert np.array_equal(host(val_g).view(np.uint16), vals.view(np.uint16))
    first_n = np.tile(np.arange(m) < n, 1024 // m)
    assert np.array_equal(tile_keep[1], first_n) and np.array_equal(tile_keep[2], first_n)


@pytest.mark.parametrize("tile_rows", [0, 128, 256])
@pytest.mark.parametrize("n,m", [(2, 4), (1, 4), (4, 8), (2, 8), (8, 16), (4, 16), (16, 32),
                                 (8, 32)])
@pytest.mark.parametrize("T,d_in,d_out,tt", [(64, 1024, 512, 32), (100, 256, 136, 32),
                                             (300, 384, 264, 64), (33, 128, 8, 32),
                                             (1, 512, 1000, 32), (257, 640, 128, 96)])
def test_nm_shared_spmm_gathering_kernel(T, d_in, d_out, tt, n, m, tile_rows):
    """The kernel that gathers WT rows per 32-row block: 1 to 16 K steps of
    64 or 128 dense rows, ragged rows and columns, tiles of 32 to 96 rows,
    both tile heights."""
    assert shared_per_block(d_in, n, m, tt) and not shared_whole_tile(d_in, n, m, tt)
    assert sa.lib().sa_nm_shared_spmm_workspace_bytes(T, d_in, n, m, tt) == 0
    X = syn.gaussian_f16((T, d_in), 1.0, T + d_in + n)
    wt = syn.weight_t(d_out, d_in, d_out + m)
    _, tile_keep, vals = sparsify.nm_shared_sparsify(X, n, m, tt)
    mask_g, val_g = sa.act_sparsify_nm_shared(dev(X), n, m, tt)
    try:
        sa.set_gemm_tuning(tile_rows, 0, 0)
        Y = sa.nm_shared_spmm(val_g, mask_g, n, m, tt, dev(wt))
    finally:
        sa.set_gemm_tuning(0, 0, 0)
    assert_close(Y, spmm.nm_shared_spmm(vals, tile_keep, tt, wt))


def shared_g32(d_in, n, m, tt):
    """Conditions of the 32-row-tile gather."""
    return (tt % 32 == 0 and 32 % n == 0 and d_in % m == 0 and d_in <= 32768
            and (d_in // m * n) % 32 == 0)


G32_CASES = [(T, d_in, d_out, tt, n, m)
             for (T, d_in, d_out, tt) in [(64, 1024, 512, 32), (100, 128, 136, 32),
                                          (33, 256, 8, 32), (1, 512, 1000, 64),
                                          (257, 640, 128, 96), (300, 384, 264, 160),
                                          (70, 2048, 256, 32)]
             for (n, m) in [(8, 16), (16, 32), (2, 4), (1, 4), (4, 16), (1, 8), (32, 32)]
             if shared_g32(d_in, n, m, tt) and not shared_whole_tile(d_in, n, m, tt)]


@pytest.mark.parametrize("engine", [0, 3])
@pytest.mark.parametrize("stages", [3, 4])
@pytest.mark.parametrize("T,d_in,d_out,tt,n,m", G32_CASES)
def test_nm_shared_spmm_g32(T, d_in, d_out, tt, n, m, stages, engine):
    """32-row tiles of one pattern, only the pattern's kept WT rows loaded:
    1 to 64 K steps of 32 compressed entries, ragged rows and columns,
    tiles of 32 to 160 rows, both stage counts, 128- and 256-column tiles
    (engine 3).  Against the oracle, and
    bit for bit against the per-32-row-block gather where that kernel takes
    the shape (the same MFMA sequence per output block)."""
    X = syn.gaussian_f16((T, d_in), 1.0, 3 * T + d_in + n)
    X[0, :] = np.float16(0.5)  # a tile of ties
    wt = syn.weight_t(d_out, d_in, d_out + 2 * m)
    _, tile_keep, vals = sparsify.nm_shared_sparsify(X, n, m, tt)
    mask_g, val_g = sa.act_sparsify_nm_shared(dev(X), n, m, tt)
    wt_g = dev(wt)
    try:
        sa.set_gemm_tuning(0, engine, stages)
        Y = sa.nm_shared_spmm(val_g, mask_g, n, m, tt, wt_g).clone()
        if shared_per_block(d_in, n, m, tt):
            sa.set_gemm_tuning(128, 0, 0)
            Yb = sa.nm_shared_spmm(val_g, mask_g, n, m, tt, wt_g)
            assert torch.equal(Y, Yb)
    finally:
        sa.set_gemm_tuning(0, 0, 0)
    assert_close(Y, spmm.nm_shared_spmm(vals, tile_keep, tt, wt))


@pytest.mark.parametrize("n,m", [(8, 16), (16, 32), (2, 4)])
def test_nm_shared_g32_long_k(n, m):
    """32-row tiles past 4096 kept entries per row: the kept positions come
    from the mask words instead of the byte table."""
    T, d_in, d_out, tt = 96, 16384, 264, 32
    assert d_in // m * n > 4096
    X = syn.gaussian_f16((T, d_in), 1.0, d_in + 3 * n)
    wt = syn.weight_t(d_out, d_in, 19 + m)
    _, tile_keep, vals = sparsify.nm_shared_sparsify(X, n, m, tt)
    mask_g, val_g = sa.act_sparsify_nm_shared(dev(X), n, m, tt)
    Y = sa.nm_shared_spmm(val_g, mask_g, n, m, tt, dev(wt))
    assert_close(Y, spmm.nm_shared_spmm(vals, tile_keep, tt, wt))


@pytest.mark.parametrize("n,m,tt", [(3, 4, 32), (5, 16, 32), (7, 8, 64), (8, 16, 1), (8, 16, 16),
                                    (2, 4, 7), (16, 32, 48), (1, 8, 48), (4, 32, 40), (32, 32, 16),
                                    (4, 4, 48), (3, 4, 128), (5, 8, 256)])
def test_nm_shared_spmm_expanded(n, m, tt):
    """Tiles and patterns outside the gathering kernels: expansion into the
    workspace, then the dense matmul."""
    T, d_in, d_out = 130, 256, 264
    assert not shared_per_block(d_in, n, m, tt) and not shared_whole_tile(d_in, n, m, tt)
    assert not shared_g32(d_in, n, m, tt)
    assert sa.lib().sa_nm_shared_spmm_workspace_bytes(T, d_in, n, m, tt) == T * d_in * 2
    X = syn.gaussian_f16((T, d_in), 1.0, n * 7 + m + tt)
    wt = syn.weight_t(d_out, d_in, 3 * m)
    _, tile_keep, vals = sparsify.nm_shared_sparsify(X, n, m, tt)
    mask_g, val_g = sa.act_sparsify_nm_shared(dev(X), n, m, tt)
    Y = sa.nm_shared_spmm(val_g, mask_g, n, m, tt, dev(wt))
    assert_close(Y, spmm.nm_shared_spmm(vals, tile_keep, tt, wt))


WHOLE_TILE_CASES = [(T, d_in, d_out, tt, n, m)
                    for (T, d_in, d_out, tt) in [(256, 1024, 512, 128), (300, 512, 136, 128),
                                                 (129, 2048, 264, 256), (1, 4096, 8, 128),
                                                 (513, 768, 1000, 256), (640, 256, 128, 128)]
                    for (n, m) in [(2, 4), (1, 4), (8, 16), (4, 16), (16, 32), (8, 32), (1, 8),
                                   (2, 32), (32, 32), (4, 8)]
                    if shared_whole_tile(d_in, n, m, tt)]


@pytest.mark.parametrize("tile_rows", [0, 128, 256])
@pytest.mark.parametrize("T,d_in,d_out,tt,n,m", WHOLE_TILE_CASES)
def test_nm_shared_spmm_whole_tile(T, d_in, d_out, tt, n, m, tile_rows):
    """One pattern per row tile: only the kept WT rows are loaded and the
    dense engine runs over d_in n / m compressed entries (1 to 64 K steps
    of 32), ragged rows and columns, both tile heights where the tile
    allows them."""
    assert sa.lib().sa_nm_shared_spmm_workspace_bytes(T, d_in, n, m, tt) == 0
    X = syn.gaussian_f16((T, d_in), 1.0, 2 * T + d_in + n)
    wt = syn.weight_t(d_out, d_in, d_out + m + 1)
    _, tile_keep, vals = sparsify.nm_shared_sparsify(X, n, m, tt)
    mask_g, val_g = sa.act_sparsify_nm_shared(dev(X), n, m, tt)
    assert np.array_equal(words(mask_g), sparsify.pack_mask(tile_keep))
    try:
        sa.set_gemm_tuning(tile_rows, 0, 0)
        Y = sa.nm_shared_spmm(val_g, mask_g, n, m, tt, dev(wt))
    finally:
        sa.set_gemm_tuning(0, 0, 0)
    assert_close(Y, spmm.nm_shared_spmm(vals, tile_keep, tt, wt))


@pytest.mark.parametrize("d_in,n,m", [(d, n, m) for d in [8256, 16384]
                                      for (n, m) in [(8, 16), (1, 4), (16, 32), (2, 4), (4, 8)]
                                      if shared_whole_tile(d, n, m, 128)])
def test_nm_shared_whole_tile_long_k(d_in, n, m):
    """The kept positions come from a byte table up to 4096 kept entries per
    row and from the mask words beyond: both sides of that limit."""
    T, d_out, tt = 130, 264, 128
    X = syn.gaussian_f16((T, d_in), 1.0, d_in + n)
    wt = syn.weight_t(d_out, d_in, 9 + m)
    _, tile_keep, vals = sparsify.nm_shared_sparsify(X, n, m, tt)
    mask_g, val_g = sa.act_sparsify_nm_shared(dev(X), n, m, tt)
    Y = sa.nm_shared_spmm(val_g, mask_g, n, m, tt, dev(wt))
    assert_close(Y, spmm.nm_shared_spmm(vals, tile_keep, tt, wt))


@pytest.mark.parametrize("stages", [3, 4, 6])
def test_nm_shared_whole_tile_stages_agree(stages):
    """Every stage count gives the same bits (the MFMA sequence does not
    depend on it)."""
    T, d_in, d_out, tt = 384, 2048, 264, 128
    X = syn.gaussian_f16((T, d_in), 1.0, 77)
    wt_g = dev(syn.weight_t(d_out, d_in, 78))
    mask_g, val_g = sa.act_sparsify_nm_shared(dev(X), 8, 16, tt)
    base = sa.nm_shared_spmm(val_g, mask_g, 8, 16, tt, wt_g).clone()
    try:
        sa.set_gemm_tuning(0, 0, stages)
        Y = sa.nm_shared_spmm(val_g, mask_g, 8, 16, tt, wt_g)
    finally:
        sa.set_gemm_tuning(0, 0, 0)
    assert torch.equal(Y, base)


@pytest.mark.parametrize("T,d_in,d_out", [(4096, 1024, 1024), (2048, 4096, 11008)])
@pytest.mark.parametrize("n,m,tt", [(2, 4, 32), (8, 16, 32), (16, 32, 32), (4, 16, 32),
                                    (8, 16, 128), (4, 16, 128), (8, 16, 256), (2, 4, 256)])
def test_nm_shared_full_shapes(T, d_in, d_out, n, m, tt):
    """Full sizes in the benchmarked launches: every tile's mask and every
    row's values bit-exact, every output row against the oracle's fp64
    masked matmul with each tile's mask applied to its tokens."""
    X = syn.gaussian_f16((T, d_in), 1.0, 5)
    wt = syn.weight_t(d_out, d_in, 41)
    X_g, wt_g = dev(X), dev(wt)
    mask_g, val_g = sa.act_sparsify_nm_shared(X_g, n, m, tt)
    Y = sa.nm_shared_spmm(val_g, mask_g, n, m, tt, wt_g)
    keep, tile_keep, vals = sparsify.nm_shared_sparsify(X, n, m, tt)
    assert np.array_equal(words(mask_g), sparsify.pack_mask(tile_keep))
    assert np.array_equal(host(val_g).view(np.uint16), vals.view(np.uint16))
    assert_close(Y, spmm.masked_matmul(X, keep, wt))


# ---------------------------------------------------------------------------
# roofline calibration kernel
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("nbytes", [16, 1 << 20, 45_020_672, (1 << 25) + 48])
def test_read_stream_reads_every_byte_once(nbytes):
    """The xor of the sink words equals the xor of every 32-bit word read:
    each 16-byte chunk is loaded exactly once, and nothing past nbytes."""
    words = nbytes // 4 + 64
    a = np.random.default_rng(nbytes % 997).integers(-2**31, 2**31 - 1, size=words,
                                                     dtype=np.int64).astype(np.int32)
    src = torch.from_numpy(a).to(DEV)
    sink = sa.read_stream(src, nbytes)
    got = np.bitwise_xor.reduce(host(sink).view(np.uint32))
    want = np.bitwise_xor.reduce(a[: nbytes // 4].view(np.uint32))
    assert got == want


def test_plan_query_matches_the_device():
    """The host-side plan with this device's facts equals the one computed
    for a 256-CU part with 8 resident workgroups (what the CPU tests pin)."""
    for op, d_out, d_in, b in [("threshold", 4096, 11008, 1), ("dense", 1024, 4096, 1),
                               ("threshold", 22016, 4096, 1), ("masked", 4096, 4096, 8)]:
        here = sa.gemv_plan(op, d_out, d_in, b)
        fixed = sa.gemv_plan(op, d_out, d_in, b, cus=256, resident=8)
        assert here == fixed, (op, d_out, d_in, b, here, fixed)


def _zero_region_is_zero(shapes):
    """The workspace's leading region (the hand-off counters) is all zero, as
    every call must leave it, for each (d_out, d_in, batch)."""
    torch.cuda.synchronize()
    ws = sa.workspace(DEV, 0)
    for d_out, d_in, b in shapes:
        nz = sa.workspace_zero_bytes(d_out, d_in, b)
        assert int(torch.count_nonzero(ws[:nz]).cpu()) == 0, (d_out, d_in, b)


def test_l2_handoff_recomputes_mixed_tiles():
    """The L2-local hand-off checks that every slice of a tile ran on one
    XCD.  With the placement reported wrong on purpose (host-set hook; every
    kernel still exits normally) the last workgroup of each tile recomputes
    the other slices' partials itself: every one-launch entry point gives
    its normal bits, and the counters come back to zero."""
    d_out, d_in, _ = syn.LLAMA2_7B["down"]
    wt = syn.weight_t(d_out, d_in, 21)
    x = syn.laplace_f16((d_in,), 1.0, 22)
    t = 0.69
    keep = sparsify.threshold_sparsify(x, t)[0]
    wt_g, x_g = dev(wt), dev(x)
    xb = dev(syn.laplace_f16((2, d_in), 1.0, 23))
    g, u = (dev(a) for a in syn.swiglu_gate_up(d_in, d_out, 24))
    cn = sa.weight_col_norms(wt_g)
    mu = dev(syn.gaussian_f16((d_in,), 0.25, 25))
    _, i1, v1, n1 = sa.act_sparsify_threshold(x_g, t)
    for op in ("threshold", "dense", "list"):
        assert sa.gemv_plan(op, d_out, d_in)["handoff"] == 3
    assert sa.gemv_plan("threshold", d_out, d_in, 2)["handoff"] == 3

    def run():
        return [sa.sparse_gemv_threshold(wt_g, x_g, t), sa.dense_gemv(wt_g, x_g),
                sa.sparse_gemv_threshold(wt_g, xb, t), sa.sparse_gemv(wt_g, i1, v1, n1),
                *sa.masked_swiglu_down(g, u, wt_g, 0.02, "rana", cn),
                *sa.masked_swiglu_down(g, u, wt_g, 0.02, "cats"),
                sa.sparse_gemv_scored(wt_g, x_g, 0.7, mu=mu, colnorm=cn, var=True)]

    ref = [o.clone() for o in run()]
    try:
        sa.set_gemv_test_hooks(1)
        for _ in range(3):
            for j, (a, b) in enumerate(zip(run(), ref)):
                assert torch.equal(a, b), j
    finally:
        sa.set_gemv_test_hooks(0)
    for _ in range(2):
        for j, (a, b) in enumerate(zip(run(), ref)):
            assert torch.equal(a, b), j
    _zero_region_is_zero([(d_out, d_in, 1), (d_out, d_in, 2)])
    assert_close(ref[0], gemv.masked_gemv(wt, x, keep))
    assert_close(ref[1], gemv.dense_gemv(wt, x))


def test_workspace_growth_keeps_graphs_valid():
    """A graph captured with the GEMV workspace at one size keeps replaying
    correctly after a larger eager call has grown the workspace (the old
    buffer stays allocated and zero); growing during a capture is refused;
    the matmul scratch does not touch the GEMV workspace."""
    small = dev(syn.weight_t(1024, 2048, 51))
    xs = dev(syn.laplace_f16((2048,), 1.0, 52))
    big = dev(syn.weight_t(8192, 16384, 53))
    xl = dev(syn.laplace_f16((16384,), 1.0, 54))
    sa.sparse_gemv_threshold(small, xs, 0.7)
    eager = sa.sparse_gemv_threshold(small, xs, 0.7).clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = sa.sparse_gemv_threshold(small, xs, 0.7)
    before = sa.workspace(DEV, 0)
    sa.workspace(DEV, before.numel() + 1)  # an eager call of a larger shape grows it like this
    y_big = sa.sparse_gemv_threshold(big, xl, 0.7)
    X = dev(syn.gaussian_f16((256, 1024), 1.0, 55))
    W = dev(syn.weight_t(512, 1024, 56))
    xm, xv = sa.act_sparsify_nm(X, 8, 16)
    sa.nm_act_spmm(xv, xm, 8, 16, W)  # scratch of its own
    torch.cuda.synchronize()
    assert sa.workspace(DEV, 0).data_ptr() != before.data_ptr()
    for _ in range(3):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        assert torch.equal(sa.sparse_gemv_threshold(big, xl, 0.7), y_big)
    need = sa.workspace(DEV, 0).numel() + 1
    g2 = torch.cuda.CUDAGraph()
    with pytest.raises(RuntimeError):
        with torch.cuda.graph(g2):
            sa.workspace(DEV, need)
    _zero_region_is_zero([(1024, 2048, 1), (8192, 16384, 1)])


def test_graph_replays_match_eager():
    """Calls captured in a HIP graph and replayed several times, with eager
    calls and synchronisations between the replays, give the eager results
    bit for bit: the one-launch hand-off's counters, in L2 or written
    through, come back to zero on every replay, and the two-launch and
    full-K paths hold no state."""
    d_out, d_in = 4096, 11008
    wt = dev(syn.weight_t(d_out, d_in, 41))
    x = dev(syn.laplace_f16((d_in,), 1.0, 42))
    xb = dev(syn.laplace_f16((4, d_in), 1.0, 43))
    t = 0.69
    _, i1, v1, n1 = sa.act_sparsify_threshold(x, t)
    mb = sa.act_sparsify_threshold(xb, t)[0]
    tall = dev(syn.weight_t(11008, 4096, 44))
    xt = dev(syn.gaussian_f16((2, 4096), 1.0, 45))
    small = dev(syn.weight_t(1024, 4096, 46))
    xs = dev(syn.gaussian_f16((4096,), 1.0, 47))
    g, u = (dev(a) for a in syn.swiglu_gate_up(d_in, d_out, 6))
    X = dev(syn.gaussian_f16((256, 1024), 1.0, 48))
    W = dev(syn.weight_t(512, 1024, 49))
    xm, xv = sa.act_sparsify_nm(X, 2, 4)

    def run():
        outs = [sa.sparse_gemv_threshold(wt, x, t),          # one launch, in L2
                sa.dense_gemv(wt, x),
                sa.sparse_gemv_threshold(tall, xt[0], 0.6745),  # one launch, written through
                sa.sparse_gemv_threshold(tall, xt, 0.6745),     # batch 2: two launches
                sa.masked_gemv(wt, xb, mb),                     # batch 4: two launches
                sa.sparse_gemv(wt, i1, v1, n1),
                sa.sparse_gemv_threshold(small, xs, 0.6745),    # small weight, narrow tiles
                sa.nm_act_spmm(xv, xm, 2, 4, W)]
        outs += list(sa.masked_swiglu_down(g, u, wt, 0.02, "cats"))
        outs += list(sa.act_sparsify_topk(xb, 5504))
        return outs

    eager = [o.clone() for o in run()]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = run()
    for r in range(4):
        sa.sparse_gemv_threshold(wt, x, t)  # eager work on the same workspace
        sa.masked_gemv(wt, xb, mb)
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(zip(outs, eager)):
            assert torch.equal(a, b), (r, j)

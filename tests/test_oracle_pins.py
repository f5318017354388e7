"""Pins of the CPU oracle to facts outside itself (run with -m "not gpu").

Each test checks the oracle against something the pages or the mathematics
fix: values the pages print (golden files), closed forms, invariants, special
cases that reduce to a library routine, and brute-force enumeration on tiny
inputs.  Together they are meant to fail on any plausible slip in the oracle
(a dropped term, a wrong comparator, sign or index, a transposed operand).
"""

import math

import numpy as np
import pytest
from scipy import stats

import synthetic as syn
from oracle import brute, calibrate, correct, gemv, rana, sparsify, spmm, swiglu


# --------------------------------------------------------------------------
# threshold sparsifier
# --------------------------------------------------------------------------

def test_threshold_hand_case_keeps_equal_magnitude():
    x = np.array([0.5, -0.5, 0.25, 0.0, -1.0, -0.0, 0.75], dtype=np.float16)
    keep, idx, val, nnz = sparsify.threshold_sparsify(x, 0.5)
    assert keep.tolist() == [True, True, False, False, True, False, True]
    assert idx.tolist() == [0, 1, 4, 6]
    assert val.astype(np.float64).tolist() == [0.5, -0.5, -1.0, 0.75]
    assert nnz == 4


def test_threshold_matches_python_loop():
    for seed in range(5):
        x = syn.laplace_f16((257,), 1.0, seed)
        t = float(np.float32(0.3 + 0.1 * seed))
        keep = sparsify.threshold_sparsify(x, t)[0]
        assert np.array_equal(keep, brute.threshold_loop(x, t))


def test_threshold_zero_is_dense_product():
    """t = 0 keeps every nonzero, so W x_s equals the dense product W x."""
    x = syn.gaussian_f16((300,), 1.0, 7)
    x[::17] = 0
    wt = syn.weight_t(96, 300, 11)
    keep, idx, val, nnz = sparsify.threshold_sparsify(x, 0.0)
    assert nnz == np.count_nonzero(x)
    y = gemv.sparse_gemv(wt, idx, val)
    ref = x.astype(np.float64) @ wt.astype(np.float64)  # numpy matmul
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_sparsity_definition_identity():
    """Q-Sparse replies: sparsity is the fraction of zeros of the activation."""
    for seed in range(4):
        x = syn.gaussian_f16((1024,), 1.0, seed)
        t = float(np.float32(0.6745))
        keep, idx, val, nnz = sparsify.threshold_sparsify(x, t)
        xs = sparsify.apply_mask(x, keep)
        assert sparsify.activation_sparsity(xs) == 1.0 - nnz / 1024


def test_threshold_equals_topk_with_distinct_magnitudes():
    x = (np.random.default_rng(3).permutation(512).astype(np.float32) + 1) / 64
    x = (x * np.where(np.arange(512) % 3 == 0, -1, 1)).astype(np.float16)
    assert len(np.unique(np.abs(x))) == 512
    t = float(np.sort(np.abs(x.astype(np.float64)))[200])
    keep = sparsify.threshold_sparsify(x, t)[0]
    keep_k = sparsify.topk_sparsify(x, int(keep.sum()))[0]
    assert np.array_equal(keep, keep_k)


def test_threshold_rows():
    X = syn.gaussian_f16((3, 64), 1.0, 5)
    keep, idx, val, nnz = sparsify.threshold_sparsify(X, 0.5)
    for r in range(3):
        k1, i1, v1, n1 = sparsify.threshold_sparsify(X[r], 0.5)
        assert np.array_equal(keep[r], k1) and np.array_equal(idx[r], i1) and nnz[r] == n1


# --------------------------------------------------------------------------
# Top-K
# --------------------------------------------------------------------------

def test_topk_hand_ties_to_lower_index():
    x = np.array([1.0, -2.0, 2.0, 1.0, -1.0, 0.0], dtype=np.float16)
    assert sparsify.topk_sparsify(x, 2)[1].tolist() == [1, 2]
    assert sparsify.topk_sparsify(x, 3)[1].tolist() == [0, 1, 2]
    assert sparsify.topk_sparsify(x, 4)[1].tolist() == [0, 1, 2, 3]
    assert sparsify.topk_sparsify(x, 0)[3] == 0
    assert sparsify.topk_sparsify(x, 6)[1].tolist() == [0, 1, 2, 3, 4, 5]


def test_topk_signed_zero_is_a_tie():
    x = np.array([-0.0, 0.0, -0.0, 1.0], dtype=np.float16)
    assert sparsify.topk_sparsify(x, 2)[1].tolist() == [0, 3]


@pytest.mark.parametrize("seed", range(12))
def test_topk_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    d = int(rng.integers(1, 13))
    # few distinct magnitudes so ties are common; includes signed zeros
    pool = np.array([0.0, -0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0, 0.125], dtype=np.float16)
    x = pool[rng.integers(0, len(pool), size=d)]
    for k in range(0, d + 1):
        keep = sparsify.topk_sparsify(x, k)[0]
        assert np.array_equal(keep, brute.topk_brute(x, k)), (x, k)
        assert keep.sum() == k


def test_topk_percent_to_sparsity(golden):
    """TopK = 60/50/40 % keeps 60/50/40 % of entries: sparsity 40/50/60 %."""
    for topk_pct, sp_pct in golden("topk_sparsity.txt"):
        for d in (4096, 11008):
            k = syn.topk_k(int(topk_pct), d)
            x = syn.laplace_f16((d,), 1.0, 0)
            keep = sparsify.topk_sparsify(x, k)[0]
            sp = sparsify.activation_sparsity(sparsify.apply_mask(x, keep))
            assert abs(sp - int(sp_pct) / 100) < 1.0 / d


# --------------------------------------------------------------------------
# N:M
# --------------------------------------------------------------------------

def test_nm_layout_counts_match_pages(golden):
    for n, m, count in golden("nm_layout_counts.txt"):
        assert len(brute.nm_layouts(int(n), int(m))) == int(count)


def test_nm_hand_case():
    x = np.array([3, -1, 4, 1, -5, 9, 2, -6], dtype=np.float16)
    keep, vals = sparsify.nm_sparsify(x, 2, 4)
    assert keep.tolist() == [True, False, True, False, False, True, False, True]
    assert vals.astype(np.float64).tolist() == [3.0, 4.0, 9.0, -6.0]


@pytest.mark.parametrize("n,m", [(1, 4), (2, 4), (3, 4), (2, 8), (4, 8), (7, 8)])
def test_nm_brute_force(n, m):
    rng = np.random.default_rng(n * 31 + m)
    pool = np.array([0.0, -0.0, 0.5, -0.5, 1.0, -1.0, 3.0, 0.25], dtype=np.float16)
    x = pool[rng.integers(0, len(pool), size=4 * m)]
    keep, vals = sparsify.nm_sparsify(x, n, m)
    assert np.array_equal(keep, brute.nm_brute(x, n, m))
    assert np.all(keep.reshape(-1, m).sum(axis=1) == n)
    assert np.array_equal(vals, x[keep])


def test_nm_brute_force_16():
    rng = np.random.default_rng(5)
    pool = np.array([0.0, 0.5, -0.5, 1.0, -1.0, 2.0], dtype=np.float16)
    x = pool[rng.integers(0, len(pool), size=32)]
    keep = sparsify.nm_sparsify(x, 8, 16)[0]
    assert np.array_equal(keep, brute.nm_brute(x, 8, 16))


def test_nm_whole_row_equals_topk_and_full_is_dense():
    x = syn.gaussian_f16((2, 64), 1.0, 9)
    for r in range(2):
        keep_nm = sparsify.nm_sparsify(x[r], 20, 64)[0]
        keep_k = sparsify.topk_sparsify(x[r], 20)[0]
        assert np.array_equal(keep_nm, keep_k)
    keep, vals = sparsify.nm_sparsify(x, 8, 8)
    assert keep.all() and np.array_equal(vals, x)


# --------------------------------------------------------------------------
# tile-shared N:M
# --------------------------------------------------------------------------

def test_nm_shared_hand_case():
    # per token the 2:4 choices differ ({0,2} / {1,3} in the first group); the
    # tile's summed magnitudes are [4, 3, 2, 2] and [2, 2, 5, 3]
    X = np.array([[4, 0, 1, 0, 1, 2, 0, 3],
                  [0, 3, -1, 2, -1, 0, 5, 0]], dtype=np.float16)
    keep, tile_keep, vals = sparsify.nm_shared_sparsify(X, 2, 4, 2)
    assert tile_keep.tolist() == [[True, True, False, False, False, False, True, True]]
    assert np.array_equal(keep, np.repeat(tile_keep, 2, axis=0))
    assert vals.astype(np.float64).tolist() == [[4, 0, 0, 3], [0, 3, 5, 0]]
    # equal scores: the lower positions
    ties = np.array([[1, -1, 1, 1], [-1, 1, 1, 1]], dtype=np.float16)
    assert sparsify.nm_shared_sparsify(ties, 2, 4, 2)[1].tolist() == [[True, True, False, False]]


@pytest.mark.parametrize("n,m", [(2, 4), (1, 4), (8, 16), (16, 32), (4, 8)])
def test_nm_shared_one_token_tiles_are_per_token(n, m):
    X = syn.gaussian_f16((9, 64), 1.0, 11)
    keep, tile_keep, vals = sparsify.nm_shared_sparsify(X, n, m, 1)
    k1, v1 = sparsify.nm_sparsify(X, n, m)
    assert np.array_equal(keep, k1) and np.array_equal(tile_keep, k1)
    assert np.array_equal(vals, v1)


def test_nm_shared_identical_rows_take_the_row_pattern():
    row = syn.gaussian_f16((1, 64), 1.0, 12)
    X = np.repeat(row, 32, axis=0)
    keep, tile_keep, _ = sparsify.nm_shared_sparsify(X, 8, 16, 32)
    assert np.array_equal(tile_keep[0], sparsify.nm_sparsify(row, 8, 16)[0][0])


@pytest.mark.parametrize("n,m,tt,T", [(2, 4, 2, 5), (1, 4, 3, 7), (3, 8, 4, 9), (8, 16, 32, 40),
                                      (5, 8, 6, 6)])
def test_nm_shared_brute_force(n, m, tt, T):
    """Exhaustive layouts on the tile scores, summed by a plain loop; ragged
    last tiles and tied scores included."""
    rng = np.random.default_rng(n * 97 + m * 7 + tt)
    pool = np.array([0.0, -0.0, 0.5, -0.5, 1.0, -1.0, 2.0, 0.25], dtype=np.float16)
    d = 2 * m
    X = pool[rng.integers(0, len(pool), size=T * d)].reshape(T, d)
    keep, tile_keep, vals = sparsify.nm_shared_sparsify(X, n, m, tt)
    tiles = (T + tt - 1) // tt
    assert tile_keep.shape == (tiles, d)
    for g in range(tiles):
        rows = range(g * tt, min(T, (g + 1) * tt))
        scores = np.array([sum(abs(float(X[t][k])) for t in rows) for k in range(d)])
        assert np.array_equal(tile_keep[g], brute.nm_brute(scores, n, m))
        for t in rows:
            assert np.array_equal(keep[t], tile_keep[g])
            assert np.array_equal(vals[t], X[t][tile_keep[g]])
    assert np.all(keep.reshape(T, -1, m).sum(axis=-1) == n)


def test_nm_shared_score_is_exact():
    """The largest and smallest fp16 magnitudes in one 256-token tile: the
    exact sums (rational arithmetic) decide, where an fp32 sum would tie."""
    from fractions import Fraction
    T = 256
    X = np.zeros((T, 4), dtype=np.float16)
    X[:255, 0] = 65504.0
    X[:255, 1] = -65504.0
    X[255, 1] = np.float16(2.0 ** -24)   # smallest subnormal
    X[:, 2] = np.float16(2.0 ** -14)
    X[7, 3] = np.float16(-3.0)
    exact = [sum(Fraction(abs(float(v))) for v in X[:, k]) for k in range(4)]
    assert exact[1] > exact[0]
    f32 = np.float32(0)
    for v in X[:, 1]:
        f32 = np.float32(f32 + np.float32(abs(float(v))))
    assert f32 == np.float32(255 * 65504.0)   # fp32 loses the last term
    _, tile_keep, _ = sparsify.nm_shared_sparsify(X, 1, 4, 256)
    assert tile_keep.tolist() == [[False, True, False, False]]
    _, tile_keep, _ = sparsify.nm_shared_sparsify(X, 2, 4, 256)
    assert tile_keep.tolist() == [[True, True, False, False]]
    _, tile_keep, _ = sparsify.nm_shared_sparsify(X, 3, 4, 256)
    assert tile_keep.tolist() == [[True, True, False, True]]  # 3 > 256 * 2^-14


def test_nm_shared_spmm_is_the_masked_matmul():
    X = syn.gaussian_f16((40, 64), 1.0, 13)
    wt = syn.weight_t(24, 64, 14)
    for (n, m, tt) in [(8, 16, 16), (2, 4, 32), (1, 4, 7)]:
        keep, tile_keep, vals = sparsify.nm_shared_sparsify(X, n, m, tt)
        np.testing.assert_allclose(spmm.nm_shared_spmm(vals, tile_keep, tt, wt),
                                   spmm.nm_spmm(X, keep, wt), rtol=1e-12, atol=1e-13)
    keep, tile_keep, vals = sparsify.nm_shared_sparsify(X, 4, 4, 32)
    np.testing.assert_allclose(spmm.nm_shared_spmm(vals, tile_keep, 32, wt),
                               X.astype(np.float64) @ wt.astype(np.float64), rtol=1e-12,
                               atol=1e-13)


# --------------------------------------------------------------------------
# mask packing
# --------------------------------------------------------------------------

def test_pack_mask_bit_order():
    keep = np.zeros(40, dtype=bool)
    keep[[0, 3, 31, 32, 39]] = True
    w = sparsify.pack_mask(keep)
    assert w.tolist() == [(1 << 0) | (1 << 3) | (1 << 31), (1 << 0) | (1 << 7)]
    assert np.array_equal(sparsify.unpack_mask(w, 40), keep)


# --------------------------------------------------------------------------
# GEMV
# --------------------------------------------------------------------------

def test_gemv_identity_weight_returns_sparse_activation():
    d = 64
    wt = np.eye(d, dtype=np.float16)
    x = syn.gaussian_f16((d,), 1.0, 2)
    keep, idx, val, _ = sparsify.threshold_sparsify(x, 0.7)
    y = gemv.sparse_gemv(wt, idx, val)
    assert np.array_equal(y, sparsify.apply_mask(x, keep))


def test_gemv_rank_one_closed_form():
    """W = b a^T (W[o][k] = b_o a_k) gives y = b * (a . x_s)."""
    a = np.array([1, 2, -1, 0.5, 4, -2], dtype=np.float16)
    b = np.array([1, -3, 0.25, 2], dtype=np.float16)
    wt = np.outer(a, b).astype(np.float16)  # WT[k][o] = a_k b_o, exact
    x = np.array([0.5, -1, 2, 0.25, -0.125, 1], dtype=np.float16)
    keep, idx, val, _ = sparsify.threshold_sparsify(x, 0.5)  # keeps 0,1,2,5
    y = gemv.sparse_gemv(wt, idx, val)
    dot = 1 * 0.5 + 2 * -1 + -1 * 2 + -2 * 1
    assert y.tolist() == [1 * dot, -3 * dot, 0.25 * dot, 2 * dot]


def test_gemv_order_free_and_linear():
    wt = syn.weight_t(128, 200, 3)
    x = syn.laplace_f16((200,), 1.0, 4)
    _, idx, val, _ = sparsify.threshold_sparsify(x, 0.69)
    y = gemv.sparse_gemv(wt, idx, val)
    perm = np.random.default_rng(0).permutation(len(idx))
    np.testing.assert_allclose(gemv.sparse_gemv(wt, idx[perm], val[perm]), y, rtol=1e-12, atol=1e-13)
    y2 = gemv.sparse_gemv(wt, idx, (val.astype(np.float64) * 2))
    assert np.array_equal(y2, 2 * y)


def test_gemv_dense_matches_library_matmul():
    wt = syn.weight_t(72, 130, 8)
    x = syn.gaussian_f16((130,), 1.0, 1)
    ref = x.astype(np.float64) @ wt.astype(np.float64)
    np.testing.assert_allclose(gemv.dense_gemv(wt, x), ref, rtol=1e-12, atol=1e-13)


def test_gemv_flops_formula(golden):
    for d, flops in golden("gemv_flops.txt"):
        assert gemv.gemv_flops(int(d), int(d)) == int(flops)
    assert gemv.gemv_flops(4096, 5504) == 45088768


def test_batched_union_and_rows():
    wt = syn.weight_t(64, 96, 5)
    X = syn.laplace_f16((4, 96), 1.0, 6)
    keep = np.stack([sparsify.topk_sparsify(X[b], 40)[0] for b in range(4)])
    Y = gemv.batched_masked_gemv(wt, X, keep)
    for b in range(4):
        ref = sparsify.apply_mask(X[b], keep[b]) @ wt.astype(np.float64)
        np.testing.assert_allclose(Y[b], ref, rtol=1e-12, atol=1e-13)
    assert gemv.union_columns(keep[:1]) == 40


def test_union_columns_hand_case():
    """Rows {0, 1}, {1, 2} and {4} of 5 columns: the union has 4 columns, the
    intersection of the first two 1 and no single row more than 2, so a
    union/intersection or row slip gives another count."""
    keep = np.zeros((3, 5), dtype=bool)
    keep[0, [0, 1]] = True
    keep[1, [1, 2]] = True
    keep[2, 4] = True
    assert gemv.union_columns(keep) == 4
    assert gemv.union_columns(keep[:2]) == 3
    assert gemv.union_columns(keep[[0, 2]]) == 3
    assert gemv.union_columns(keep[2:]) == 1
    assert gemv.union_columns(np.zeros((2, 5), dtype=bool)) == 0


# --------------------------------------------------------------------------
# SiLU / masked SwiGLU down
# --------------------------------------------------------------------------

def test_fused_projection_is_the_members_side_by_side():
    """A fused projection (one sparsified input, the members' weights side by
    side) gives each member's own sparse GEMV in its output block, computed
    here member by member with numpy's matmul on the masked input."""
    x = syn.activation((4096,), "gaussian", 3)
    t = 0.6745
    keep, idx, val, nnz = sparsify.threshold_sparsify(x, t)
    xs = np.where(keep, x.astype(np.float64), 0.0)
    for name, (members, inp) in syn.LLAMA2_7B_FUSED.items():
        assert syn.LLAMA2_7B_INPUTS[inp][0] == 4096
        wt = syn.fused_weight_t(name)
        y = gemv.sparse_gemv(wt, idx, val)
        o = 0
        for m in members:
            d_out, d_in, m_inp = syn.LLAMA2_7B[m]
            assert (d_in, m_inp) == (4096, inp)
            w = syn.weight_t(d_out, d_in, syn.weight_seed(m))
            assert np.array_equal(wt[:, o:o + d_out], w)
            np.testing.assert_allclose(y[o:o + d_out], xs @ w.astype(np.float64), rtol=1e-12,
                                       atol=1e-12)
            o += d_out
        assert o == wt.shape[1] == len(y)


# --------------------------------------------------------------------------
# RaNA linear-layer rank adapter
# --------------------------------------------------------------------------

def test_rank_adapter_t0_is_the_dense_chain_and_large_t_is_zero():
    """t = 0 keeps every entry: y = A fp16(B x) by numpy's matmul; a
    threshold above every v_i^2 keeps none: y = 0."""
    bt, at = syn.weight_t(64, 96, 1), syn.weight_t(40, 64, 2)
    x = syn.gaussian_f16((96,), 1.0, 3)
    v, v16, keep, y = rana.rank_adapter(bt, at, x, 0.0)
    np.testing.assert_allclose(v, x.astype(np.float64) @ bt.astype(np.float64), rtol=1e-12,
                               atol=1e-14)
    assert keep.all() and np.array_equal(v16, v.astype(np.float16))
    np.testing.assert_allclose(y, v16.astype(np.float64) @ at.astype(np.float64), rtol=1e-12,
                               atol=1e-14)
    _, _, keep, y = rana.rank_adapter(bt, at, x, 1e6)
    assert not keep.any() and np.all(y == 0)


def test_rank_adapter_mask_at_an_exact_square():
    """With B = A = I, v = x and y = m ⊙ x.  At t = 0.25 the mask is
    |x| >= 0.5 exactly: +-0.5 are kept, the fp16 neighbours below are not."""
    below = float(np.nextafter(np.float16(0.5), np.float16(0)))
    x = np.array([0.5, -0.5, below, -below, 0.0, 2.0, -0.25, 0.75], dtype=np.float16)
    eye = np.eye(8, dtype=np.float16)
    v, v16, keep, y = rana.rank_adapter(eye, eye, x, 0.25)
    assert np.array_equal(v16, x)
    assert keep.tolist() == [True, True, False, False, False, True, False, True]
    assert np.array_equal(y, np.where(keep, x.astype(np.float64), 0.0))


def test_rank_adapter_given_v_decides_the_mask():
    """A v from another implementation (fp16) is masked and multiplied as
    given; here it differs from the oracle's own rounding by one ulp at one
    entry placed exactly on the threshold."""
    bt, at = syn.weight_t(16, 32, 4), syn.weight_t(24, 16, 5)
    x = syn.gaussian_f16((32,), 1.0, 6)
    v, v16, _, _ = rana.rank_adapter(bt, at, x, 0.0)
    other = v16.copy()
    other[3] = np.nextafter(v16[3], np.float16(np.inf) if v16[3] >= 0 else np.float16(-np.inf))
    t = float(np.float64(other[3]) ** 2)
    _, _, keep_o, y_o = rana.rank_adapter(bt, at, x, t, v16=other)
    assert keep_o[3]
    idx = np.flatnonzero(keep_o)
    np.testing.assert_allclose(y_o, other[idx].astype(np.float64) @ at[idx].astype(np.float64),
                               rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("seed", range(4))
def test_rank_adapter_matches_scalar_loops(seed):
    r, d_in, d_out = 12, 20, 9 + seed
    bt, at = syn.weight_t(r, d_in, 10 + seed, std=0.3), syn.weight_t(d_out, r, 20 + seed)
    x = syn.gaussian_f16((d_in,), 1.0, 30 + seed)
    v, v16, keep, y = rana.rank_adapter(bt, at, x, 0.5)
    assert 0 < keep.sum() < r
    np.testing.assert_allclose(y, brute.rank_adapter_loop(bt, at, x, 0.5), rtol=1e-12,
                               atol=1e-13)


# --------------------------------------------------------------------------
# weight-aware selection, static shift, variance correction
# --------------------------------------------------------------------------

def test_scored_selection_reduces_to_the_plain_rules():
    """No shift and no weights: the scored threshold and N:M are the plain
    magnitude threshold and N:M; weights all equal to 2 halve the threshold."""
    x = syn.laplace_f16((256,), 1.0, 8)
    for t in (0.0, 0.5, 1.25):
        plain = sparsify.threshold_sparsify(x, t)[0]
        assert np.array_equal(correct.threshold_keep(correct.shift(x, None), None, t), plain)
        assert np.array_equal(correct.threshold_keep(x, np.full(256, 2.0), 2 * t), plain)
    x[::9] = np.float16(0.5)  # ties
    for n, m in ((2, 4), (8, 16), (16, 32)):
        plain = sparsify.nm_sparsify(x[None], n, m)[0][0]
        assert np.array_equal(correct.nm_keep(x, None, n, m), plain)
        assert np.array_equal(correct.nm_keep(x, np.full(256, 3.0), n, m), plain)


def test_scored_selection_hand_case():
    """Weights reorder the choice: entry 1 is smaller than entry 0 but its
    column is three times as large; equal scores keep the lower index."""
    x = np.array([2.0, -1.0, 0.5, -0.5], dtype=np.float16)
    c = np.array([1.0, 3.0, 4.0, 2.0])
    assert correct.scores(x, c).tolist() == [2.0, 3.0, 2.0, 1.0]
    assert correct.nm_keep(x, c, 2, 4).tolist() == [True, True, False, False]
    assert correct.threshold_keep(x, c, 2.0).tolist() == [True, True, True, False]


def test_shift_and_bias_give_back_the_dense_product():
    """t = 0 and an exactly representable shift: W s(x - mu) + W mu = W x,
    checked against numpy's matmul (the bias term and the shift's sign)."""
    wt = syn.weight_t(48, 64, 9)
    rng = np.random.default_rng(10)
    x = (rng.integers(-64, 64, size=64) / 16.0).astype(np.float16)  # multiples of 1/16
    mu = np.full(64, 0.5, dtype=np.float16)
    xs = correct.shift(x, mu)
    np.testing.assert_array_equal(xs.astype(np.float64), x.astype(np.float64) - 0.5)
    _, keep, alpha, y = correct.corrected_gemv(
        wt, x, mu, None, lambda v, c: correct.threshold_keep(v, c, 0.0), var=True)
    assert alpha == 1.0  # only exact zeros are dropped
    np.testing.assert_allclose(y, x.astype(np.float64) @ wt.astype(np.float64), rtol=1e-12,
                               atol=1e-13)


def test_variance_correction_hand_case():
    """x' = [3, 4, 0, 0] keeping only 3: alpha = sqrt(25 / 9) = 5/3, so the
    output is 5 times column 0 of W."""
    x = np.array([3.0, 4.0, 0.0, 0.0], dtype=np.float16)
    wt = syn.weight_t(8, 4, 11)
    keep1 = np.array([True, False, False, False])
    assert correct.var_alpha(x, keep1) == pytest.approx(5.0 / 3.0, rel=1e-15)
    assert correct.var_alpha(x, np.zeros(4, bool)) == 1.0
    _, _, alpha1, y1 = correct.corrected_gemv(wt, x, None, None, lambda v, c: keep1, var=True)
    np.testing.assert_allclose(y1, 5.0 * wt[0].astype(np.float64), rtol=1e-14)


def test_column_norms_match_the_swiglu_oracle():
    wt = syn.weight_t(24, 40, 12)
    np.testing.assert_allclose(correct.column_norms(wt), swiglu.column_norms(wt), rtol=1e-15)


def test_silu_closed_forms():
    assert swiglu.silu(np.array([0.0]))[0] == 0.0
    # sigmoid(ln 3) = 3/4
    z = math.log(3.0)
    assert abs(swiglu.silu(np.array([z]))[0] - 0.75 * z) < 1e-15
    # SiLU(z) - SiLU(-z) = z (sigmoid(z) + sigmoid(-z) = 1)
    zs = np.linspace(-12, 12, 97)
    np.testing.assert_allclose(swiglu.silu(zs) - swiglu.silu(-zs), zs, rtol=1e-13, atol=1e-14)
    # tails: -> z for large z, -> 0 for very negative z
    assert abs(swiglu.silu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(swiglu.silu(np.array([-40.0]))[0]) < 1e-15
    assert swiglu.silu(np.array([-60000.0]))[0] == 0.0


def test_column_norms():
    wdt = np.array([[3, 4, 0], [1, 0, 0], [0, 0, 0], [1, 1, 1]], dtype=np.float16)
    c = swiglu.column_norms(wdt)
    assert c[:3].tolist() == [5.0, 1.0, 0.0]
    assert abs(c[3] - math.sqrt(3)) < 1e-15
    w = syn.weight_t(64, 48, 2)
    np.testing.assert_allclose(swiglu.column_norms(w), np.linalg.norm(w.astype(np.float64), axis=1),
                               rtol=1e-14)


@pytest.mark.parametrize("mode", ["cats", "rana"])
def test_swiglu_t0_is_dense_down(mode):
    g, u = syn.swiglu_gate_up(256, 64, 1)
    wdt = syn.weight_t(48, 256, 12)
    keep, y = swiglu.masked_swiglu_down(g, u, wdt, 0.0, mode)
    assert keep.all()
    h = swiglu.silu(g) * u.astype(np.float64)
    np.testing.assert_allclose(y, h @ wdt.astype(np.float64), rtol=1e-12, atol=1e-13)


def test_swiglu_special_cases():
    g, u = syn.swiglu_gate_up(512, 256, 2)
    wdt = syn.weight_t(32, 512, 13)
    h = swiglu.silu(g) * u.astype(np.float64)
    # all column norms equal: RaNA is a threshold on |h|
    c = np.full(512, 2.0)
    sc = swiglu.scores(g, u, "rana", c)
    assert np.array_equal(sc >= 0.8, np.abs(h) >= 0.4)
    # u = 1: RaNA score is the CATS score times the column norm
    ones = np.ones(512, dtype=np.float16)
    cn = swiglu.column_norms(wdt)
    np.testing.assert_allclose(swiglu.scores(g, ones, "rana", cn),
                               swiglu.scores(g, ones, "cats") * cn, rtol=1e-15)
    # the masked sum is the dense product of the masked hidden vector
    keep, y = swiglu.masked_swiglu_down(g, u, wdt, 0.3, "cats")
    assert np.array_equal(keep, np.abs(swiglu.silu(g)) >= 0.3)
    np.testing.assert_allclose(y, np.where(keep, h, 0.0) @ wdt.astype(np.float64), rtol=1e-12,
                               atol=1e-13)


@pytest.mark.parametrize("rate", [0.5, 0.7])
def test_mask_rate_threshold(rate):
    sc = np.random.default_rng(4).random(1000) + 0.1
    t = swiglu.threshold_for_mask_rate(sc, rate)
    assert np.count_nonzero(sc < t) == int(rate * 1000)
    gap = np.min(np.abs(sc - t))
    assert gap > 0
    g, u = syn.swiglu_gate_up(14336, 4096, 0)
    sc = swiglu.scores(g, u, "cats")
    t = swiglu.threshold_for_mask_rate(sc, rate)
    masked = np.count_nonzero(sc < t)
    assert abs(masked / 14336 - rate) < 0.01
    assert np.min(np.abs(sc - t)) > 1e-6 * t


# --------------------------------------------------------------------------
# batched N:M matmul
# --------------------------------------------------------------------------

def test_spmm_full_pattern_is_dense_matmul():
    X = syn.gaussian_f16((6, 32), 1.0, 3)
    wt = syn.weight_t(24, 32, 4)
    keep = sparsify.nm_sparsify(X, 4, 4)[0]
    Y = spmm.nm_spmm(X, keep, wt)
    np.testing.assert_allclose(Y, X.astype(np.float64) @ wt.astype(np.float64), rtol=1e-12,
                               atol=1e-13)


def test_masked_matmul_hand_case():
    """Token 0 keeps column 0 and token 1 column 1 of X = [[1, 2], [3, 4]];
    WT = [[1, 2, 3], [4, 5, 6]] gives Y = [[1, 2, 3], [16, 20, 24]].  A
    transposed operand or an unapplied mask gives other values."""
    X = np.array([[1, 2], [3, 4]], dtype=np.float16)
    keep = np.array([[True, False], [False, True]])
    wt = np.array([[1, 2, 3], [4, 5, 6]], dtype=np.float16)
    Y = spmm.masked_matmul(X, keep, wt)
    assert Y.tolist() == [[1.0, 2.0, 3.0], [16.0, 20.0, 24.0]]
    assert spmm.nm_spmm(X, keep, wt).tolist() == Y.tolist()


@pytest.mark.parametrize("n,m", [(2, 4), (8, 16), (16, 32)])
def test_masked_matmul_is_the_per_token_sum(n, m):
    """The one-matmul form equals the per-token sums over kept columns, for
    N:M masks, for an arbitrary mask, and for a tile-shared mask expanded to
    its tokens."""
    X = syn.gaussian_f16((37, 96), 1.0, 40 + m)
    wt = syn.weight_t(56, 96, 41 + m)
    keep = sparsify.nm_sparsify(X, n, m)[0]
    np.testing.assert_allclose(spmm.masked_matmul(X, keep, wt), spmm.nm_spmm(X, keep, wt),
                               rtol=1e-12, atol=1e-13)
    rnd = np.random.default_rng(m).random(X.shape) < 0.3
    np.testing.assert_allclose(spmm.masked_matmul(X, rnd, wt), spmm.nm_spmm(X, rnd, wt),
                               rtol=1e-12, atol=1e-13)
    _, tile_keep, vals = sparsify.nm_shared_sparsify(X, n, m, 8)
    expanded = np.repeat(tile_keep, 8, axis=0)[:X.shape[0]]
    np.testing.assert_allclose(spmm.masked_matmul(X, expanded, wt),
                               spmm.nm_shared_spmm(vals, tile_keep, 8, wt), rtol=1e-12,
                               atol=1e-13)


def test_spmm_rows_are_sparse_gemvs():
    X = syn.gaussian_f16((5, 64), 1.0, 6)
    wt = syn.weight_t(40, 64, 7)
    keep, vals = sparsify.nm_sparsify(X, 2, 4)
    Y = spmm.nm_spmm(X, keep, wt)
    for t in range(5):
        idx = np.flatnonzero(keep[t])
        assert np.array_equal(Y[t], gemv.sparse_gemv(wt, idx, vals[t]))
    assert spmm.nm_spmm_flops(4096, 1024, 1024, 2, 4) == 2 * 4096 * 1024 * 512


# --------------------------------------------------------------------------
# calibration
# --------------------------------------------------------------------------

def test_quantile_hand_cases():
    assert calibrate.quantile_linear([1, 2, 3, 4], 0.5) == 2.5
    assert calibrate.quantile_linear([4, 1, 3, 2], 0.0) == 1.0
    assert calibrate.quantile_linear([4, 1, 3, 2], 1.0) == 4.0
    assert calibrate.quantile_linear([5], 0.3) == 5.0
    assert calibrate.quantile_linear([0, 10], 0.25) == 2.5


def test_quantile_matches_numpy_linear():
    v = np.abs(syn.laplace_f16((10_000,), 1.0, 1).astype(np.float64))
    for s in (0.0, 0.1, 0.4, 0.5, 0.6, 0.9, 1.0):
        assert calibrate.quantile_linear(v, s) == pytest.approx(np.quantile(v, s), rel=0, abs=1e-15)


@pytest.mark.parametrize("s", [0.4, 0.5, 0.6])
def test_calibration_closed_forms(s):
    """|N(0,1)| quantile = Phi^-1((1+s)/2); |Laplace(0,1)| quantile = -ln(1-s)."""
    n = 10_000
    xg = syn.calibration_samples("attn_in", n)
    q = stats.norm.ppf((1 + s) / 2)
    sigma = math.sqrt(s * (1 - s) / n) / (2 * stats.norm.pdf(q))
    assert abs(float(calibrate.magnitude_threshold(xg, s)) - q) < 5 * sigma + 1e-3
    xl = syn.calibration_samples("down_in", n)
    ql = -math.log(1 - s)
    sigma_l = math.sqrt(s * (1 - s) / n) / math.exp(-ql)
    assert abs(float(calibrate.magnitude_threshold(xl, s)) - ql) < 5 * sigma_l + 1e-3
    # a calibrated threshold gives about the target sparsity on a fresh draw
    t = float(calibrate.magnitude_threshold(xl, s))
    x = syn.laplace_f16((11008,), 1.0, 42)
    keep = sparsify.threshold_sparsify(x, t)[0]
    assert abs((1 - keep.mean()) - s) < 0.03

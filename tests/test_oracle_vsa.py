"""Pins for the oracle's VSA block selection: pooling, FP64 block scores and
top-k (no GPU). Anchors: an exact int64 fixed-point sum, exact small-integer
dot products, numpy's lexsort as an independent ranking, and the planted,
all-equal and full-set special cases."""
import numpy as np
import torch

import oracle


def test_pool_equals_exact_fixed_point_mean():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((1, 2, 256, 16)).astype(np.float16)
    x[0, 0, :64, 0] = 65504.0  # largest FP16 values: the sum needs more than FP32
    x[0, 0, :64, 1] = np.float16(2.0 ** -24)
    ours = oracle.vsa_pool(x, 64)
    # every FP16 value is an integer multiple of 2^-24
    ints = (x.astype(np.float64) * 2.0 ** 24).astype(np.int64)
    sums = ints.reshape(1, 2, 4, 64, 16).sum(axis=3)
    exact = sums.astype(np.float64) / (2.0 ** 24 * 64)  # exact: |sums| < 2^53
    assert np.all(np.abs(sums) < 2 ** 53)
    assert np.array_equal(ours, exact.astype(np.float32))
    # torch float64 mean agrees for data whose sum is exact in any order
    tm = torch.from_numpy(x.astype(np.float64)).reshape(1, 2, 4, 64, 16).mean(3).float().numpy()
    assert np.array_equal(ours, tm)


def _nearest_f32(fr):
    """The float32 nearest to a Fraction, ties to even, by exact rational comparison."""
    from fractions import Fraction
    f = np.float32(float(fr))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - fr), int(np.array(c).view(np.uint32)) & 1))
    return best


def test_pool_partial_tile_is_the_exact_mean_rounded_once():
    """A last block of 37 valid rows: every mean equals the exactly computed
    rational sum / 37 rounded once to FP32 (not twice)."""
    from fractions import Fraction
    rng = np.random.default_rng(3)
    L, D = 64 + 37, 24
    x = (rng.standard_normal((1, 1, L, D)) * 100).astype(np.float16)
    ours = oracle.vsa_pool(x, 64)
    assert ours.shape == (1, 1, 2, D)
    ints = (x.astype(np.float64) * 2.0 ** 24).astype(np.int64)[0, 0]
    for t, (lo, hi) in enumerate([(0, 64), (64, L)]):
        for d in range(D):
            exact = Fraction(int(ints[lo:hi, d].sum()), 2 ** 24 * (hi - lo))
            assert ours[0, 0, t, d] == _nearest_f32(exact), (t, d)


def test_scores_exact_on_integer_vectors_and_within_bound_otherwise():
    rng = np.random.default_rng(1)
    qi = rng.integers(-50, 50, (1, 2, 10, 128)).astype(np.float32)
    ki = rng.integers(-50, 50, (1, 2, 10, 128)).astype(np.float32)
    s = oracle.vsa_scores(qi, ki)
    ref = np.einsum("bhid,bhjd->bhij", qi.astype(np.int64), ki.astype(np.int64))
    assert np.array_equal(s, ref.astype(np.float64))
    qf = rng.standard_normal((1, 1, 9, 128)).astype(np.float32)
    kf = rng.standard_normal((1, 1, 9, 128)).astype(np.float32)
    s = oracle.vsa_scores(qf, kf)
    from fractions import Fraction
    for i in range(9):
        for j in range(9):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qf[0, 0, i], kf[0, 0, j]))
            bound = 128 * 2.0 ** -53 * float(np.abs(qf[0, 0, i].astype(np.float64) * kf[0, 0, j]).sum())
            assert abs(float(Fraction(s[0, 0, i, j]) - exact)) <= bound


def _lexsort_topk(s, k):
    B, H, NB, _ = s.shape
    out = np.empty((B, H, NB, k), np.int32)
    cols = np.arange(NB)
    for b in range(B):
        for h in range(H):
            for i in range(NB):
                order = np.lexsort((cols, -s[b, h, i]))  # primary: score desc, then index asc
                out[b, h, i] = np.sort(order[:k])
    return out


def test_topk_matches_lexsort_with_many_ties():
    rng = np.random.default_rng(2)
    s = rng.integers(0, 7, (1, 3, 40, 40)).astype(np.float64)  # heavy ties
    for k in (1, 5, 13, 40):
        assert np.array_equal(oracle.vsa_topk(s, k), _lexsort_topk(s, k))
    s2 = rng.standard_normal((2, 2, 33, 33))
    assert np.array_equal(oracle.vsa_topk(s2, 8), _lexsort_topk(s2, 8))


def test_topk_special_cases():
    nb = 24
    eq = np.zeros((1, 1, nb, nb))
    assert np.array_equal(oracle.vsa_topk(eq, 5)[0, 0], np.broadcast_to(np.arange(5), (nb, 5)))
    full = oracle.vsa_topk(np.random.default_rng(3).standard_normal((1, 1, nb, nb)), nb)
    assert np.array_equal(full[0, 0], np.broadcast_to(np.arange(nb), (nb, nb)))


def test_select_picks_planted_dominant_block():
    rng = np.random.default_rng(4)
    L, D, blk = 512, 128, 64
    q = (rng.standard_normal((1, 2, L, D)) * 0.1).astype(np.float16)
    k = (rng.standard_normal((1, 2, L, D)) * 0.1).astype(np.float16)
    q[0, :, :, 0] = 1.0
    k[0, :, 5 * blk: 6 * blk, 0] = 4.0  # block 5 has a dominant mean along d=0
    idx, s = oracle.vsa_select(q, k, blk, 1)
    assert np.all(idx == 5)
    idx3, _ = oracle.vsa_select(q, k, blk, 3)
    assert np.all(np.any(idx3 == 5, axis=-1)) and np.all(np.diff(idx3, axis=-1) > 0)

"""Pins for the oracle's VSA block selection: pooling, FP64 block scores and
top-k (no GPU). Anchors: an exact int64 fixed-point sum, exact small-integer
dot products, numpy's lexsort as an independent ranking, and the planted,
all-equal and full-set special cases."""
import numpy as np
import pytest
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


# ---------------------------------------------------------------- block lists
# The list format of "[perf] FastH3 two-Spark: gather packed FP4 inputs before
# head projections", block_lists.py: 128-token blocks built from two 64-token
# halves, descending variable-length key-block lists, per-half valid counts
# and 4-bit quadrant masks (query half x 2 + key half).

def test_block_lists_tile128_is_the_mask_itself():
    """With 128-token tiles every tile is one block: a block is listed with all
    four quadrant bits exactly when the mask selects the tile."""
    rng = np.random.default_rng(3)
    mask = rng.random((2, 3, 9, 9)) < 0.3
    idx, counts, kv, quad = oracle.block_lists(mask, np.full(9, 128, np.int32), 128)
    assert np.array_equal(counts, mask.sum(-1))
    assert np.array_equal(kv, np.full(18, 64))
    for b, h, r in np.ndindex(2, 3, 9):
        want = np.nonzero(mask[b, h, r])[0][::-1]
        n = len(want)
        assert np.array_equal(idx[b, h, r, :n], want) and not idx[b, h, r, n:].any()
        assert np.all(quad[b, h, r, :n] == 15) and not quad[b, h, r, n:].any()


@pytest.mark.parametrize("i,j", [(0, 0), (0, 1), (1, 0), (1, 1), (6, 3), (3, 6)])
def test_block_lists_one_selected_tile_sets_one_quadrant_bit(i, j):
    """A single selected 64-token tile (query tile i, key tile j) lists exactly
    key block j // 2 for query block i // 2, with quadrant bit
    2 * (i % 2) + (j % 2): a transposed mask or swapped bits fail here."""
    T = 8
    mask = np.zeros((1, 1, T, T), bool)
    mask[0, 0, i, j] = True
    idx, counts, kv, quad = oracle.block_lists(mask, np.full(T, 64, np.int32), 64)
    nz = np.argwhere(counts[0, 0] > 0).ravel()
    assert list(nz) == [i // 2]
    assert counts[0, 0, i // 2] == 1 and idx[0, 0, i // 2, 0] == j // 2
    assert quad[0, 0, i // 2, 0] == 1 << (2 * (i % 2) + (j % 2))


def test_block_lists_any_quadrant_lists_the_block_and_bits_count_pairs():
    """64-token tiles, all valid, even count: a key block is listed iff any of
    its four (query half, key half) tiles is selected, and the quadrant bits of
    a row add up to the selected tile pairs of its two query tiles."""
    rng = np.random.default_rng(4)
    T = 12
    mask = rng.random((1, 2, T, T)) < 0.15
    idx, counts, kv, quad = oracle.block_lists(mask, np.full(T, 64, np.int32), 64)
    nb = T // 2
    pooled = mask.reshape(1, 2, nb, 2, nb, 2).any(axis=(3, 5))
    assert np.array_equal(counts, pooled.sum(-1))
    bits = np.unpackbits(quad[..., None], axis=-1).sum(-1)
    assert np.array_equal(bits.sum(-1), mask.reshape(1, 2, nb, 2, T).sum(axis=(3, 4)))
    for h, r in np.ndindex(2, nb):
        n = counts[0, h, r]
        assert np.all(np.diff(idx[0, h, r, :n]) < 0)  # strictly descending
        assert set(idx[0, h, r, :n]) == set(np.nonzero(pooled[0, h, r])[0])


def test_block_lists_valid_counts_and_empty_halves():
    """Per-half valid counts come from the tiles' counts (64-token halves of a
    128-token tile split them); a half with no valid token is never selected."""
    # 128-token tiles, the last holding 70 tokens: halves 64 64 64 6
    _, _, kv, _ = oracle.block_lists(np.ones((1, 1, 2, 2), bool), np.array([128, 70], np.int32), 128)
    assert list(kv) == [64, 64, 64, 6]
    # 64-token tiles, the second one empty: its half contributes no bit
    mask = np.ones((1, 1, 4, 4), bool)
    idx, counts, kv, quad = oracle.block_lists(mask, np.array([64, 0, 64, 30], np.int32), 64)
    assert list(kv) == [64, 0, 64, 30]
    assert list(idx[0, 0, 0, :2]) == [1, 0] and list(quad[0, 0, 0, :2]) == [15, 5]  # key half 1 has no token
    assert int(kv.sum()) == 64 + 0 + 64 + 30


def test_block_lists_odd_half_count_pads_with_key_half_zero():
    """An odd count of 64-token halves: the last block's second query half is
    padding that sees key half 0 only (whatever the mask says)."""
    T = 5  # 64-token tiles: halves 0..4, blocks of halves (8, 9): half 9 is padding
    mask = np.zeros((1, 1, T, T), bool)
    idx, counts, kv, quad = oracle.block_lists(mask, np.full(T, 64, np.int32), 64)
    assert list(kv) == [64] * 5 + [0]
    assert counts[0, 0, :2].sum() == 0
    assert counts[0, 0, 2] == 1 and idx[0, 0, 2, 0] == 0 and quad[0, 0, 2, 0] == 4
    mask[0, 0, 4, 3] = True   # query half 8 -> key half 3 (block 1, second half)
    idx, counts, _, quad = oracle.block_lists(mask, np.full(T, 64, np.int32), 64)
    assert list(idx[0, 0, 2, :2]) == [1, 0] and list(quad[0, 0, 2, :2]) == [2, 4]


def test_block_lists_of_a_topk_selection():
    """Lists built from a top-k selection (64-token tiles): every listed block's
    bits are exactly the selected tiles among its four, and the union of the
    lists covers every selected tile."""
    q = np.random.default_rng(5).standard_normal((1, 2, 64 * 10, 128)).astype(np.float16)
    k = np.random.default_rng(6).standard_normal((1, 2, 64 * 10, 128)).astype(np.float16)
    sel, _ = oracle.vsa_select(q, k, 64, 3)
    mask = np.zeros((1, 2, 10, 10), bool)
    for h, i in np.ndindex(2, 10):
        mask[0, h, i, sel[0, h, i]] = True
    idx, counts, _, quad = oracle.block_lists(mask, np.full(10, 64, np.int32), 64)
    for h, r in np.ndindex(2, 5):
        got = set()
        for t in range(counts[0, h, r]):
            c, bits = idx[0, h, r, t], quad[0, h, r, t]
            for qh, kh in np.ndindex(2, 2):
                on = bool(bits & (1 << (2 * qh + kh)))
                assert on == mask[0, h, 2 * r + qh, 2 * c + kh]
                if on:
                    got.add((2 * r + qh, 2 * c + kh))
        assert got == {(2 * r + qh, j) for qh in range(2) for j in sel[0, h, 2 * r + qh]}

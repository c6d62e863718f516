"""Pins for the oracle's attention, causal/prefix masking, GQA, block lists
and merge (no GPU).

Independent anchors: torch's float64 scaled_dot_product_attention on the CPU
(a library special case of the same definition), closed forms (identical keys
give mean(V), a dominant logit returns its V row, constant V gives V) and
invariants (key shift, joint permutation of keys and values, causality,
full-set block lists equal dense, merge over any split equals the whole).
"""
import numpy as np
import pytest
import torch

import oracle


def _rand(shape, rng, lo=-4, hi=4):
    # multiples of 2^-8 in [lo, hi): exact in FP16, so shifted copies stay exact
    return (rng.integers(lo * 256, hi * 256, size=shape) / 256.0).astype(np.float16)


def _sdpa(q, k, v, scale, mask=None):
    group = q.shape[1] // k.shape[1]
    qt = torch.from_numpy(q.astype(np.float64))
    kt = torch.from_numpy(k.astype(np.float64)).repeat_interleave(group, dim=1)
    vt = torch.from_numpy(v.astype(np.float64)).repeat_interleave(group, dim=1)
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale).numpy()


@pytest.mark.parametrize("B,Hq,Hkv,Lq,Lkv,D", [(1, 2, 2, 37, 53, 16), (2, 6, 1, 20, 31, 32),
                                                (1, 4, 2, 5, 200, 8)])
def test_dense_matches_torch_sdpa(B, Hq, Hkv, Lq, Lkv, D):
    rng = np.random.default_rng(B * 100 + Lq)
    q, k, v = (rng.standard_normal(s).astype(np.float16) for s in
               ((B, Hq, Lq, D), (B, Hkv, Lkv, D), (B, Hkv, Lkv, D)))
    scale = float(np.float32(1 / np.sqrt(D)))
    out, lse = oracle.attention(q, k, v, scale)
    ref = _sdpa(q, k, v, scale)
    assert np.abs(out - ref.reshape(-1, D)).max() < 1e-12
    # lse against torch.logsumexp of the scaled scores
    g = Hq // Hkv
    kk = torch.from_numpy(k.astype(np.float64)).repeat_interleave(g, 1)
    s = torch.from_numpy(q.astype(np.float64)) @ kk.transpose(-1, -2) * scale
    assert np.abs(lse - torch.logsumexp(s, -1).numpy().ravel()).max() < 1e-12


def test_bf16_operands_match_torch_sdpa():
    """bfloat16 operands (as bit patterns) against torch float64 SDPA of the same values."""
    rng = np.random.default_rng(11)
    B, H, Lq, Lkv, D = 1, 3, 29, 47, 16
    tq, tk, tv = (torch.from_numpy(rng.standard_normal(s)).to(torch.bfloat16) for s in
                  ((B, H, Lq, D), (B, H, Lkv, D), (B, H, Lkv, D)))
    bits = [t.view(torch.int16).numpy().view(np.uint16) for t in (tq, tk, tv)]
    scale = float(np.float32(1 / np.sqrt(D)))
    out, lse = oracle.attention(*bits, scale, bf16=True)
    ref = torch.nn.functional.scaled_dot_product_attention(tq.double(), tk.double(), tv.double(), scale=scale)
    assert np.abs(out - ref.numpy().reshape(-1, D)).max() < 1e-12
    s = tq.double() @ tk.double().transpose(-1, -2) * scale
    assert np.abs(lse - torch.logsumexp(s, -1).numpy().ravel()).max() < 1e-12


@pytest.mark.parametrize("q_rows,q_real,kv_len", [(64, 64, 96), (64, 40, 100), (128, 100, 101)])
def test_causal_offset_matches_torch_masked_sdpa(q_rows, q_real, kv_len):
    rng = np.random.default_rng(q_real)
    Hq, Hkv, D = 6, 1, 32
    q = rng.standard_normal((1, Hq, q_rows, D)).astype(np.float16)
    k = rng.standard_normal((1, Hkv, kv_len, D)).astype(np.float16)
    v = rng.standard_normal((1, Hkv, kv_len, D)).astype(np.float16)
    offset = kv_len - q_real
    mask = np.arange(kv_len)[None, :] <= (offset + np.arange(q_rows)[:, None])
    out, _ = oracle.attention(q, k, v, 0.0625, mode=oracle.MODE_CAUSAL, offset=offset)
    ref = _sdpa(q, k, v, 0.0625, mask=mask)
    assert np.abs(out - ref.reshape(-1, D)).max() < 1e-12
    # padded rows (i >= q_real) see every key: they equal dense attention
    dense, _ = oracle.attention(q, k, v, 0.0625)
    o3 = out.reshape(Hq, q_rows, D)
    d3 = dense.reshape(Hq, q_rows, D)
    assert np.abs(o3[:, q_real:] - d3[:, q_real:]).max() < 1e-13 if q_rows > q_real else True


def test_causality_future_keys_do_not_matter():
    rng = np.random.default_rng(5)
    q_rows, q_real, kv_len, D = 32, 32, 80, 16
    q = rng.standard_normal((1, 2, q_rows, D)).astype(np.float16)
    k = rng.standard_normal((1, 1, kv_len, D)).astype(np.float16)
    v = rng.standard_normal((1, 1, kv_len, D)).astype(np.float16)
    off = kv_len - q_real
    a, _ = oracle.attention(q, k, v, 0.25, mode=oracle.MODE_CAUSAL, offset=off)
    i = 10
    k2, v2 = k.copy(), v.copy()
    k2[:, :, off + i + 1:] = rng.standard_normal(k2[:, :, off + i + 1:].shape).astype(np.float16)
    v2[:, :, off + i + 1:] = 9.0
    b, _ = oracle.attention(q, k2, v2, 0.25, mode=oracle.MODE_CAUSAL, offset=off)
    a3, b3 = a.reshape(2, q_rows, D), b.reshape(2, q_rows, D)
    assert np.array_equal(a3[:, : i + 1], b3[:, : i + 1])
    assert not np.array_equal(a3[:, i + 1:], b3[:, i + 1:])


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(1)
    D, L = 32, 77
    q = rng.standard_normal((1, 2, 9, D)).astype(np.float16)
    k = np.repeat(rng.standard_normal((1, 1, 1, D)).astype(np.float16), L, axis=2)
    v = rng.standard_normal((1, 1, L, D)).astype(np.float16)
    out, lse = oracle.attention(q, k, v, 0.3)
    mean = v.astype(np.float64).mean(axis=2).reshape(1, D)
    assert np.abs(out - mean).max() < 1e-14
    # lse = s + ln L for every row
    s = 0.3 * (q.astype(np.float64).reshape(-1, D) @ k[0, 0, 0].astype(np.float64))
    assert np.abs(lse - (s + np.log(L))).max() < 1e-12


def test_dominant_logit_returns_its_value_row():
    rng = np.random.default_rng(2)
    D, L, j = 16, 50, 17
    q = np.zeros((1, 1, 3, D), np.float16)
    q[..., 0] = 8.0
    k = (rng.standard_normal((1, 1, L, D)) * 0.01).astype(np.float16)
    k[0, 0, j, 0] = 16.0  # logit 128 above every other key
    v = rng.standard_normal((1, 1, L, D)).astype(np.float16)
    out, _ = oracle.attention(q, k, v, 1.0)
    assert np.abs(out - v[0, 0, j].astype(np.float64)).max() < 1e-40


def test_constant_values_weights_sum_to_one():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 3, 11, 8)).astype(np.float16)
    k = rng.standard_normal((1, 3, 70, 8)).astype(np.float16)
    v = np.full((1, 3, 70, 8), 0.75, np.float16)
    out, _ = oracle.attention(q, k, v, 0.9)
    assert np.abs(out - 0.75).max() < 1e-15


def test_key_shift_and_joint_permutation_invariance():
    rng = np.random.default_rng(6)
    D, L = 16, 45
    q, k, v = _rand((1, 2, 7, D), rng), _rand((1, 2, L, D), rng), _rand((1, 2, L, D), rng)
    base, lse = oracle.attention(q, k, v, 0.25)
    c = _rand((1, 1, 1, D), rng, -2, 2)
    shifted, _ = oracle.attention(q, (k.astype(np.float64) - c).astype(np.float16), v, 0.25)
    assert np.abs(base - shifted).max() < 1e-12
    perm = rng.permutation(L)
    permuted, lse2 = oracle.attention(q, k[:, :, perm], v[:, :, perm], 0.25)
    assert np.abs(base - permuted).max() < 1e-13 and np.abs(lse - lse2).max() < 1e-13


def test_strided_views_equal_contiguous():
    rng = np.random.default_rng(8)
    big = rng.standard_normal((1, 30, 3, 16)).astype(np.float16)  # [B, L, H, D] storage
    q = big.transpose(0, 2, 1, 3)
    out_v, _ = oracle.attention(q, q, q, 0.5)
    qc = np.ascontiguousarray(q)
    out_c, _ = oracle.attention(qc, qc, qc, 0.5)
    assert np.array_equal(out_v, out_c)


def test_full_block_list_equals_dense_and_prefix_rows_are_dense():
    rng = np.random.default_rng(9)
    B, H, L, D, blk = 1, 2, 256, 16, 32
    nb = L // blk
    q, k, v = (rng.standard_normal((B, H, L, D)).astype(np.float16) for _ in range(3))
    dense, _ = oracle.attention(q, k, v, 0.25)
    full = np.broadcast_to(np.arange(nb, dtype=np.int32), (B, H, nb, nb)).copy()
    sparse, _ = oracle.attention(q, k, v, 0.25, mode=oracle.MODE_BLOCKS, idx=full, block=blk)
    assert np.abs(dense - sparse).max() < 1e-14
    # a one-block list equals dense attention over that block's keys
    one = np.full((B, H, nb, 1), 3, np.int32)
    o1, _ = oracle.attention(q, k, v, 0.25, mode=oracle.MODE_BLOCKS, idx=one, block=blk, dense_prefix=2)
    sub, _ = oracle.attention(q, k[:, :, 3 * blk: 4 * blk], v[:, :, 3 * blk: 4 * blk], 0.25)
    o1 = o1.reshape(H, L, D)
    assert np.abs(o1[:, 2 * blk:] - sub.reshape(H, L, D)[:, 2 * blk:]).max() < 1e-14
    assert np.abs(o1[:, : 2 * blk] - dense.reshape(H, L, D)[:, : 2 * blk]).max() < 1e-14


def test_partial_last_block_list_equals_dense():
    """L not a multiple of the block: a full list still equals dense attention,
    and a list holding only the partial last block sees only its valid keys."""
    rng = np.random.default_rng(12)
    B, H, L, D, blk = 1, 2, 200, 16, 32  # 7 blocks, the last one of 8 keys
    nb = (L + blk - 1) // blk
    q, k, v = (rng.standard_normal((B, H, L, D)).astype(np.float16) for _ in range(3))
    dense, _ = oracle.attention(q, k, v, 0.25)
    full = np.broadcast_to(np.arange(nb, dtype=np.int32), (B, H, nb, nb)).copy()
    sparse, _ = oracle.attention(q, k, v, 0.25, mode=oracle.MODE_BLOCKS, idx=full, block=blk)
    assert np.abs(dense - sparse).max() < 1e-14
    last = np.full((B, H, nb, 1), nb - 1, np.int32)
    o1, _ = oracle.attention(q, k, v, 0.25, mode=oracle.MODE_BLOCKS, idx=last, block=blk)
    sub, _ = oracle.attention(q, k[:, :, (nb - 1) * blk:], v[:, :, (nb - 1) * blk:], 0.25)
    assert np.abs(o1 - sub).max() < 1e-14


def test_merge_over_any_split_equals_whole():
    rng = np.random.default_rng(10)
    D, L = 24, 300
    q = rng.standard_normal((1, 1, 1, D)).astype(np.float16)
    k = (rng.standard_normal((1, 1, L, D)) * 2).astype(np.float16)
    v = rng.standard_normal((1, 1, L, D)).astype(np.float16)
    whole, lse_whole = oracle.attention(q, k, v, 0.5)
    for cuts in ([0, 64, 300], [0, 1, 2, 150, 299, 300], [0, 300]):
        ms, ls, os_ = [], [], []
        for a, b in zip(cuts[:-1], cuts[1:]):
            o, lse = oracle.attention(q, k[:, :, a:b], v[:, :, a:b], 0.5)
            # a segment's state: any (m, l) with m + ln l = lse
            ms.append(lse[0] - 1.0)
            ls.append(np.e)
            os_.append(o[0])
        out, lse = oracle.merge(np.array(ms), np.array(ls), np.array(os_))
        assert np.abs(out - whole[0]).max() < 1e-13 and abs(lse - lse_whole[0]) < 1e-12


def test_row_subset_matches_full_run():
    rng = np.random.default_rng(12)
    q, k, v = (rng.standard_normal((1, 3, 40, 8)).astype(np.float16) for _ in range(3))
    full, lse_full = oracle.attention(q, k, v, 0.3)
    rows = np.array([[0, 2, 39], [0, 0, 0], [0, 1, 17]], np.int32)
    sub, lse = oracle.attention(q, k, v, 0.3, rows=rows)
    flat = rows[:, 1] * 40 + rows[:, 2]
    assert np.array_equal(sub, full[flat]) and np.array_equal(lse, lse_full[flat])


def test_float64_operands_match_torch_sdpa():
    """FP64 operands (the FP8 path's dequantized queries and keys) against
    torch float64 scaled_dot_product_attention, dense and causal."""
    rng = np.random.default_rng(41)
    q = rng.standard_normal((1, 3, 21, 64)) * 3.0
    k = rng.standard_normal((1, 3, 40, 64))
    v = rng.standard_normal((1, 3, 40, 64))
    out, lse = oracle.attention(q, k, v, 0.125)
    ref = _sdpa(q, k, v, 0.125)
    assert np.abs(out.reshape(ref.shape) - ref).max() < 1e-12
    mask = np.arange(40)[None, :] <= (40 - 21) + np.arange(21)[:, None]
    out_c, _ = oracle.attention(q, k, v, 0.125, mode=oracle.MODE_CAUSAL, offset=40 - 21)
    ref_c = _sdpa(q, k, v, 0.125, mask)
    assert np.abs(out_c.reshape(ref_c.shape) - ref_c).max() < 1e-12

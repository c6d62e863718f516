"""GPU parity over a seeded sweep of shapes for every attention entry point
(marked gpu): sizes drawn at random within each entry point's domain (the
causal and paged calls take query rows in multiples of 64 for prefill, and
cache lengths in whole 32-key pages), so that
tile tails, ragged key ranges, split plans, GQA groups, page tables and
block lists meet in combinations the hand-picked cases do not name. Each
case is compared with the FP64 oracle on every row at the FP16 (or BF16)
bounds; the drawn shape is printed before the launch."""
import numpy as np
import pytest

import oracle
import synth
from parity_util import BF16_LSE_ABS, BF16_MAX_ABS, BF16_REL_L2, LSE_ABS, assert_close, qkv, qkv_bf16, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def draw(case, salt):
    return np.random.default_rng(7919 * case + salt)


@pytest.mark.parametrize("case", range(10))
def test_sweep_dense(lib, case):
    r = draw(case, 1)
    B, H = int(r.integers(1, 3)), int(r.integers(1, 4))
    D = int(r.choice([128, 256]))
    Lq, Lkv = int(r.integers(1, 520)), int(r.integers(1, 2600))
    bf16 = D == 128 and case % 3 == 2
    say(f"sweep dense {case}: B{B} H{H} Lq{Lq} Lkv{Lkv} D{D} {'bf16' if bf16 else 'fp16'}")
    scale = lib.default_scale(D)
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device="cuda")
    if bf16:
        q, k, v = qkv_bf16(200 + case, B, H, Lq, Lkv, D)
        dq, dk, dv = (dev(x.view(np.int16)).view(torch.bfloat16) for x in (q, k, v))
        out = lib.attn_fwd_dense(dq, dk, dv, lse=lse)
        torch.cuda.synchronize()
        ref, ref_lse = oracle.attention(q, k, v, scale, bf16=True)
        assert_close(out.double().cpu().numpy().reshape(-1, D), ref, "O bf16", BF16_MAX_ABS, BF16_REL_L2)
        assert np.abs(lse.cpu().numpy().ravel() - ref_lse).max() < BF16_LSE_ABS
    else:
        q, k, v = qkv(200 + case, B, H, H, Lq, Lkv, D)
        out = lib.attn_fwd_dense(dev(q), dev(k), dev(v), lse=lse)
        torch.cuda.synchronize()
        ref, ref_lse = oracle.attention(q, k, v, scale)
        assert_close(out.cpu().numpy().reshape(-1, D), ref, "O")
        assert np.abs(lse.cpu().numpy().ravel() - ref_lse).max() < LSE_ABS


GROUPS = [(2, 1), (4, 2), (6, 1), (3, 3), (8, 2)]


@pytest.mark.parametrize("case", range(10))
def test_sweep_causal(lib, case):
    r = draw(case, 2)
    Hq, Hkv = GROUPS[int(r.integers(0, len(GROUPS)))]
    B, D = 1, int(r.choice([128, 256]))
    q_real = int(r.integers(1, 300))
    q_rows = (q_real + int(r.integers(0, 60)) + 63) // 64 * 64
    kv_len = (q_real + 1 + int(r.integers(0, 3000)) + 31) // 32 * 32
    nws = lib.prefix_causal_workspace(B, Hq, Hkv, D, q_rows, kv_len)
    say(f"sweep causal {case}: B{B} Hq{Hq} Hkv{Hkv} D{D} rows{q_rows} real{q_real} kv{kv_len} ws={nws}")
    q, k, v = qkv(300 + case, B, Hq, Hkv, q_rows, kv_len, D)
    scale = lib.default_scale(D)
    lse = torch.empty((B, Hq, q_rows), dtype=torch.float32, device="cuda")
    out = lib.attn_fwd_prefix_causal(dev(q), dev(k), dev(v), q_real, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention(q, k, v, scale, mode=oracle.MODE_CAUSAL, offset=kv_len - q_real)
    assert_close(out.cpu().numpy().reshape(-1, D), ref, "O")
    assert np.abs(lse.cpu().numpy().ravel() - ref_lse).max() < LSE_ABS


def _paged_case(case, salt, decode):
    r = draw(case, salt)
    Hq, Hkv = GROUPS[int(r.integers(0, len(GROUPS)))]
    D = int(r.choice([128, 256]))
    B = int(r.integers(1, 3))
    if decode:
        q_rows = int(r.integers(1, 17))
        q_real = int(r.integers(1, q_rows + 1))
    else:
        q_real = int(r.integers(1, 200))
        q_rows = (q_real + int(r.integers(0, 40)) + 63) // 64 * 64
    kv_len = (q_real + 1 + int(r.integers(0, 9000 if decode else 2500)) + 31) // 32 * 32
    per_seq = kv_len // 32
    pages = B * per_seq + int(r.integers(0, 8))
    pow2 = case % 2 == 0
    ks = float(2.0 ** -int(r.integers(1, 6))) if pow2 else float(np.float32(r.uniform(0.01, 0.1)))
    vs = float(np.float32(r.uniform(0.01, 0.1)))
    seed = (500 if decode else 400) + case
    q = synth.normal_f16(seed, synth.TID_Q, (B, Hq, q_rows, D))
    kc = synth.e4m3_codes(seed, synth.TID_K, (pages, 32, Hkv, D), ks)
    vc = synth.e4m3_codes(seed, synth.TID_V, (pages, 32, Hkv, D), vs)
    table = synth.permutation(seed, synth.TID_TABLE, pages)[: B * per_seq].reshape(B, per_seq).copy()
    return B, Hq, Hkv, D, q_rows, q_real, kv_len, ks, vs, q, kc, vc, table


def _paged_ref(lib, q, kc, vc, table, kv_len, q_real, ks, vs, D):
    kf = oracle.e4m3_to_f16(oracle.paged_gather(kc, table, kv_len), ks).view(np.float16)
    vf = oracle.e4m3_to_f16(oracle.paged_gather(vc, table, kv_len), vs).view(np.float16)
    return oracle.attention(q, kf, vf, lib.default_scale(D), mode=oracle.MODE_CAUSAL, offset=kv_len - q_real)


@pytest.mark.parametrize("case", range(6))
def test_sweep_paged_prefill(lib, case):
    B, Hq, Hkv, D, q_rows, q_real, kv_len, ks, vs, q, kc, vc, table = _paged_case(case, 3, False)
    bridged = case % 3 != 1
    say(f"sweep paged {case}: B{B} Hq{Hq} Hkv{Hkv} D{D} rows{q_rows} real{q_real} kv{kv_len} "
        f"scales {ks} {vs} bridged {bridged}")
    lse = torch.empty((B, Hq, q_rows), dtype=torch.float32, device="cuda")
    out = lib.attn_fwd_paged_e4m3(dev(q), dev(kc), dev(vc), dev(table), kv_len, q_real, ks, vs, lse=lse,
                                  bridged=bridged)
    torch.cuda.synchronize()
    ref, ref_lse = _paged_ref(lib, q, kc, vc, table, kv_len, q_real, ks, vs, D)
    assert_close(out.cpu().numpy().reshape(-1, D), ref, "O")
    assert np.abs(lse.cpu().numpy().ravel() - ref_lse).max() < LSE_ABS


@pytest.mark.parametrize("case", range(6))
def test_sweep_paged_decode(lib, case):
    B, Hq, Hkv, D, q_rows, q_real, kv_len, ks, vs, q, kc, vc, table = _paged_case(case, 4, True)
    say(f"sweep decode {case}: B{B} Hq{Hq} Hkv{Hkv} D{D} rows{q_rows} real{q_real} kv{kv_len} scales {ks} {vs}")
    lse = torch.empty((B, Hq, q_rows), dtype=torch.float32, device="cuda")
    out = lib.attn_fwd_paged_e4m3_decode(dev(q), dev(kc), dev(vc), dev(table), kv_len, q_real, ks, vs, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = _paged_ref(lib, q, kc, vc, table, kv_len, q_real, ks, vs, D)
    assert_close(out.cpu().numpy().reshape(-1, D), ref, "O")
    assert np.abs(lse.cpu().numpy().ravel() - ref_lse).max() < LSE_ABS


@pytest.mark.parametrize("case", range(6))
def test_sweep_paged_decode_mid_rows(lib, case):
    """33..64 packed rows at D256 (the 16-row-wave decode): random groups, positions, lengths and scales."""
    r = draw(case, 6)
    Hq, Hkv = [(6, 1), (8, 2), (4, 1), (8, 1), (12, 3)][int(r.integers(0, 5))]
    group = Hq // Hkv
    q_rows = int(r.integers((32 // group) + 1, min(16, 64 // group) + 1))
    q_real = int(r.integers(1, q_rows + 1))
    B, D = int(r.integers(1, 3)), 256
    kv_len = (q_real + 1 + int(r.integers(0, 12000)) + 31) // 32 * 32
    per_seq = kv_len // 32
    pages = B * per_seq + int(r.integers(0, 8))
    ks = float(np.float32(r.uniform(0.01, 0.1))) if case % 2 else float(2.0 ** -int(r.integers(1, 6)))
    vs = float(np.float32(r.uniform(0.01, 0.1)))
    say(f"sweep decode rows {group * q_rows}: B{B} Hq{Hq} Hkv{Hkv} q{q_rows} real{q_real} kv{kv_len} scales {ks} {vs}")
    seed = 700 + case
    q = synth.normal_f16(seed, synth.TID_Q, (B, Hq, q_rows, D))
    kc = synth.e4m3_codes(seed, synth.TID_K, (pages, 32, Hkv, D), ks)
    vc = synth.e4m3_codes(seed, synth.TID_V, (pages, 32, Hkv, D), vs)
    table = synth.permutation(seed, synth.TID_TABLE, pages)[: B * per_seq].reshape(B, per_seq).copy()
    lse = torch.empty((B, Hq, q_rows), dtype=torch.float32, device="cuda")
    out = lib.attn_fwd_paged_e4m3_decode(dev(q), dev(kc), dev(vc), dev(table), kv_len, q_real, ks, vs, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = _paged_ref(lib, q, kc, vc, table, kv_len, q_real, ks, vs, D)
    assert_close(out.cpu().numpy().reshape(-1, D), ref, "O")
    assert np.abs(lse.cpu().numpy().ravel() - ref_lse).max() < LSE_ABS


@pytest.mark.parametrize("case", range(6))
def test_sweep_vsa(lib, case):
    r = draw(case, 5)
    B, H = int(r.integers(1, 3)), int(r.integers(1, 4))
    L = int(r.integers(64, 3000))
    NB = (L + 63) // 64
    topk = int(r.integers(1, NB + 1))
    dense_prefix = int(r.integers(0, min(NB, 4) + 1))
    say(f"sweep vsa {case}: B{B} H{H} L{L} NB{NB} topk{topk} dense_prefix{dense_prefix}")
    shape = (B, H, L, 128)
    q = synth.normal_f16(600 + case, synth.TID_Q, shape)
    k = synth.normal_f16(600 + case, synth.TID_K, shape)
    v = synth.normal_f16(600 + case, synth.TID_V, shape)
    dq, dk, dv = dev(q), dev(k), dev(v)
    idx = lib.vsa_block_select(dq, dk, topk)
    lse = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    out = lib.vsa_block_sparse_attn(dq, dk, dv, idx, dense_prefix_qblocks=dense_prefix, lse=lse)
    torch.cuda.synchronize()
    want_idx, _ = oracle.vsa_select(q, k, 64, topk)
    got_idx = idx.cpu().numpy()
    assert np.array_equal(got_idx, want_idx)
    ref, ref_lse = oracle.attention(q, k, v, lib.default_scale(128), mode=oracle.MODE_BLOCKS, idx=want_idx,
                                    block=64, dense_prefix=dense_prefix)
    assert_close(out.cpu().numpy().reshape(-1, 128), ref, "O")
    assert np.abs(lse.cpu().numpy().ravel() - ref_lse).max() < LSE_ABS

"""GPU parity of every entry point against the FP64 oracle on small seeded
shapes that span several tiles and ragged tails (marked gpu)."""
import numpy as np
import pytest

import oracle
import synth
from parity_util import BF16_MAX_ABS, BF16_REL_L2, LSE_ABS, assert_close, qkv, qkv_bf16, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


@pytest.mark.parametrize("B,H,Lq,Lkv,D", [(1, 2, 256, 256, 128),     # the tiny dense workload
                                          (2, 3, 300, 1000, 128),    # ragged query and key tails
                                          (1, 2, 129, 65, 256),
                                          (1, 2, 200, 100, 128),     # one full 64-key tile, then a partial one
                                          (1, 1, 130, 321, 128),     # an odd count of full tiles, then one key
                                          (1, 2, 600, 4100, 128),    # five query tiles, the last ragged; many key tiles
                                          (1, 1, 1, 1, 128)])        # single row, single key
def test_dense_parity(lib, B, H, Lq, Lkv, D):
    say(f"dense B{B} H{H} Lq{Lq} Lkv{Lkv} D{D}")
    q, k, v = qkv(1, B, H, H, Lq, Lkv, D)
    scale = lib.default_scale(D)
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device="cuda")
    out = lib.attn_fwd_dense(dev(q), dev(k), dev(v), lse=lse, scale=scale)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention(q, k, v, scale)
    assert_close(out.cpu().numpy().reshape(-1, D), ref, "O")
    assert np.abs(lse.cpu().numpy().ravel() - ref_lse).max() < LSE_ABS


@pytest.mark.parametrize("B,H,Lq,Lkv,D", [(1, 2, 256, 256, 128), (2, 3, 300, 1000, 128), (1, 2, 129, 65, 256)])
def test_dense_bf16_parity(lib, B, H, Lq, Lkv, D):
    say(f"dense bf16 B{B} H{H} Lq{Lq} Lkv{Lkv} D{D}")
    q, k, v = qkv_bf16(12, B, H, Lq, Lkv, D)
    dq, dk, dv = (dev(x.view(np.int16)).view(torch.bfloat16) for x in (q, k, v))
    scale = lib.default_scale(D)
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device="cuda")
    out = lib.attn_fwd_dense(dq, dk, dv, lse=lse, scale=scale)
    torch.cuda.synchronize()
    assert out.dtype == torch.bfloat16
    ref, ref_lse = oracle.attention(q, k, v, scale, bf16=True)
    assert_close(out.double().cpu().numpy().reshape(-1, D), ref, "O bf16", BF16_MAX_ABS, BF16_REL_L2)
    assert np.abs(lse.cpu().numpy().ravel() - ref_lse).max() < LSE_ABS


def test_dense_strided_views(lib):
    """[B, L, H, D] storage passed as BHSD views with a unit D stride."""
    say("dense strided views")
    B, H, L, D = 1, 4, 200, 128
    rng = np.random.default_rng(0)
    base = [rng.standard_normal((B, L, H, D)).astype(np.float16) for _ in range(3)]
    qd, kd, vd = (dev(x).transpose(1, 2) for x in base)
    out_store = torch.zeros((B, L, H, D), dtype=torch.float16, device="cuda")
    lib.attn_fwd_dense(qd, kd, vd, out=out_store.transpose(1, 2))
    torch.cuda.synchronize()
    q, k, v = (x.transpose(0, 2, 1, 3) for x in base)
    ref, _ = oracle.attention(q, k, v, lib.default_scale(D))
    assert_close(out_store.transpose(1, 2).cpu().numpy().reshape(-1, D), ref, "O strided")


@pytest.mark.parametrize("B,Hq,Hkv,D,q_rows,q_real,kv_len", [
    (1, 6, 1, 256, 256, 200, 4096),   # split over the key range, padded rows
    (1, 6, 1, 256, 128, 128, 160),    # one segment, KV tail not a multiple of 64
    (1, 4, 2, 128, 192, 150, 2400),   # GQA groups of 2, D128
    (1, 2, 1, 256, 64, 64, 16480),    # 16 segments of 17 units, the last 3 units with a 32-key tail
    (1, 3, 1, 128, 64, 40, 9024),     # 9 segments at D128, padded rows
    (2, 4, 2, 256, 128, 90, 3072),    # two batches: their items and merges side by side
])
def test_prefix_causal_parity(lib, B, Hq, Hkv, D, q_rows, q_real, kv_len):
    say(f"causal B{B} Hq{Hq} Hkv{Hkv} D{D} rows{q_rows} real{q_real} kv{kv_len} "
        f"ws={lib.prefix_causal_workspace(B, Hq, Hkv, D, q_rows, kv_len)}")
    q, k, v = qkv(3, B, Hq, Hkv, q_rows, kv_len, D)
    scale = lib.default_scale(D)
    lse = torch.empty((B, Hq, q_rows), dtype=torch.float32, device="cuda")
    out = lib.attn_fwd_prefix_causal(dev(q), dev(k), dev(v), q_real, lse=lse, scale=scale)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention(q, k, v, scale, mode=oracle.MODE_CAUSAL, offset=kv_len - q_real)
    assert_close(out.cpu().numpy().reshape(-1, D), ref, "O")
    assert np.abs(lse.cpu().numpy().ravel() - ref_lse).max() < LSE_ABS


def test_prefix_causal_real_rows_ignore_padding(lib):
    """Real rows are bitwise independent of what the padded query rows hold."""
    say("causal padding independence")
    Hq, Hkv, D, q_rows, q_real, kv_len = 6, 1, 256, 128, 70, 2048
    q, k, v = qkv(4, 1, Hq, Hkv, q_rows, kv_len, D)
    a = lib.attn_fwd_prefix_causal(dev(q), dev(k), dev(v), q_real)
    a2 = lib.attn_fwd_prefix_causal(dev(q), dev(k), dev(v), q_real)
    q2 = q.copy()
    q2[:, :, q_real:] = np.float16(7.0)
    b = lib.attn_fwd_prefix_causal(dev(q2), dev(k), dev(v), q_real)
    torch.cuda.synchronize()
    # a row maximum read from the MFMA accumulators before they are final
    # shows up first here: repeated calls and padding changes then disagree
    assert torch.equal(a, a2)
    assert torch.equal(a[:, :, :q_real], b[:, :, :q_real])


def _paged_inputs(seed, Hkv, D, kv_len, pages, ks, vs):
    k_codes = synth.e4m3_codes(seed, synth.TID_K, (pages, 32, Hkv, D), ks)
    v_codes = synth.e4m3_codes(seed, synth.TID_V, (pages, 32, Hkv, D), vs)
    table = synth.permutation(seed, synth.TID_TABLE, pages)[None, : kv_len // 32].copy()
    return k_codes, v_codes, table


@pytest.mark.parametrize("Hq,Hkv,D,q_rows,q_real,kv_len,pages,ks,vs", [
    (6, 1, 256, 128, 100, 2048, 80, 1.0, 1.0),
    (6, 1, 256, 128, 100, 2048, 80, 0.0625, 0.03125),
    (6, 1, 256, 128, 100, 2048, 80, 0.0371, 0.0815),
    (4, 2, 128, 192, 150, 1056, 40, 0.0371, 0.0815),   # D128 byte swizzle, two kv heads, a 32-key tail
])
@pytest.mark.parametrize("bridged", [True, False])  # with a non-power-of-two k_scale: the two plans
def test_paged_e4m3_parity(lib, Hq, Hkv, D, q_rows, q_real, kv_len, pages, ks, vs, bridged):
    say(f"paged e4m3 Hq{Hq} Hkv{Hkv} D{D} q{q_rows} real{q_real} kv{kv_len} scales {ks} {vs} bridged {bridged}")
    ks, vs = float(np.float32(ks)), float(np.float32(vs))
    q = synth.normal_f16(5, synth.TID_Q, (1, Hq, q_rows, D))
    kc, vc, table = _paged_inputs(5, Hkv, D, kv_len, pages, ks, vs)
    scale = lib.default_scale(D)
    out = lib.attn_fwd_paged_e4m3(dev(q), dev(kc), dev(vc), dev(table), kv_len, q_real, ks, vs, scale=scale,
                                  bridged=bridged)
    torch.cuda.synchronize()
    kf = oracle.e4m3_to_f16(oracle.paged_gather(kc, table, kv_len), ks).view(np.float16)
    vf = oracle.e4m3_to_f16(oracle.paged_gather(vc, table, kv_len), vs).view(np.float16)
    ref, _ = oracle.attention(q, kf, vf, scale, mode=oracle.MODE_CAUSAL, offset=kv_len - q_real)
    assert_close(out.cpu().numpy().reshape(-1, D), ref, "O")


@pytest.mark.parametrize("Hq,Hkv,D,q_rows,q_real,kv_len,pages,ks,vs", [
    (6, 1, 256, 16, 16, 4096, 130, 1.0, 1.0),          # the decode shape, short cache
    (6, 1, 256, 5, 3, 2080, 70, 0.0625, 0.03125),      # padded rows, 32-key tail
    (4, 2, 128, 1, 1, 1024, 40, 0.0371, 0.0815),       # one position, two kv heads
    (8, 1, 128, 16, 16, 8192, 260, 1.0, 1.0),          # 8 heads x 16 rows fill the 128-row tile
    (4, 2, 128, 2, 2, 16416, 520, 0.0625, 1.0),        # 64 segments: the wide merge
    # one-wave workgroups (at most 32 packed rows): K converted in registers
    # (scaled) or decoded exactly (power-of-two k_scale), many short segments,
    # the merge in 16-column slices
    (6, 1, 256, 1, 1, 131072, 4100, 0.0371, 0.0815),   # one position: 6 rows, 512 segments
    (6, 1, 256, 5, 4, 32768, 1030, 0.0703, 0.05),      # 30 rows, padded, scaled
    (6, 1, 256, 4, 4, 8192, 260, 1.0, 1.0),            # 24 rows, power-of-two scale
    (2, 1, 128, 16, 16, 65536, 2050, 0.0371, 0.0815),  # 32 rows fill the wave, D128
    (8, 2, 128, 4, 3, 32800, 1030, 0.125, 0.0815),     # two kv heads, D128, a 32-key tail
    (6, 1, 256, 8, 8, 8192, 260, 0.0703, 0.05),        # 48 rows, scaled
    (4, 1, 256, 16, 11, 32992, 1040, 0.0625, 0.0815),  # 64 rows, power-of-two scale, padded positions
    (6, 1, 256, 11, 9, 20000, 630, 0.0371, 0.0815),    # 66 rows, scaled, padded
    (6, 1, 256, 16, 16, 1056, 40, 0.0703, 0.05),       # one short segment: an odd tile count
])
def test_paged_decode_parity(lib, Hq, Hkv, D, q_rows, q_real, kv_len, pages, ks, vs):
    say(f"paged decode Hq{Hq} Hkv{Hkv} D{D} q{q_rows} real{q_real} kv{kv_len} scales {ks} {vs}")
    ks, vs = float(np.float32(ks)), float(np.float32(vs))
    q = synth.normal_f16(9, synth.TID_Q, (1, Hq, q_rows, D))
    kc, vc, table = _paged_inputs(9, Hkv, D, kv_len, pages, ks, vs)
    scale = lib.default_scale(D)
    lse = torch.empty((1, Hq, q_rows), dtype=torch.float32, device="cuda")
    out = lib.attn_fwd_paged_e4m3_decode(dev(q), dev(kc), dev(vc), dev(table), kv_len, q_real, ks, vs, lse=lse,
                                         scale=scale)
    torch.cuda.synchronize()
    kf = oracle.e4m3_to_f16(oracle.paged_gather(kc, table, kv_len), ks).view(np.float16)
    vf = oracle.e4m3_to_f16(oracle.paged_gather(vc, table, kv_len), vs).view(np.float16)
    ref, ref_lse = oracle.attention(q, kf, vf, scale, mode=oracle.MODE_CAUSAL, offset=kv_len - q_real)
    assert_close(out.cpu().numpy().reshape(-1, D), ref, "O")
    assert np.abs(lse.cpu().numpy().ravel() - ref_lse).max() < LSE_ABS


@pytest.mark.parametrize("B,N,H,rows", [(2, 300, 3, 200), (1, 64, 1, 64), (1, 5, 2, 9)])
def test_prefix_fp8_gather_bit_exact(lib, B, N, H, rows):
    import synth.workloads as wl
    say(f"prefix fp8 gather B{B} N{N} H{H} rows{rows}")
    w = dict(wl.PREFIX_FP8, B=B, N=N, H=H, rows=min(rows, N))
    k, v, index = wl.prefix_fp8_inputs(w)
    if rows > N:  # repeated rows
        index = np.resize(index, rows).astype(np.int32)
    k[0, 0, 0] = 0                      # an all-zero (row, head): scale 0
    k[0, 1 % N, 0, :5] = 0x8000          # negative zeros
    k[0, 1 % N, 0, 5:9] = 0x0001         # tiny values: subnormal E4M3 codes after scaling
    dk, dv = (dev(x.view(np.int16)).view(torch.bfloat16) for x in (k, v))
    ko, vo = lib.kv_prefix_fp8_gather(dk, dv, dev(index))
    torch.cuda.synchronize()
    rk, rv = oracle.prefix_fp8_gather(k, v, index)
    got_k = ko.view(torch.int16).cpu().numpy().view(np.uint16)
    got_v = vo.view(torch.int16).cpu().numpy().view(np.uint16)
    bad = np.nonzero(got_k != rk)
    assert bad[0].size == 0, f"{bad[0].size} K mismatches, first {[hex(got_k[t]) for t in zip(*bad)][:4]} vs {[hex(rk[t]) for t in zip(*bad)][:4]}"
    assert np.array_equal(got_v, rv)


def test_prefix_fp8_then_bf16_attention(lib):
    """The pages' use: attention of BF16 queries over the FP8-round-tripped prefix keys."""
    import synth.workloads as wl
    say("prefix fp8 + attention")
    w = dict(wl.PREFIX_FP8, N=500, H=2, rows=300)
    k, v, index = wl.prefix_fp8_inputs(w)
    q = synth.normal_bf16(9, synth.TID_Q, (1, 2, 200, 128))
    dk, dv = (dev(x.view(np.int16)).view(torch.bfloat16) for x in (k, v))
    ko, vo = lib.kv_prefix_fp8_gather(dk, dv, dev(index))
    dq = dev(q.view(np.int16)).view(torch.bfloat16)
    scale = lib.default_scale(128)
    out = lib.attn_fwd_dense(dq, ko.transpose(1, 2), vo.transpose(1, 2), scale=scale)
    torch.cuda.synchronize()
    rk, rv = oracle.prefix_fp8_gather(k, v, index)
    ref, _ = oracle.attention(q, rk.transpose(0, 2, 1, 3), rv.transpose(0, 2, 1, 3), scale, bf16=True)
    assert_close(out.double().cpu().numpy().reshape(-1, 128), ref, "O", BF16_MAX_ABS, BF16_REL_L2)


def _bits_equal(got, want, codes, what):
    got = np.asarray(got).view(np.uint16).ravel()
    want = np.asarray(want).ravel()
    bad = np.nonzero(got != want)[0]
    if bad.size:
        c = np.asarray(codes).ravel()[bad[:8]]
        raise AssertionError(f"{what}: {bad.size} mismatches; codes {[hex(x) for x in c]} "
                             f"got {[hex(x) for x in got[bad[:8]]]} want {[hex(x) for x in want[bad[:8]]]}")


def test_bridge_bit_exact_all_codes_many_scales(lib):
    say("bridge all codes")
    D, Hkv, kv_len = 256, 1, 64
    codes = np.arange(256, dtype=np.uint8)
    cache = np.tile(codes, (2 * 32 * Hkv * D) // 256).reshape(2, 32, Hkv, D)
    rng = np.random.default_rng(9)
    cache_v = rng.integers(0, 256, cache.shape, dtype=np.uint8)
    table = np.array([[1, 0]], dtype=np.int32)
    scales = np.concatenate([[1.0, 0.5, 2.0, 1 / 3, 0.01, 0.1, 146.0, 2.0 ** -16, 1e-7],
                             rng.uniform(0.01, 0.1, 40), np.ldexp(rng.uniform(1, 2, 40), rng.integers(-20, 8, 40))])
    kd, vd, td = dev(cache), dev(cache_v), dev(table)
    for s in scales.astype(np.float32):
        s = float(s)
        ko, vo = lib.kv_e4m3_paged_to_fp16(kd, vd, td, 1, kv_len, s, 0.5 * s)
        torch.cuda.synchronize()
        g = oracle.paged_gather(cache, table, kv_len)
        gv = oracle.paged_gather(cache_v, table, kv_len)
        _bits_equal(ko.cpu().numpy(), oracle.e4m3_to_f16(g, s), g, f"K scale {s}")
        _bits_equal(vo.cpu().numpy(), oracle.e4m3_to_f16(gv, float(np.float32(0.5 * s))), gv, f"V scale {0.5 * s}")


def test_bridge_paged_layout_bit_exact(lib):
    say("bridge paged layout")
    Hkv, D, kv_len, pages = 2, 128, 1000, 40
    kc = synth.e4m3_codes(6, synth.TID_K, (pages, 32, Hkv, D), 0.05)
    vc = synth.e4m3_codes(6, synth.TID_V, (pages, 32, Hkv, D), 0.05)
    table = np.stack([synth.permutation(6, synth.TID_TABLE, pages)[:32],
                      synth.permutation(7, synth.TID_TABLE, pages)[:32]]).astype(np.int32)
    ko, vo = lib.kv_e4m3_paged_to_fp16(dev(kc), dev(vc), dev(table), 2, kv_len, 0.05, 0.07)
    torch.cuda.synchronize()
    for b in range(2):
        g = oracle.paged_gather(kc, table[b:b + 1], kv_len)
        assert np.array_equal(ko[b:b + 1].cpu().numpy().view(np.uint16), oracle.e4m3_to_f16(g, 0.05))
        g = oracle.paged_gather(vc, table[b:b + 1], kv_len)
        assert np.array_equal(vo[b:b + 1].cpu().numpy().view(np.uint16),
                              oracle.e4m3_to_f16(g, float(np.float32(0.07))))


@pytest.mark.parametrize("B,H,L,topk", [(1, 2, 4096, 8), (2, 1, 64 * 300, 64), (1, 1, 128, 2),
                                         (1, 2, 64 * 20 + 37, 6), (1, 1, 50, 1),  # partial last blocks
                                         (1, 1, 64 * 1000 + 17, 64)])  # 1001 blocks: 16 keys per lane in the top-k
def test_vsa_select_bit_exact(lib, B, H, L, topk):
    say(f"vsa select B{B} H{H} L{L} k{topk}")
    q = synth.normal_f16(8, synth.TID_Q, (B, H, L, 128))
    k = synth.normal_f16(8, synth.TID_K, (B, H, L, 128))
    idx, s = lib.vsa_block_select(dev(q), dev(k), topk, scores=True)
    torch.cuda.synchronize()
    ref_idx, ref_s = oracle.vsa_select(q, k, 64, topk)
    assert np.array_equal(s.cpu().numpy(), ref_s)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)


@pytest.mark.parametrize("k_sign", [1.0, -1.0])
def test_vsa_select_scores_of_one_sign(lib, k_sign):
    # every score near +-128: all keys share their sign and leading exponent bits
    say(f"vsa select one-sign scores {k_sign:+.0f}")
    B, H, L, topk = 1, 2, 64 * 24 + 5, 7
    nq = synth.normal_f16(11, synth.TID_Q, (B, H, L, 128)).astype(np.float32)
    nk = synth.normal_f16(11, synth.TID_K, (B, H, L, 128)).astype(np.float32)
    q = (1.0 + 0.05 * nq).astype(np.float16)
    k = (k_sign + 0.05 * nk).astype(np.float16)
    idx, s = lib.vsa_block_select(dev(q), dev(k), topk, scores=True)
    torch.cuda.synchronize()
    ref_idx, ref_s = oracle.vsa_select(q, k, 64, topk)
    assert np.all(np.sign(ref_s) == k_sign)
    assert np.array_equal(s.cpu().numpy(), ref_s)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)


def test_vsa_select_ties_take_lower_index(lib):
    say("vsa select ties")
    L = 64 * 40
    q = np.ones((1, 1, L, 128), np.float16)
    k = np.ones((1, 1, L, 128), np.float16)  # every block scores the same
    idx = lib.vsa_block_select(dev(q), dev(k), 5)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy()[0, 0], np.broadcast_to(np.arange(5), (40, 5)))


@pytest.mark.parametrize("B,H,L,topk,dp", [(1, 2, 2048, 8, 2), (1, 2, 64 * 20, 20, 0), (1, 2, 1024, 3, 16),
                                           (1, 2, 64 * 30 + 37, 7, 2), (1, 2, 64 * 6 + 1, 7, 7),  # partial last blocks
                                           (2, 3, 64 * 12 + 5, 5, 1)])  # two batches, three heads
def test_vsa_sparse_attn_parity(lib, B, H, L, topk, dp):
    say(f"vsa sparse B{B} H{H} L{L} k{topk} dp{dp}")
    D = 128
    q, k, v = qkv(10, B, H, H, L, L, D)
    ref_idx, _ = oracle.vsa_select(q, k, 64, topk)
    scale = lib.default_scale(D)
    lse = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    out = lib.vsa_block_sparse_attn(dev(q), dev(k), dev(v), dev(ref_idx), dense_prefix_qblocks=dp, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention(q, k, v, scale, mode=oracle.MODE_BLOCKS, idx=ref_idx, block=64,
                                    dense_prefix=dp)
    assert_close(out.cpu().numpy().reshape(-1, D), ref, "O")
    assert np.abs(lse.cpu().numpy().ravel() - ref_lse).max() < LSE_ABS


def test_bitwise_repeatability_without_sync(lib):
    """Three complete runs with no synchronisation in between give identical bits."""
    say("repeatability")
    q, k, v = (dev(x) for x in qkv(11, 1, 6, 1, 256, 4096, 256))
    outs = [lib.attn_fwd_prefix_causal(q, k, v, 256) for _ in range(3)]
    qd, kd, vd = (dev(x) for x in qkv(12, 1, 2, 2, 333, 777, 128))
    dens = [lib.attn_fwd_dense(qd, kd, vd) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    for o in dens[1:]:
        assert torch.equal(o, dens[0])


@pytest.mark.parametrize("decode,Hq,Hkv,D,q_rows,q_real,kv_len", [
    (False, 4, 2, 128, 128, 100, 640),   # prefill, two sequences with their own page lists
    (True, 6, 1, 256, 16, 16, 1056),     # decode, two sequences, a 32-key tail
    (True, 8, 2, 256, 12, 10, 4128),     # decode, two sequences and kv heads, 48 rows (16-row waves)
    (True, 4, 2, 256, 3, 3, 2080),       # decode, two sequences and kv heads, 6 rows (one-wave workgroups)
])
def test_paged_two_sequences_parity(lib, decode, Hq, Hkv, D, q_rows, q_real, kv_len):
    say(f"paged {'decode' if decode else 'prefill'} B2 Hq{Hq} Hkv{Hkv} D{D} q{q_rows} real{q_real} kv{kv_len}")
    B, ks, vs = 2, float(np.float32(0.0371)), float(np.float32(0.0815))
    per = kv_len // 32
    pages = 2 * per + 7
    q = synth.normal_f16(13, synth.TID_Q, (B, Hq, q_rows, D))
    kc = synth.e4m3_codes(13, synth.TID_K, (pages, 32, Hkv, D), ks)
    vc = synth.e4m3_codes(13, synth.TID_V, (pages, 32, Hkv, D), vs)
    perm = synth.permutation(13, synth.TID_TABLE, pages)
    table = np.stack([perm[:per], perm[per:2 * per]]).astype(np.int32)
    fn = lib.attn_fwd_paged_e4m3_decode if decode else lib.attn_fwd_paged_e4m3
    scale = lib.default_scale(D)
    out = fn(dev(q), dev(kc), dev(vc), dev(table), kv_len, q_real, ks, vs, scale=scale)
    torch.cuda.synchronize()
    kf = oracle.e4m3_to_f16(oracle.paged_gather(kc, table, kv_len), ks).view(np.float16)
    vf = oracle.e4m3_to_f16(oracle.paged_gather(vc, table, kv_len), vs).view(np.float16)
    ref, _ = oracle.attention(q, kf, vf, scale, mode=oracle.MODE_CAUSAL, offset=kv_len - q_real)
    assert_close(out.cpu().numpy().reshape(-1, D), ref, "O")

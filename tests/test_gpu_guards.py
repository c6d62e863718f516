"""Guard canaries around the outputs and workspaces of the entry points that
are not attention proper: the E4M3 bridge, the FP8 prefix gather, the VSA
selection, tile means and block lists, the FP8-QK prefix attention and the
allocation-free decode. Every output is a view inside a sentinel-filled
buffer; after the call (and a synchronisation) the sentinels must be intact,
and the results must equal the oracle's (or, bit for bit, an unguarded call
of the same entry point). Marked gpu."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from parity_util import say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

PAD = 4096  # sentinel elements before and after each flat output


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


class Flat:
    """A contiguous output of `shape` in the middle of a flat sentinel-filled
    buffer of a same-width integer type."""

    def __init__(self, shape, dtype, bits_dtype, sentinel):
        n = int(np.prod(shape))
        self.sentinel = sentinel
        self.full = torch.full((n + 2 * PAD,), sentinel, dtype=bits_dtype, device="cuda")
        self.view = self.full[PAD:PAD + n].view(dtype).view(shape)
        self.n = n

    def check(self, what):
        bits = self.full.cpu().numpy()
        outside = np.concatenate([bits[:PAD], bits[PAD + self.n:]])
        bad = int(np.count_nonzero(outside != np.array(self.sentinel).astype(bits.dtype)))
        assert bad == 0, f"{what}: {bad} elements written outside the output"


def test_bridge_guarded(lib):
    B, Hkv, D, kv_len, pages = 2, 2, 256, 1000, 70  # a partial last page per sequence
    say("guarded bridge", B, Hkv, D, kv_len)
    rng = np.random.default_rng(31)
    kc = rng.integers(0, 256, (pages, 32, Hkv, D), dtype=np.uint8)
    vc = rng.integers(0, 256, (pages, 32, Hkv, D), dtype=np.uint8)
    kc[kc == 0x7F] = 0
    kc[kc == 0xFF] = 0
    vc[vc == 0x7F] = 0
    vc[vc == 0xFF] = 0
    table = np.stack([rng.permutation(pages)[:32] for _ in range(B)]).astype(np.int32)
    ks, vs = 0.0371, 0.0815
    shape = (B, Hkv, kv_len, D)
    ko = Flat(shape, torch.float16, torch.int16, -21555)
    vo = Flat(shape, torch.float16, torch.int16, -21555)
    lib.kv_e4m3_paged_to_fp16(dev(kc), dev(vc), dev(table), B, kv_len, ks, vs, k_out=ko.view, v_out=vo.view)
    torch.cuda.synchronize()
    ko.check("bridge K")
    vo.check("bridge V")
    kf = oracle.e4m3_to_f16(oracle.paged_gather(kc, table, kv_len), ks)
    vf = oracle.e4m3_to_f16(oracle.paged_gather(vc, table, kv_len), vs)
    assert np.array_equal(ko.view.cpu().numpy().view(np.uint16), kf)
    assert np.array_equal(vo.view.cpu().numpy().view(np.uint16), vf)


def test_prefix_fp8_gather_guarded(lib):
    B, N, H, D, rows = 2, 300, 3, 128, 201
    say("guarded prefix gather", B, N, H, rows)
    k = synth.normal_bf16(32, synth.TID_K, (B, N, H, D))
    v = synth.normal_bf16(32, synth.TID_V, (B, N, H, D))
    index = np.sort(np.random.default_rng(32).choice(N, rows, replace=False)).astype(np.int32)
    dk = dev(k.view(np.int16)).view(torch.bfloat16)
    dv = dev(v.view(np.int16)).view(torch.bfloat16)
    di = dev(index)
    ko = Flat((B, rows, H, D), torch.bfloat16, torch.int16, -21555)
    vo = Flat((B, rows, H, D), torch.bfloat16, torch.int16, -21555)
    lib.kv_prefix_fp8_gather(dk, dv, di, k_out=ko.view, v_out=vo.view)
    rk, rv = lib.kv_prefix_fp8_gather(dk, dv, di)
    torch.cuda.synchronize()
    ko.check("gather K")
    vo.check("gather V")
    assert torch.equal(ko.view.view(torch.int16), rk.view(torch.int16))
    assert torch.equal(vo.view.view(torch.int16), rv.view(torch.int16))
    want_k, want_v = oracle.prefix_fp8_gather(k, v, index)
    assert np.array_equal(rk.view(torch.int16).cpu().numpy().view(np.uint16), want_k)
    assert np.array_equal(rv.view(torch.int16).cpu().numpy().view(np.uint16), want_v)


def test_vsa_select_and_means_guarded(lib):
    B, H, L, D, topk = 1, 2, 64 * 40 + 23, 128, 9  # a partial last block
    say("guarded VSA select", B, H, L, topk)
    q = synth.normal_f16(33, synth.TID_Q, (B, H, L, D))
    k = synth.normal_f16(33, synth.TID_K, (B, H, L, D))
    NB = (L + 63) // 64
    dq, dk = dev(q), dev(k)
    idx = Flat((B, H, NB, topk), torch.int32, torch.int32, 0x5A5A5A5A)
    nws = int(lib.load().vsa_block_select_workspace(B, H, L, D, 64))
    ws = Flat((nws,), torch.uint8, torch.uint8, 0xA5)
    lib.vsa_block_select(dq, dk, topk, workspace=ws.view, out=idx.view)
    means = Flat((B, H, NB, D), torch.float32, torch.int32, 0x5A5A5A5A)
    lib.vsa_tile_means(dq, out=means.view)
    torch.cuda.synchronize()
    idx.check("selection indices")
    ws.check("selection workspace")
    means.check("tile means")
    want_idx, _ = oracle.vsa_select(q, k, 64, topk)
    assert np.array_equal(idx.view.cpu().numpy(), want_idx)
    assert np.array_equal(means.view.cpu().numpy().view(np.uint32), oracle.tile_means(q, 64).view(np.uint32))


def test_block_lists_guarded(lib):
    B, H, T, tile = 1, 2, 37, 64  # an odd half count: the last query block has a padded half
    say("guarded block lists", B, H, T, tile)
    rng = np.random.default_rng(34)
    mask = (rng.random((B, H, T, T)) < 0.3).astype(np.uint8)
    valid = np.full(T, 64, dtype=np.int32)
    valid[-1] = 23
    dm, dvl = dev(mask), dev(valid)
    nb = (T + 1) // 2
    gi = Flat((B, H, nb, nb), torch.int32, torch.int32, 0x5A5A5A5A)
    gc = Flat((B, H, nb), torch.int32, torch.int32, 0x5A5A5A5A)
    gk = Flat((2 * nb,), torch.int32, torch.int32, 0x5A5A5A5A)
    gq = Flat((B, H, nb, nb), torch.uint8, torch.uint8, 0xA5)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.load().vsa_tile_mask_to_block_lists(dm.data_ptr(), dvl.data_ptr(), B, H, T, tile, gi.view.data_ptr(),
                                                 gc.view.data_ptr(), gk.view.data_ptr(), gq.view.data_ptr(),
                                                 stream)
    assert rc == 0
    ri, rcnt, rkv, rq = lib.vsa_tile_mask_to_block_lists(dm, dvl, tile)
    torch.cuda.synchronize()
    for g, what in ((gi, "indices"), (gc, "counts"), (gk, "kv_valid"), (gq, "quadrants")):
        g.check(f"block lists {what}")
    assert torch.equal(gi.view, ri) and torch.equal(gc.view, rcnt) and torch.equal(gk.view, rkv)
    assert torch.equal(gq.view, rq)


def test_prefix_fp8_attention_guarded(lib):
    B, H, Lq, Lkv, D = 1, 2, 300, 700, 128
    say("guarded FP8 prefix attention", B, H, Lq, Lkv)
    q = dev(synth.normal_bf16(35, synth.TID_Q, (B, H, Lq, D)).view(np.int16)).view(torch.bfloat16)
    k = dev(synth.normal_bf16(35, synth.TID_K, (B, H, Lkv, D)).view(np.int16)).view(torch.bfloat16)
    v = dev(synth.normal_bf16(35, synth.TID_V, (B, H, Lkv, D)).view(np.int16)).view(torch.bfloat16)
    out = Flat((B, H, Lq, D), torch.bfloat16, torch.int16, -21555)
    lse = Flat((B, H, Lq), torch.float32, torch.int32, 0x5A5A5A5A)
    ws = Flat((lib.prefix_fp8_workspace(B, H, Lq, Lkv),), torch.uint8, torch.uint8, 0xA5)
    lib.attn_fwd_prefix_fp8(q, k, v, out=out.view, lse=lse.view, workspace=ws.view)
    ref_lse = torch.empty((B, H, Lq), dtype=torch.float32, device="cuda")
    ref = lib.attn_fwd_prefix_fp8(q, k, v, lse=ref_lse)
    torch.cuda.synchronize()
    out.check("FP8 attention O")
    lse.check("FP8 attention LSE")
    ws.check("FP8 attention workspace")
    assert torch.equal(out.view.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(lse.view.view(torch.int32), ref_lse.view(torch.int32))


def test_noalloc_decode_guarded(lib):
    Hq, Hkv, D, q_rows, kv_len, pages = 6, 1, 256, 16, 4096, 130
    say("guarded allocation-free decode", Hq, Hkv, D, q_rows, kv_len)
    rng = np.random.default_rng(36)
    q = synth.normal_f16(36, synth.TID_Q, (1, Hq, q_rows, D))
    kc = rng.integers(0, 126, (pages, 32, Hkv, D), dtype=np.uint8)
    vc = rng.integers(0, 126, (pages, 32, Hkv, D), dtype=np.uint8)
    table = rng.permutation(pages)[:kv_len // 32].astype(np.int32)[None, :].copy()
    dq, dkc, dvc, dt = dev(q), dev(kc), dev(vc), dev(table)
    out = Flat((1, Hq, q_rows, D), torch.float16, torch.int16, -21555)
    lse = Flat((1, Hq, q_rows), torch.float32, torch.int32, 0x5A5A5A5A)
    lib.attn_fwd_paged_e4m3_decode_noalloc(dq, dkc, dvc, dt, kv_len, out.view, q_rows, 0.0371, 0.0815,
                                           lse=lse.view)
    ref_lse = torch.empty((1, Hq, q_rows), dtype=torch.float32, device="cuda")
    ref = lib.attn_fwd_paged_e4m3_decode(dq, dkc, dvc, dt, kv_len, q_rows, 0.0371, 0.0815, lse=ref_lse)
    torch.cuda.synchronize()
    out.check("decode O")
    lse.check("decode LSE")
    assert torch.equal(out.view.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(lse.view.view(torch.int32), ref_lse.view(torch.int32))

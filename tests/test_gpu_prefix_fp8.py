"""GPU parity of the FP8-MFMA prefix attention (attn_fwd_prefix_fp8, marked
gpu) against the oracle: the quantized queries and keys bit-exact, the output
within the BF16 bounds of (a) FP64 attention over the dequantized values
decode(code) * scale (the path's reading), and (b) the pages' own pipeline,
the bfloat16 round trip of queries and keys followed by bfloat16 attention
("[perf] FastH3 two-Spark: gather packed FP4 inputs before head
projections", query_pool.py PREFIX_FP8 and prefix_quant.py), on N(0,1) data.
Queries scaled by 16 drive the online softmax through its rescale."""
import numpy as np
import pytest

import oracle
import synth
from parity_util import BF16_LSE_ABS, BF16_MAX_ABS, BF16_REL_L2, assert_close, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def dev_bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)


def _inputs(seed, B, H, Lq, Lkv, D=128, qmul=1):
    q = synth.normal_bf16(seed, synth.TID_Q, (B, H, Lq, D))
    if qmul != 1:  # an exact power-of-two multiple: add to the exponent of the normal values
        e = (q >> 7) & 0xFF
        q = np.where((e > 0) & (e < 250), q + (int(np.log2(qmul)) << 7), q).astype(np.uint16)
    k = synth.normal_bf16(seed, synth.TID_K, (B, H, Lkv, D))
    v = synth.normal_bf16(seed, synth.TID_V, (B, H, Lkv, D))
    return q, k, v


def _bf16_to_f64(x):
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("B,H,Lq,Lkv,qmul", [(1, 2, 256, 256, 1), (2, 3, 300, 1000, 1), (1, 2, 600, 4100, 1),
                                             (1, 1, 1, 1, 1), (1, 2, 200, 100, 1),
                                             (1, 2, 300, 2000, 16)])   # scores span > 2^8: the rescale runs
def test_prefix_fp8_parity(lib, B, H, Lq, Lkv, qmul):
    say(f"prefix fp8 B{B} H{H} Lq{Lq} Lkv{Lkv} q x{qmul}")
    q, k, v = _inputs(15, B, H, Lq, Lkv, qmul=qmul)
    scale = lib.default_scale(128)
    ws = torch.empty(lib.prefix_fp8_workspace(B, H, Lq, Lkv), dtype=torch.uint8, device="cuda")
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device="cuda")
    out = lib.attn_fwd_prefix_fp8(dev_bf16(q), dev_bf16(k), dev_bf16(v), lse=lse, scale=scale, workspace=ws)
    torch.cuda.synchronize()
    # the codes and scales in the workspace: bit-exact
    qc, qs = oracle.fp8_quantize_rows(q)
    kc, ks = oracle.fp8_quantize_rows(k)
    w = ws.cpu().numpy()
    pad = lambda n: (n + 255) // 256 * 256
    nq, nk = B * H * Lq * 128, B * H * Lkv * 128
    assert np.array_equal(w[:nq].reshape(qc.shape), qc)
    assert np.array_equal(w[pad(nq):pad(nq) + nk].reshape(kc.shape), kc)
    o0 = pad(nq) + pad(nk)
    assert np.array_equal(w[o0:o0 + 4 * B * H * Lq].view(np.float32).reshape(qs.shape), qs)
    o1 = o0 + pad(4 * B * H * Lq)
    assert np.array_equal(w[o1:o1 + 4 * B * H * Lkv].view(np.float32).reshape(ks.shape), ks)
    # (a) attention over the dequantized values
    qd, kd = oracle.fp8_dequant(qc, qs), oracle.fp8_dequant(kc, ks)
    if qmul != 1:
        # the inputs force a raise of the reference maximum after the first 64-key tile
        s = np.einsum("bhid,bhjd->bhij", qd, kd) * scale * 1.4426950408889634
        forced = int((s[..., 64:].max(-1) > s[..., :64].max(-1) + 8).sum())
        say(f"  rows forced to raise: {forced} of {B * H * Lq}")
        assert forced >= B * H * Lq // 4
    got = out.double().cpu().numpy().reshape(-1, 128)
    ref, ref_lse = oracle.attention(qd, kd, _bf16_to_f64(v), scale)
    assert_close(got, ref, "O vs dequantized-value attention", BF16_MAX_ABS, BF16_REL_L2)
    assert np.abs(lse.cpu().numpy().ravel() - ref_lse).max() < BF16_LSE_ABS
    if qmul == 1:
        # (b) the pages' pipeline: bfloat16 round trips, then bfloat16 attention
        qr, _ = oracle.prefix_fp8_gather(q.reshape(1, -1, 1, 128), q.reshape(1, -1, 1, 128),
                                         np.arange(B * H * Lq, dtype=np.int32))
        kr, _ = oracle.prefix_fp8_gather(k.reshape(1, -1, 1, 128), k.reshape(1, -1, 1, 128),
                                         np.arange(B * H * Lkv, dtype=np.int32))
        ref_b, _ = oracle.attention(qr.reshape(q.shape), kr.reshape(k.shape), v, scale, bf16=True)
        assert_close(got, ref_b, "O vs bfloat16 round trip + attention", BF16_MAX_ABS, BF16_REL_L2)


def test_prefix_fp8_strided_views(lib):
    """[B, L, H, D] storage (the pages' BSHD layout) passed as BHSD views."""
    say("prefix fp8 strided views")
    B, H, L = 1, 4, 200
    rng = np.random.default_rng(3)
    base = [torch.from_numpy(rng.standard_normal((B, L, H, 128))).to(torch.bfloat16) for _ in range(3)]
    q, k, v = (t.cuda().transpose(1, 2) for t in base)
    out_store = torch.zeros((B, L, H, 128), dtype=torch.bfloat16, device="cuda")
    lib.attn_fwd_prefix_fp8(q, k, v, out=out_store.transpose(1, 2))
    torch.cuda.synchronize()
    qb, kb, vb = (t.transpose(1, 2).contiguous().view(torch.int16).numpy().view(np.uint16) for t in base)
    qc, qs = oracle.fp8_quantize_rows(qb)
    kc, ks = oracle.fp8_quantize_rows(kb)
    ref, _ = oracle.attention(oracle.fp8_dequant(qc, qs), oracle.fp8_dequant(kc, ks), _bf16_to_f64(vb),
                              lib.default_scale(128))
    got = out_store.transpose(1, 2).double().cpu().numpy().reshape(-1, 128)
    assert_close(got, ref, "O strided", BF16_MAX_ABS, BF16_REL_L2)

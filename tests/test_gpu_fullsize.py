"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (same entry points, shapes and split plans), on sampled outputs the
FP64 oracle computes one row at a time; E4M3 conversion and block indices
are compared bit-exactly over the whole output (marked gpu)."""
import numpy as np
import pytest

import oracle
import synth.workloads as wl
from parity_util import BF16_LSE_ABS, BF16_MAX_ABS, BF16_REL_L2, LSE_ABS, assert_close, sample_rows, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _rows_of(out_np, rows):
    return out_np[rows[:, 0], rows[:, 1], rows[:, 2]].astype(np.float64)


def test_video_dense_full(lib):
    w = wl.VIDEO_DENSE
    say("full dense", w["name"])
    q, k, v = wl.dense_inputs(w)
    lse = torch.empty((w["B"], w["H"], w["Lq"]), dtype=torch.float32, device="cuda")
    out = lib.attn_fwd_dense(dev(q), dev(k), dev(v), lse=lse)
    torch.cuda.synchronize()
    rows = sample_rows(w["B"], w["H"], w["Lq"], 24, seed=2)
    ref, ref_lse = oracle.attention(q, k, v, lib.default_scale(w["D"]), rows=rows)
    assert_close(_rows_of(out.cpu().numpy(), rows), ref, f"O ({len(rows)} rows)")
    got_lse = lse.cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
    assert np.abs(got_lse - ref_lse).max() < LSE_ABS


def test_ragged_dense_full(lib):
    """The GB10 page's dense shape: 56 heads, Lq 15360 against Lkv 29678 (a 14-key tail)."""
    w = wl.RAGGED_DENSE
    say("full ragged dense", w["name"])
    q, k, v = wl.dense_inputs(w)
    lse = torch.empty((w["B"], w["H"], w["Lq"]), dtype=torch.float32, device="cuda")
    out = lib.attn_fwd_dense(dev(q), dev(k), dev(v), lse=lse)
    torch.cuda.synchronize()
    rows = sample_rows(w["B"], w["H"], w["Lq"], 8, seed=6)
    ref, ref_lse = oracle.attention(q, k, v, lib.default_scale(w["D"]), rows=rows)
    assert_close(_rows_of(out.cpu().numpy(), rows), ref, f"O ({len(rows)} rows)")
    got_lse = lse.cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
    assert np.abs(got_lse - ref_lse).max() < LSE_ABS


def test_ragged_dense_bf16_full(lib):
    """The GB10 page's BF16 variant of the same ragged dense shape."""
    import synth
    w = wl.RAGGED_DENSE
    say("full ragged dense bf16", w["name"])
    shape_q, shape_kv = (w["B"], w["H"], w["Lq"], w["D"]), (w["B"], w["H"], w["Lkv"], w["D"])
    q = synth.normal_bf16(w["seed"], synth.TID_Q, shape_q)
    k = synth.normal_bf16(w["seed"], synth.TID_K, shape_kv)
    v = synth.normal_bf16(w["seed"], synth.TID_V, shape_kv)
    dq, dk, dv = (dev(x.view(np.int16)).view(torch.bfloat16) for x in (q, k, v))
    lse = torch.empty((w["B"], w["H"], w["Lq"]), dtype=torch.float32, device="cuda")
    out = lib.attn_fwd_dense(dq, dk, dv, lse=lse)
    torch.cuda.synchronize()
    rows = sample_rows(w["B"], w["H"], w["Lq"], 8, seed=7)
    ref, ref_lse = oracle.attention(q, k, v, lib.default_scale(w["D"]), rows=rows, bf16=True)
    got = out.double().cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
    assert_close(got, ref, f"O bf16 ({len(rows)} rows)", BF16_MAX_ABS, BF16_REL_L2)
    got_lse = lse.cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
    assert np.abs(got_lse - ref_lse).max() < LSE_ABS


def test_prefix_causal_full(lib):
    w = wl.PREFIX_CAUSAL
    say("full causal", w["name"])
    q, k, v = wl.causal_inputs(w)
    lse = torch.empty((w["B"], w["Hq"], w["q_rows"]), dtype=torch.float32, device="cuda")
    out = lib.attn_fwd_prefix_causal(dev(q), dev(k), dev(v), w["q_real"], lse=lse)
    torch.cuda.synchronize()
    rows = sample_rows(w["B"], w["Hq"], w["q_rows"], 12, seed=3, tile=2048)
    ref, ref_lse = oracle.attention(q, k, v, lib.default_scale(w["D"]), mode=oracle.MODE_CAUSAL,
                                    offset=w["kv_len"] - w["q_real"], rows=rows)
    assert_close(_rows_of(out.cpu().numpy(), rows), ref, f"O ({len(rows)} rows)")
    got_lse = lse.cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
    assert np.abs(got_lse - ref_lse).max() < LSE_ABS


@pytest.mark.parametrize("unit_scales,bridged", [(True, True), (False, True), (False, False)])
def test_paged_e4m3_full(lib, unit_scales, bridged):
    w = wl.PAGED_E4M3
    q, kc, vc, table, ks, vs = wl.paged_inputs(w, unit_scales)
    say("full paged", w["name"], "scales", ks, vs, "bridged", bridged)
    dq, dkc, dvc, dt = dev(q), dev(kc), dev(vc), dev(table)
    out = lib.attn_fwd_paged_e4m3(dq, dkc, dvc, dt, w["kv_len"], w["q_real"], ks, vs, bridged=bridged)
    ko, vo = lib.kv_e4m3_paged_to_fp16(dkc, dvc, dt, w["B"], w["kv_len"], ks, vs)
    torch.cuda.synchronize()
    # the bridge, bit-exact over every converted element
    kf = oracle.e4m3_to_f16(oracle.paged_gather(kc, table, w["kv_len"]), ks)
    vf = oracle.e4m3_to_f16(oracle.paged_gather(vc, table, w["kv_len"]), vs)
    assert np.array_equal(ko.cpu().numpy().view(np.uint16), kf), "bridge K bits differ"
    assert np.array_equal(vo.cpu().numpy().view(np.uint16), vf), "bridge V bits differ"
    del ko, vo
    rows = sample_rows(w["B"], w["Hq"], w["q_rows"], 8, seed=4, tile=2048)
    ref, _ = oracle.attention(q, kf.view(np.float16), vf.view(np.float16), lib.default_scale(w["D"]),
                              mode=oracle.MODE_CAUSAL, offset=w["kv_len"] - w["q_real"], rows=rows)
    assert_close(_rows_of(out.cpu().numpy(), rows), ref, f"O ({len(rows)} rows)")


@pytest.mark.parametrize("positions", [16, 1])
def test_paged_decode_full(lib, positions):
    """Every (head, position) row of the decode workload, non-unit scales: its 16 positions (96 rows, the
    128-row workgroups), and its first position alone (6 rows, the one-wave workgroups, 1000 segments)."""
    w = wl.PAGED_DECODE
    q, kc, vc, table, ks, vs = wl.paged_inputs(w, unit_scales=False)
    if positions != w["q_rows"]:
        w = dict(w, q_rows=positions, q_real=positions)
        q = np.ascontiguousarray(q[:, :, :positions])
    say("full paged decode", w["name"], "positions", positions, "scales", ks, vs)
    lse = torch.empty((w["B"], w["Hq"], w["q_rows"]), dtype=torch.float32, device="cuda")
    out = lib.attn_fwd_paged_e4m3_decode(dev(q), dev(kc), dev(vc), dev(table), w["kv_len"], w["q_real"], ks, vs,
                                         lse=lse)
    torch.cuda.synchronize()
    kf = oracle.e4m3_to_f16(oracle.paged_gather(kc, table, w["kv_len"]), ks).view(np.float16)
    vf = oracle.e4m3_to_f16(oracle.paged_gather(vc, table, w["kv_len"]), vs).view(np.float16)
    ref, ref_lse = oracle.attention(q, kf, vf, lib.default_scale(w["D"]), mode=oracle.MODE_CAUSAL,
                                    offset=w["kv_len"] - w["q_real"])
    assert_close(out.cpu().numpy().reshape(-1, w["D"]), ref, "O (all rows)")
    assert np.abs(lse.cpu().numpy().ravel() - ref_lse).max() < LSE_ABS


def test_prefix_fp8_gather_full(lib):
    """The video-shape gather (32768 of 36864 rows, 8 heads): V exactly everywhere, K bit-exact
    on a seeded sample of output rows (the oracle computes those rows' index entries only)."""
    w = wl.PREFIX_FP8
    say("full prefix fp8", w["name"])
    k, v, index = wl.prefix_fp8_inputs(w)
    dk, dv = (dev(x.view(np.int16)).view(torch.bfloat16) for x in (k, v))
    ko, vo = lib.kv_prefix_fp8_gather(dk, dv, dev(index))
    torch.cuda.synchronize()
    got_v = vo.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got_v, v[:, index]), "V gather differs"
    rng = np.random.default_rng(8)
    sample = np.unique(np.concatenate([[0, w["rows"] - 1], rng.integers(0, w["rows"], 1024)])).astype(np.int64)
    rk, _ = oracle.prefix_fp8_gather(k, v, index[sample])
    got_k = ko.view(torch.int16).cpu().numpy().view(np.uint16)[:, sample]
    assert np.array_equal(got_k, rk), f"{int((got_k != rk).sum())} K mismatches on {sample.size} rows"


def test_vsa_full(lib):
    w = wl.VSA
    say("full vsa", w["name"])
    q, k, v = wl.vsa_inputs(w)
    dq, dk, dv = dev(q), dev(k), dev(v)
    idx = lib.vsa_block_select(dq, dk, w["topk"], block=w["block"])
    torch.cuda.synchronize()
    ref_idx, _ = oracle.vsa_select(q, k, w["block"], w["topk"])
    assert np.array_equal(idx.cpu().numpy(), ref_idx), "selected blocks differ"
    out = lib.vsa_block_sparse_attn(dq, dk, dv, idx, dense_prefix_qblocks=w["dense_prefix"], block=w["block"])
    torch.cuda.synchronize()
    # dense prefix rows (query blocks 0-1) and sparse rows
    rows = sample_rows(w["B"], w["H"], w["L"], 16, seed=5, extra=(63, 64, 127, 128))
    ref, _ = oracle.attention(q, k, v, lib.default_scale(w["D"]), mode=oracle.MODE_BLOCKS, idx=ref_idx,
                              block=w["block"], dense_prefix=w["dense_prefix"], rows=rows)
    assert_close(_rows_of(out.cpu().numpy(), rows), ref, f"O ({len(rows)} rows)")


def test_prefix_fp8_attention_full(lib):
    """The FP8-QK prefix attention at the video shape the benchmark times (B1 H8 D128 Lq = Lkv = 36864,
    BF16 N(0,1) operands): the E4M3 codes and row scales of all of Q and K bit-exact, sampled output rows
    and their LSE within the BF16 bounds of FP64 attention over the dequantized values."""
    import synth
    w = wl.VIDEO_DENSE
    B, H, L, D = w["B"], w["H"], w["Lq"], w["D"]
    say("full FP8 prefix attention", B, H, L, D)
    q = synth.normal_bf16(w["seed"], synth.TID_Q, (B, H, L, D))
    k = synth.normal_bf16(w["seed"], synth.TID_K, (B, H, L, D))
    v = synth.normal_bf16(w["seed"], synth.TID_V, (B, H, L, D))
    as_bf16 = lambda x: torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    ws = torch.empty(lib.prefix_fp8_workspace(B, H, L, L), dtype=torch.uint8, device="cuda")
    lse = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    out = lib.attn_fwd_prefix_fp8(as_bf16(q), as_bf16(k), as_bf16(v), lse=lse, workspace=ws)
    torch.cuda.synchronize()
    qc, qs = oracle.fp8_quantize_rows(q)
    kc, ks = oracle.fp8_quantize_rows(k)
    wsn = ws.cpu().numpy()
    n = B * H * L * D
    pad = lambda x: (x + 255) // 256 * 256
    assert np.array_equal(wsn[:n].reshape(qc.shape), qc), "Q codes differ"
    assert np.array_equal(wsn[pad(n):pad(n) + n].reshape(kc.shape), kc), "K codes differ"
    o0 = 2 * pad(n)
    assert np.array_equal(wsn[o0:o0 + 4 * B * H * L].view(np.float32).reshape(qs.shape), qs), "Q scales differ"
    o1 = o0 + pad(4 * B * H * L)
    assert np.array_equal(wsn[o1:o1 + 4 * B * H * L].view(np.float32).reshape(ks.shape), ks), "K scales differ"
    del wsn, ws
    rows = sample_rows(B, H, L, 8, seed=9, tile=4096)
    vd = (v.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref, ref_lse = oracle.attention(oracle.fp8_dequant(qc, qs), oracle.fp8_dequant(kc, ks), vd,
                                    lib.default_scale(D), rows=rows)
    got = out.float().cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]].astype(np.float64)
    assert_close(got, ref, f"O ({len(rows)} rows)", BF16_MAX_ABS, BF16_REL_L2)
    got_lse = lse.cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
    assert np.abs(got_lse - ref_lse).max() < BF16_LSE_ABS

"""GPU check of the allocation-free decode entry point (marked gpu): two
calls in a row through the C ABI, the second on a smaller input, each equal
to attn_fwd_paged_e4m3_decode (the entry point with a caller workspace) on
the same inputs, and within the FP16 tolerance of the FP64 oracle."""
import numpy as np
import pytest

import oracle
import synth
import synth.workloads as wl
from parity_util import LSE_ABS, assert_close, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _check_pair(lib, q, kc, vc, table, kv_len, q_real, ks, vs, what):
    dq, dkc, dvc, dt = dev(q), dev(kc), dev(vc), dev(table)
    B, Hq, q_rows, D = q.shape
    ref_out = torch.empty_like(dq)
    ref_lse = torch.empty((B, Hq, q_rows), dtype=torch.float32, device="cuda")
    lib.attn_fwd_paged_e4m3_decode(dq, dkc, dvc, dt, kv_len, q_real, ks, vs, out=ref_out, lse=ref_lse)
    out = torch.full_like(dq, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    lib.attn_fwd_paged_e4m3_decode_noalloc(dq, dkc, dvc, dt, kv_len, out, q_real, ks, vs, lse=lse)
    torch.cuda.synchronize()
    say(f"  {what}: equal to the workspace entry point: {torch.equal(out, ref_out)}")
    assert torch.equal(out, ref_out), what
    assert torch.equal(lse, ref_lse), what
    return out, lse


def test_noalloc_decode_two_calls_second_smaller(lib):
    # call 1: the decode workload (16 positions x 6 heads, KV 256000, D256)
    w = wl.PAGED_DECODE
    q, kc, vc, table, ks, vs = wl.paged_inputs(w, unit_scales=False)
    need = lib.load().attn_fwd_paged_e4m3_decode_workspace(1, w["Hq"], w["Hkv"], w["D"], w["q_rows"], w["kv_len"])
    say(f"noalloc decode call 1: {w['name']}, partial states {need} of {lib.NOALLOC_SCRATCH_BYTES} bytes")
    out, _ = _check_pair(lib, q, kc, vc, table, w["kv_len"], w["q_real"], ks, vs, "call 1")
    rows = np.array([(0, h, i) for h in range(w["Hq"]) for i in (0, 7, 15)], dtype=np.int32)
    kf = oracle.e4m3_to_f16(oracle.paged_gather(kc, table, w["kv_len"]), ks).view(np.float16)
    vf = oracle.e4m3_to_f16(oracle.paged_gather(vc, table, w["kv_len"]), vs).view(np.float16)
    ref, _ = oracle.attention(q, kf, vf, lib.default_scale(w["D"]), mode=oracle.MODE_CAUSAL,
                              offset=w["kv_len"] - w["q_real"], rows=rows)
    got = out.cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
    assert_close(got, ref, "call 1 vs oracle (18 rows)")
    del kf, vf

    # call 2: smaller (D128, two kv heads, 5 positions of which 3 real, 2080 keys),
    # over whatever call 1 left in the scratch array
    Hq, Hkv, D, q_rows, q_real, kv_len = 4, 2, 128, 5, 3, 2080
    ks2, vs2 = float(np.float32(0.0371)), float(np.float32(0.0815))
    pages = kv_len // 32 + 3
    q2 = synth.normal_f16(31, synth.TID_Q, (1, Hq, q_rows, D))
    kc2 = synth.e4m3_codes(31, synth.TID_K, (pages, 32, Hkv, D), ks2)
    vc2 = synth.e4m3_codes(31, synth.TID_V, (pages, 32, Hkv, D), vs2)
    table2 = synth.permutation(31, synth.TID_TABLE, pages)[None, : kv_len // 32].copy()
    say(f"noalloc decode call 2: Hq{Hq} Hkv{Hkv} D{D} q{q_rows} real{q_real} kv{kv_len}")
    out2, lse2 = _check_pair(lib, q2, kc2, vc2, table2, kv_len, q_real, ks2, vs2, "call 2")
    kf = oracle.e4m3_to_f16(oracle.paged_gather(kc2, table2, kv_len), ks2).view(np.float16)
    vf = oracle.e4m3_to_f16(oracle.paged_gather(vc2, table2, kv_len), vs2).view(np.float16)
    ref, ref_lse = oracle.attention(q2, kf, vf, lib.default_scale(D), mode=oracle.MODE_CAUSAL, offset=kv_len - q_real)
    assert_close(out2.cpu().numpy().reshape(-1, D), ref, "call 2 vs oracle")
    assert np.abs(lse2.cpu().numpy().ravel() - ref_lse).max() < LSE_ABS

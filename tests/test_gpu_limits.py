"""GPU parity at the edges of the prefill and decode domains the library
accepts: the largest prefill (8192 query rows against 262144 cached
positions, FP16 and paged E4M3) and decode against the largest cache, and
the smallest causal shapes (one real query row, one 32-key page). Checked
against the FP64 oracle at the FP16 bounds (marked gpu)."""
import numpy as np
import pytest

import oracle
import synth.workloads as wl
from parity_util import LSE_ABS, assert_close, sample_rows, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _rows_of(out_np, rows):
    return out_np[rows[:, 0], rows[:, 1], rows[:, 2]].astype(np.float64)


# the largest prefill the ABI accepts: q_rows <= 8192, kv_len <= 262144
MAX_PREFILL = dict(name="causal prefill at the domain maxima B1 Hq6 Hkv1 D256 Q8192 KV262144", seed=11, B=1,
                   Hq=6, Hkv=1, D=256, q_rows=8192, q_real=8192, kv_len=262144, page_size=32)


def test_prefix_causal_domain_maxima(lib):
    w = MAX_PREFILL
    say("causal", w["name"])
    q, k, v = wl.causal_inputs(w)
    lse = torch.empty((w["B"], w["Hq"], w["q_rows"]), dtype=torch.float32, device="cuda")
    out = lib.attn_fwd_prefix_causal(dev(q), dev(k), dev(v), w["q_real"], lse=lse)
    torch.cuda.synchronize()
    rows = sample_rows(w["B"], w["Hq"], w["q_rows"], 10, seed=11, tile=2048)
    ref, ref_lse = oracle.attention(q, k, v, lib.default_scale(w["D"]), mode=oracle.MODE_CAUSAL,
                                    offset=w["kv_len"] - w["q_real"], rows=rows)
    assert_close(_rows_of(out.cpu().numpy(), rows), ref, f"O ({len(rows)} rows)")
    got_lse = lse.cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
    assert np.abs(got_lse - ref_lse).max() < LSE_ABS


def test_paged_prefill_and_decode_domain_maxima(lib):
    w = dict(MAX_PREFILL, name="paged E4M3 prefill at the domain maxima B1 Hq6 Hkv1 D256 Q8192 KV262144 page32")
    q, kc, vc, table, ks, vs = wl.paged_inputs(w, unit_scales=False)
    say("paged", w["name"], "scales", ks, vs)
    dq, dkc, dvc, dt = dev(q), dev(kc), dev(vc), dev(table)
    out = lib.attn_fwd_paged_e4m3(dq, dkc, dvc, dt, w["kv_len"], w["q_real"], ks, vs)
    # decode: the 16 last positions of every head against the same (largest) cache
    qd = q[:, :, -16:].copy()
    lse_d = torch.empty((w["B"], w["Hq"], 16), dtype=torch.float32, device="cuda")
    out_d = lib.attn_fwd_paged_e4m3_decode(dev(qd), dkc, dvc, dt, w["kv_len"], 16, ks, vs, lse=lse_d)
    torch.cuda.synchronize()
    kf = oracle.e4m3_to_f16(oracle.paged_gather(kc, table, w["kv_len"]), ks).view(np.float16)
    vf = oracle.e4m3_to_f16(oracle.paged_gather(vc, table, w["kv_len"]), vs).view(np.float16)
    rows = sample_rows(w["B"], w["Hq"], w["q_rows"], 8, seed=12, tile=2048)
    ref, _ = oracle.attention(q, kf, vf, lib.default_scale(w["D"]), mode=oracle.MODE_CAUSAL,
                              offset=w["kv_len"] - w["q_real"], rows=rows)
    assert_close(_rows_of(out.cpu().numpy(), rows), ref, f"prefill O ({len(rows)} rows)")
    ref_d, ref_lse_d = oracle.attention(qd, kf, vf, lib.default_scale(w["D"]), mode=oracle.MODE_CAUSAL,
                                        offset=w["kv_len"] - 16)
    assert_close(out_d.cpu().numpy().reshape(-1, w["D"]), ref_d, "decode O (all 96 rows)")
    assert np.abs(lse_d.cpu().numpy().ravel() - ref_lse_d).max() < LSE_ABS


@pytest.mark.parametrize("D", [128, 256])
def test_causal_smallest_shapes(lib, D):
    """One real query row of a 64-row tile against one 32-key page: FP16
    prefill, paged prefill, and a one-position decode."""
    w = dict(name=f"smallest causal B1 Hq2 Hkv1 D{D} Q64 (1 real) KV32", seed=13, B=1, Hq=2, Hkv=1, D=D,
             q_rows=64, q_real=1, kv_len=32, page_size=32)
    say(w["name"])
    q, k, v = wl.causal_inputs(w)
    out = lib.attn_fwd_prefix_causal(dev(q), dev(k), dev(v), w["q_real"])
    q8, kc, vc, table, ks, vs = wl.paged_inputs(w, unit_scales=False)
    dkc, dvc, dt = dev(kc), dev(vc), dev(table)
    out_p = lib.attn_fwd_paged_e4m3(dev(q8), dkc, dvc, dt, w["kv_len"], w["q_real"], ks, vs)
    qd = q8[:, :, :1].copy()
    out_d = lib.attn_fwd_paged_e4m3_decode(dev(qd), dkc, dvc, dt, w["kv_len"], 1, ks, vs)
    torch.cuda.synchronize()
    off = w["kv_len"] - w["q_real"]
    ref, _ = oracle.attention(q, k, v, lib.default_scale(D), mode=oracle.MODE_CAUSAL, offset=off)
    assert_close(out.cpu().numpy().reshape(-1, D), ref, "prefill O (all rows)")
    kf = oracle.e4m3_to_f16(oracle.paged_gather(kc, table, w["kv_len"]), ks).view(np.float16)
    vf = oracle.e4m3_to_f16(oracle.paged_gather(vc, table, w["kv_len"]), vs).view(np.float16)
    ref_p, _ = oracle.attention(q8, kf, vf, lib.default_scale(D), mode=oracle.MODE_CAUSAL, offset=off)
    assert_close(out_p.cpu().numpy().reshape(-1, D), ref_p, "paged prefill O (all rows)")
    ref_d, _ = oracle.attention(qd, kf, vf, lib.default_scale(D), mode=oracle.MODE_CAUSAL, offset=w["kv_len"] - 1)
    assert_close(out_d.cpu().numpy().reshape(-1, D), ref_d, "decode O")

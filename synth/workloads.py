"""The five seeded synthetic workloads of the attention hot path (shapes and
seeds only; no attention arithmetic).

Shapes follow the pages' workloads:
  * dense non-causal D128 attention of a video diffusion transformer, one
    GPU's share of heads ("[Kernel] Share SM70 projection, attention and row
    reduction paths", Purpose);
  * the long causal D256 GQA prefill against a prefix KV, Hq6/Hkv1, Q8000,
    KV 128000 and 256000, paged E4M3 cache with 32-token pages ("[Kernel][SM70]
    Integrate FP32 v37 prefill and exact E4M3 bridge", Implementation and
    Test plan);
  * VSA block-sparse video attention, top-k = 64 of 64-token blocks with two
    dense prefix query blocks ("[Video] Integrate H3 SM70 execution, metrics
    and VSA diagnostics", Purpose).
Values are N(0,1) FP16 draws from synth's counter-based generator with
seed = workload number and tensor ids Q=1, K=2, V=3, page table=4, scales=5.
"""
from __future__ import annotations

import numpy as np

from . import (TID_K, TID_Q, TID_SCALES, TID_TABLE, TID_V, e4m3_codes, normal_bf16, normal_f16, permutation,
               uniform, uniform_f32)

TINY_DENSE = dict(name="tiny dense attention B1 H2 D128 L256 non-causal", seed=1, B=1, H=2, D=128,
                  Lq=256, Lkv=256)
VIDEO_DENSE = dict(name="video-DiT dense attention B1 H8 D128 L36864 non-causal", seed=2, B=1, H=8,
                   D=128, Lq=36864, Lkv=36864)
# the dense shape of the GB10 page: 56 heads, a key length that is not a multiple of 32 or 64
RAGGED_DENSE = dict(name="ragged dense D128 B1 H56 Lq15360 Lkv29678 non-causal", seed=6, B=1, H=56, D=128,
                    Lq=15360, Lkv=29678)
PREFIX_CAUSAL = dict(name="causal prefill B1 Hq6 Hkv1 D256 Q8000 KV128000 (prefix 120000)", seed=3, B=1,
                     Hq=6, Hkv=1, D=256, q_rows=8000, q_real=8000, kv_len=128000)
PAGED_E4M3 = dict(name="paged E4M3 causal prefill B1 Hq6 Hkv1 D256 Q8000 KV256000 page32", seed=4, B=1,
                  Hq=6, Hkv=1, D=256, q_rows=8000, q_real=8000, kv_len=256000, page_size=32)
PAGED_DECODE = dict(name="paged E4M3 decode B1 Hq6 Hkv1 D256 Q16 KV256000 page32", seed=4, B=1, Hq=6, Hkv=1,
                    D=256, q_rows=16, q_real=16, kv_len=256000, page_size=32)
# valid-row gather with the FP8 round trip of the prefix keys, at the video shape
PREFIX_FP8 = dict(name="FP8 prefix-key round trip + gather B1 N36864 H8 D128, 32768 valid rows", seed=8, B=1,
                  N=36864, H=8, D=128, rows=32768)
VSA = dict(name="VSA block-sparse attention B1 H8 D128 L36864 block64 top-k 64 dense-prefix 2", seed=5,
           B=1, H=8, D=128, L=36864, block=64, topk=64, dense_prefix=2)


def dense_inputs(w):
    s = w["seed"]
    q = normal_f16(s, TID_Q, (w["B"], w["H"], w["Lq"], w["D"]))
    k = normal_f16(s, TID_K, (w["B"], w["H"], w["Lkv"], w["D"]))
    v = normal_f16(s, TID_V, (w["B"], w["H"], w["Lkv"], w["D"]))
    return q, k, v


def causal_inputs(w):
    s = w["seed"]
    q = normal_f16(s, TID_Q, (w["B"], w["Hq"], w["q_rows"], w["D"]))
    k = normal_f16(s, TID_K, (w["B"], w["Hkv"], w["kv_len"], w["D"]))
    v = normal_f16(s, TID_V, (w["B"], w["Hkv"], w["kv_len"], w["D"]))
    return q, k, v


def paged_scales(w, unit: bool):
    """(k_scale, v_scale): 1.0 each, or U(0.01, 0.1) draws rounded to FP32."""
    if unit:
        return 1.0, 1.0
    ks, vs = uniform_f32(w["seed"], TID_SCALES, 0.01, 0.1, 2)
    return float(ks), float(vs)


def paged_inputs(w, unit_scales: bool):
    """q FP16, E4M3 caches uint8 [pages, 32, Hkv, D], page table int32 [B, pages] (a
    permutation of the physical pages), and the two scales. The cache holds
    RNE_e4m3(x / scale) for x ~ N(0,1), so decode(code) * scale ~ N(0,1)."""
    s = w["seed"]
    ks, vs = paged_scales(w, unit_scales)
    pages = w["B"] * w["kv_len"] // w["page_size"]
    q = normal_f16(s, TID_Q, (w["B"], w["Hq"], w["q_rows"], w["D"]))
    kc = e4m3_codes(s, TID_K, (pages, w["page_size"], w["Hkv"], w["D"]), ks)
    vc = e4m3_codes(s, TID_V, (pages, w["page_size"], w["Hkv"], w["D"]), vs)
    table = permutation(s, TID_TABLE, pages).reshape(w["B"], -1).copy()
    return q, kc, vc, table, ks, vs


def vsa_inputs(w):
    s = w["seed"]
    shape = (w["B"], w["H"], w["L"], w["D"])
    return normal_f16(s, TID_Q, shape), normal_f16(s, TID_K, shape), normal_f16(s, TID_V, shape)


def prefix_fp8_inputs(w):
    """k, v: bfloat16 bit patterns [B, N, H, D] of N(0,1) draws times a per-(token, head)
    magnitude spread over 2^-8 .. 2^8; index: the sorted valid rows (a seeded subset)."""
    s = w["seed"]
    shape = (w["B"], w["N"], w["H"], w["D"])
    k = normal_bf16(s, TID_K, shape)
    v = normal_bf16(s, TID_V, shape)
    # spread K's per-row magnitude: add a per-(token, head) exponent offset in [-8, 8] to the bfloat16 bits
    e = (uniform(s, TID_SCALES, w["B"] * w["N"] * w["H"]) * 17).astype(np.int32) - 8
    e = np.repeat(e.reshape(w["B"], w["N"], w["H"], 1), w["D"], axis=3)
    expo = ((k >> 7) & 0xFF).astype(np.int32)
    nz = expo > 0
    k = np.where(nz, (k & 0x807F) | (np.clip(expo + e, 1, 254).astype(np.uint16) << 7), k).astype(np.uint16)
    index = np.sort(permutation(s, TID_TABLE, w["N"])[: w["rows"]]).astype(np.int32)
    return k, v, index

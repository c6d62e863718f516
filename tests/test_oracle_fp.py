"""Pins for the oracle's FP16 and E4M3 arithmetic (no GPU).

The oracle's conversions are checked against independent library routines
(numpy's correctly rounded float casts, torch's float8_e4m3fn dtype) and the
printed spot values of the format, never against a re-typed formula.
"""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_f16_decode_exhaustive_matches_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_bf16_decode_exhaustive_matches_torch():
    """All 65536 bfloat16 codes against torch's own bfloat16 -> float64 conversion."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_f64_to_f16_rounding_matches_numpy():
    rng = np.random.default_rng(7)
    h = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)  # all finite positive halves
    v = h.view(np.float16).astype(np.float64)
    nxt = np.append(v[1:], 65536.0)
    mids = (v + nxt) / 2.0  # exact ties: must round to even
    near = np.concatenate([mids * (1 + 2.0 ** -40), mids * (1 - 2.0 ** -40)])
    rand = np.ldexp(rng.random(200000) + 0.5, rng.integers(-30, 18, 200000))
    edge = np.array([65504.0, 65519.999, 65520.0, 1e6, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001,
                     2.0 ** -14, 2.0 ** -14 * (1 - 2.0 ** -12), 0.0, np.inf])
    x = np.concatenate([v, mids, near, rand, edge])
    x = np.concatenate([x, -x])
    ours = oracle.f64_to_f16(x)
    with np.errstate(over="ignore"):  # values past the FP16 range round to infinity, as intended
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def _golden_spots():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_spot_values.txt")) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if line:
                c, val = line.split()
                rows.append((int(c, 16), float(val)))
    return rows


def test_e4m3_spot_values_from_format_definition():
    table = oracle.e4m3_decode_table()
    spots = _golden_spots()
    assert len(spots) >= 10
    for code, val in spots:
        if np.isnan(val):
            assert np.isnan(table[code])
        else:
            assert table[code] == val and np.signbit(table[code]) == np.signbit(val), hex(code)


def test_e4m3_table_matches_torch_dtype_and_round_trips():
    table = oracle.e4m3_decode_table()
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    torch_vals = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(torch_vals)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(np.isnan(table), nan)
    assert np.array_equal(table[~nan], torch_vals[~nan])
    # decode -> encode gives the code back for all 254 finite codes
    finite = np.nonzero(~nan)[0]
    enc = torch.from_numpy(table[finite].astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8)
    back = enc.numpy().astype(np.int64)
    # +0 and -0 are distinct codes and must both come back
    assert np.array_equal(back, finite)
    assert np.nanmax(np.abs(table)) == 448.0


def test_e4m3_scaled_conversion_exhaustive_vs_numpy_two_roundings():
    """256 codes x 10^4 scales against numpy float32 multiply then float16 cast."""
    table = oracle.e4m3_decode_table()
    rng = np.random.default_rng(11)
    scales = np.concatenate([
        rng.uniform(0.01, 0.1, 4000), rng.uniform(0.5, 2.0, 2000),
        np.ldexp(rng.uniform(1, 2, 3990), rng.integers(-20, 8, 3990)),
        [1.0, 0.5, 2.0, 1.0 / 3.0, 0.01, 0.1, 7.0, 146.0, 2.0 ** -16, 1e-7]]).astype(np.float32)
    codes = np.arange(256, dtype=np.uint8)
    finite = ~np.isnan(table)
    for s in scales:
        ours = oracle.e4m3_to_f16(codes, float(s))
        prod = table[finite].astype(np.float32) * np.float32(s)  # one FP32 rounding
        with np.errstate(over="ignore"):  # large scales overflow FP16 to infinity, as intended
            ref = prod.astype(np.float16).view(np.uint16)  # one FP16 rounding
        assert np.array_equal(ours[finite], ref), float(s)
        assert ours[0x7F] == 0x7E00 and ours[0xFF] == 0xFE00


def test_e4m3_unit_scale_is_exact_decode():
    table = oracle.e4m3_decode_table()
    ours = oracle.e4m3_to_f16(np.arange(256, dtype=np.uint8), 1.0).view(np.float16).astype(np.float64)
    finite = ~np.isnan(table)
    assert np.array_equal(ours[finite], table[finite])
    # subnormal FP16 results are kept, not flushed: code 0x01 * 0.01 < 2^-14
    tiny = oracle.e4m3_to_f16(np.array([0x01, 0x81], dtype=np.uint8), 0.01)
    assert tiny[0] != 0 and tiny[0] < 0x0400 and tiny[1] == (tiny[0] | 0x8000)


def test_paged_gather_identity_and_permutation():
    rng = np.random.default_rng(3)
    pages, ps, hkv, d, kv_len = 12, 4, 2, 8, 43
    cache = rng.integers(0, 256, (pages, ps, hkv, d), dtype=np.uint8)
    ident = np.arange(pages, dtype=np.int32)[None]
    g = oracle.paged_gather(cache, ident, kv_len)
    contiguous = cache.reshape(pages * ps, hkv, d).transpose(1, 0, 2)[None, :, :kv_len]
    assert np.array_equal(g, contiguous)
    perm = rng.permutation(pages).astype(np.int32)
    g2 = oracle.paged_gather(cache, perm[None], kv_len)
    for t in range(kv_len):
        assert np.array_equal(g2[0, :, t], cache[perm[t // ps], t % ps])
    # a permutation of physical pages moved together with the table changes nothing
    inv = np.empty_like(perm)
    inv[perm] = np.arange(pages)
    moved = cache[np.argsort(inv)]  # page perm[t] of the old cache sits at slot t
    assert np.array_equal(oracle.paged_gather(moved, np.arange(pages, dtype=np.int32)[None], kv_len), g2)
    with pytest.raises(ValueError):
        oracle.paged_gather(cache, np.full((1, pages), pages, dtype=np.int32), kv_len)


def test_f32_to_e4m3_matches_torch_float8():
    """Every finite code value, every midpoint between neighbours (the ties) and
    random values in [-448, 448], against torch's float32 -> float8_e4m3fn cast."""
    vals = oracle.e4m3_decode_table()
    fin = np.sort(vals[np.isfinite(vals)])
    mids = (fin[:-1] + fin[1:]) / 2  # exact in FP32: E4M3 values have 4 significant bits
    rng = np.random.default_rng(21)
    rand = np.concatenate([rng.uniform(-448, 448, 4000), rng.uniform(-1, 1, 2000) * 2.0 ** -6])
    x = np.concatenate([fin, mids, rand, [0.0, -0.0]]).astype(np.float32)
    ours = oracle.f32_to_e4m3(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_f32_to_bf16_matches_torch():
    """Random FP32 values and exact ties (low 16 bits 0x8000) against torch's bfloat16 cast."""
    rng = np.random.default_rng(22)
    u = rng.integers(0, 0x7F7F0000, 6000, dtype=np.uint64).astype(np.uint32)
    ties = (u & 0xFFFF0000) | 0x8000
    bits = np.concatenate([u, ties, u | 0x80000000]).astype(np.uint32)
    x = bits.view(np.float32)
    ours = oracle.f32_to_bf16(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_prefix_fp8_gather_matches_torch_dtype_casts():
    """The round trip against torch float32 arithmetic with its float8_e4m3fn and
    bfloat16 casts (independent conversion routines), plus the gather of V."""
    rng = np.random.default_rng(23)
    B, N, H, D = 2, 40, 3, 128
    tk = torch.from_numpy(rng.standard_normal((B, N, H, D)) * rng.uniform(0.01, 30, (B, N, H, 1))).to(torch.bfloat16)
    tv = torch.from_numpy(rng.standard_normal((B, N, H, D))).to(torch.bfloat16)
    tk[0, 5, 1] = 0  # an all-zero row: scale 0
    index = rng.permutation(N)[:25].astype(np.int32)
    kb = tk.view(torch.int16).numpy().view(np.uint16)
    vb = tv.view(torch.int16).numpy().view(np.uint16)
    ko, vo = oracle.prefix_fp8_gather(kb, vb, index)
    kg = tk.float()[:, torch.from_numpy(index).long()]
    scale = kg.abs().amax(-1, keepdim=True) / 448.0
    inv = torch.where(scale == 0, torch.zeros_like(scale), 1.0 / scale)
    q8 = torch.clamp(kg * inv, -448.0, 448.0).to(torch.float8_e4m3fn).float()
    ref = (q8 * scale).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ko, ref)
    assert np.array_equal(vo, vb[:, index])


def test_fp8_quantize_rows_matches_torch_dtype_casts():
    """The per-row E4M3 quantization (prefix queries and keys) against torch
    float32 arithmetic and its float8_e4m3fn cast; its dequantized values,
    rounded to bfloat16, are the round trip's output."""
    rng = np.random.default_rng(29)
    t = torch.from_numpy(rng.standard_normal((3, 50, 128)) * rng.uniform(0.01, 40, (3, 50, 1))).to(torch.bfloat16)
    t[1, 7] = 0  # an all-zero row: scale 0, codes 0
    xb = t.view(torch.int16).numpy().view(np.uint16)
    codes, scales = oracle.fp8_quantize_rows(xb)
    x = t.float()
    scale = x.abs().amax(-1, keepdim=True) / 448.0
    inv = torch.where(scale == 0, torch.zeros_like(scale), 1.0 / scale)
    q8 = torch.clamp(x * inv, -448.0, 448.0).to(torch.float8_e4m3fn)
    assert np.array_equal(codes, q8.view(torch.uint8).numpy())
    assert np.array_equal(scales, scale[..., 0].numpy())
    assert scales[1, 7] == 0 and not codes[1, 7].any()
    # the dequantized values, exact in float64, equal the FP8 round trip before its bfloat16 storage
    deq = oracle.fp8_dequant(codes, scales)
    assert np.array_equal(deq, (q8.double() * scale.double()).numpy())
    # ... and rounded to bfloat16 they are the prefix round trip's keys
    ko, _ = oracle.prefix_fp8_gather(xb.reshape(1, 3 * 50, 1, 128), xb.reshape(1, 3 * 50, 1, 128),
                                     np.arange(150, dtype=np.int32))
    ref = torch.from_numpy(deq).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ko.reshape(3, 50, 128), ref)

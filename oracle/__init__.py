"""numpy front end of the FP64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the fp16_attention_amd package.
It shares no code with the HIP library; both sides only share the seeded
generators in synth/.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_i64p = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (plain -O2, no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                               "-fno-fast-math", "-pthread", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        lib.or_f16_to_f64.restype = ctypes.c_double
        lib.or_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.or_f32_to_e4m3.restype = ctypes.c_uint8
        lib.or_f32_to_e4m3.argtypes = [ctypes.c_float]
        lib.or_f32_to_bf16.restype = ctypes.c_uint16
        lib.or_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.or_fp8_quantize_rows.restype = None
        lib.or_fp8_quantize_rows.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                             ctypes.c_void_p]
        lib.or_prefix_fp8_gather.restype = None
        lib.or_prefix_fp8_gather.argtypes = [ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int] * 4 + [
            ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        lib.or_bf16_to_f64.restype = ctypes.c_double
        lib.or_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.or_f64_to_f16.restype = ctypes.c_uint16
        lib.or_f64_to_f16.argtypes = [ctypes.c_double]
        lib.or_e4m3_decode.restype = ctypes.c_double
        lib.or_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.or_e4m3_to_f16.restype = ctypes.c_uint16
        lib.or_e4m3_to_f16.argtypes = [ctypes.c_uint8, ctypes.c_float]
        lib.or_e4m3_to_f16_array.restype = None
        lib.or_e4m3_to_f16_array.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_float,
                                             ctypes.c_void_p]
        lib.or_paged_gather.restype = ctypes.c_int
        lib.or_paged_gather.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int64, ctypes.c_void_p]
        lib.or_attention.restype = ctypes.c_int
        lib.or_attention.argtypes = [ctypes.c_void_p, _i64p, ctypes.c_void_p, _i64p, ctypes.c_void_p,
                                     _i64p] + [ctypes.c_int] * 6 + [ctypes.c_double, ctypes.c_int,
                                     ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
        lib.or_merge.restype = None
        lib.or_merge.argtypes = [ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 5
        lib.or_vsa_pool.restype = None
        lib.or_vsa_pool.argtypes = [ctypes.c_void_p] + [ctypes.c_int] * 5 + [ctypes.c_void_p]
        lib.or_vsa_scores.restype = None
        lib.or_vsa_scores.argtypes = [ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int] * 4 + [
            ctypes.c_void_p]
        lib.or_block_lists.restype = None
        lib.or_block_lists.argtypes = [ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int] * 4 + [ctypes.c_void_p] * 4
        lib.or_vsa_topk.restype = None
        lib.or_vsa_topk.argtypes = [ctypes.c_void_p] + [ctypes.c_int] * 4 + [ctypes.c_void_p]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _strides(a: np.ndarray):
    st = [s // a.itemsize for s in a.strides]
    if st[3] != 1:
        raise ValueError("oracle expects a unit stride along D")
    return (ctypes.c_int64 * 3)(st[0], st[1], st[2])


def _threads(threads):
    return threads if threads else max(1, os.cpu_count() or 1)


# ---------------------------------------------------------------- FP16 / E4M3

def f16_to_f64(bits) -> np.ndarray:
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.or_f16_to_f64(int(x)) for x in b], dtype=np.float64)


def bf16_to_f64(bits) -> np.ndarray:
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.or_bf16_to_f64(int(x)) for x in b], dtype=np.float64)


def f64_to_f16(values) -> np.ndarray:
    lib = _load()
    v = np.asarray(values, dtype=np.float64).ravel()
    return np.array([lib.or_f64_to_f16(float(x)) for x in v], dtype=np.uint16)


def e4m3_decode_table() -> np.ndarray:
    """float64[256]: the value of each OCP E4M3FN byte code (NaN for 0x7F/0xFF)."""
    lib = _load()
    return np.array([lib.or_e4m3_decode(c) for c in range(256)], dtype=np.float64)


def e4m3_to_f16(codes: np.ndarray, scale: float) -> np.ndarray:
    """FP16 bits (uint16) of RNE16(RNE32(decode(code) * scale)), same shape."""
    lib = _load()
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.uint16)
    lib.or_e4m3_to_f16_array(_ptr(c), c.size, ctypes.c_float(np.float32(scale)), _ptr(out))
    return out


def f32_to_e4m3(x) -> np.ndarray:
    lib = _load()
    a = np.asarray(x, dtype=np.float32).ravel()
    return np.array([lib.or_f32_to_e4m3(float(v)) for v in a], dtype=np.uint8)


def f32_to_bf16(x) -> np.ndarray:
    lib = _load()
    a = np.asarray(x, dtype=np.float32).ravel()
    return np.array([lib.or_f32_to_bf16(float(v)) for v in a], dtype=np.uint16)


def prefix_fp8_gather(k: np.ndarray, v: np.ndarray, index: np.ndarray):
    """k, v: bfloat16 bit patterns (uint16) [B, N, H, D]; index: int32 source rows.
    Returns (ko, vo) uint16 [B, rows, H, D]: K's FP8 round trip with a per-(row, head)
    amax / 448 scale, and V, both gathered."""
    lib = _load()
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    index = np.ascontiguousarray(index, dtype=np.int32)
    B, N, H, D = k.shape
    rows = index.size
    ko = np.empty((B, rows, H, D), dtype=np.uint16)
    vo = np.empty_like(ko)
    lib.or_prefix_fp8_gather(_ptr(k), _ptr(v), B, N, H, D, _ptr(index), rows, _ptr(ko), _ptr(vo))
    return ko, vo


def fp8_quantize_rows(x: np.ndarray):
    """Per-row E4M3 quantization of bfloat16 bit patterns x [..., D]: returns (codes uint8
    [..., D], scales float32 [...]) with scale = max|x| / 448 (the round trip's first steps)."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.uint16)
    D = x.shape[-1]
    rows = x.size // D
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(x.shape[:-1], dtype=np.float32)
    lib.or_fp8_quantize_rows(_ptr(x), rows, D, _ptr(codes), _ptr(scales))
    return codes, scales


def fp8_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 decode(code) * scale, exact (a 4-bit E4M3 significand times an FP32 scale)."""
    return e4m3_decode_table()[codes] * scales.astype(np.float64)[..., None]


def paged_gather(cache: np.ndarray, table: np.ndarray, kv_len: int) -> np.ndarray:
    """cache uint8 [pages, page_size, Hkv, D], table int32 [B, pages_per_seq]
    -> contiguous uint8 [B, Hkv, kv_len, D]."""
    lib = _load()
    cache = np.ascontiguousarray(cache, dtype=np.uint8)
    table = np.ascontiguousarray(table, dtype=np.int32)
    pages, page_size, hkv, d = cache.shape
    bsz = table.shape[0]
    out = np.empty((bsz, hkv, kv_len, d), dtype=np.uint8)
    rc = lib.or_paged_gather(_ptr(cache), pages, page_size, _ptr(table), table.shape[1], bsz, hkv, d,
                             kv_len, _ptr(out))
    if rc:
        raise ValueError("page table entry out of range")
    return out


# ------------------------------------------------------------------ attention

MODE_DENSE, MODE_CAUSAL, MODE_BLOCKS = 0, 1, 2


def all_rows(B: int, H: int, L: int) -> np.ndarray:
    b, h, i = np.meshgrid(np.arange(B), np.arange(H), np.arange(L), indexing="ij")
    return np.stack([b.ravel(), h.ravel(), i.ravel()], axis=1).astype(np.int32)


def attention(q, k, v, scale: float, mode: int = MODE_DENSE, offset: int = 0, idx=None,
              block: int = 64, dense_prefix: int = 0, rows=None, threads: int = 0, bf16: bool = False):
    """FP64 attention of FP16 q [B,Hq,Lq,D], k/v [B,Hkv,Lkv,D] (any D-contiguous strides).

    bf16: the arrays are uint16 bit patterns of bfloat16 values instead.
    float64 arrays (all three) are used as they are.
    rows: int32 [n,3] (b, h, i) triples to compute (default: all rows).
    Returns (out float64 [n, D], lse float64 [n]) in the order of rows.
    """
    lib = _load()
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    if q.dtype == np.float64:
        fmt, want = 2, np.float64
    else:
        fmt, want = (1, np.uint16) if bf16 else (0, np.float16)
    for name, a in (("q", q), ("k", k), ("v", v)):
        if a.dtype != want or a.ndim != 4:
            raise TypeError(f"{name} must be a 4-D {np.dtype(want).name} array")
    B, Hq, Lq, D = q.shape
    _, Hkv, Lkv, _ = k.shape
    if rows is None:
        rows = all_rows(B, Hq, Lq)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    n = rows.shape[0]
    out = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    idx_arr = None
    if mode == MODE_BLOCKS:
        idx_arr = np.ascontiguousarray(idx, dtype=np.int32)
        topk = idx_arr.shape[-1]
    else:
        topk = 0
    rc = lib.or_attention(_ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v), B, Hq, Hkv,
                          Lq, Lkv, D, float(scale), mode, int(offset),
                          _ptr(idx_arr) if idx_arr is not None else None, block, topk, dense_prefix,
                          _ptr(rows), n, _ptr(out), _ptr(lse), _threads(threads), fmt)
    if rc:
        raise ValueError("invalid oracle arguments")
    return out, lse


def merge(m, l, o):
    """Merge per-segment (m, l, o) states; returns (out [D], lse)."""
    lib = _load()
    m = np.ascontiguousarray(m, dtype=np.float64)
    l = np.ascontiguousarray(l, dtype=np.float64)
    o = np.ascontiguousarray(o, dtype=np.float64)
    nseg, D = o.shape
    out = np.empty(D, dtype=np.float64)
    lse = np.empty(1, dtype=np.float64)
    lib.or_merge(nseg, D, _ptr(m), _ptr(l), _ptr(o), _ptr(out), _ptr(lse))
    return out, float(lse[0])


# ------------------------------------------------------------------------ VSA

def vsa_pool(x: np.ndarray, block: int) -> np.ndarray:
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float16)
    B, H, L, D = x.shape
    out = np.empty((B, H, (L + block - 1) // block, D), dtype=np.float32)
    lib.or_vsa_pool(_ptr(x), B, H, L, D, block, _ptr(out))
    return out


def vsa_scores(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    lib = _load()
    qbar = np.ascontiguousarray(qbar, dtype=np.float32)
    kbar = np.ascontiguousarray(kbar, dtype=np.float32)
    B, H, NB, D = qbar.shape
    s = np.empty((B, H, NB, NB), dtype=np.float64)
    lib.or_vsa_scores(_ptr(qbar), _ptr(kbar), B, H, NB, D, _ptr(s))
    return s


def vsa_topk(s: np.ndarray, topk: int) -> np.ndarray:
    lib = _load()
    s = np.ascontiguousarray(s, dtype=np.float64)
    B, H, NB, _ = s.shape
    idx = np.empty((B, H, NB, topk), dtype=np.int32)
    lib.or_vsa_topk(_ptr(s), B, H, NB, topk, _ptr(idx))
    return idx


def vsa_select(q: np.ndarray, k: np.ndarray, block: int, topk: int):
    """Pool, score, select. Returns (idx int32 [B,H,NB,topk], scores f64 [B,H,NB,NB])."""
    s = vsa_scores(vsa_pool(q, block), vsa_pool(k, block))
    return vsa_topk(s, topk), s


def block_lists(mask: np.ndarray, valid: np.ndarray, tile: int, quadrants: bool = True):
    """128-token block lists from a square tile mask [B,H,T,T] (bool or uint8) and the
    valid-token counts of the T tiles of `tile` tokens. Returns (idx int32 [B,H,NB,NB],
    counts int32 [B,H,NB], kv_valid int32 [2*NB], quad uint8 [B,H,NB,NB] or None)."""
    lib = _load()
    m = np.ascontiguousarray(mask, dtype=np.uint8)
    v = np.ascontiguousarray(valid, dtype=np.int32)
    B, H, T, T2 = m.shape
    assert T == T2 and v.shape == (T,) and tile % 64 == 0
    nb = (T * (tile // 64) + 1) // 2
    idx = np.empty((B, H, nb, nb), dtype=np.int32)
    counts = np.empty((B, H, nb), dtype=np.int32)
    kv = np.empty((2 * nb,), dtype=np.int32)
    quad = np.empty((B, H, nb, nb), dtype=np.uint8) if quadrants else None
    lib.or_block_lists(_ptr(m), _ptr(v), B, H, T, tile, _ptr(idx), _ptr(counts), _ptr(kv),
                       _ptr(quad) if quad is not None else None)
    return idx, counts, kv, quad


def tile_means(x: np.ndarray, block: int) -> np.ndarray:
    """FP32 means of the valid rows of each `block`-row tile of x [B,H,L,D] FP16 (the
    exact sum divided by the count, rounded once): the pooled V of the VSA coarse branch."""
    return vsa_pool(x, block)

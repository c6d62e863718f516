"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle.

This module holds no attention arithmetic: it only draws numbers. Every value
is a pure function of (seed, tensor_id, element index), so the GPU side and the
oracle side see the same inputs without either importing the other.

Generator (counter based, written from the published definitions):
  * SplitMix64 finaliser (Steele, Lea, Flood, "Fast splittable pseudorandom
    number generators", OOPSLA 2014) applied to key + (i+1)*golden-gamma.
  * Uniform in (0, 1]: ((x >> 11) + 1) * 2**-53.
  * Normal pairs by the Box-Muller transform in float64, rounded to FP16
    with round-to-nearest-even (numpy's float64 -> float16 cast).

Tensor ids: Q=1, K=2, V=3, page table=4, scales=5.
"""
from __future__ import annotations

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 20

TID_Q, TID_K, TID_V, TID_TABLE, TID_SCALES = 1, 2, 3, 4, 5


def _mix_inplace(z: np.ndarray, tmp: np.ndarray) -> np.ndarray:
    """SplitMix64 finaliser, in place (fresh large arrays are slow to fault in)."""
    np.right_shift(z, np.uint64(30), out=tmp)
    np.bitwise_xor(z, tmp, out=z)
    np.multiply(z, _M1, out=z)
    np.right_shift(z, np.uint64(27), out=tmp)
    np.bitwise_xor(z, tmp, out=z)
    np.multiply(z, _M2, out=z)
    np.right_shift(z, np.uint64(31), out=tmp)
    np.bitwise_xor(z, tmp, out=z)
    return z


def _key(seed: int, tensor_id: int) -> np.uint64:
    base = np.array([((seed & 0xFFFFFFFF) << 16) | (tensor_id & 0xFFFF)], dtype=np.uint64)
    np.multiply(base, _GAMMA, out=base)
    np.add(base, _GAMMA, out=base)
    return _mix_inplace(base, np.empty_like(base))[0]


def raw_u64(seed: int, tensor_id: int, start: int, count: int) -> np.ndarray:
    """64-bit words number start .. start+count-1 of the stream (seed, tensor_id)."""
    key = _key(seed, tensor_id)
    z = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    np.multiply(z, _GAMMA, out=z)
    np.add(z, key, out=z)
    return _mix_inplace(z, np.empty_like(z))


def uniform(seed: int, tensor_id: int, count: int, start: int = 0) -> np.ndarray:
    """float64 uniforms in (0, 1]."""
    x = raw_u64(seed, tensor_id, start, count)
    return ((x >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)


def normal_f64(seed: int, tensor_id: int, count: int) -> np.ndarray:
    """count N(0,1) draws in float64; element 2j and 2j+1 share one Box-Muller pair."""
    out = np.empty(count, dtype=np.float64)
    npairs = (count + 1) // 2
    for p0 in range(0, npairs, _CHUNK):
        n = min(_CHUNK, npairs - p0)
        u = uniform(seed, tensor_id, 2 * n, start=2 * p0)
        r = np.sqrt(-2.0 * np.log(u[0::2]))
        t = 2.0 * np.pi * u[1::2]
        pair = np.empty(2 * n, dtype=np.float64)
        pair[0::2] = r * np.cos(t)
        pair[1::2] = r * np.sin(t)
        lo = 2 * p0
        hi = min(count, lo + 2 * n)
        out[lo:hi] = pair[: hi - lo]
    return out


def _threads() -> int:
    import os
    return max(1, min(8, os.cpu_count() or 1))


def _blocks(n: int):
    step = 2 * _CHUNK
    return [(lo, min(n, lo + step)) for lo in range(0, n, step)]


def normal_f16(seed: int, tensor_id: int, shape) -> np.ndarray:
    """FP16 tensor of N(0,1) draws (float64 Box-Muller, RNE to FP16)."""
    from concurrent.futures import ThreadPoolExecutor

    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.float16)

    def fill(span):
        lo, hi = span
        out[lo:hi] = normal_f64_block(seed, tensor_id, lo, hi).astype(np.float16)

    with ThreadPoolExecutor(_threads()) as pool:
        list(pool.map(fill, _blocks(n)))
    return out.reshape(shape)


def normal_bf16(seed: int, tensor_id: int, shape) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of the same N(0,1) draws: float64 -> float32
    (numpy, nearest even) -> the upper 16 bits, nearest even."""
    from concurrent.futures import ThreadPoolExecutor

    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.uint16)

    def fill(span):
        lo, hi = span
        u = normal_f64_block(seed, tensor_id, lo, hi).astype(np.float32).view(np.uint32)
        out[lo:hi] = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)

    with ThreadPoolExecutor(_threads()) as pool:
        list(pool.map(fill, _blocks(n)))
    return out.reshape(shape)


def normal_f64_block(seed: int, tensor_id: int, lo: int, hi: int) -> np.ndarray:
    """Elements lo..hi-1 of the normal stream; lo must be even."""
    assert lo % 2 == 0
    p0, p1 = lo // 2, (hi + 1) // 2
    u = uniform(seed, tensor_id, 2 * (p1 - p0), start=2 * p0)
    r = np.sqrt(-2.0 * np.log(u[0::2]))
    t = 2.0 * np.pi * u[1::2]
    pair = np.empty(2 * (p1 - p0), dtype=np.float64)
    pair[0::2] = r * np.cos(t)
    pair[1::2] = r * np.sin(t)
    return pair[: hi - lo]


def permutation(seed: int, tensor_id: int, n: int) -> np.ndarray:
    """Fisher-Yates shuffle of 0..n-1 driven by the uniform stream (int32)."""
    perm = np.arange(n, dtype=np.int64)
    u = uniform(seed, tensor_id, max(n - 1, 0))
    for step, i in enumerate(range(n - 1, 0, -1)):
        j = min(int(u[step] * (i + 1)), i)
        perm[i], perm[j] = perm[j], perm[i]
    return perm.astype(np.int32)


def uniform_f32(seed: int, tensor_id: int, lo: float, hi: float, count: int) -> np.ndarray:
    """count draws of U(lo, hi) in float64, rounded to float32."""
    return (lo + (hi - lo) * uniform(seed, tensor_id, count)).astype(np.float32)


def e4m3_codes(seed: int, tensor_id: int, shape, scale: float) -> np.ndarray:
    """OCP E4M3FN byte codes of N(0,1)/scale, saturated to +-448 (uint8).

    The encoding uses torch's float8_e4m3fn cast (round to nearest even) on
    values clamped to the finite range, so no code is NaN.
    """
    from concurrent.futures import ThreadPoolExecutor

    import torch

    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint8)

    def fill(span):
        lo, hi = span
        x = normal_f64_block(seed, tensor_id, lo, hi) / float(scale)
        x = np.clip(x, -448.0, 448.0).astype(np.float32)
        out[lo:hi] = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()

    with ThreadPoolExecutor(_threads()) as pool:
        list(pool.map(fill, _blocks(n)))
    return out.reshape(shape)

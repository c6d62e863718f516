"""Shared helpers of the GPU parity tests: seeded inputs (synth), tolerance
checks against the FP64 oracle, row sampling."""
import sys

import numpy as np

import synth

# FP16-output tolerance of the hot path: max-abs 2e-3 and relative L2 1e-3
# against the FP64 oracle.
MAX_ABS = 2e-3
REL_L2 = 1e-3
# LSE is FP32: compare it with an absolute bound. The GPU's row sum l adds
# the probabilities after they are rounded to FP16 (each once, relative error
# at most 2^-11), so ln l is off by at most ~2^-11 = 4.9e-4, plus the FP32
# rounding of the maximum.
LSE_ABS = 1e-3
# BF16 outputs (and BF16 P): the same bounds in units of the format's unit
# roundoff, which is 2^-8 for BF16 against 2^-11 for FP16, i.e. 8x
BF16_MAX_ABS = 8 * MAX_ABS
BF16_REL_L2 = 8 * REL_L2
# with BF16 probabilities ln l is off by up to 2^-9 = 2.0e-3 (reached when one
# or two keys dominate a row); the same 8x scaling as the other BF16 bounds
BF16_LSE_ABS = 8 * LSE_ABS


def say(*msg):
    print(*msg, flush=True)
    sys.stdout.flush()


def assert_close(out, ref, what="", max_abs=MAX_ABS, rel_l2=REL_L2):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert out.shape == ref.shape, (out.shape, ref.shape)
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    err = out - ref
    ma = float(np.abs(err).max()) if err.size else 0.0
    rl = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-30))
    say(f"  {what}: max_abs={ma:.3e} rel_l2={rl:.3e}")
    assert ma <= max_abs, f"{what}: max-abs {ma} > {max_abs}"
    assert rl <= rel_l2, f"{what}: rel-L2 {rl} > {rel_l2}"


def qkv_bf16(seed, B, H, Lq, Lkv, D):
    """bfloat16 bit patterns (uint16) of the seeded N(0,1) draws."""
    q = synth.normal_bf16(seed, synth.TID_Q, (B, H, Lq, D))
    k = synth.normal_bf16(seed, synth.TID_K, (B, H, Lkv, D))
    v = synth.normal_bf16(seed, synth.TID_V, (B, H, Lkv, D))
    return q, k, v


def qkv(seed, B, Hq, Hkv, Lq, Lkv, D):
    q = synth.normal_f16(seed, synth.TID_Q, (B, Hq, Lq, D))
    k = synth.normal_f16(seed, synth.TID_K, (B, Hkv, Lkv, D))
    v = synth.normal_f16(seed, synth.TID_V, (B, Hkv, Lkv, D))
    return q, k, v


def sample_rows(B, H, L, per_head, seed, tile=128, extra=()):
    """First/last rows, tile boundaries and seeded random rows of every (b, h)."""
    rng = np.random.default_rng(seed)
    base = {0, 1, L - 1, L - 2}
    for t in range(tile, L, tile * max(1, (L // tile) // 8)):
        base.update({t - 1, t})
    base.update(e for e in extra if 0 <= e < L)
    rows = []
    for b in range(B):
        for h in range(H):
            sel = set(base)
            sel.update(rng.integers(0, L, max(0, per_head - len(sel))).tolist())
            rows += [(b, h, i) for i in sorted(sel)]
    return np.array(rows, dtype=np.int32)

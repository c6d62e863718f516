"""GPU parity of the dense launch whose last partial round runs as 8-wave
workgroups that split each item's keys between their two halves and merge the
two online-softmax states in LDS (marked gpu).

The shapes have 520 work items (B1 H4, 130 query tiles of 128 rows): four
whole rounds' worth of slots (512) run the 4-wave kernel and the last 8 items
(head 3, query tiles 122-129) the split one. Key counts cover a second half
with a ragged last tile, with one key, with fewer tiles than the first half
(its last iteration sees no key at all), and many tiles. Every row of the
split items and a sample of the others are compared with the FP64 oracle; O
and LSE sit inside sentinel-filled buffers. The rescale cases force, on the
CPU, maxima that differ between the halves, so the merge weights both ways.
"""
import numpy as np
import pytest

import oracle
import work_items
from parity_util import BF16_LSE_ABS, BF16_MAX_ABS, BF16_REL_L2, LSE_ABS, assert_close, qkv, qkv_bf16, sample_rows, say
from test_gpu_rescale_edges import check_guards, guarded_lse, guarded_out, plant

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

B, H, LQ, D = 1, 4, 16640, 128


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def split_rows():
    """(b, h, i) of every real row of the items the split launch runs."""
    rows = [(0, 3, i) for i in range(122 * 128, LQ)]
    return np.array(rows, dtype=np.int32)


def key_split(Lkv):
    out = work_items.check("dense_tail", B, H, LQ, Lkv, D)
    return int(out.rsplit(" ", 1)[1])


def run_and_check(lib, q, k, v, rows, what):
    Lkv = k.shape[2]
    o, lse = guarded_out(B, H, LQ, D), guarded_lse(B, H, LQ)
    lib.attn_fwd_dense(dev(q), dev(k), dev(v), out=o.view, lse=lse.view)
    torch.cuda.synchronize()
    check_guards(o, lse)
    ref, ref_lse = oracle.attention(q, k, v, lib.default_scale(D), rows=rows)
    got = o.view.cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]].astype(np.float64)
    assert_close(got, ref, f"{what} O ({len(rows)} rows, Lkv {Lkv})")
    got_lse = lse.view.cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
    assert np.abs(got_lse - ref_lse).max() < LSE_ABS
    return o


@pytest.mark.parametrize("Lkv", [200, 130, 65, 4100])
def test_dense_tail_split_parity(lib, Lkv):
    ks = key_split(Lkv)
    say(f"dense tail split B{B} H{H} Lq{LQ} Lkv{Lkv} D{D}: key split {ks}")
    q, k, v = qkv(41, B, H, H, LQ, Lkv, D)
    rows = np.concatenate([split_rows(), sample_rows(B, H, LQ, 16, seed=41)])
    run_and_check(lib, q, k, v, rows, "split")


@pytest.mark.parametrize("case", ["q16", "planted"])
def test_dense_tail_split_rescale(lib, case):
    Lkv = 4100
    ks = key_split(Lkv)
    say(f"dense tail split rescale {case}: Lkv {Lkv}, key split {ks}")
    q, k, v = qkv(42, B, H, H, LQ, Lkv, D)
    chosen = [122 * 128, 122 * 128 + 77, 125 * 128 + 5, LQ - 1]
    if case == "q16":
        q = (q.astype(np.float32) * 16).astype(np.float16)
    else:
        # dominant keys in the last tile of the second half for two rows and
        # in the last tile of the first half for the other two: each half's
        # state then loses to the other's in the merge for some rows
        for n, i in enumerate(chosen):
            plant(q, k, 0, 3, 3, i, (Lkv - 1 - n) if n % 2 == 0 else (ks - 1 - n))
    scale = lib.default_scale(D)
    # the halves' maxima (log2 units) differ by more than the rescale slack
    # for some of the split rows: the merge must weight the states both ways
    s = (q[0, 3, 122 * 128:].astype(np.float64) @ k[0, 3].astype(np.float64).T) * scale * 1.4426950408889634
    m0, m1 = s[:, :ks].max(axis=1), s[:, ks:].max(axis=1)
    say(f"  rows with m0 > m1 + 8: {(m0 > m1 + 8).sum()}, m1 > m0 + 8: {(m1 > m0 + 8).sum()}")
    assert (m0 > m1 + 8).sum() >= 1 and (m1 > m0 + 8).sum() >= 1
    rows = split_rows()
    o = run_and_check(lib, q, k, v, rows, case)
    if case == "planted":
        for n, i in enumerate(chosen):
            j = (Lkv - 1 - n) if n % 2 == 0 else (ks - 1 - n)
            got = o.view[0, 3, i].double().cpu().numpy()
            assert np.abs(got - v[0, 3, j].astype(np.float64)).max() < 2e-3


def test_dense_tail_split_bf16(lib):
    """The same split on BF16 operands (P and O in BF16), at the BF16 bounds."""
    Lkv = 4100
    say(f"dense tail split bf16: Lkv {Lkv}, key split {key_split(Lkv)}")
    q, k, v = qkv_bf16(43, B, H, LQ, Lkv, D)
    rows = np.concatenate([split_rows(), sample_rows(B, H, LQ, 16, seed=43)])
    o, lse = guarded_out(B, H, LQ, D, torch.bfloat16), guarded_lse(B, H, LQ)
    dq, dk, dv = (dev(x.view(np.int16)).view(torch.bfloat16) for x in (q, k, v))
    lib.attn_fwd_dense(dq, dk, dv, out=o.view, lse=lse.view)
    torch.cuda.synchronize()
    check_guards(o, lse)
    ref, ref_lse = oracle.attention(q, k, v, lib.default_scale(D), bf16=True, rows=rows)
    got = o.view.double().cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
    assert_close(got, ref, f"bf16 O ({len(rows)} rows)", BF16_MAX_ABS, BF16_REL_L2)
    got_lse = lse.view.cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
    assert np.abs(got_lse - ref_lse).max() < BF16_LSE_ABS

"""GPU parity of every attention kernel instantiation the workloads use on
inputs that drive the online softmax through its rescale and the method's
degenerate cases, with guard canaries around every output (marked gpu).

Online softmax ("[Kernel][SM70] Integrate FP32 v37 prefill and exact E4M3
bridge", Implementation: FP32 running state per key segment and a final
merge): each kernel keeps a reference maximum per row and rescales its FP32
output and row sum only when a later score exceeds it by more than 2^8 (log2
units). N(0,1) inputs never do that, so these cases use
  * queries scaled by 16: scores spread over ~25 log2 units per sigma;
  * a dominant key planted at the last key a chosen row sees (the last tile
    of its last segment): the row's output is then that key's value row;
  * identical keys: every row's output is the mean of the values it sees;
  * causal rows whose last key segment is entirely past their last key.
Every test asserts on the CPU, from the work items the launcher uses, that
its inputs force a raise after the first tile of some segment for many rows,
so none can pass without running the rescale.

Canaries: O is a strided view inside a larger buffer (extra rows before and
after, 16 extra columns per row), LSE a view inside a larger FP32 buffer,
and the workspace a slice of a larger byte buffer; every element outside the
views must keep its sentinel bits. The VSA cases with a partial last block
also check that rows past L are not written.
"""
import numpy as np
import pytest

import oracle
import synth
import work_items
from parity_util import BF16_LSE_ABS, BF16_MAX_ABS, BF16_REL_L2, LSE_ABS, assert_close, qkv, qkv_bf16, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634
SLACK = 8.0          # log2 units a score must exceed the reference maximum by
O_SENT = 0x7D5B      # FP16 NaN payload no kernel writes
LSE_SENT = 0x7FA0BAD5
WS_SENT = 0xA5
PAD_ROWS = 3
PAD_COLS = 16


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


# ------------------------------------------------------------------------ canaries

class Guarded:
    """An output view inside a sentinel-filled buffer."""

    def __init__(self, full, view, interior_mask):
        self.full, self.view, self.mask = full, view, interior_mask

    def check(self, what, sentinel):
        bits = self.full.cpu().numpy()
        outside = bits[~self.mask]
        bad = int(np.count_nonzero(outside != np.array(sentinel).astype(bits.dtype)))
        assert bad == 0, f"{what}: {bad} elements written outside the view"


def guarded_out(B, H, L, D, dtype=torch.float16):
    full = torch.full((B, H, L + 2 * PAD_ROWS, D + PAD_COLS), O_SENT, dtype=torch.int16, device="cuda")
    view = full.view(dtype)[:, :, PAD_ROWS:PAD_ROWS + L, :D]
    mask = np.zeros(full.shape, dtype=bool)
    mask[:, :, PAD_ROWS:PAD_ROWS + L, :D] = True
    return Guarded(full, view, mask)


def guarded_lse(B, H, L):
    n = B * H * L
    full = torch.full((n + 128,), LSE_SENT, dtype=torch.int32, device="cuda")
    view = full[64:64 + n].view(torch.float32).view(B, H, L)
    mask = np.zeros(n + 128, dtype=bool)
    mask[64:64 + n] = True
    return Guarded(full, view, mask)


def guarded_ws(nbytes):
    full = torch.full((nbytes + 8192,), WS_SENT, dtype=torch.uint8, device="cuda")
    view = full[4096:4096 + nbytes]
    mask = np.zeros(nbytes + 8192, dtype=bool)
    mask[4096:4096 + nbytes] = True
    return Guarded(full, view, mask)


def check_guards(o, lse=None, ws=None):
    o.check("O", np.int16(O_SENT))
    if lse is not None:
        lse.check("LSE", np.int32(LSE_SENT))
    if ws is not None:
        ws.check("workspace", np.uint8(WS_SENT))


# -------------------------------------------------- raises the inputs force (CPU)

def raises_forced(q, k, scale, row_keys, first_tile):
    """Number of rows whose scores, streamed in the order given, exceed the
    maximum of their segment's first tile by more than the slack: row_keys is
    a list of (b, h, g, i, [segment key arrays in stream order])."""
    n = 0
    for b, h, g, i, segs in row_keys:
        qi = q[b, h, i].astype(np.float64)
        for keys in segs:
            if len(keys) <= first_tile:
                continue
            s = (k[b, g, keys].astype(np.float64) @ qi) * scale * LOG2E
            if s[first_tile:].max() > s[:first_tile].max() + SLACK:
                n += 1
                break
    return n


def causal_row_keys(mode, shape, rows_of_item, offset, q_rows, group):
    """(b, h, g, i, segments) for the rows of a causal or decode launch, from
    the launcher's own work items; a segment's keys are clipped to the row's
    causal limit."""
    out = []
    for it in work_items.items(mode, *shape):
        if it["empty"]:
            continue
        for h, i in rows_of_item(it):
            lim = min(it["key_stop"], offset + i + 1)
            keys = np.arange(it["key_begin"], max(it["key_begin"], lim))
            out.append((it["b"], h, h // group, i, [keys]))
    return out


def plant(q, k, b, h, g, i, j, gain=8.0):
    """Key j of kv head g becomes gain x query row i of head h: that row's score
    for j is then ~gain * |q_i|^2 * scale, far above every other."""
    k[b, g, j] = (gain * q[b, h, i].astype(np.float32)).astype(k.dtype)


# ----------------------------------------------------------------------- dense

@pytest.mark.parametrize("D,case", [(128, "q16"), (128, "planted"), (256, "q16"), (256, "planted")])
def test_dense_rescale(lib, D, case):
    B, H, Lq, Lkv = 1, 2, 300, 2000
    say(f"dense rescale D{D} {case}: B{B} H{H} Lq{Lq} Lkv{Lkv}")
    q, k, v = qkv(21, B, H, H, Lq, Lkv, D)
    chosen = [0, 37, 128, 299]
    if case == "q16":
        q = (q.astype(np.float32) * 16).astype(np.float16)
    else:
        for n, i in enumerate(chosen):
            plant(q, k, 0, n % H, n % H, i, Lkv - 1 - n)  # in the last 64-key tile
    scale = lib.default_scale(D)
    first = 64 if D == 128 else 32
    rows = [(0, h, h, i, [np.arange(Lkv)]) for h in range(H) for i in (range(Lq) if case == "q16" else chosen)]
    forced = raises_forced(q, k, scale, rows, first)
    say(f"  rows forced to raise: {forced} of {len(rows)}")
    assert forced >= (len(rows) // 4 if case == "q16" else len(chosen))
    o, lse = guarded_out(B, H, Lq, D), guarded_lse(B, H, Lq)
    lib.attn_fwd_dense(dev(q), dev(k), dev(v), out=o.view, lse=lse.view, scale=scale)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention(q, k, v, scale)
    assert_close(o.view.cpu().numpy().reshape(-1, D), ref, "O")
    assert np.abs(lse.view.cpu().numpy().ravel() - ref_lse).max() < LSE_ABS
    if case == "planted":
        for n, i in enumerate(chosen):
            got = o.view[0, n % H, i].double().cpu().numpy()
            assert np.abs(got - v[0, n % H, Lkv - 1 - n].astype(np.float64)).max() < 2e-3
    check_guards(o, lse)


def test_dense_bf16_rescale(lib):
    B, H, Lq, Lkv, D = 1, 2, 200, 1000, 128
    say(f"dense bf16 rescale: B{B} H{H} Lq{Lq} Lkv{Lkv}")
    q, k, v = qkv_bf16(22, B, H, Lq, Lkv, D)
    # x16 is exact on BF16 bit patterns: add 4 to the exponent of every normal value
    e = (q >> 7) & 0xFF
    q = np.where((e > 0) & (e < 250), q + (4 << 7), q).astype(np.uint16)
    qf = (q.astype(np.uint32) << 16).view(np.float32)
    kf = (k.astype(np.uint32) << 16).view(np.float32)
    scale = lib.default_scale(D)
    rows = [(0, h, h, i, [np.arange(Lkv)]) for h in range(H) for i in range(Lq)]
    forced = raises_forced(qf, kf, scale, rows, 64)
    assert forced >= len(rows) // 4, forced
    o, lse = guarded_out(B, H, Lq, D, torch.bfloat16), guarded_lse(B, H, Lq)
    dq, dk, dv = (dev(x.view(np.int16)).view(torch.bfloat16) for x in (q, k, v))
    lib.attn_fwd_dense(dq, dk, dv, out=o.view, lse=lse.view, scale=scale)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention(q, k, v, scale, bf16=True)
    assert_close(o.view.double().cpu().numpy().reshape(-1, D), ref, "O bf16", BF16_MAX_ABS, BF16_REL_L2)
    assert np.abs(lse.view.cpu().numpy().ravel() - ref_lse).max() < BF16_LSE_ABS
    check_guards(o, lse)


@pytest.mark.parametrize("D", [128, 256])
def test_dense_identical_keys_give_mean_of_values(lib, D):
    B, H, Lq, Lkv = 1, 2, 130, 777
    say(f"dense identical keys D{D}")
    q, k, v = qkv(23, B, H, H, Lq, Lkv, D)
    k[:] = k[:, :, :1]
    o = guarded_out(B, H, Lq, D)
    lib.attn_fwd_dense(dev(q), dev(k), dev(v), out=o.view)
    torch.cuda.synchronize()
    mean = v.astype(np.float64).mean(axis=2, keepdims=True)
    got = o.view.double().cpu().numpy()
    assert_close(got.reshape(-1, D), np.broadcast_to(mean, got.shape).reshape(-1, D), "O vs mean(V)")
    ref, _ = oracle.attention(q, k, v, lib.default_scale(D))
    assert_close(got.reshape(-1, D), ref, "O vs oracle")
    check_guards(o)


# ---------------------------------------------------------------------- causal

def _causal_rows(shape, q_real, q_rows, rows=128):
    B, Hq, Hkv, D, _, _, kv_len = shape
    group = Hq // Hkv

    def rows_of(it):
        q0 = it["qt"] * rows
        return [(it["h"], i) for i in range(q0, min(q0 + rows, q_rows))]
    return causal_row_keys("causal", shape, rows_of, kv_len - q_real, q_rows, group)


@pytest.mark.parametrize("split,case", [(True, "q16"), (True, "planted"), (False, "q16"), (False, "planted")])
def test_causal_d256_rescale(lib, split, case):
    # split: 4096 keys in several segments per query tile; unsplit: 1920 keys
    # (30 units of 64) are too few for two segments of at least 16 units
    B, Hq, Hkv, D, q_rows, q_real = 1, 6, 1, 256, 256, 200
    kv_len = 4096 if split else 1920
    shape = (B, Hq, Hkv, D, q_rows, q_real, kv_len)
    nws = lib.prefix_causal_workspace(B, Hq, Hkv, D, q_rows, kv_len)
    say(f"causal D256 rescale {case} split={split}: q{q_rows} real{q_real} kv{kv_len} ws={nws}")
    assert (nws > 0) == split
    q, k, v = qkv(24, B, Hq, Hkv, q_rows, kv_len, D)
    off = kv_len - q_real
    # (head, row, planted key): each real row's last visible key; row 255 is
    # padding (it sees every key) and takes the one before the last
    chosen = [(0, 0, off), (1, 63, off + 63), (2, 130, off + 130), (5, 199, off + 199), (3, 255, kv_len - 2)]
    if case == "q16":
        q = (q.astype(np.float32) * 16).astype(np.float16)
    else:
        for h, i, j in chosen:
            plant(q, k, 0, h, 0, i, j)
    rk = _causal_rows(shape, q_real, q_rows)
    if case == "planted":
        rk = [r for r in rk if (r[1], r[3]) in {(h, i) for h, i, _ in chosen}]
    forced = raises_forced(q, k, lib.default_scale(D), rk, 32)
    say(f"  (row, segment) pairs forced to raise: {forced} of {len(rk)}")
    assert forced >= (len(rk) // 4 if case == "q16" else len(chosen))
    o, lse = guarded_out(B, Hq, q_rows, D), guarded_lse(B, Hq, q_rows)
    ws = guarded_ws(nws) if nws else None
    lib.attn_fwd_prefix_causal(dev(q), dev(k), dev(v), q_real, out=o.view, lse=lse.view,
                               workspace=None if ws is None else ws.view)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention(q, k, v, lib.default_scale(D), mode=oracle.MODE_CAUSAL, offset=off)
    assert_close(o.view.cpu().numpy().reshape(-1, D), ref, "O")
    assert np.abs(lse.view.cpu().numpy().ravel() - ref_lse).max() < LSE_ABS
    if case == "planted":
        for h, i, j in chosen:
            assert np.abs(o.view[0, h, i].double().cpu().numpy() - v[0, 0, j].astype(np.float64)).max() < 2e-3
    check_guards(o, lse, ws)


def _find_masked_late_segment(D, Hq, q_rows, q_real):
    """A kv_len (multiple of 32) whose last key segment of some query tile lies
    entirely past the last key of some of that tile's rows."""
    for kv_len in range(2400, 40000, 32):
        if kv_len <= q_real:
            continue
        shape = (1, Hq, 1, D, q_rows, q_real, kv_len)
        if lib_ws(shape) == 0:
            continue
        off = kv_len - q_real
        for it in work_items.items("causal", *shape):
            if it["empty"] or it["seg"] == 0:
                continue
            q0 = it["qt"] * 128
            masked = [i for i in range(q0, min(q0 + 128, q_rows)) if off + i < it["key_begin"]]
            if masked and it["key_stop"] == it["key_end"]:
                return kv_len, it, masked
    return None


def lib_ws(shape):
    import fp16_attention_amd as fa
    B, Hq, Hkv, D, q_rows, _, kv_len = shape
    return fa.prefix_causal_workspace(B, Hq, Hkv, D, q_rows, kv_len)


@pytest.mark.parametrize("D", [256, 128])
def test_causal_fully_masked_late_segment(lib, D):
    Hq, q_rows, q_real = 2, 128, 128
    found = _find_masked_late_segment(D, Hq, q_rows, q_real)
    assert found is not None, "no shape with a fully masked late segment"
    kv_len, it, masked = found
    say(f"causal D{D} masked late segment: kv{kv_len} segment {it['seg']} keys [{it['key_begin']}, "
        f"{it['key_stop']}) fully masked for {len(masked)} rows")
    q, k, v = qkv(25, 1, Hq, 1, q_rows, kv_len, D)
    q = (q.astype(np.float32) * 16).astype(np.float16)
    nws = lib.prefix_causal_workspace(1, Hq, 1, D, q_rows, kv_len)
    o, lse, ws = guarded_out(1, Hq, q_rows, D), guarded_lse(1, Hq, q_rows), guarded_ws(nws)
    lib.attn_fwd_prefix_causal(dev(q), dev(k), dev(v), q_real, out=o.view, lse=lse.view, workspace=ws.view)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention(q, k, v, lib.default_scale(D), mode=oracle.MODE_CAUSAL, offset=kv_len - q_real)
    assert_close(o.view.cpu().numpy().reshape(-1, D), ref, "O")
    assert np.abs(lse.view.cpu().numpy().ravel() - ref_lse).max() < LSE_ABS
    check_guards(o, lse, ws)


def test_causal_identical_keys_give_mean_of_visible_values(lib):
    B, Hq, Hkv, D, q_rows, q_real, kv_len = 1, 2, 1, 256, 128, 100, 3072
    say("causal identical keys")
    q, k, v = qkv(26, B, Hq, Hkv, q_rows, kv_len, D)
    k[:] = k[:, :, :1]
    off = kv_len - q_real
    o = guarded_out(B, Hq, q_rows, D)
    ws = guarded_ws(lib.prefix_causal_workspace(B, Hq, Hkv, D, q_rows, kv_len))
    lib.attn_fwd_prefix_causal(dev(q), dev(k), dev(v), q_real, out=o.view, workspace=ws.view)
    torch.cuda.synchronize()
    csum = np.cumsum(v[0, 0].astype(np.float64), axis=0)
    n = np.minimum(off + np.arange(q_rows) + 1, kv_len)
    mean = csum[n - 1] / n[:, None]
    got = o.view.double().cpu().numpy()[0]
    for h in range(Hq):
        assert_close(got[h], mean, f"head {h} vs mean of visible V")
    check_guards(o, None, ws)


# ----------------------------------------------------------------------- paged

def _paged(seed, Hkv, D, kv_len, ks, vs):
    pages = kv_len // 32 + 5
    kc = synth.e4m3_codes(seed, synth.TID_K, (pages, 32, Hkv, D), ks)
    vc = synth.e4m3_codes(seed, synth.TID_V, (pages, 32, Hkv, D), vs)
    table = synth.permutation(seed, synth.TID_TABLE, pages)[None, : kv_len // 32].copy()
    return kc, vc, table


def _plant_code(q, kc, table, h, i, j, ks, gain=8.0):
    """Logical key j's codes become E4M3(gain * q_i / ks) (kv head 0)."""
    import torch as _t
    x = np.clip(gain * q[0, h, i].astype(np.float32) / ks, -448, 448).astype(np.float32)
    kc[table[0, j // 32], j % 32, 0] = _t.from_numpy(x).to(_t.float8_e4m3fn).view(_t.uint8).numpy()


def _decoded(kc, vc, table, kv_len, ks, vs):
    kf = oracle.e4m3_to_f16(oracle.paged_gather(kc, table, kv_len), ks).view(np.float16)
    vf = oracle.e4m3_to_f16(oracle.paged_gather(vc, table, kv_len), vs).view(np.float16)
    return kf, vf


@pytest.mark.parametrize("case,ks,vs,D,bridged", [("q16", 0.0371, 0.0815, 256, False),
                                                  ("planted", 0.0371, 0.0815, 256, False),
                                                  ("q16", 0.0625, 0.5, 256, False),
                                                  ("q16", 0.0703418, 0.0493912, 128, False),
                                                  ("q16", 0.0371, 0.0815, 256, True),
                                                  ("planted", 0.0371, 0.0815, 256, True)])
def test_paged_prefill_rescale(lib, case, ks, vs, D, bridged):
    # power-of-two k_scale: the exact decode; otherwise the K conversion in
    # LDS (in place) or the bridge into the workspace and the FP16 kernel
    Hq, Hkv, q_rows, q_real, kv_len = 6, 1, 128, 100, 4096
    ks, vs = float(np.float32(ks)), float(np.float32(vs))
    shape = (1, Hq, Hkv, D, q_rows, q_real, kv_len)
    say(f"paged prefill rescale {case}: q{q_rows} real{q_real} kv{kv_len}")
    q = synth.normal_f16(27, synth.TID_Q, (1, Hq, q_rows, D))
    kc, vc, table = _paged(27, Hkv, D, kv_len, ks, vs)
    off = kv_len - q_real
    # (head, row, planted key); row 127 is padding and takes the key before the last
    chosen = [(0, 5, off + 5), (3, 99, off + 99), (5, 127, kv_len - 2)]
    if case == "q16":
        q = (q.astype(np.float32) * 16).astype(np.float16)
    else:
        for h, i, j in chosen:
            _plant_code(q, kc, table, h, i, j, ks)
    kf, vf = _decoded(kc, vc, table, kv_len, ks, vs)
    rk = _causal_rows(shape, q_real, q_rows)
    if case == "planted":
        rk = [r for r in rk if (r[1], r[3]) in {(h, i) for h, i, _ in chosen}]
    forced = raises_forced(q, kf, lib.default_scale(D), rk, 32)
    say(f"  (row, segment) pairs forced to raise: {forced} of {len(rk)}")
    assert forced >= (len(rk) // 4 if case == "q16" else len(chosen))
    nws = lib.paged_e4m3_workspace(1, Hq, Hkv, D, q_rows, kv_len, ks if bridged else None)
    assert nws > 0
    if bridged:
        assert nws >= 4 * Hkv * kv_len * D  # the FP16 K and V are in it
    o, lse, ws = guarded_out(1, Hq, q_rows, D), guarded_lse(1, Hq, q_rows), guarded_ws(nws)
    lib.attn_fwd_paged_e4m3(dev(q), dev(kc), dev(vc), dev(table), kv_len, q_real, ks, vs, out=o.view,
                            lse=lse.view, workspace=ws.view)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention(q, kf, vf, lib.default_scale(D), mode=oracle.MODE_CAUSAL, offset=off)
    assert_close(o.view.cpu().numpy().reshape(-1, D), ref, "O")
    assert np.abs(lse.view.cpu().numpy().ravel() - ref_lse).max() < LSE_ABS
    check_guards(o, lse, ws)


@pytest.mark.parametrize("kv_len,case,ks,vs", [(4096, "q16", 0.0625, 0.03125), (4096, "q16", 0.0371, 0.0815),
                                              (4096, "planted", 0.0371, 0.0815), (16416, "q16", 0.0703418, 0.0493912)])
def test_paged_decode_rescale(lib, kv_len, case, ks, vs):
    # power-of-two scales take the exact decode, others the in-register K
    # conversion; 16416 keys: 16 segments, merged by the workgroup-per-row merge
    Hq, Hkv, D, q_rows, q_real = 6, 1, 256, 16, 16
    ks, vs = float(np.float32(ks)), float(np.float32(vs))
    shape = (1, Hq, Hkv, D, q_rows, q_real, kv_len)
    say(f"paged decode rescale {case}: q{q_rows} kv{kv_len}")
    q = synth.normal_f16(28, synth.TID_Q, (1, Hq, q_rows, D))
    kc, vc, table = _paged(28, Hkv, D, kv_len, ks, vs)
    off = kv_len - q_real
    chosen = [(0, 0), (2, 7), (5, 15)]
    if case == "q16":
        q = (q.astype(np.float32) * 16).astype(np.float16)
    else:
        for h, i in chosen:
            _plant_code(q, kc, table, h, i, off + i, ks)
    kf, vf = _decoded(kc, vc, table, kv_len, ks, vs)

    def rows_of(it):
        return [(it["h"] + j, i) for j in range(Hq // Hkv) for i in range(q_rows)]
    rk = causal_row_keys("decode", shape, rows_of, off, q_rows, Hq // Hkv)
    if case == "planted":
        rk = [r for r in rk if (r[1], r[3]) in chosen]
    forced = raises_forced(q, kf, lib.default_scale(D), rk, 32)
    say(f"  (row, segment) pairs forced to raise: {forced} of {len(rk)}")
    assert forced >= (len(rk) // 4 if case == "q16" else len(chosen))
    nws = int(lib.load().attn_fwd_paged_e4m3_decode_workspace(1, Hq, Hkv, D, q_rows, kv_len))
    o, lse, ws = guarded_out(1, Hq, q_rows, D), guarded_lse(1, Hq, q_rows), guarded_ws(nws)
    lib.attn_fwd_paged_e4m3_decode(dev(q), dev(kc), dev(vc), dev(table), kv_len, q_real, ks, vs, out=o.view,
                                   lse=lse.view, workspace=ws.view)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention(q, kf, vf, lib.default_scale(D), mode=oracle.MODE_CAUSAL, offset=off)
    assert_close(o.view.cpu().numpy().reshape(-1, D), ref, "O")
    assert np.abs(lse.view.cpu().numpy().ravel() - ref_lse).max() < LSE_ABS
    check_guards(o, lse, ws)


# -------------------------------------------------------------------------- VSA

@pytest.mark.parametrize("L,case", [(64 * 30 + 37, "q16"), (64 * 30 + 37, "planted"), (64 * 24, "q16")])
def test_vsa_sparse_rescale(lib, L, case):
    B, H, D, topk, dp = 1, 2, 128, 7, 2
    NB = (L + 63) // 64
    say(f"vsa sparse rescale {case}: L{L} NB{NB} k{topk} dense prefix {dp}")
    q, k, v = qkv(29, B, H, H, L, L, D)
    # block lists: distinct ascending blocks drawn per (head, query block); the
    # kernel reads them as given, however they were chosen
    rng = np.random.default_rng(29)
    idx = np.stack([np.stack([np.sort(rng.choice(NB, topk, replace=False)) for _ in range(NB)])
                    for _ in range(H)])[None].astype(np.int32)
    chosen = [(0, 2 * 64 + 3), (1, 10 * 64 + 63), (0, (NB - 1) * 64 + 1), (1, 5)]  # (head, row); row 5: dense prefix
    if case == "q16":
        q = (q.astype(np.float32) * 16).astype(np.float16)
    else:
        for h, i in chosen:
            bq = i // 64
            last_blk = NB - 1 if bq < dp else int(idx[0, h, bq, -1])
            j = min(last_blk * 64 + 63, L - 1)
            plant(q, k, 0, h, h, i, j)
    # stream order of each row's keys: dense-prefix rows by their item's
    # segment, sparse rows along their list (two 32-key tiles per block)
    its = work_items.items("blocks", B, H, L, D, 64, topk, dp)
    rk = []
    for it in its:
        if it["empty"]:
            continue
        q0 = it["qt"] * 64
        for i in range(q0, min(q0 + 64, L)):
            if case == "planted" and (it["h"], i) not in chosen:
                continue
            if it["list"]:
                keys = np.concatenate([np.arange(b * 64, min(b * 64 + 64, L)) for b in idx[0, it["h"], it["qt"]]])
            else:
                keys = np.arange(it["key_begin"], it["key_stop"])
            rk.append((0, it["h"], it["h"], i, [keys]))
    forced = raises_forced(q, k, lib.default_scale(D), rk, 32)
    say(f"  (row, item) pairs forced to raise: {forced} of {len(rk)}")
    assert forced >= (len(rk) // 4 if case == "q16" else len(chosen))
    nws = lib.vsa_block_sparse_attn_workspace(B, H, L, D, 64, topk, dp)
    o, lse, ws = guarded_out(B, H, L, D), guarded_lse(B, H, L), guarded_ws(max(nws, 256))
    lib.vsa_block_sparse_attn(dev(q), dev(k), dev(v), dev(idx), dense_prefix_qblocks=dp, out=o.view, lse=lse.view,
                              workspace=ws.view if nws else None)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention(q, k, v, lib.default_scale(D), mode=oracle.MODE_BLOCKS, idx=idx, block=64,
                                    dense_prefix=dp)
    assert_close(o.view.cpu().numpy().reshape(-1, D), ref, "O")
    assert np.abs(lse.view.cpu().numpy().ravel() - ref_lse).max() < LSE_ABS
    check_guards(o, lse, ws)

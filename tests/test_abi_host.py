"""Host-side checks of the C-ABI library (no GPU, no compute calls).

The library must load, export every function include/fa16attn.h declares,
and reject invalid arguments with the documented codes before any HIP call.
"""
import ctypes
import os
import re
import subprocess

import pytest

import fp16_attention_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa16attn.h")
MEASURE_HEADER = os.path.join(ROOT, "include", "fa16measure.h")

# fake, 256-byte aligned, distinct host addresses: only ever validated, never dereferenced
A, B_, C, O, L, W = (0x10000000 * (i + 1) for i in range(6))


def _declared(header=HEADER):
    with open(header) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b([a-z_0-9]+)\s*\([^;{]*\)\s*;", text)) - {"if", "while"}


def test_header_declarations_are_all_exported():
    declared = _declared()
    assert declared == set(fa.EXPORTS), declared ^ set(fa.EXPORTS)
    out = subprocess.check_output(["nm", "-D", "--defined-only", fa.LIB_PATH]).decode()
    exported = {line.split()[-1] for line in out.splitlines()}
    assert declared <= exported
    lib = fa.load()
    for name in declared:
        assert hasattr(lib, name)
    assert lib.fa_abi_version() == 1


def test_measurement_library_is_separate():
    """The measurement aid has a header and library of its own; the attention
    library neither declares nor exports it."""
    from fp16_attention_amd import measure
    declared = _declared(MEASURE_HEADER)
    assert declared == set(measure.EXPORTS)
    out = subprocess.check_output(["nm", "-D", "--defined-only", measure.LIB_PATH]).decode()
    assert declared <= {line.split()[-1] for line in out.splitlines()}
    attn = subprocess.check_output(["nm", "-D", "--defined-only", fa.LIB_PATH]).decode()
    assert "fa_mfma_ceiling" not in attn
    assert not (declared & _declared())


def test_library_has_no_undefined_kernel_stubs():
    """Every kernel launch stub the host code calls is defined in the library."""
    out = subprocess.check_output(["nm", "-C", "--undefined-only", fa.LIB_PATH]).decode()
    stubs = [line for line in out.splitlines() if "__device_stub__" in line]
    assert not stubs, stubs


def test_error_strings():
    for code in range(7):
        assert fa.error_string(code)
    assert "HIP" in fa.error_string(1000 + 1)


def T(addr, sb=1 << 20, sh=1 << 16, ss=128):
    return fa.FaTensor(addr, sb, sh, ss)


def dense(**kw):
    args = dict(q=T(A), k=T(B_), v=T(C), o=T(O), lse=None, B=1, H=2, Lq=256, Lkv=256, D=128, scale=0.088)
    args.update(kw)
    return fa.load().attn_fwd_dense(args["q"], args["k"], args["v"], args["o"], args["lse"], args["B"],
                                    args["H"], args["Lq"], args["Lkv"], args["D"], args["scale"], None)


def test_dense_rejections():
    assert dense(q=T(0)) == fa.FA_ERR_NULL
    assert dense(q=T(A + 2)) == fa.FA_ERR_ALIGN
    assert dense(k=T(B_, ss=130)) == fa.FA_ERR_ALIGN
    assert dense(D=64) == fa.FA_ERR_UNSUPPORTED
    assert dense(Lkv=0) == fa.FA_ERR_SHAPE
    assert dense(B=0) == fa.FA_ERR_SHAPE
    assert dense(scale=0.0) == fa.FA_ERR_SHAPE
    assert dense(scale=float("nan")) == fa.FA_ERR_SHAPE
    assert dense(o=T(A)) == fa.FA_ERR_ALIAS            # output aliases q
    assert dense(o=T(A + (1 << 16) * 2)) == fa.FA_ERR_ALIAS  # overlaps q's second head
    assert dense(lse=O) == fa.FA_ERR_ALIAS
    assert dense(Lq=0) == fa.FA_OK                     # empty query: a no-op, no launch


def causal(**kw):
    args = dict(q=T(A), k=T(B_, sh=1 << 22, sb=1 << 22, ss=256), v=T(C, sh=1 << 22, sb=1 << 22, ss=256),
                o=T(O), lse=None, B=1, Hq=6, Hkv=1, D=256, q_rows=128, q_real=100, kv_len=4096, scale=0.0625,
                ws=W, ws_bytes=1 << 30)
    args.update(kw)
    a = args
    return fa.load().attn_fwd_prefix_causal(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"],
                                            a["Hkv"], a["D"], a["q_rows"], a["q_real"], a["kv_len"],
                                            a["scale"], a["ws"], a["ws_bytes"], None)


def test_causal_domain_rejections():
    q = T(A, sb=1 << 20, sh=128 * 256, ss=256)
    assert causal(q=q, q_rows=100) == fa.FA_ERR_SHAPE       # not a multiple of 64
    assert causal(q=q, q_rows=8256) == fa.FA_ERR_SHAPE      # above 8192
    assert causal(q=q, q_real=0) == fa.FA_ERR_SHAPE
    assert causal(q=q, q_real=129) == fa.FA_ERR_SHAPE       # more real rows than rows
    assert causal(q=q, kv_len=100) == fa.FA_ERR_SHAPE       # q_real >= kv_len
    assert causal(q=q, kv_len=4000 + 16) == fa.FA_ERR_SHAPE  # not a multiple of 32
    assert causal(q=q, kv_len=262144 + 32) == fa.FA_ERR_SHAPE
    assert causal(q=q, Hq=5, Hkv=2) == fa.FA_ERR_SHAPE
    assert causal(q=q, D=192) == fa.FA_ERR_UNSUPPORTED
    need = fa.prefix_causal_workspace(1, 6, 1, 256, 128, 4096)
    assert need > 0
    assert causal(q=q, ws=0) == fa.FA_ERR_WORKSPACE
    assert causal(q=q, ws_bytes=need - 1) == fa.FA_ERR_WORKSPACE
    assert causal(q=q, ws=W + 16) == fa.FA_ERR_ALIGN
    assert causal(q=q, ws=A) == fa.FA_ERR_ALIAS             # workspace over q


def test_decode_rejections_and_workspace():
    lib = fa.load()

    def decode(**kw):
        a = dict(q_rows=16, q_real=16, Hq=6, Hkv=1, D=256, kv_len=4096, page_size=32, ws=W, ws_bytes=1 << 30,
                 ks=1.0, stride=4096 // 32)
        a.update(kw)
        return lib.attn_fwd_paged_e4m3_decode(T(A), B_, C, L, a["stride"], 200, a["page_size"], a["ks"], 1.0,
                                              T(O), None, 1, a["Hq"], a["Hkv"], a["D"], a["q_rows"], a["q_real"],
                                              a["kv_len"], 0.0625, a["ws"], a["ws_bytes"], None)
    assert decode(q_rows=17, q_real=17) == fa.FA_ERR_SHAPE
    assert decode(Hq=16) == fa.FA_ERR_SHAPE           # 16 heads x 16 rows exceed one 128-row tile
    assert decode(q_real=0) == fa.FA_ERR_SHAPE
    assert decode(q_real=17) == fa.FA_ERR_SHAPE
    assert decode(kv_len=4100) == fa.FA_ERR_SHAPE
    assert decode(page_size=16) == fa.FA_ERR_UNSUPPORTED
    assert decode(D=64) == fa.FA_ERR_UNSUPPORTED
    assert decode(ks=0.0) == fa.FA_ERR_SHAPE
    assert decode(stride=10) == fa.FA_ERR_SHAPE
    assert decode(ws=0) == fa.FA_ERR_WORKSPACE
    need = lib.attn_fwd_paged_e4m3_decode_workspace(1, 6, 1, 256, 16, 4096)
    assert decode(ws_bytes=need - 1) == fa.FA_ERR_WORKSPACE
    # 64 key units of 64 allow 4 segments of 1024 keys; 96 packed rows each
    assert need == 4 * 6 * 16 * (256 * 4 + 8)
    # 256000 keys: one segment per CU (256), capped at 1024-key segments (250)
    assert lib.attn_fwd_paged_e4m3_decode_workspace(1, 6, 1, 256, 16, 256000) == 250 * 96 * (256 * 4 + 8)
    assert lib.attn_fwd_paged_e4m3_decode_workspace(1, 6, 1, 256, 17, 256000) == 0   # invalid shape


def test_paged_bridged_workspace():
    """The bridged plan's size: the split-KV states rounded up to 256 bytes plus FP16 K and V, only for a
    k_scale whose products with the E4M3 values are not all FP16 values (else the in-place size)."""
    lib = fa.load()
    shape = (1, 6, 1, 256, 8000, 256000)
    base = lib.attn_fwd_paged_e4m3_workspace(*shape)
    partial = (base + 255) // 256 * 256
    assert lib.attn_fwd_paged_e4m3_bridged_workspace(*shape, 0.0703418) == partial + 4 * 256000 * 256
    for pow2 in (1.0, 0.0625, 2.0 ** -15, 128.0):
        assert lib.attn_fwd_paged_e4m3_bridged_workspace(*shape, pow2) == base
    assert lib.attn_fwd_paged_e4m3_bridged_workspace(*shape, 256.0) == partial + 4 * 256000 * 256
    assert lib.attn_fwd_paged_e4m3_bridged_workspace(1, 6, 1, 256, 100, 256000, 0.07) == 0  # invalid shape
    assert fa.paged_e4m3_workspace(*shape) == base
    assert fa.paged_e4m3_workspace(*shape, k_scale=0.0703418) == partial + 4 * 256000 * 256


def test_workspace_queries_are_pure_functions_of_shape():
    lib = fa.load()
    a = lib.attn_fwd_prefix_causal_workspace(1, 6, 1, 256, 8000, 128000)
    assert a == lib.attn_fwd_prefix_causal_workspace(1, 6, 1, 256, 8000, 128000) > 0
    assert lib.attn_fwd_paged_e4m3_workspace(1, 6, 1, 256, 8000, 256000) >= a
    assert lib.attn_fwd_prefix_causal_workspace(1, 6, 1, 256, 100, 128000) == 0  # invalid shape -> 0
    # a short key range needs no split and no workspace
    assert lib.attn_fwd_prefix_causal_workspace(1, 6, 1, 256, 64, 512) == 0
    # 378 query tiles of D256 on one workgroup per CU: two key segments per tile
    # fill three rounds of 256 slots best (756 items)
    assert a == 2 * 6 * 8000 * (256 * 4 + 8)
    # two query tiles: as many segments as 1024-key minimum segments allow (16)
    assert lib.attn_fwd_prefix_causal_workspace(1, 2, 1, 256, 64, 16480) == 16 * 2 * 64 * (256 * 4 + 8)
    # pooled FP32 means (256-byte aligned) then the FP64 block scores
    assert lib.vsa_block_select_workspace(1, 8, 36864, 128, 64) == 2 * 8 * 576 * 128 * 4 + 8 * 576 * 576 * 8
    # 576 blocks, top-k 64: the two dense-prefix query blocks of each head split into 9 segments
    rows = 9 * 8 * 2 * 64
    assert lib.vsa_block_sparse_attn_workspace(1, 8, 36864, 128, 64, 64, 2) == rows * 128 * 4 + rows * 8
    assert lib.vsa_block_sparse_attn_workspace(1, 8, 36864, 128, 64, 64, 0) == 0    # nothing dense
    assert lib.vsa_block_sparse_attn_workspace(1, 8, 36864, 128, 64, 576, 2) == 0   # one segment
    assert lib.vsa_block_sparse_attn_workspace(1, 8, 36864, 128, 32, 64, 2) == 0    # unsupported block


def test_paged_and_bridge_rejections():
    lib = fa.load()
    q = T(A, sb=1 << 20, sh=128 * 256, ss=256)

    def paged(**kw):
        a = dict(page_size=32, ks=1.0, vs=1.0, table_stride=128, pages=128, kv_len=4096, kc=B_, vc=C)
        a.update(kw)
        return lib.attn_fwd_paged_e4m3(q, a["kc"], a["vc"], L, a["table_stride"], a["pages"], a["page_size"],
                                       a["ks"], a["vs"], T(O), None, 1, 6, 1, 256, 128, 100, a["kv_len"],
                                       0.0625, W, 1 << 30, None)
    assert paged(page_size=16) == fa.FA_ERR_UNSUPPORTED
    assert paged(ks=0.0) == fa.FA_ERR_SHAPE
    assert paged(vs=float("inf")) == fa.FA_ERR_SHAPE
    assert paged(table_stride=10) == fa.FA_ERR_SHAPE
    assert paged(pages=0) == fa.FA_ERR_SHAPE
    assert paged(kc=0) == fa.FA_ERR_NULL
    assert paged(kc=B_ + 1) == fa.FA_ERR_ALIGN

    def bridge(**kw):
        a = dict(kc=B_, vc=C, ko=O, vo=O + (1 << 24), D=256, kv_len=4096, page_size=32)
        a.update(kw)
        return lib.kv_e4m3_paged_to_fp16(a["kc"], a["vc"], L, 128, 128, a["page_size"], 1, 1, a["D"],
                                         a["kv_len"], 1.0, 1.0, a["ko"], a["vo"], None)
    assert bridge(kc=0) == fa.FA_ERR_NULL
    assert bridge(D=64) == fa.FA_ERR_UNSUPPORTED
    assert bridge(page_size=64) == fa.FA_ERR_UNSUPPORTED
    assert bridge(kv_len=0) == fa.FA_ERR_SHAPE
    assert bridge(kv_len=(1 << 26) + 32) == fa.FA_ERR_SHAPE
    assert bridge(vo=O + 64) == fa.FA_ERR_ALIAS       # k_out and v_out overlap
    assert bridge(ko=B_) == fa.FA_ERR_ALIAS           # output over the cache


def test_vsa_rejections():
    lib = fa.load()

    def select(**kw):
        a = dict(L=4096, D=128, block=64, topk=8, ws=W, ws_bytes=1 << 30, idx=O)
        a.update(kw)
        return lib.vsa_block_select(A, B_, 1, 2, a["L"], a["D"], a["block"], a["topk"], a["idx"], None, a["ws"],
                                    a["ws_bytes"], None)
    assert select(block=128) == fa.FA_ERR_UNSUPPORTED
    assert select(D=256) == fa.FA_ERR_UNSUPPORTED
    assert select(L=0) == fa.FA_ERR_SHAPE
    # a length that is not a multiple of the block: the last block is partial
    assert lib.vsa_block_select_workspace(1, 2, 4000, 128, 64) == 2 * 2 * 63 * 128 * 4 + 2 * 63 * 63 * 8
    assert select(topk=0) == fa.FA_ERR_SHAPE
    assert select(topk=65) == fa.FA_ERR_SHAPE         # more than NB = 64
    assert select(L=64 * 1025, topk=4) == fa.FA_ERR_SHAPE
    assert select(ws=0) == fa.FA_ERR_WORKSPACE
    assert select(idx=0) == fa.FA_ERR_NULL
    assert select(idx=A) == fa.FA_ERR_ALIAS

    def sparse(**kw):
        a = dict(topk=8, dp=2, L=4096, o=O, ws=W, ws_bytes=1 << 30)
        a.update(kw)
        return lib.vsa_block_sparse_attn(T(A), T(B_), T(C), T(a["o"]), L, None, 1, 2, a["L"], 128, 64, a["topk"],
                                         a["dp"], 0.088, a["ws"], a["ws_bytes"], None)
    need = lib.vsa_block_sparse_attn_workspace(1, 2, 4096, 128, 64, 8, 2)
    assert need == 8 * 2 * 2 * 64 * (128 + 2) * 4  # 8 segments of 8 blocks, 2 heads, 2 dense blocks
    assert sparse(ws=0) == fa.FA_ERR_WORKSPACE
    assert sparse(ws_bytes=need - 1) == fa.FA_ERR_WORKSPACE
    assert sparse(ws=W + 16) == fa.FA_ERR_ALIGN
    assert sparse(ws=C - 256) == fa.FA_ERR_ALIAS      # workspace runs into v
    assert sparse(topk=65) == fa.FA_ERR_SHAPE
    assert sparse(dp=65) == fa.FA_ERR_SHAPE
    assert sparse(dp=-1) == fa.FA_ERR_SHAPE
    assert sparse(o=C) == fa.FA_ERR_ALIAS


def test_kernels_take_no_values_from_inline_asm():
    """Inline asm in the kernels may only fence the compiler or pin a value to
    a register class: the compiler inserts no hazard wait states before an asm
    statement, so an asm that computes on an MFMA result can read it early."""
    csrc = os.path.join(ROOT, "fp16_attention_amd", "csrc")
    # an empty template (a compiler fence, or a value pinned to its register
    # class) issues no instruction; a comment-only template neither
    allowed = ('asm volatile("" ::: "memory")', 'asm volatile("; q fragment to AGPRs"', 'asm volatile("" : "+v"(')
    for name in sorted(os.listdir(csrc)):
        if not name.endswith((".hip", ".h", ".cpp")):
            continue
        with open(os.path.join(csrc, name)) as f:
            lines = f.read().splitlines()
        for n, line in enumerate(lines, 1):
            code = line.split("//")[0]
            if re.search(r"\basm\b", code):
                assert any(a in code for a in allowed), f"{name}:{n}: {line.strip()}"


def test_vsa_keep_ratio():
    assert fa.vsa_topk_for_sparsity(36864, 0.8) == 116    # 576 blocks, 115.2 kept
    assert fa.vsa_topk_for_sparsity(36864, 0.0) == 576
    assert fa.vsa_topk_for_sparsity(64 * 3 + 1, 0.5) == 2  # 4 blocks, the last partial
    assert fa.vsa_topk_for_sparsity(64, 0.99) == 1         # never below one block
    assert fa.vsa_topk_for_sparsity(640, 0.7) == 3         # (1 - 0.7) * 10 is 3.0000000000000004
    assert fa.vsa_topk_for_sparsity(1280, 0.9) == 2        # (1 - 0.9) * 20 is 1.9999999999999996
    assert fa.vsa_topk_for_sparsity(36864, 1 - 64 / 576) == 64
    with pytest.raises(fa.FaError):
        fa.vsa_topk_for_sparsity(36864, 1.0)


def test_mfma_ceiling_rejections():
    from fp16_attention_amd import measure
    lib = measure.load()
    assert lib.fa_mfma_ceiling(16, None, None) == measure.FAM_ERR_NULL
    # the pointer is never dereferenced on the host, and no launch happens
    assert lib.fa_mfma_ceiling(0, 256, None) == measure.FAM_ERR_SHAPE
    assert lib.fa_mfma_ceiling((1 << 20) + 1, 256, None) == measure.FAM_ERR_SHAPE
    assert measure.mfma_ceiling_flop(1000) == 512.0 * 4 * 1000 * 4 * 32768


def test_binding_validates_every_tensor_before_the_library():
    """The C side receives bare pointers and cannot check dtypes or extents, so
    the binding rejects bad outputs, LSE buffers, operands and workspaces first
    (CPU tensors here: every check runs before the device check and before any
    library call)."""
    import torch
    h, f32, bf = torch.float16, torch.float32, torch.bfloat16
    q = torch.zeros(1, 2, 64, 128, dtype=h)
    k = torch.zeros(1, 2, 96, 128, dtype=h)

    def rejects(fn, match):
        with pytest.raises(ValueError, match=match):
            fn()

    d = fa.attn_fwd_dense
    rejects(lambda: d(q, k, k, lse=torch.zeros(1, 2, 64, dtype=h)), "lse must be float32")
    rejects(lambda: d(q, k, k, lse=torch.zeros(1, 2, 63, dtype=f32)), "lse must have shape")
    rejects(lambda: d(q, k, k, lse=torch.zeros(1, 2, 128, dtype=f32)[..., ::2]), "lse must be contiguous")
    rejects(lambda: d(q, k, k, out=torch.zeros(1, 2, 64, 128, dtype=bf)), "out must be float16")
    rejects(lambda: d(q, k, k, out=torch.zeros(1, 2, 32, 128, dtype=h)), "out must have shape")
    rejects(lambda: d(q, k, k, out=torch.zeros(1, 2, 128, 64, dtype=h).transpose(2, 3)), "stride 1")
    rejects(lambda: d(q, k.to(bf), k), "k must be float16")
    rejects(lambda: d(q, k, k[:, :, :90]), "v must have shape")
    rejects(lambda: d(q.float(), k, k), "q must be float16 or bfloat16")
    rejects(lambda: d(q, k, k), "CUDA")  # well-formed CPU tensors still never reach the library

    c = fa.attn_fwd_prefix_causal
    kc = torch.zeros(1, 1, 96, 128, dtype=h)
    rejects(lambda: c(q.to(bf), kc, kc, 64), "q must be float16")
    rejects(lambda: c(q, kc, kc, 64, lse=torch.zeros(1, 2, 64, dtype=torch.float64)), "lse must be float32")
    rejects(lambda: c(q, kc, kc, 64, out=torch.zeros(1, 1, 64, 128, dtype=h)), "out must have shape")

    cache = torch.zeros(4, 32, 1, 128, dtype=torch.uint8)
    table = torch.zeros(1, 4, dtype=torch.int32)
    p = fa.attn_fwd_paged_e4m3
    rejects(lambda: p(q.to(bf), cache, cache, table, 96, 64), "q must be float16")
    rejects(lambda: p(q, cache.to(torch.int8), cache, table, 96, 64), "k_cache must be uint8")
    rejects(lambda: p(q, cache, cache[:2], table, 96, 64), "v_cache must have shape")
    rejects(lambda: p(q, cache, cache, table.long(), 96, 64), "page_table must be int32")
    rejects(lambda: p(q, cache, cache, table, 96, 64, lse=torch.zeros(1, 2, 64, dtype=h)), "lse must be float32")

    b = fa.kv_e4m3_paged_to_fp16
    rejects(lambda: b(cache, cache, table, 1, 96, k_out=torch.zeros(1, 1, 96, 128, dtype=f32)), "k_out must be")
    rejects(lambda: b(cache, cache, table, 1, 96, v_out=torch.zeros(1, 1, 95, 128, dtype=h)), "v_out must have")

    s = fa.vsa_block_sparse_attn
    qv = torch.zeros(1, 2, 128, 128, dtype=h)
    idx = torch.zeros(1, 2, 2, 1, dtype=torch.int32)
    rejects(lambda: s(qv, qv, qv, idx.long()), "idx must be int32")
    rejects(lambda: s(qv, qv, qv, torch.zeros(1, 2, 3, 1, dtype=torch.int32)), "idx must have shape")
    rejects(lambda: s(qv.to(bf), qv, qv, idx), "q must be float16")
    rejects(lambda: s(qv, qv, qv, idx, lse=torch.zeros(1, 2, 128, dtype=h)), "lse must be float32")
    rejects(lambda: fa.vsa_block_select(qv, qv, 1, out=torch.zeros(1, 2, 2, 2, dtype=torch.int32)),
            "out must have shape")
    rejects(lambda: fa.vsa_block_select(qv.to(bf), qv, 1), "q must be float16")

    g = fa.kv_prefix_fp8_gather
    kb = torch.zeros(1, 8, 2, 128, dtype=bf)
    ix = torch.zeros(4, dtype=torch.int32)
    rejects(lambda: g(kb.to(h), kb, ix), "k must be bfloat16")
    rejects(lambda: g(kb, kb, ix.long()), "index must be int32")
    rejects(lambda: g(kb, kb, ix, k_out=torch.zeros(1, 3, 2, 128, dtype=bf)), "k_out must have shape")


def test_noalloc_decode_rejects_before_any_hip_call():
    """The allocation-free decode validates every argument, and that the
    shape's partial states fit its fixed scratch, before any HIP call (these
    calls run without a GPU)."""
    lib = fa.load()

    def call(**kw):
        a = dict(q_rows=16, q_real=16, Hq=6, Hkv=1, D=256, kv_len=4096, page_size=32, ks=1.0, kc=B_,
                 stride=262144 // 32)
        a.update(kw)
        return lib.attn_fwd_paged_e4m3_decode_noalloc(T(A), a["kc"], C, L, a["stride"], 9000, a["page_size"],
                                                      a["ks"], 1.0, T(O), None, 1, a["Hq"], a["Hkv"], a["D"],
                                                      a["q_rows"], a["q_real"], a["kv_len"], 0.0625, None)
    scratch = fa.NOALLOC_SCRATCH_BYTES
    assert scratch == 32 << 20
    # the workload decode fits; 8 heads at the longest cache do not
    assert lib.attn_fwd_paged_e4m3_decode_workspace(1, 6, 1, 256, 16, 256000) <= scratch
    assert lib.attn_fwd_paged_e4m3_decode_workspace(1, 8, 1, 256, 16, 262144) > scratch
    assert call(Hq=8, kv_len=262144) == fa.FA_ERR_WORKSPACE
    assert call(q_rows=17, q_real=17) == fa.FA_ERR_SHAPE
    assert call(kc=0) == fa.FA_ERR_NULL
    assert call(page_size=16) == fa.FA_ERR_UNSUPPORTED
    assert call(ks=float("nan")) == fa.FA_ERR_SHAPE
    assert call(kc=B_ + 4) == fa.FA_ERR_ALIGN


def test_block_list_and_tile_mean_rejections():
    lib = fa.load()

    def lists(**kw):
        a = dict(mask=A, valid=B_, T=576, tile=64, idx=O, counts=C, kv=L, quad=W)
        a.update(kw)
        return lib.vsa_tile_mask_to_block_lists(a["mask"], a["valid"], 1, 8, a["T"], a["tile"], a["idx"],
                                                a["counts"], a["kv"], a["quad"], None)
    assert lists(mask=0) == fa.FA_ERR_NULL
    assert lists(tile=96) == fa.FA_ERR_UNSUPPORTED
    assert lists(tile=128) == fa.FA_ERR_UNSUPPORTED      # quadrant masks only for 64-token tiles
    assert lists(T=0) == fa.FA_ERR_SHAPE
    assert lists(T=1025) == fa.FA_ERR_SHAPE
    assert lists(tile=128, T=513, quad=0) == fa.FA_ERR_SHAPE
    assert lists(counts=C + 2) == fa.FA_ERR_ALIGN
    assert lists(counts=O + 64) == fa.FA_ERR_ALIAS       # counts inside the index lists
    assert lists(idx=A) == fa.FA_ERR_ALIAS                # lists over the mask

    def means(**kw):
        a = dict(x=A, out=O, D=128, block=64, L=1000)
        a.update(kw)
        return lib.vsa_tile_means(a["x"], 1, 2, a["L"], a["D"], a["block"], a["out"], None)
    assert means(x=0) == fa.FA_ERR_NULL
    assert means(D=256) == fa.FA_ERR_UNSUPPORTED
    assert means(block=128) == fa.FA_ERR_UNSUPPORTED
    assert means(L=0) == fa.FA_ERR_SHAPE
    assert means(out=O + 4) == fa.FA_ERR_ALIGN
    assert means(out=A + 256) == fa.FA_ERR_ALIAS


def test_abi_from_plain_c(tmp_path):
    """include/fa16attn.h compiles as C99 (gcc -pedantic -Werror) and the library links and answers through
    it: version, error strings, workspace queries and host-side rejections (tests/abi_c_check.c)."""
    import shutil
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    lib_dir = os.path.dirname(fa.LIB_PATH)
    exe = str(tmp_path / "abi_c_check")
    src = os.path.join(os.path.dirname(__file__), "abi_c_check.c")
    inc = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")
    subprocess.check_call([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", inc, src, "-L",
                           lib_dir, "-l:libfa16attn.so", f"-Wl,-rpath,{lib_dir}", "-o", exe])
    out = subprocess.run([exe], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.strip() == "OK", out.stdout + out.stderr

"""Python binding of libfa16attn.so (include/fa16attn.h).

Argument marshalling only: every function takes torch CUDA tensors, passes
their device pointers, strides and the current HIP stream to the C ABI, and
raises RuntimeError on a nonzero return code. torch provides device memory
and streams; all computation happens in the library's HIP kernels. There is
no fallback: if the library is missing the import of a function fails loudly.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa16attn.so")
_lib = None

FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_ALIGN, FA_ERR_WORKSPACE, FA_ERR_ALIAS = range(7)
FA_ERR_HIP = 1000

# Every symbol include/fa16attn.h declares.
EXPORTS = ("fa_abi_version", "fa_error_string", "attn_fwd_dense", "attn_fwd_dense_bf16",
           "attn_fwd_prefix_fp8_workspace", "attn_fwd_prefix_fp8",
           "attn_fwd_prefix_causal_workspace",
           "attn_fwd_prefix_causal", "attn_fwd_paged_e4m3_workspace", "attn_fwd_paged_e4m3_bridged_workspace",
           "attn_fwd_paged_e4m3",
           "attn_fwd_paged_e4m3_decode_workspace", "attn_fwd_paged_e4m3_decode",
           "attn_fwd_paged_e4m3_decode_noalloc",
           "kv_e4m3_paged_to_fp16", "kv_prefix_fp8_gather", "vsa_topk_for_sparsity", "vsa_block_select_workspace",
           "vsa_block_select",
           "vsa_block_sparse_attn_workspace", "vsa_block_sparse_attn", "vsa_tile_means",
           "vsa_tile_mask_to_block_lists")


class FaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64),
                ("stride_s", ctypes.c_int64)]


class FaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (code {code})")
        self.code = code


_vp, _i, _i64, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t

_SIGS = {
    "fa_abi_version": (_i, []),
    "fa_error_string": (ctypes.c_char_p, [_i]),
    "attn_fwd_dense": (_i, [FaTensor] * 4 + [_vp] + [_i] * 5 + [_f, _vp]),
    "attn_fwd_dense_bf16": (_i, [FaTensor] * 4 + [_vp] + [_i] * 5 + [_f, _vp]),
    "attn_fwd_prefix_fp8_workspace": (_sz, [_i] * 5),
    "attn_fwd_prefix_fp8": (_i, [FaTensor] * 4 + [_vp] + [_i] * 5 + [_f, _vp, _sz, _vp]),
    "attn_fwd_prefix_causal_workspace": (_sz, [_i] * 6),
    "attn_fwd_prefix_causal": (_i, [FaTensor] * 4 + [_vp] + [_i] * 7 + [_f, _vp, _sz, _vp]),
    "attn_fwd_paged_e4m3_workspace": (_sz, [_i] * 6),
    "attn_fwd_paged_e4m3_bridged_workspace": (_sz, [_i] * 6 + [_f]),
    "attn_fwd_paged_e4m3": (_i, [FaTensor, _vp, _vp, _vp, _i64, _i, _i, _f, _f, FaTensor, _vp]
                            + [_i] * 7 + [_f, _vp, _sz, _vp]),
    "attn_fwd_paged_e4m3_decode_workspace": (_sz, [_i] * 6),
    "attn_fwd_paged_e4m3_decode": (_i, [FaTensor, _vp, _vp, _vp, _i64, _i, _i, _f, _f, FaTensor, _vp]
                                   + [_i] * 7 + [_f, _vp, _sz, _vp]),
    "attn_fwd_paged_e4m3_decode_noalloc": (_i, [FaTensor, _vp, _vp, _vp, _i64, _i, _i, _f, _f, FaTensor, _vp]
                                           + [_i] * 7 + [_f, _vp]),
    "kv_e4m3_paged_to_fp16": (_i, [_vp, _vp, _vp, _i64] + [_i] * 6 + [_f, _f, _vp, _vp, _vp]),
    "kv_prefix_fp8_gather": (_i, [_vp, _vp] + [_i] * 4 + [_vp, _i, _vp, _vp, _vp]),
    "vsa_topk_for_sparsity": (_i, [_i, _i, ctypes.c_double]),
    "vsa_block_select_workspace": (_sz, [_i] * 5),
    "vsa_block_select": (_i, [_vp, _vp] + [_i] * 6 + [_vp, _vp, _vp, _sz, _vp]),
    "vsa_block_sparse_attn_workspace": (_sz, [_i] * 7),
    "vsa_block_sparse_attn": (_i, [FaTensor] * 4 + [_vp, _vp] + [_i] * 7 + [_f, _vp, _sz, _vp]),
    "vsa_tile_means": (_i, [_vp] + [_i] * 5 + [_vp, _vp]),
    "vsa_tile_mask_to_block_lists": (_i, [_vp, _vp] + [_i] * 4 + [_vp] * 5),
}


def load():
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m fp16_attention_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if lib.fa_abi_version() != 1:
            raise ImportError("libfa16attn.so ABI version mismatch")
        _lib = lib
    return _lib


def error_string(code: int) -> str:
    return load().fa_error_string(code).decode()


def _check(rc: int):
    if rc != FA_OK:
        raise FaError(rc, error_string(rc))


def _view(t) -> FaTensor:
    if t.dim() != 4:
        raise ValueError("expected a 4-D [B, H, S, D] tensor")
    if t.stride(3) != 1 and t.size(3) > 1:
        raise ValueError("the D dimension must have stride 1")
    return FaTensor(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(t):
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _need_cuda(*ts):
    """Every given tensor is a CUDA (HIP) tensor on the device of the first."""
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("fp16_attention_amd operates on CUDA (HIP) tensors only")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors of a call must be on the same device")


def _dtype_name(t):
    return str(t.dtype).replace("torch.", "")


def _want(t, name, dtypes, ndim=None, shape=None, contiguous=False, unit_d=False):
    """Check a tensor's dtype, rank, exact shape, contiguity and (for BHSD views)
    the unit stride along D, before anything is handed to the library."""
    if t is None:
        return
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be {' or '.join(str(d).replace('torch.', '') for d in dtypes)}, "
                         f"not {_dtype_name(t)}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, not {t.dim()}-D")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if unit_d and t.stride(-1) != 1 and t.size(-1) > 1:
        raise ValueError(f"{name}: the D dimension must have stride 1")


def _lse_shape_ok(lse, shape):
    import torch
    _want(lse, "lse", (torch.float32,), shape=shape, contiguous=True)


def default_scale(D: int) -> float:
    """1/sqrt(D) rounded to FP32, the softmax scale the pages use."""
    import numpy as np
    return float(np.float32(1.0 / math.sqrt(D)))


# --------------------------------------------------------------------------- attention
#
# Every wrapper checks dtypes, shapes, contiguity and devices of all its
# tensors (outputs, LSE and workspaces included) before the library sees a
# pointer: the C side gets bare device pointers and cannot check them itself.

def _f16():
    import torch
    return (torch.float16,)


def attn_fwd_dense(q, k, v, out=None, lse=None, scale=None):
    """Dense non-causal attention. q [B,H,Lq,D], k/v [B,H,Lkv,D] FP16 or BF16 -> out of the same type.
    BF16 operands go to attn_fwd_dense_bf16. lse: optional float32 [B,H,Lq] contiguous."""
    import torch
    dt = q.dtype
    if dt not in (torch.float16, torch.bfloat16):
        raise ValueError("q must be float16 or bfloat16")
    _want(q, "q", (dt,), ndim=4, unit_d=True)
    B, H, Lq, D = q.shape
    _want(k, "k", (dt,), ndim=4, unit_d=True)
    Lkv = k.shape[2]
    _want(k, "k", (dt,), shape=(B, H, Lkv, D))
    _want(v, "v", (dt,), shape=(B, H, Lkv, D), unit_d=True)
    _want(out, "out", (dt,), shape=(B, H, Lq, D), unit_d=True)
    _lse_shape_ok(lse, (B, H, Lq))
    _need_cuda(q, k, v, out, lse)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    scale = default_scale(D) if scale is None else scale
    fn = load().attn_fwd_dense_bf16 if dt == torch.bfloat16 else load().attn_fwd_dense
    _check(fn(_view(q), _view(k), _view(v), _view(out), _ptr(lse), B, H, Lq, Lkv, D, scale, _stream(q)))
    return out


def prefix_fp8_workspace(B, H, Lq, Lkv, D=128) -> int:
    return int(load().attn_fwd_prefix_fp8_workspace(B, H, Lq, Lkv, D))


def attn_fwd_prefix_fp8(q, k, v, out=None, lse=None, scale=None, workspace=None):
    """Dense attention with FP8 (E4M3, per-row amax/448 scale) queries and keys on the FP8
    matrix cores; q [B,H,Lq,128], k/v [B,H,Lkv,128] bfloat16 -> out bfloat16."""
    import torch
    bf = (torch.bfloat16,)
    _want(q, "q", bf, ndim=4, unit_d=True)
    B, H, Lq, D = q.shape
    _want(k, "k", bf, ndim=4, unit_d=True)
    Lkv = k.shape[2]
    _want(k, "k", bf, shape=(B, H, Lkv, D))
    _want(v, "v", bf, shape=(B, H, Lkv, D), unit_d=True)
    _want(out, "out", bf, shape=(B, H, Lq, D), unit_d=True)
    _lse_shape_ok(lse, (B, H, Lq))
    _need_cuda(q, k, v, out, lse)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    scale = default_scale(D) if scale is None else scale
    ws = _workspace(prefix_fp8_workspace(B, H, Lq, Lkv, D), q.device, workspace)
    _check(load().attn_fwd_prefix_fp8(_view(q), _view(k), _view(v), _view(out), _ptr(lse), B, H, Lq, Lkv, D, scale,
                                      _ptr(ws), _nbytes(ws), _stream(q)))
    return out


def prefix_causal_workspace(B, Hq, Hkv, D, q_rows, kv_len) -> int:
    return int(load().attn_fwd_prefix_causal_workspace(B, Hq, Hkv, D, q_rows, kv_len))


def _workspace(nbytes, device, workspace):
    """The caller's workspace (a CUDA uint8 tensor of at least nbytes on the
    call's device), or a fresh one; None when nothing is needed."""
    import torch
    if nbytes == 0:
        return workspace
    if workspace is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    _want(workspace, "workspace", (torch.uint8,), contiguous=True)
    if not workspace.is_cuda or workspace.device != device:
        raise ValueError("workspace must be a CUDA tensor on the device of the operands")
    if workspace.numel() < nbytes:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, {nbytes} needed")
    return workspace


def _nbytes(ws):
    return 0 if ws is None else ws.numel() * ws.element_size()


def attn_fwd_prefix_causal(q, k, v, q_real, out=None, lse=None, scale=None, workspace=None):
    """Causal prefill against a prefix KV (GQA). q [B,Hq,q_rows,D], k/v [B,Hkv,kv_len,D] FP16;
    lse: optional float32 [B,Hq,q_rows] contiguous."""
    import torch
    _want(q, "q", _f16(), ndim=4, unit_d=True)
    B, Hq, q_rows, D = q.shape
    _want(k, "k", _f16(), ndim=4, unit_d=True)
    Hkv, kv_len = k.shape[1], k.shape[2]
    _want(k, "k", _f16(), shape=(B, Hkv, kv_len, D))
    _want(v, "v", _f16(), shape=(B, Hkv, kv_len, D), unit_d=True)
    _want(out, "out", _f16(), shape=(B, Hq, q_rows, D), unit_d=True)
    _lse_shape_ok(lse, (B, Hq, q_rows))
    _need_cuda(q, k, v, out, lse)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    scale = default_scale(D) if scale is None else scale
    ws = _workspace(prefix_causal_workspace(B, Hq, Hkv, D, q_rows, kv_len), q.device, workspace)
    _check(load().attn_fwd_prefix_causal(_view(q), _view(k), _view(v), _view(out), _ptr(lse), B, Hq, Hkv,
                                         D, q_rows, q_real, kv_len, scale, _ptr(ws), _nbytes(ws), _stream(q)))
    return out


def attn_fwd_paged_e4m3(q, k_cache, v_cache, page_table, kv_len, q_real, k_scale=1.0, v_scale=1.0,
                        out=None, lse=None, scale=None, workspace=None, bridged=True):
    """Causal prefill reading an E4M3 paged cache [pages, 32, Hkv, D] (uint8) via an int32 page table
    [B, pages_per_seq]. bridged: size the workspace this call allocates (when none is given) for the
    bridged plan (FP16 K and V converted into the workspace first; used for a k_scale that is not a
    power of two); False allocates only the split-KV states, so the cache is attended in place. A
    given workspace selects the plan by its size (see paged_e4m3_workspace)."""
    return _paged(False, q, k_cache, v_cache, page_table, kv_len, q_real, k_scale, v_scale, out, lse, scale,
                  workspace, bridged=bridged)


def paged_e4m3_workspace(B, Hq, Hkv, D, q_rows, kv_len, k_scale=None) -> int:
    """Workspace bytes of attn_fwd_paged_e4m3: the in-place plan's (k_scale None), or the size that
    selects the bridged plan for that k_scale."""
    lib = load()
    if k_scale is None:
        return int(lib.attn_fwd_paged_e4m3_workspace(B, Hq, Hkv, D, q_rows, kv_len))
    return int(lib.attn_fwd_paged_e4m3_bridged_workspace(B, Hq, Hkv, D, q_rows, kv_len, k_scale))


def attn_fwd_paged_e4m3_decode(q, k_cache, v_cache, page_table, kv_len, q_real=None, k_scale=1.0, v_scale=1.0,
                               out=None, lse=None, scale=None, workspace=None):
    """Decode: q [B,Hq,1..16,D] new positions against an E4M3 paged cache (see attn_fwd_paged_e4m3)."""
    q_real = q.shape[2] if q_real is None else q_real
    return _paged(True, q, k_cache, v_cache, page_table, kv_len, q_real, k_scale, v_scale, out, lse, scale,
                  workspace)


NOALLOC_SCRATCH_BYTES = 32 << 20  # FA_NOALLOC_SCRATCH_BYTES


def attn_fwd_paged_e4m3_decode_noalloc(q, k_cache, v_cache, page_table, kv_len, out, q_real=None, k_scale=1.0,
                                       v_scale=1.0, lse=None, scale=None):
    """attn_fwd_paged_e4m3_decode without a workspace: the split-KV partial states go to the
    library's own per-GPU scratch array (no device allocation in the call). out must be given
    (a caller that cannot allocate owns it); calls that overlap on one GPU race."""
    q_real = q.shape[2] if q_real is None else q_real
    return _paged(True, q, k_cache, v_cache, page_table, kv_len, q_real, k_scale, v_scale, out, lse, scale,
                  None, noalloc=True)


def _paged(decode, q, k_cache, v_cache, page_table, kv_len, q_real, k_scale, v_scale, out, lse, scale, workspace,
           noalloc=False, bridged=False):
    import torch
    _want(q, "q", _f16(), ndim=4, unit_d=True)
    B, Hq, q_rows, D = q.shape
    _want(k_cache, "k_cache", (torch.uint8,), ndim=4, contiguous=True)
    pages, page_size, Hkv, Dc = k_cache.shape
    if Dc != D:
        raise ValueError("the caches' D differs from q's")
    _want(v_cache, "v_cache", (torch.uint8,), shape=k_cache.shape, contiguous=True)
    _want(page_table, "page_table", (torch.int32,), ndim=2, contiguous=True)
    if page_table.shape[0] != B:
        raise ValueError("page_table must have one row per sequence")
    _want(out, "out", _f16(), shape=(B, Hq, q_rows, D), unit_d=True)
    _lse_shape_ok(lse, (B, Hq, q_rows))
    _need_cuda(q, k_cache, v_cache, page_table, out, lse)
    scale = default_scale(D) if scale is None else scale
    lib = load()
    if noalloc:
        if out is None:
            raise ValueError("the allocation-free decode writes into a caller-provided out")
        _check(lib.attn_fwd_paged_e4m3_decode_noalloc(
            _view(q), k_cache.data_ptr(), v_cache.data_ptr(), page_table.data_ptr(), page_table.stride(0), pages,
            page_size, k_scale, v_scale, _view(out), _ptr(lse), B, Hq, Hkv, D, q_rows, q_real, kv_len, scale,
            _stream(q)))
        return out
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    fn = lib.attn_fwd_paged_e4m3_decode if decode else lib.attn_fwd_paged_e4m3
    if decode:
        need = lib.attn_fwd_paged_e4m3_decode_workspace(B, Hq, Hkv, D, q_rows, kv_len)
    elif bridged and workspace is None:
        # allocate what the bridged plan needs (a given workspace only has to hold the split-KV
        # states: the library takes the bridged plan when it is large enough)
        need = lib.attn_fwd_paged_e4m3_bridged_workspace(B, Hq, Hkv, D, q_rows, kv_len, k_scale)
    else:
        need = lib.attn_fwd_paged_e4m3_workspace(B, Hq, Hkv, D, q_rows, kv_len)
    ws = _workspace(int(need), q.device, workspace)
    _check(fn(_view(q), k_cache.data_ptr(), v_cache.data_ptr(), page_table.data_ptr(), page_table.stride(0),
              pages, page_size, k_scale, v_scale, _view(out), _ptr(lse), B, Hq, Hkv, D, q_rows, q_real, kv_len,
              scale, _ptr(ws), _nbytes(ws), _stream(q)))
    return out


def kv_e4m3_paged_to_fp16(k_cache, v_cache, page_table, B, kv_len, k_scale=1.0, v_scale=1.0,
                          k_out=None, v_out=None):
    """Exact paged E4M3 -> FP16 bridge. Returns contiguous FP16 (k, v) [B, Hkv, kv_len, D]."""
    import torch
    _want(k_cache, "k_cache", (torch.uint8,), ndim=4, contiguous=True)
    pages, page_size, Hkv, D = k_cache.shape
    _want(v_cache, "v_cache", (torch.uint8,), shape=k_cache.shape, contiguous=True)
    _want(page_table, "page_table", (torch.int32,), ndim=2, contiguous=True)
    if page_table.shape[0] != B:
        raise ValueError("page_table must have one row per sequence")
    shape = (B, Hkv, kv_len, D)
    _want(k_out, "k_out", _f16(), shape=shape, contiguous=True)
    _want(v_out, "v_out", _f16(), shape=shape, contiguous=True)
    _need_cuda(k_cache, v_cache, page_table, k_out, v_out)
    if k_out is None:
        k_out = torch.empty(shape, dtype=torch.float16, device=k_cache.device)
    if v_out is None:
        v_out = torch.empty(shape, dtype=torch.float16, device=k_cache.device)
    _check(load().kv_e4m3_paged_to_fp16(k_cache.data_ptr(), v_cache.data_ptr(), page_table.data_ptr(),
                                        page_table.stride(0), pages, page_size, B, Hkv, D, kv_len, k_scale,
                                        v_scale, k_out.data_ptr(), v_out.data_ptr(), _stream(k_cache)))
    return k_out, v_out


# ---------------------------------------------------------------------------------- VSA

def kv_prefix_fp8_gather(k, v, index, k_out=None, v_out=None):
    """FP8 round trip of K per (row, head) with the row gather. k, v: bfloat16 [B, N, H, 128]
    contiguous; index: int32 [rows]. Returns (k_out, v_out) bfloat16 [B, rows, H, 128]."""
    import torch
    _want(k, "k", (torch.bfloat16,), ndim=4, contiguous=True)
    B, N, H, D = k.shape
    _want(v, "v", (torch.bfloat16,), shape=k.shape, contiguous=True)
    _want(index, "index", (torch.int32,), ndim=1, contiguous=True)
    rows = index.numel()
    _want(k_out, "k_out", (torch.bfloat16,), shape=(B, rows, H, D), contiguous=True)
    _want(v_out, "v_out", (torch.bfloat16,), shape=(B, rows, H, D), contiguous=True)
    _need_cuda(k, v, index, k_out, v_out)
    if k_out is None:
        k_out = torch.empty((B, rows, H, D), dtype=torch.bfloat16, device=k.device)
    if v_out is None:
        v_out = torch.empty_like(k_out)
    _check(load().kv_prefix_fp8_gather(k.data_ptr(), v.data_ptr(), B, N, H, D, index.data_ptr(), rows,
                                       k_out.data_ptr(), v_out.data_ptr(), _stream(k)))
    return k_out, v_out


def vsa_topk_for_sparsity(L: int, sparsity: float, block: int = 64) -> int:
    """Blocks kept per query block for a VSA keep ratio (1 - sparsity)."""
    k = int(load().vsa_topk_for_sparsity(L, block, sparsity))
    if k < 0:
        raise FaError(-k, error_string(-k))
    return k


def vsa_block_select(q, k, topk, block=64, scores=False, workspace=None, out=None):
    """Top-k KV blocks per query block. q, k: FP16 [B,H,L,D] contiguous. Returns idx int32
    [B,H,NB,topk] (and FP64 scores [B,H,NB,NB] if asked)."""
    import torch
    _want(q, "q", _f16(), ndim=4, contiguous=True)
    B, H, L, D = q.shape
    _want(k, "k", _f16(), shape=q.shape, contiguous=True)
    NB = (L + block - 1) // block  # the last block may be partial
    _want(out, "out", (torch.int32,), shape=(B, H, NB, topk), contiguous=True)
    _need_cuda(q, k, out)
    idx = out
    if idx is None:
        idx = torch.empty((B, H, NB, topk), dtype=torch.int32, device=q.device)
    s = torch.empty((B, H, NB, NB), dtype=torch.float64, device=q.device) if scores else None
    ws = _workspace(int(load().vsa_block_select_workspace(B, H, L, D, block)), q.device, workspace)
    _check(load().vsa_block_select(q.data_ptr(), k.data_ptr(), B, H, L, D, block, topk, idx.data_ptr(),
                                   _ptr(s), _ptr(ws), _nbytes(ws), _stream(q)))
    return (idx, s) if scores else idx


def vsa_block_sparse_attn_workspace(B, H, L, D, block, topk, dense_prefix_qblocks) -> int:
    return int(load().vsa_block_sparse_attn_workspace(B, H, L, D, block, topk, dense_prefix_qblocks))


def vsa_block_sparse_attn(q, k, v, idx, dense_prefix_qblocks=2, block=64, out=None, lse=None, scale=None,
                          workspace=None):
    """Block-sparse attention over per-query-block KV block lists idx [B,H,ceil(L/block),topk] (int32,
    contiguous). q, k, v, out: FP16 [B,H,L,D] views; lse: optional float32 [B,H,L] contiguous."""
    import torch
    _want(q, "q", _f16(), ndim=4, unit_d=True)
    B, H, L, D = q.shape
    _want(k, "k", _f16(), shape=q.shape, unit_d=True)
    _want(v, "v", _f16(), shape=q.shape, unit_d=True)
    _want(idx, "idx", (torch.int32,), ndim=4, contiguous=True)
    NB = (L + block - 1) // block
    topk = idx.shape[-1]
    _want(idx, "idx", (torch.int32,), shape=(B, H, NB, topk))
    _want(out, "out", _f16(), shape=q.shape, unit_d=True)
    _lse_shape_ok(lse, (B, H, L))
    _need_cuda(q, k, v, idx, out, lse)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    scale = default_scale(D) if scale is None else scale
    ws = _workspace(vsa_block_sparse_attn_workspace(B, H, L, D, block, topk, dense_prefix_qblocks), q.device,
                    workspace)
    _check(load().vsa_block_sparse_attn(_view(q), _view(k), _view(v), _view(out), idx.data_ptr(), _ptr(lse),
                                        B, H, L, D, block, topk, dense_prefix_qblocks, scale, _ptr(ws),
                                        _nbytes(ws), _stream(q)))
    return out


def vsa_tile_means(x, block=64, out=None):
    """FP32 means of each 64-row tile of x [B,H,L,128] FP16 contiguous (the last tile may be
    partial): the pooled V of the VSA coarse branch. Returns float32 [B,H,ceil(L/64),128]."""
    import torch
    _want(x, "x", _f16(), ndim=4, contiguous=True)
    B, H, L, D = x.shape
    NB = (L + block - 1) // block
    _want(out, "out", (torch.float32,), shape=(B, H, NB, D), contiguous=True)
    _need_cuda(x, out)
    if out is None:
        out = torch.empty((B, H, NB, D), dtype=torch.float32, device=x.device)
    _check(load().vsa_tile_means(x.data_ptr(), B, H, L, D, block, out.data_ptr(), _stream(x)))
    return out


def vsa_tile_mask_to_block_lists(mask, valid, tile, quadrants=True):
    """128-token block lists from a square tile mask [B,H,T,T] (bool or uint8) and the valid
    tokens of the T tiles (int32 [T]). Returns (indices int32 [B,H,NB,NB] descending then zero,
    counts int32 [B,H,NB], kv_valid int32 [2*NB], quadrants uint8 [B,H,NB,NB] or None)."""
    import torch
    if mask.dtype == torch.bool:
        mask = mask.view(torch.uint8)
    _want(mask, "mask", (torch.uint8,), ndim=4, contiguous=True)
    B, H, T, T2 = mask.shape
    if T2 != T:
        raise ValueError("mask must be square over the tiles")
    _want(valid, "valid", (torch.int32,), shape=(T,), contiguous=True)
    _need_cuda(mask, valid)
    nb = (T * (tile // 64) + 1) // 2
    dev = mask.device
    idx = torch.empty((B, H, nb, nb), dtype=torch.int32, device=dev)
    counts = torch.empty((B, H, nb), dtype=torch.int32, device=dev)
    kv = torch.empty((2 * nb,), dtype=torch.int32, device=dev)
    quad = torch.empty((B, H, nb, nb), dtype=torch.uint8, device=dev) if quadrants and tile == 64 else None
    _check(load().vsa_tile_mask_to_block_lists(mask.data_ptr(), valid.data_ptr(), B, H, T, tile, idx.data_ptr(),
                                               counts.data_ptr(), kv.data_ptr(), _ptr(quad), _stream(mask)))
    return idx, counts, kv, quad

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
           "attn_fwd_prefix_causal_workspace",
           "attn_fwd_prefix_causal", "attn_fwd_paged_e4m3_workspace", "attn_fwd_paged_e4m3",
           "attn_fwd_paged_e4m3_decode_workspace", "attn_fwd_paged_e4m3_decode",
           "kv_e4m3_paged_to_fp16", "kv_prefix_fp8_gather", "vsa_topk_for_sparsity", "vsa_block_select_workspace",
           "vsa_block_select",
           "vsa_block_sparse_attn_workspace", "vsa_block_sparse_attn", "fa_mfma_ceiling")


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
    "attn_fwd_prefix_causal_workspace": (_sz, [_i] * 6),
    "attn_fwd_prefix_causal": (_i, [FaTensor] * 4 + [_vp] + [_i] * 7 + [_f, _vp, _sz, _vp]),
    "attn_fwd_paged_e4m3_workspace": (_sz, [_i] * 6),
    "attn_fwd_paged_e4m3": (_i, [FaTensor, _vp, _vp, _vp, _i64, _i, _i, _f, _f, FaTensor, _vp]
                            + [_i] * 7 + [_f, _vp, _sz, _vp]),
    "attn_fwd_paged_e4m3_decode_workspace": (_sz, [_i] * 6),
    "attn_fwd_paged_e4m3_decode": (_i, [FaTensor, _vp, _vp, _vp, _i64, _i, _i, _f, _f, FaTensor, _vp]
                                   + [_i] * 7 + [_f, _vp, _sz, _vp]),
    "kv_e4m3_paged_to_fp16": (_i, [_vp, _vp, _vp, _i64] + [_i] * 6 + [_f, _f, _vp, _vp, _vp]),
    "kv_prefix_fp8_gather": (_i, [_vp, _vp] + [_i] * 4 + [_vp, _i, _vp, _vp, _vp]),
    "vsa_topk_for_sparsity": (_i, [_i, _i, ctypes.c_double]),
    "vsa_block_select_workspace": (_sz, [_i] * 5),
    "vsa_block_select": (_i, [_vp, _vp] + [_i] * 6 + [_vp, _vp, _vp, _sz, _vp]),
    "vsa_block_sparse_attn_workspace": (_sz, [_i] * 7),
    "vsa_block_sparse_attn": (_i, [FaTensor] * 4 + [_vp, _vp] + [_i] * 7 + [_f, _vp, _sz, _vp]),
    "fa_mfma_ceiling": (_i, [_i, _vp, _vp]),
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
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("fp16_attention_amd operates on CUDA (HIP) tensors only")


def default_scale(D: int) -> float:
    """1/sqrt(D) rounded to FP32, the softmax scale the pages use."""
    import numpy as np
    return float(np.float32(1.0 / math.sqrt(D)))


# --------------------------------------------------------------------------- attention

def attn_fwd_dense(q, k, v, out=None, lse=None, scale=None):
    """Dense non-causal attention. q [B,H,Lq,D], k/v [B,H,Lkv,D] FP16 or BF16 -> out of the same type.
    BF16 operands go to attn_fwd_dense_bf16."""
    import torch
    _need_cuda(q, k, v, out, lse)
    dt = q.dtype
    if dt not in (torch.float16, torch.bfloat16) or k.dtype != dt or v.dtype != dt:
        raise ValueError("q, k, v must all be float16 or all bfloat16")
    B, H, Lq, D = q.shape
    Lkv = k.shape[2]
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    elif out.dtype != dt:
        raise ValueError("out must have the dtype of q")
    scale = default_scale(D) if scale is None else scale
    fn = load().attn_fwd_dense_bf16 if dt == torch.bfloat16 else load().attn_fwd_dense
    _check(fn(_view(q), _view(k), _view(v), _view(out), _ptr(lse), B, H, Lq, Lkv, D, scale, _stream(q)))
    return out


def prefix_causal_workspace(B, Hq, Hkv, D, q_rows, kv_len) -> int:
    return int(load().attn_fwd_prefix_causal_workspace(B, Hq, Hkv, D, q_rows, kv_len))


def _workspace(nbytes, device, workspace):
    import torch
    if nbytes == 0:
        return workspace
    if workspace is None or workspace.numel() * workspace.element_size() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return workspace


def attn_fwd_prefix_causal(q, k, v, q_real, out=None, lse=None, scale=None, workspace=None):
    """Causal prefill against a prefix KV (GQA). q [B,Hq,q_rows,D], k/v [B,Hkv,kv_len,D]."""
    import torch
    _need_cuda(q, k, v, out, lse)
    B, Hq, q_rows, D = q.shape
    Hkv, kv_len = k.shape[1], k.shape[2]
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    scale = default_scale(D) if scale is None else scale
    ws = _workspace(prefix_causal_workspace(B, Hq, Hkv, D, q_rows, kv_len), q.device, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().attn_fwd_prefix_causal(_view(q), _view(k), _view(v), _view(out), _ptr(lse), B, Hq, Hkv,
                                         D, q_rows, q_real, kv_len, scale, _ptr(ws), nbytes, _stream(q)))
    return out


def attn_fwd_paged_e4m3(q, k_cache, v_cache, page_table, kv_len, q_real, k_scale=1.0, v_scale=1.0,
                        out=None, lse=None, scale=None, workspace=None):
    """Causal prefill reading an E4M3 paged cache [pages, 32, Hkv, D] (uint8) via an int32 page table."""
    return _paged(False, q, k_cache, v_cache, page_table, kv_len, q_real, k_scale, v_scale, out, lse, scale,
                  workspace)


def attn_fwd_paged_e4m3_decode(q, k_cache, v_cache, page_table, kv_len, q_real=None, k_scale=1.0, v_scale=1.0,
                               out=None, lse=None, scale=None, workspace=None):
    """Decode: q [B,Hq,1..16,D] new positions against an E4M3 paged cache (see attn_fwd_paged_e4m3)."""
    q_real = q.shape[2] if q_real is None else q_real
    return _paged(True, q, k_cache, v_cache, page_table, kv_len, q_real, k_scale, v_scale, out, lse, scale,
                  workspace)


def _paged(decode, q, k_cache, v_cache, page_table, kv_len, q_real, k_scale, v_scale, out, lse, scale, workspace):
    import torch
    _need_cuda(q, k_cache, v_cache, page_table, out, lse)
    B, Hq, q_rows, D = q.shape
    pages, page_size, Hkv, Dc = k_cache.shape
    if Dc != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shape mismatch")
    for t in (k_cache, v_cache, page_table):
        if not t.is_contiguous():
            raise ValueError("caches and the page table must be contiguous")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    scale = default_scale(D) if scale is None else scale
    lib = load()
    wsq = lib.attn_fwd_paged_e4m3_decode_workspace if decode else lib.attn_fwd_paged_e4m3_workspace
    fn = lib.attn_fwd_paged_e4m3_decode if decode else lib.attn_fwd_paged_e4m3
    ws = _workspace(int(wsq(B, Hq, Hkv, D, q_rows, kv_len)), q.device, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(fn(_view(q), k_cache.data_ptr(), v_cache.data_ptr(), page_table.data_ptr(), page_table.stride(0),
              pages, page_size, k_scale, v_scale, _view(out), _ptr(lse), B, Hq, Hkv, D, q_rows, q_real, kv_len,
              scale, _ptr(ws), nbytes, _stream(q)))
    return out


def kv_e4m3_paged_to_fp16(k_cache, v_cache, page_table, B, kv_len, k_scale=1.0, v_scale=1.0,
                          k_out=None, v_out=None):
    """Exact paged E4M3 -> FP16 bridge. Returns contiguous FP16 (k, v) [B, Hkv, kv_len, D]."""
    import torch
    _need_cuda(k_cache, v_cache, page_table, k_out, v_out)
    pages, page_size, Hkv, D = k_cache.shape
    shape = (B, Hkv, kv_len, D)
    if k_out is None:
        k_out = torch.empty(shape, dtype=torch.float16, device=k_cache.device)
    if v_out is None:
        v_out = torch.empty(shape, dtype=torch.float16, device=k_cache.device)
    for t in (k_cache, v_cache, page_table, k_out, v_out):
        if not t.is_contiguous():
            raise ValueError("bridge operands must be contiguous")
    _check(load().kv_e4m3_paged_to_fp16(k_cache.data_ptr(), v_cache.data_ptr(), page_table.data_ptr(),
                                        page_table.stride(0), pages, page_size, B, Hkv, D, kv_len, k_scale,
                                        v_scale, k_out.data_ptr(), v_out.data_ptr(), _stream(k_cache)))
    return k_out, v_out


# ---------------------------------------------------------------------------------- VSA

def kv_prefix_fp8_gather(k, v, index, k_out=None, v_out=None):
    """FP8 round trip of K per (row, head) with the row gather. k, v: bfloat16 [B, N, H, 128]
    contiguous; index: int32 [rows]. Returns (k_out, v_out) bfloat16 [B, rows, H, 128]."""
    import torch
    _need_cuda(k, v, index, k_out, v_out)
    if k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16 or not k.is_contiguous() or not v.is_contiguous():
        raise ValueError("k and v must be contiguous bfloat16 [B, N, H, D]")
    if index.dtype != torch.int32 or not index.is_contiguous():
        raise ValueError("index must be contiguous int32")
    B, N, H, D = k.shape
    rows = index.numel()
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
    """Top-k KV blocks per query block. Returns idx int32 [B,H,NB,topk] (and FP64 scores if asked)."""
    import torch
    _need_cuda(q, k, out)
    if not (q.is_contiguous() and k.is_contiguous()):
        raise ValueError("q and k must be contiguous")
    B, H, L, D = q.shape
    NB = (L + block - 1) // block  # the last block may be partial
    idx = out
    if idx is None:
        idx = torch.empty((B, H, NB, topk), dtype=torch.int32, device=q.device)
    elif tuple(idx.shape) != (B, H, NB, topk) or idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("out must be a contiguous int32 [B, H, L/block, topk] tensor")
    s = torch.empty((B, H, NB, NB), dtype=torch.float64, device=q.device) if scores else None
    ws = _workspace(int(load().vsa_block_select_workspace(B, H, L, D, block)), q.device, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().vsa_block_select(q.data_ptr(), k.data_ptr(), B, H, L, D, block, topk, idx.data_ptr(),
                                   _ptr(s), _ptr(ws), nbytes, _stream(q)))
    return (idx, s) if scores else idx


def vsa_block_sparse_attn_workspace(B, H, L, D, block, topk, dense_prefix_qblocks) -> int:
    return int(load().vsa_block_sparse_attn_workspace(B, H, L, D, block, topk, dense_prefix_qblocks))


def vsa_block_sparse_attn(q, k, v, idx, dense_prefix_qblocks=2, block=64, out=None, lse=None, scale=None,
                          workspace=None):
    """Block-sparse attention over per-query-block KV block lists idx [B,H,L/block,topk]."""
    import torch
    _need_cuda(q, k, v, idx, out, lse)
    B, H, L, D = q.shape
    if not idx.is_contiguous() or idx.dtype != torch.int32:
        raise ValueError("idx must be contiguous int32")
    topk = idx.shape[-1]
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    scale = default_scale(D) if scale is None else scale
    ws = _workspace(vsa_block_sparse_attn_workspace(B, H, L, D, block, topk, dense_prefix_qblocks), q.device,
                    workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().vsa_block_sparse_attn(_view(q), _view(k), _view(v), _view(out), idx.data_ptr(), _ptr(lse),
                                        B, H, L, D, block, topk, dense_prefix_qblocks, scale, _ptr(ws), nbytes,
                                        _stream(q)))
    return out


MFMA_CEILING_OUT = 512 * 256  # FP32 values fa_mfma_ceiling writes


def mfma_ceiling_flop(iters: int) -> float:
    """FLOP of one fa_mfma_ceiling launch."""
    return 512.0 * 4 * iters * 4 * 32768


def mfma_ceiling(out, iters: int):
    """Launch the FP16 MFMA rate kernel (a measurement aid) on out's stream;
    out: CUDA float32 tensor of at least MFMA_CEILING_OUT elements."""
    _need_cuda(out)
    import torch
    if out.dtype != torch.float32 or out.numel() < MFMA_CEILING_OUT or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor of MFMA_CEILING_OUT elements")
    _check(load().fa_mfma_ceiling(int(iters), out.data_ptr(), _stream(out)))
    return out

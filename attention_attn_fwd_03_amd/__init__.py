"""Python binding of libmiattn (ctypes).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libmiattn.so. PyTorch provides device memory and the current
stream. Importing this package fails loudly when the library has not been
built; there is no fallback path.

Entry points (same names as the C ABI, without the ``miattn_`` prefix):
    attn_fwd(q, k, v, cu_seqlens, max_seqlen, *, scale, causal) -> (o, lse)
    attn_fwd_paged(q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens_k,
                   max_seqlen_q, *, scale, causal) -> (o, lse)
    attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, *, scale,
                      num_splits=0) -> (o, lse)
    attn_decode_paged_noalloc(q, k_cache, v_cache, block_table, seq_lens, *,
                              scale, num_splits=0) -> (o, lse)
    attn_decode_paged_numerics(..., *, scale, num_splits, numerics,
                               tile_pages, out_dtype) -> (o, lse)
    attn_combine(partial_o, partial_lse, *, out_dtype) -> (o, lse)
    attn_bwd(q, k, v, o, lse, dout, cu_seqlens, max_seqlen, *, scale,
             causal) -> (dq, dk, dv)
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import accounting  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmiattn.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_WORKSPACE = 0, -1, -2, -3, -4
BF16, FP32 = 0, 1
PAGE_SIZE = 16


class MiattnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libmiattn error {code}: {msg}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: run `python -m attention_attn_fwd_03_amd.build` "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.miattn_attn_fwd.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, F, I, I, P]
    lib.miattn_attn_fwd.restype = I
    lib.miattn_attn_fwd_paged.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, F, I, P]
    lib.miattn_attn_fwd_paged.restype = I
    lib.miattn_attn_decode_paged.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, F, I, P, Z, P, P, P]
    lib.miattn_attn_decode_paged.restype = I
    lib.miattn_attn_decode_paged_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, F, I, P, P, P]
    lib.miattn_attn_decode_paged_noalloc.restype = I
    lib.miattn_attn_decode_paged_numerics.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, F, I, I, I, P, Z, P,
                                                      I, P, P]
    lib.miattn_attn_decode_paged_numerics.restype = I
    lib.miattn_decode_numerics_workspace_bytes.argtypes = [I, I, I, I]
    lib.miattn_decode_numerics_workspace_bytes.restype = Z
    lib.miattn_attn_bwd.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, P, P, P, P, Z, P]
    lib.miattn_attn_bwd.restype = I
    lib.miattn_attn_bwd_workspace_bytes.argtypes = [I, I, I, I]
    lib.miattn_attn_bwd_workspace_bytes.restype = Z
    lib.miattn_attn_combine.argtypes = [P, P, I, I, I, P, P, I, P]
    lib.miattn_attn_combine.restype = I
    lib.miattn_decode_workspace_bytes.argtypes = [I, I, I, I]
    lib.miattn_decode_workspace_bytes.restype = Z
    lib.miattn_decode_pick_splits.argtypes = [I, I, I]
    lib.miattn_decode_pick_splits.restype = I
    lib.miattn_split_heuristic.argtypes = [I, I, I, I, I, I]
    lib.miattn_split_heuristic.restype = I
    lib.miattn_last_error.argtypes = []
    lib.miattn_last_error.restype = ctypes.c_char_p
    lib.miattn_version.argtypes = []
    lib.miattn_version.restype = I
    lib.miattn_device_supported.argtypes = [I]
    lib.miattn_device_supported.restype = I
    lib.miattn_release.argtypes = []
    lib.miattn_release.restype = None
    return lib


lib = _load()


def last_error() -> str:
    return lib.miattn_last_error().decode()


def _check(code: int):
    if code != OK:
        raise MiattnError(code, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_decode_tables(block_table, seq_lens, batch: int):
    # the kernels read block_table[b, :] and seq_lens[b] for every b < batch
    if block_table.dim() != 2 or block_table.shape[0] != batch or block_table.shape[1] < 1:
        raise ValueError(f"block_table must be [batch={batch}, max_pages >= 1], got {tuple(block_table.shape)}")
    if seq_lens.dim() != 1 or seq_lens.numel() != batch:
        raise ValueError(f"seq_lens must be [batch={batch}], got {tuple(seq_lens.shape)}")


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")


def attn_fwd(q, k, v, cu_seqlens, max_seqlen: int, *, scale: float, causal: bool,
             out=None, lse=None, return_lse: bool = True):
    """Prefill forward. q [T,Hq,D], k/v [T,Hkv,D] (bf16 or fp32), cu_seqlens
    int32 [n+1] on the device. Returns (o [T,Hq,D], lse [Hq,T] fp32)."""
    _need_cuda(q, k, v, cu_seqlens, out, lse)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    if q.dtype == torch.bfloat16:
        dt = BF16
    elif q.dtype == torch.float32:
        dt = FP32
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share a dtype")
    if cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if k.shape != (T, Hkv, D) or v.shape != (T, Hkv, D):
        raise ValueError("k/v must be [T, Hkv, D] like q")
    o = out if out is not None else torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
    _check(lib.miattn_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse) if return_lse else None,
                               _ptr(cu_seqlens), cu_seqlens.numel() - 1, int(max_seqlen), T, Hq, Hkv, D,
                               float(scale), int(bool(causal)), dt, _stream(q.device)))
    return o, (lse if return_lse else None)


def attn_bwd_workspace_bytes(total_tokens: int, num_q_heads: int, num_kv_heads: int, head_dim: int) -> int:
    return int(lib.miattn_attn_bwd_workspace_bytes(total_tokens, num_q_heads, num_kv_heads, head_dim))


def attn_bwd(q, k, v, o, lse, dout, cu_seqlens, max_seqlen: int, *, scale: float, causal: bool,
             dq=None, dk=None, dv=None, workspace=None):
    """Backward of attn_fwd (bf16). q/o/dout [T,Hq,D], k/v [T,Hkv,D], lse
    [Hq,T] fp32 from attn_fwd. Returns (dq [T,Hq,D], dk, dv [T,Hkv,D])."""
    _need_cuda(q, k, v, o, lse, dout, cu_seqlens, dq, dk, dv, workspace)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    for name, t_ in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if t_.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bf16")
    if k.shape != (T, Hkv, D) or v.shape != (T, Hkv, D) or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("shapes do not match")
    if lse.dtype != torch.float32 or lse.shape != (Hq, T):
        raise ValueError("lse must be fp32 [Hq, T]")
    if cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    dq = dq if dq is not None else torch.empty_like(q)
    dk = dk if dk is not None else torch.empty_like(k)
    dv = dv if dv is not None else torch.empty_like(v)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.miattn_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(cu_seqlens),
                               cu_seqlens.numel() - 1, int(max_seqlen), T, Hq, Hkv, D, float(scale),
                               int(bool(causal)), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes,
                               _stream(q.device)))
    return dq, dk, dv


def attn_fwd_paged(q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens_k, max_seqlen_q: int, *,
                   scale: float, causal: bool, out=None, lse=None, return_lse: bool = True):
    """Chunked prefill against a paged cache. q [Tq,Hq,D] bf16 packed by
    cu_seqlens_q (int32 [n+1]); caches [pages,16,Hkv,D] bf16; block_table
    int32 [n,max_pages]; seq_lens_k int32 [n] (keys per sequence, the chunk's
    own included). Returns (o [Tq,Hq,D] bf16, lse [Hq,Tq] fp32)."""
    _need_cuda(q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens_k, out, lse)
    Tq, Hq, D = q.shape
    num_pages, page, Hkv, Dk = k_cache.shape
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.bfloat16 or v_cache.dtype != torch.bfloat16:
        raise ValueError("paged prefill takes bf16 q and caches")
    if v_cache.shape != k_cache.shape or Dk != D:
        raise ValueError("cache shapes do not match q")
    for t, name in ((block_table, "block_table"), (cu_seqlens_q, "cu_seqlens_q"), (seq_lens_k, "seq_lens_k")):
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    n = cu_seqlens_q.numel() - 1
    if block_table.dim() != 2 or block_table.shape[0] != n or seq_lens_k.numel() != n:
        raise ValueError("block_table must be [n, max_pages] and seq_lens_k [n] for n sequences")
    if not block_table.is_contiguous():
        raise ValueError("block_table must be contiguous")
    o = out if out is not None else torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device)
    _check(lib.miattn_attn_fwd_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o),
                                     _ptr(lse) if return_lse else None, _ptr(cu_seqlens_q), _ptr(seq_lens_k),
                                     _ptr(block_table), n, int(max_seqlen_q), Tq, block_table.shape[1], page,
                                     num_pages, Hq, Hkv, D, float(scale), int(bool(causal)), _stream(q.device)))
    return o, (lse if return_lse else None)


def decode_workspace_bytes(batch: int, num_q_heads: int, head_dim: int, num_splits: int) -> int:
    return int(lib.miattn_decode_workspace_bytes(batch, num_q_heads, head_dim, num_splits))


def decode_pick_splits(batch: int, num_kv_heads: int, max_seq_len: int) -> int:
    return int(lib.miattn_decode_pick_splits(batch, num_kv_heads, max_seq_len))


def split_heuristic(total_tokens, work_units, cu_count, wg_per_cu, block_tokens, max_splits) -> int:
    return int(lib.miattn_split_heuristic(total_tokens, work_units, cu_count, wg_per_cu, block_tokens,
                                          max_splits))


def attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, *, scale: float, num_splits: int = 0,
                      workspace=None, out=None, lse=None, return_lse: bool = True):
    """Paged split-KV decode. q [B,Hq,D] bf16; caches [pages,16,Hkv,D] bf16;
    block_table int32 [B,max_pages]; seq_lens int32 [B]. Returns
    (o [B,Hq,D] bf16, lse [B,Hq] fp32)."""
    B, Hq, D = q.shape
    num_pages, page, Hkv, Dk = k_cache.shape
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.bfloat16 or v_cache.dtype != torch.bfloat16:
        raise ValueError("decode takes bf16 q and caches")
    if v_cache.shape != k_cache.shape or Dk != D:
        raise ValueError("cache shapes do not match q")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    _check_decode_tables(block_table, seq_lens, B)
    _need_cuda(q, k_cache, v_cache, block_table, seq_lens, out, lse, workspace)
    o = out if out is not None else torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.miattn_attn_decode_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                        _ptr(seq_lens), B, block_table.shape[1], page, num_pages, Hq, Hkv,
                                        D, float(scale), int(num_splits), _ptr(workspace), ws_bytes,
                                        _ptr(o), _ptr(lse) if return_lse else None, _stream(q.device)))
    return o, (lse if return_lse else None)


# bytes of the static device scratch behind attn_decode_paged_noalloc
NOALLOC_SCRATCH_BYTES = 32 << 20


def attn_decode_paged_noalloc(q, k_cache, v_cache, block_table, seq_lens, *, scale: float, num_splits: int = 0,
                              out=None, lse=None, return_lse: bool = True):
    """attn_decode_paged without any device allocation inside the library: the
    split partials use the library's static per-GPU scratch
    (NOALLOC_SCRATCH_BYTES). Pass `out` (and `lse`) to allocate nothing here
    either. Calls that may overlap on one GPU race on that scratch."""
    B, Hq, D = q.shape
    num_pages, page, Hkv, Dk = k_cache.shape
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.bfloat16 or v_cache.dtype != torch.bfloat16:
        raise ValueError("decode takes bf16 q and caches")
    if v_cache.shape != k_cache.shape or Dk != D:
        raise ValueError("cache shapes do not match q")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    _check_decode_tables(block_table, seq_lens, B)
    _need_cuda(q, k_cache, v_cache, block_table, seq_lens, out, lse)
    o = out if out is not None else torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check(lib.miattn_attn_decode_paged_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                                _ptr(seq_lens), B, block_table.shape[1], page, num_pages, Hq,
                                                Hkv, D, float(scale), int(num_splits), _ptr(o),
                                                _ptr(lse) if return_lse else None, _stream(q.device)))
    return o, (lse if return_lse else None)


# numerics of the decode split records (miattn_attn_decode_paged_numerics)
RECORD_LSE = 0
RECORD_NUMERATOR_F32 = 1
RECORD_NORMALIZED_BF16 = 2
RECORD_NUMERATOR_BF16 = 3
NUMERICS_ROUNDED_NORMALIZER = 4
NUMERICS_P_FP16 = 8


def decode_numerics_workspace_bytes(batch: int, num_q_heads: int, head_dim: int, num_splits: int) -> int:
    return int(lib.miattn_decode_numerics_workspace_bytes(batch, num_q_heads, head_dim, num_splits))


def attn_decode_paged_numerics(q, k_cache, v_cache, block_table, seq_lens, *, scale: float, num_splits: int,
                               numerics: int = RECORD_LSE, tile_pages: int = 0, out_dtype=torch.bfloat16,
                               workspace=None, out=None, lse=None, return_lse: bool = True):
    """Paged split-KV decode with selectable split records, rounding points
    and group geometry (see miattn_attn_decode_paged_numerics). Same inputs as
    attn_decode_paged; returns (o [B,Hq,D] of out_dtype, lse [B,Hq] fp32)."""
    B, Hq, D = q.shape
    num_pages, page, Hkv, Dk = k_cache.shape
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.bfloat16 or v_cache.dtype != torch.bfloat16:
        raise ValueError("decode takes bf16 q and caches")
    if v_cache.shape != k_cache.shape or Dk != D:
        raise ValueError("cache shapes do not match q")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    _check_decode_tables(block_table, seq_lens, B)
    _need_cuda(q, k_cache, v_cache, block_table, seq_lens, out, lse, workspace)
    dt = BF16 if out_dtype == torch.bfloat16 else FP32 if out_dtype == torch.float32 else None
    if dt is None:
        raise ValueError("out_dtype must be bf16 or fp32")
    o = out if out is not None else torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.miattn_attn_decode_paged_numerics(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens), B, block_table.shape[1], page,
        num_pages, Hq, Hkv, D, float(scale), int(num_splits), int(numerics), int(tile_pages), _ptr(workspace),
        ws_bytes, _ptr(o), dt, _ptr(lse) if return_lse else None, _stream(q.device)))
    return o, (lse if return_lse else None)


def attn_combine(partial_o, partial_lse, *, out_dtype=torch.bfloat16, out=None, lse=None,
                 return_lse: bool = True):
    """LSE-weighted merge. partial_o fp32 [rows,S,D], partial_lse fp32 [rows,S]
    (-inf = empty split). Returns (o [rows,D] of out_dtype, lse [rows] fp32)."""
    _need_cuda(partial_o, partial_lse, out, lse)
    rows, S, D = partial_o.shape
    if partial_o.dtype != torch.float32 or partial_lse.dtype != torch.float32:
        raise ValueError("partials must be fp32")
    if partial_lse.shape != (rows, S):
        raise ValueError("partial_lse must be [rows, S]")
    dt = BF16 if out_dtype == torch.bfloat16 else FP32 if out_dtype == torch.float32 else None
    if dt is None:
        raise ValueError("out_dtype must be bf16 or fp32")
    o = out if out is not None else torch.empty((rows, D), dtype=out_dtype, device=partial_o.device)
    if return_lse and lse is None:
        lse = torch.empty((rows,), dtype=torch.float32, device=partial_o.device)
    _check(lib.miattn_attn_combine(_ptr(partial_o), _ptr(partial_lse), rows, S, D, _ptr(o),
                                   _ptr(lse) if return_lse else None, dt, _stream(partial_o.device)))
    return o, (lse if return_lse else None)


def release():
    lib.miattn_release()

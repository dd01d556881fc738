"""Python binding of the gfx950 fused-attention library (libfa.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of ``include/fa.h``. PyTorch supplies device memory
and the current stream; nothing here computes attention, and there is no CPU
fallback: if ``libfa.so`` is missing, or a tensor is not on the GPU, the call
raises.

    import attention_fa_prefill_amd as fa
    o = fa.prefill(q, k, v, causal=True)                 # bf16 or fp32 [B,H,S,d]
    o = fa.decode(q, kcache, vcache, seqlens, block_table=bt)   # bf16 [B,Hq,d]
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

FA_OK = 0
STATUS_NAMES = {0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_UNSUPPORTED", 4: "FA_ERR_ALIGN",
                5: "FA_ERR_WORKSPACE", 6: "FA_ERR_HIP", 7: "FA_ERR_ARG"}
EXPORTS = ("fa_status_string", "fa_version", "fa_prefill", "fa_prefill_f32", "fa_prefill_cache", "fa_decode_split_tokens",
           "fa_decode_workspace_bytes", "fa_decode", "fa_decode_fp8", "fa_merge_lse", "fa_decode_noalloc",
           "fa_decode_int8")

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libfa.so (built in-tree by ``python -m attention_fa_prefill_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run: python -m attention_fa_prefill_amd.build")
        # libfa.so must run on the HIP runtime that owns the caller's memory and
        # streams. PyTorch ships its own copy of the runtime; once torch is
        # loaded, libfa.so's dependency on libamdhip64.so.7 resolves to that
        # copy. Loaded first, libfa.so would pull in the system runtime and the
        # process would hold two, whose streams and launches do not mix.
        # (Without torch there is only the system runtime.)
        try:
            _torch()
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        vp, ci, cf, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.fa_status_string.argtypes = [ci]
        L.fa_status_string.restype = ctypes.c_char_p
        L.fa_version.argtypes = []
        L.fa_version.restype = ci
        pre = [vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, ci, vp]
        L.fa_prefill.argtypes = pre
        L.fa_prefill.restype = ci
        L.fa_prefill_f32.argtypes = pre
        L.fa_prefill_f32.restype = ci
        L.fa_prefill_cache.argtypes = [vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, cf, ci, vp]
        L.fa_prefill_cache.restype = ci
        L.fa_decode_split_tokens.argtypes = [ci, ci, ci, ci, ci]
        L.fa_decode_split_tokens.restype = ci
        L.fa_decode_workspace_bytes.argtypes = [ci, ci, ci, ci, ci, ci]
        L.fa_decode_workspace_bytes.restype = sz
        L.fa_decode.argtypes = [vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, cf, vp, sz, vp]
        L.fa_decode.restype = ci
        L.fa_decode_fp8.argtypes = [vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, cf, cf, cf, vp, sz, vp]
        L.fa_decode_fp8.restype = ci
        L.fa_decode_int8.argtypes = L.fa_decode_fp8.argtypes
        L.fa_decode_int8.restype = ci
        L.fa_merge_lse.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, vp]
        L.fa_merge_lse.restype = ci
        L.fa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, cf, vp]
        L.fa_decode_noalloc.restype = ci
        _lib = L
    return _lib


def check(status: int) -> None:
    if status != FA_OK:
        raise FAError(status, lib().fa_status_string(status).decode())


def status_string(status: int) -> str:
    return lib().fa_status_string(status).decode()


# ----------------------------------------------------------------------------- helpers


def _torch():
    import torch

    return torch


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("fused attention runs on the GPU only: pass device tensors")


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous (row-major)")


def _stream_handle(t, stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _cache_geometry(kcache, vcache, seqlens, block_table, max_kv_len, B, d):
    """(max_kv_len, page_size) of a contiguous or paged cache, after checking
    that the tensors agree with each other and with the batch: the kernels use
    max_kv_len as the per-sequence row count of a contiguous cache and read B
    lengths and B block-table rows."""
    if kcache.shape != vcache.shape or kcache.shape[3] != d:
        raise ValueError("kcache and vcache must match and end in [Hkv, d]")
    if seqlens.dim() != 1 or seqlens.numel() != B:
        raise ValueError(f"seqlens must be int32 [B] with B = {B}")
    if block_table is None:
        if kcache.shape[0] != B:
            raise ValueError("contiguous cache must be [B, max_kv_len, Hkv, d]")
        mkl = kcache.shape[1]
        if max_kv_len is not None and int(max_kv_len) != mkl:
            raise ValueError(f"max_kv_len ({max_kv_len}) must equal the contiguous cache's length ({mkl})")
        return mkl, 0
    if kcache.shape[1] != 16 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("paged cache must be [num_pages, 16, Hkv, d] with block_table [B, pages]")
    mkl = 16 * block_table.shape[1] if max_kv_len is None else int(max_kv_len)
    if (mkl + 15) // 16 != block_table.shape[1]:
        raise ValueError("block_table must have ceil(max_kv_len/16) columns")
    return mkl, 16


def _check_out(o, q):
    """A caller's output tensor must match q in shape and dtype."""
    if o is not None and (o.shape != q.shape or o.dtype != q.dtype):
        raise ValueError(f"o must match q in shape {tuple(q.shape)} and dtype {q.dtype}")


# ----------------------------------------------------------------------------- entry points


def prefill(q, k, v, o=None, *, causal: bool = True, scale: float | None = None, stream=None):
    """Fused attention. q [B,Hq,Sq,d]; k, v [B,Hkv,Skv,d]; bf16 or fp32 (all alike).

    Returns o [B,Hq,Sq,d] (written into ``o`` if given). bf16 runs ``fa_prefill``,
    fp32 runs ``fa_prefill_f32``.
    """
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("expected q [B,Hq,Sq,d] and k, v [B,Hkv,Skv,d]")
    B, Hq, Sq, d = q.shape
    Bk, Hkv, Skv, dk = k.shape
    if Bk != B or dk != d:
        raise ValueError("q and k/v disagree on batch or head_dim")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k, v must all be bfloat16 or all float32")
    _check_out(o, q)
    _dev(q, k, v, o)
    _contig(q, k, v, o)
    if o is None:
        o = torch.empty_like(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    fn = lib().fa_prefill if q.dtype == torch.bfloat16 else lib().fa_prefill_f32
    check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, Hq, Hkv, Sq, Skv, d, float(scale), int(bool(causal)),
             _stream_handle(q, stream)))
    return o


def prefill_cache(q, kcache, vcache, seqlens, *, block_table=None, max_kv_len: int | None = None, causal: bool = True,
                  scale: float | None = None, o=None, stream=None):
    """Chunked prefill over a KV cache. q [B,Hq,Sq,d] bf16 (each sequence's Sq
    new queries); kcache, vcache bf16 in the decode layouts (contiguous
    [B, max_kv_len, Hkv, d], or pages [num_pages, 16, Hkv, d] with block_table
    int32 [B, pages_per_seq]); seqlens int32 [B] cached tokens, the new ones
    included. Returns o [B,Hq,Sq,d] bf16."""
    torch = _torch()
    if q.dtype != torch.bfloat16 or kcache.dtype != torch.bfloat16 or vcache.dtype != torch.bfloat16:
        raise ValueError("prefill_cache takes bfloat16 q and caches")
    if seqlens.dtype != torch.int32 or (block_table is not None and block_table.dtype != torch.int32):
        raise ValueError("seqlens and block_table must be int32")
    if q.dim() != 4 or kcache.dim() != 4:
        raise ValueError("expected q [B,Hq,Sq,d] and caches of 4 dims")
    B, Hq, Sq, d = q.shape
    Hkv = kcache.shape[2]
    mkl, page = _cache_geometry(kcache, vcache, seqlens, block_table, max_kv_len, B, d)
    _check_out(o, q)
    _dev(q, kcache, vcache, seqlens, block_table, o)
    _contig(q, kcache, vcache, seqlens, block_table, o)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty_like(q)
    check(lib().fa_prefill_cache(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(block_table), _ptr(seqlens), _ptr(o), B,
                                 Hq, Hkv, Sq, d, mkl, page, float(scale), int(bool(causal)), _stream_handle(q, stream)))
    return o


def decode_split_tokens(B: int, Hq: int, Hkv: int, max_kv_len: int, tokens_per_split: int = 0) -> int:
    """KV tokens per split that fa_decode uses for these sizes (0 if invalid)."""
    return int(lib().fa_decode_split_tokens(B, Hq, Hkv, max_kv_len, tokens_per_split))


def decode_workspace_bytes(B: int, Hq: int, Hkv: int, d: int, max_kv_len: int, tokens_per_split: int = 0) -> int:
    return int(lib().fa_decode_workspace_bytes(B, Hq, Hkv, d, max_kv_len, tokens_per_split))


def decode(q, kcache, vcache, seqlens, *, block_table=None, max_kv_len: int | None = None, scale: float | None = None,
           tokens_per_split: int = 0, o=None, workspace=None, stream=None):
    """Single-token decode. q [B,Hq,d] bf16; seqlens int32 [B] (device).

    Contiguous cache: kcache, vcache bf16 [B, max_kv_len, Hkv, d].
    Paged cache (block_table int32 [B, pages_per_seq]): kcache, vcache bf16
    [num_pages, 16, Hkv, d]; max_kv_len defaults to 16 * pages_per_seq.
    Returns o [B,Hq,d] bf16.
    """
    return _decode(q, kcache, vcache, seqlens, None, block_table, max_kv_len, scale, tokens_per_split, o, workspace,
                   stream)


def decode_fp8(q, kcache, vcache, seqlens, *, k_scale: float, v_scale: float, block_table=None,
               max_kv_len: int | None = None, scale: float | None = None, tokens_per_split: int = 0, o=None,
               workspace=None, stream=None):
    """decode over an FP8 cache: kcache, vcache hold OCP FP8 E4M3 codes (uint8
    or float8_e4m3fn tensors, same layouts as decode); K = k_scale * E4M3(code),
    V = v_scale * E4M3(code). q and o bf16."""
    return _decode(q, kcache, vcache, seqlens, (float(k_scale), float(v_scale)), block_table, max_kv_len, scale,
                   tokens_per_split, o, workspace, stream)


def decode_int8(q, kcache, vcache, seqlens, *, k_scale: float, v_scale: float, block_table=None,
                max_kv_len: int | None = None, scale: float | None = None, tokens_per_split: int = 0, o=None,
                workspace=None, stream=None):
    """decode over an INT8 cache: kcache, vcache hold signed 8-bit codes
    (int8 or uint8 tensors holding the two's-complement bytes, same layouts as
    decode); K = k_scale * code, V = v_scale * code. q and o bf16."""
    return _decode(q, kcache, vcache, seqlens, (float(k_scale), float(v_scale)), block_table, max_kv_len, scale,
                   tokens_per_split, o, workspace, stream, fmt="int8")


def decode_noalloc(q, kcache, vcache, seqlens, o, *, block_table=None, max_kv_len: int | None = None,
                   scale: float | None = None, tokens_per_split: int = 0, stream=None):
    """decode without a workspace (``fa_decode_noalloc``): the split partials
    live in the library's 16 MiB device array, so the call allocates nothing
    (the caller passes o). Calls that may overlap on one GPU race."""
    if o is None:
        raise ValueError("decode_noalloc writes into a caller's o")
    return _decode(q, kcache, vcache, seqlens, None, block_table, max_kv_len, scale, tokens_per_split, o, None,
                   stream, noalloc=True)


def _decode(q, kcache, vcache, seqlens, fp8_scales, block_table, max_kv_len, scale, tokens_per_split, o, workspace,
            stream, noalloc=False, fmt="fp8"):
    torch = _torch()
    if fp8_scales is None:
        if q.dtype != torch.bfloat16 or kcache.dtype != torch.bfloat16 or vcache.dtype != torch.bfloat16:
            raise ValueError("decode takes bfloat16 q and caches")
    elif fmt == "int8":
        if q.dtype != torch.bfloat16 or kcache.dtype not in (torch.int8, torch.uint8) or \
                vcache.dtype not in (torch.int8, torch.uint8):
            raise ValueError("decode_int8 takes a bfloat16 q and int8 / uint8 caches")
    else:
        byte_types = (torch.uint8,) + ((torch.float8_e4m3fn,) if hasattr(torch, "float8_e4m3fn") else ())
        if q.dtype != torch.bfloat16 or kcache.dtype not in byte_types or vcache.dtype not in byte_types:
            raise ValueError("decode_fp8 takes a bfloat16 q and uint8 / float8_e4m3fn caches")
    if seqlens.dtype != torch.int32 or (block_table is not None and block_table.dtype != torch.int32):
        raise ValueError("seqlens and block_table must be int32")
    if q.dim() != 3 or kcache.dim() != 4:
        raise ValueError("expected q [B,Hq,d] and caches of 4 dims")
    B, Hq, d = q.shape
    Hkv = kcache.shape[2]
    mkl, page = _cache_geometry(kcache, vcache, seqlens, block_table, max_kv_len, B, d)
    _check_out(o, q)
    _dev(q, kcache, vcache, seqlens, block_table, o, workspace)
    _contig(q, kcache, vcache, seqlens, block_table, o, workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty_like(q)
    if noalloc:
        check(lib().fa_decode_noalloc(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(block_table), _ptr(seqlens), _ptr(o),
                                      B, Hq, Hkv, d, mkl, page, int(tokens_per_split), float(scale),
                                      _stream_handle(q, stream)))
        return o
    need = decode_workspace_bytes(B, Hq, Hkv, d, mkl, tokens_per_split)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    common = (_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(block_table), _ptr(seqlens), _ptr(o), B, Hq, Hkv, d, mkl,
              page, int(tokens_per_split), float(scale))
    tail = (_ptr(workspace), workspace.numel() * workspace.element_size(), _stream_handle(q, stream))
    if fp8_scales is None:
        check(lib().fa_decode(*common, *tail))
    elif fmt == "int8":
        check(lib().fa_decode_int8(*common, *fp8_scales, *tail))
    else:
        check(lib().fa_decode_fp8(*common, *fp8_scales, *tail))
    return o


def merge_lse(o_parts, lse, *, out_dtype=None, o=None, lse_out=None, stream=None):
    """Log-sum-exp merge of S partial results per row.

    o_parts fp32 [R, S, d] (normalised parts), lse fp32 [R, S] (natural log).
    Returns (o [R, d] in out_dtype (bf16 default, or fp32), lse_out fp32 [R]).
    """
    torch = _torch()
    if o_parts.dtype != torch.float32 or lse.dtype != torch.float32:
        raise ValueError("o_parts and lse must be float32")
    if o_parts.dim() != 3:
        raise ValueError("o_parts must be [R, S, d]")
    R, S, d = o_parts.shape
    if tuple(lse.shape) != (R, S):
        raise ValueError(f"lse must be [R, S] = [{R}, {S}]")
    if out_dtype is None:
        out_dtype = torch.bfloat16 if o is None else o.dtype
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("the merged output is bfloat16 or float32")
    if o is not None and (tuple(o.shape) != (R, d) or o.dtype != out_dtype):
        raise ValueError(f"o must be [R, d] = [{R}, {d}] of dtype {out_dtype}")
    if lse_out is not None and (tuple(lse_out.shape) != (R,) or lse_out.dtype != torch.float32):
        raise ValueError(f"lse_out must be float32 [R] = [{R}]")
    _dev(o_parts, lse, o, lse_out)
    _contig(o_parts, lse, o, lse_out)
    if o is None:
        o = torch.empty((R, d), dtype=out_dtype, device=o_parts.device)
    if lse_out is None:
        lse_out = torch.empty((R,), dtype=torch.float32, device=o_parts.device)
    check(lib().fa_merge_lse(_ptr(o_parts), _ptr(lse), _ptr(o), _ptr(lse_out), R, S, d,
                             int(o.dtype == torch.bfloat16), _stream_handle(o_parts, stream)))
    return o, lse_out

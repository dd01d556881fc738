"""fp64 CPU oracle for fused attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and its
Python binding) never imports, links or runs it, and this package imports
nothing from the product.

``attention``, ``decode`` and ``merge`` call the plain C implementation in
``fa_oracle.c`` (the softmax-attention definition written out in fp64; the
header of that file lists the readings it takes); ``brute`` holds an
independent pure-Python formulation for tiny shapes.

Page citations: the definition is the one the tiled kernel of the "Real-time
inference optimisation" page (section "Flash Attention optimisation") reaches
in exact arithmetic; paged decode follows that page's paged-attention sketch
(page size 16) with its per-page sum replaced by the log-sum-exp merge.

Every function takes an optional ``lib`` path so that the pin suite can also be
run against deliberately broken copies of the C source (mutation testing).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "fa_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_libs: dict = {}


def build(force: bool = True, src: str = SRC, out: str = LIB_PATH) -> str:
    """Compile an oracle C source into a shared library with gcc (OpenMP, no fast-math)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall", "-o", tmp, src, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def _load(path: str | None = None):
    if path is None:
        path = LIB_PATH
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(SRC):
            build(force=True)
    lib = _libs.get(path)
    if lib is None:
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        ci = ctypes.c_int
        lib.oracle_attention_f64.argtypes = [dp, dp, dp, dp, dp, ci, ci, ci, ci, ci, ci, ctypes.c_double, ci]
        lib.oracle_attention_f64.restype = ci
        lib.oracle_decode_f64.argtypes = [dp, dp, dp, ip, ci, ip, dp, dp, ci, ci, ci, ci, ci, ci, ctypes.c_double]
        lib.oracle_decode_f64.restype = ci
        lib.oracle_merge_f64.argtypes = [dp, dp, dp, dp, ci, ci, ci]
        lib.oracle_merge_f64.restype = ci
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ci
        _libs[path] = lib
    return lib


def _dptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _iptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def num_threads(lib: str | None = None) -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS, else all visible cores)."""
    return int(_load(lib).oracle_num_threads())


def attention(q, k, v, scale: float, causal: bool, lib: str | None = None):
    """Plain softmax attention in fp64.

    q: [B, Hq, Sq, d]; k, v: [B, Hkv, Skv, d] (any real dtype, converted exactly
    to float64). Returns (o [B, Hq, Sq, d], lse [B, Hq, Sq]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Sq, d = q.shape
    Bk, Hkv, Skv, dk = k.shape
    assert Bk == B and dk == d and v.shape == k.shape
    o = np.empty((B, Hq, Sq, d), dtype=np.float64)
    lse = np.empty((B, Hq, Sq), dtype=np.float64)
    rc = _load(lib).oracle_attention_f64(_dptr(q), _dptr(k), _dptr(v), _dptr(o), _dptr(lse),
                                         B, Hq, Hkv, Sq, Skv, d, float(scale), int(bool(causal)))
    if rc != 0:
        raise ValueError("oracle_attention_f64: invalid shape")
    return o, lse


def decode(q, kcache, vcache, seqlens, scale: float, block_table=None, page_size: int = 16, max_kv_len=None,
           lib: str | None = None):
    """Single-query attention over each sequence's cached tokens, in fp64.

    q: [B, Hq, d]. Contiguous cache (block_table None): kcache, vcache
    [B, max_kv_len, Hkv, d]. Paged cache: [num_pages, page_size, Hkv, d] with
    block_table int32 [B, pages_per_seq]. seqlens int32 [B].
    Returns (o [B, Hq, d], lse [B, Hq]).
    """
    q, kc, vc = _f64(q), _f64(kcache), _f64(vcache)
    B, Hq, d = q.shape
    Hkv = kc.shape[2]
    seqlens = np.ascontiguousarray(seqlens, dtype=np.int32)
    if block_table is None:
        mkl = kc.shape[1] if max_kv_len is None else int(max_kv_len)
        bt, pps, page = None, 0, 1
    else:
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        pps = bt.shape[1]
        page = int(page_size)
        mkl = pps * page if max_kv_len is None else int(max_kv_len)
    o = np.empty((B, Hq, d), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64)
    rc = _load(lib).oracle_decode_f64(_dptr(q), _dptr(kc), _dptr(vc), _iptr(bt), pps, _iptr(seqlens),
                                      _dptr(o), _dptr(lse), B, Hq, Hkv, d, mkl, page, float(scale))
    if rc != 0:
        raise ValueError("oracle_decode_f64: invalid shape")
    return o, lse


def prefill_cache(q, kcache, vcache, seqlens, scale: float, causal: bool, block_table=None, page_size: int = 16,
                  max_kv_len=None, lib: str | None = None):
    """Chunked prefill over a KV cache, in fp64: sequence b's keys are its
    first L_b = clamp(seqlens[b], 0, max_kv_len) cached tokens, gathered from
    the cache (contiguous [B, max_kv_len, Hkv, d], or pages [P, page, Hkv, d]
    through block_table [B, pages]), and its Sq queries q[b] are the last Sq
    of them: with causal, row i sees tokens j <= i + L_b - Sq. A row that sees
    no token is zero (softmax over an empty set taken as an empty sum).
    Returns o [B, Hq, Sq, d]."""
    q, kc, vc = _f64(q), _f64(kcache), _f64(vcache)
    B, Hq, Sq, d = q.shape
    Hkv = kc.shape[2]
    lens = np.asarray(seqlens, dtype=np.int64)
    if block_table is None:
        mkl = kc.shape[1] if max_kv_len is None else int(max_kv_len)
    else:
        bt = np.asarray(block_table, dtype=np.int64)
        mkl = bt.shape[1] * int(page_size) if max_kv_len is None else int(max_kv_len)
    o = np.zeros((B, Hq, Sq, d), dtype=np.float64)
    for b in range(B):
        L = int(min(max(lens[b], 0), mkl))
        if L == 0:
            continue
        t = np.arange(L)
        if block_table is None:
            kb, vb = kc[b, :L], vc[b, :L]                      # [L, Hkv, d]
        else:
            rows = bt[b, t // page_size], t % page_size
            kb, vb = kc[rows], vc[rows]
        kb = np.ascontiguousarray(kb.transpose(1, 0, 2))[None]  # [1, Hkv, L, d]
        vb = np.ascontiguousarray(vb.transpose(1, 0, 2))[None]
        if causal and L < Sq:
            # rows i < Sq - L see nothing; the rest are the last L rows over L keys
            ob, _ = attention(q[b:b + 1, :, Sq - L:], kb, vb, scale, True, lib=lib)
            o[b, :, Sq - L:] = ob[0]
        else:
            ob, _ = attention(q[b:b + 1], kb, vb, scale, causal, lib=lib)
            o[b] = ob[0]
    return o


def e4m3_to_f64(codes) -> np.ndarray:
    """OCP 8-bit floating point E4M3 (the "FN" variant: no infinities) to
    fp64, from the definition of the format: bit 7 sign, bits 6..3 exponent
    field E with bias 7, bits 2..0 mantissa field M. E = 0 is subnormal,
    (M / 8) * 2^-6; E = 15 with M = 7 is NaN; otherwise (1 + M / 8) * 2^(E - 7).
    The largest finite value is 448 (E = 15, M = 6). This is the 8-bit KV-cache
    element of the fp8 decode (FasterTransformer walkthrough, section 3.3: an
    8-bit KV cache; FlashRT summary: FP8 with one scale per tensor)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    mag = np.where((e == 15) & (c & 7 == 7), np.nan, mag)
    return sign * mag


def decode_fp8(q, kcodes, vcodes, seqlens, scale: float, k_scale: float, v_scale: float, block_table=None,
               page_size: int = 16, max_kv_len=None, lib: str | None = None):
    """decode over an FP8 E4M3 cache with one scale per tensor: the cache is
    dequantised (K = k_scale * E4M3(code), V = v_scale * E4M3(code)) and the
    same definition applied in fp64. Returns (o [B, Hq, d], lse [B, Hq])."""
    kc = e4m3_to_f64(kcodes) * float(k_scale)
    vc = e4m3_to_f64(vcodes) * float(v_scale)
    return decode(q, kc, vc, seqlens, scale, block_table=block_table, page_size=page_size, max_kv_len=max_kv_len,
                  lib=lib)


def int8_to_f64(codes) -> np.ndarray:
    """Signed 8-bit integers (two's complement) to fp64, from the definition:
    a byte c = 0..255 holds c when c < 128 and c - 256 otherwise, so the
    range is -128..127. This is the element of the INT8 KV cache of the
    FasterTransformer walkthrough (section 3.3: an 8-bit KV cache that halves
    the bytes a decode step reads), with one scale per tensor."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(c >= 128, c - 256, c).astype(np.float64)


def decode_int8(q, kcodes, vcodes, seqlens, scale: float, k_scale: float, v_scale: float, block_table=None,
                page_size: int = 16, max_kv_len=None, lib: str | None = None):
    """decode over an INT8 cache with one scale per tensor: the cache is
    dequantised (K = k_scale * code, V = v_scale * code) and the same
    definition applied in fp64. Returns (o [B, Hq, d], lse [B, Hq])."""
    kc = int8_to_f64(kcodes) * float(k_scale)
    vc = int8_to_f64(vcodes) * float(v_scale)
    return decode(q, kc, vc, seqlens, scale, block_table=block_table, page_size=page_size, max_kv_len=max_kv_len,
                  lib=lib)


def merge(o_parts, lse_parts, lib: str | None = None):
    """Log-sum-exp merge. o_parts [R, S, d] (normalised parts), lse_parts [R, S].
    Returns (o [R, d], lse [R])."""
    op, lp = _f64(o_parts), _f64(lse_parts)
    R, S, d = op.shape
    assert lp.shape == (R, S)
    o = np.empty((R, d), dtype=np.float64)
    lse = np.empty((R,), dtype=np.float64)
    _load(lib).oracle_merge_f64(_dptr(op), _dptr(lp), _dptr(o), _dptr(lse), R, S, d)
    return o, lse

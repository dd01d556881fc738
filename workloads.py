"""Seeded synthetic workloads for the attention kernels and the oracle.

This module only draws and lays out inputs; it holds none of the attention
arithmetic. Both the GPU path (through the binding) and the fp64 oracle consume
exactly what it returns: bf16 data is produced as bf16 bit patterns (uint16),
and the oracle reads the same bits converted exactly to float64.

Generator: numpy's PCG64 seeded with SeedSequence([seed, stream]); normal
values come from ``Generator.standard_normal`` in float32 and are rounded to
bf16 with round-to-nearest-even. Streams are numbered so that adding a draw
never changes an earlier one.

Workloads (shapes from the small-batch inference setting of the pages: 32
heads of dimension 128 as in the FlashRT-HF-kernels usage example, 32k
contexts as on the TensorRT page, 256K contexts as on the FlashRT page, page
size 16 as in the paged sketch of the real-time inference page):

  prefill_f32_b1h1s128d64            fp32 causal, B=1, H=1, Sq=Skv=128, d=64
  prefill_gqa_b1h32x8s2048d128       bf16 GQA causal, B=1, Hq=32, Hkv=8, Sq=Skv=2048, d=128
  decode_contig_b4h32x8kv32768d128   bf16 decode, B=4, Hq=32, Hkv=8, 32768 cached tokens each
  decode_paged_b8h32x8kv1k16kd128    bf16 paged decode, B=8, lengths U{1024..16384}, page 16
  decode_long_b1h16x2kv256kd128      bf16 paged decode, B=1, Hq=16, Hkv=2, 262144 tokens
"""
from __future__ import annotations

import math
import zlib
from dataclasses import dataclass, field

import numpy as np

PAGE = 16
BF16_NAN = np.uint16(0x7FC0)


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(stream)])))


def normal_f32(seed: int, stream: int, shape) -> np.ndarray:
    return rng(seed, stream).standard_normal(size=shape, dtype=np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round-to-nearest-even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = BF16_NAN
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


def normal_bf16(seed: int, stream: int, shape) -> np.ndarray:
    return f32_to_bf16_bits(normal_f32(seed, stream, shape))


# --------------------------------------------------------------------------- prefill


@dataclass
class PrefillCase:
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Skv: int
    d: int
    causal: bool
    dtype: str  # "bf16" (uint16 bits) or "f32"
    scale: float
    q: np.ndarray = field(repr=False)
    k: np.ndarray = field(repr=False)
    v: np.ndarray = field(repr=False)

    def as_f64(self):
        conv = bf16_bits_to_f64 if self.dtype == "bf16" else (lambda a: a.astype(np.float64))
        return conv(self.q), conv(self.k), conv(self.v)


def device_normal_bf16(shape, seed: int, device="cuda"):
    """N(0, 1) values rounded to bf16, drawn on the device by torch's seeded
    generator: inputs too large to build on the host (several GB). Tests copy
    the slices the oracle needs back to the host."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def prefill_case(B, Hq, Hkv, Sq, Skv, d, causal=True, dtype="bf16", seed=1, scale=None, name=None) -> PrefillCase:
    """q [B,Hq,Sq,d], k/v [B,Hkv,Skv,d], i.i.d. N(0,1) from (seed, stream 0/1/2)."""
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    shp_q, shp_kv = (B, Hq, Sq, d), (B, Hkv, Skv, d)
    if dtype == "bf16":
        q, k, v = normal_bf16(seed, 0, shp_q), normal_bf16(seed, 1, shp_kv), normal_bf16(seed, 2, shp_kv)
    elif dtype == "f32":
        q, k, v = normal_f32(seed, 0, shp_q), normal_f32(seed, 1, shp_kv), normal_f32(seed, 2, shp_kv)
    else:
        raise ValueError(dtype)
    if name is None:
        name = f"prefill_{dtype}_b{B}h{Hq}x{Hkv}sq{Sq}skv{Skv}d{d}{'_causal' if causal else ''}"
    return PrefillCase(name, B, Hq, Hkv, Sq, Skv, d, bool(causal), dtype, float(scale), q, k, v)


def prefill_f32_small() -> PrefillCase:
    """fp32 single-head causal forward: B=1, H=1, Sq=Skv=128, d=64, scale 1/8."""
    return prefill_case(1, 1, 1, 128, 128, 64, True, "f32", seed=1001, scale=1.0 / math.sqrt(64),
                        name="prefill_f32_b1h1s128d64")


def prefill_gqa_2k() -> PrefillCase:
    """bf16 GQA causal prefill: B=1, Hq=32, Hkv=8, Sq=Skv=2048, d=128, scale 1/sqrt(128)."""
    return prefill_case(1, 32, 8, 2048, 2048, 128, True, "bf16", seed=1002, scale=1.0 / math.sqrt(128),
                        name="prefill_gqa_b1h32x8s2048d128")


def prefill_gqa_d256() -> PrefillCase:
    """bf16 GQA causal prefill at head dim 256: B=1, Hq=16, Hkv=8, Sq=Skv=2048, scale 1/16."""
    return prefill_case(1, 16, 8, 2048, 2048, 256, True, "bf16", seed=1007, scale=1.0 / 16.0,
                        name="prefill_gqa_b1h16x8s2048d256")


def prefill_mha_d96() -> PrefillCase:
    """bf16 MHA causal prefill at head dim 96: B=1, Hq=Hkv=32, Sq=Skv=2048, scale 1/sqrt(96)."""
    return prefill_case(1, 32, 32, 2048, 2048, 96, True, "bf16", seed=1008, scale=1.0 / math.sqrt(96),
                        name="prefill_mha_b1h32s2048d96")


def prefill_gqa_d32() -> PrefillCase:
    """bf16 GQA causal prefill at head dim 32: the headline prefill's shape
    (B=1, Hq=32, Hkv=8, Sq=Skv=2048) at d=32, scale 1/sqrt(32)."""
    return prefill_case(1, 32, 8, 2048, 2048, 32, True, "bf16", seed=1013, scale=1.0 / math.sqrt(32),
                        name="prefill_gqa_b1h32x8s2048d32")


# --------------------------------------------------------------------------- decode


@dataclass
class DecodeCase:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    max_kv_len: int
    scale: float
    seqlens: np.ndarray  # int32 [B]
    q: np.ndarray = field(repr=False)  # bf16 bits [B,Hq,d]
    kcache: np.ndarray = field(repr=False)  # bf16 bits: [B,max_kv_len,Hkv,d] or pool [P,16,Hkv,d]
    vcache: np.ndarray = field(repr=False)
    block_table: np.ndarray | None = field(default=None, repr=False)  # int32 [B, ceil(max_kv_len/16)]
    fp8: bool = False        # kcache / vcache hold uint8 OCP FP8 E4M3 codes
    k_scale: float = 1.0     # per-tensor scales of an fp8 or int8 cache
    v_scale: float = 1.0
    int8: bool = False       # kcache / vcache hold signed 8-bit integer codes (as uint8 bytes)

    @property
    def paged(self) -> bool:
        return self.block_table is not None

    def total_tokens(self) -> int:
        return int(np.clip(self.seqlens, 0, self.max_kv_len).sum())


def decode_contiguous(B, Hq, Hkv, d, max_kv_len, seqlens=None, seed=7, name=None, poison=False) -> DecodeCase:
    """Contiguous cache [B, max_kv_len, Hkv, d]; q [B,Hq,d]; N(0,1).
    seqlens default to max_kv_len. With poison, slots t >= seqlens[b] hold NaN."""
    q = normal_bf16(seed, 0, (B, Hq, d))
    kc = normal_bf16(seed, 1, (B, max_kv_len, Hkv, d))
    vc = normal_bf16(seed, 2, (B, max_kv_len, Hkv, d))
    if seqlens is None:
        seqlens = np.full((B,), max_kv_len, dtype=np.int32)
    seqlens = np.asarray(seqlens, dtype=np.int32)
    if poison:
        for b in range(B):
            L = max(0, min(int(seqlens[b]), max_kv_len))
            kc[b, L:] = BF16_NAN
            vc[b, L:] = BF16_NAN
    if name is None:
        name = f"decode_contig_b{B}h{Hq}x{Hkv}kv{max_kv_len}d{d}"
    return DecodeCase(name, B, Hq, Hkv, d, int(max_kv_len), 1.0 / math.sqrt(d), seqlens, q, kc, vc, None)


def decode_paged(B, Hq, Hkv, d, seqlens, max_kv_len, seed=11, slack_pages=7, name=None, poison=False) -> DecodeCase:
    """Shared page pool [P, 16, Hkv, d] with P = sum ceil(len_b/16) + slack pages.
    The pool order is a seeded random permutation: sequence b owns
    perm[off_b : off_b + ceil(len_b/16)]. Unused block-table entries point at the
    first slack page. With poison, tail slots past len_b and all slack pages are NaN."""
    seqlens = np.asarray(seqlens, dtype=np.int32)
    npages = [(int(min(max(L, 0), max_kv_len)) + PAGE - 1) // PAGE for L in seqlens]
    used = sum(npages)
    P = used + max(1, slack_pages)
    perm = rng(seed, 3).permutation(P).astype(np.int32)
    q = normal_bf16(seed, 0, (B, Hq, d))
    kp = normal_bf16(seed, 1, (P, PAGE, Hkv, d))
    vp = normal_bf16(seed, 2, (P, PAGE, Hkv, d))
    pps = (max_kv_len + PAGE - 1) // PAGE
    slack0 = int(perm[used])
    bt = np.full((B, pps), slack0, dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, : npages[b]] = perm[off : off + npages[b]]
        off += npages[b]
    if poison:
        for s in perm[used:]:
            kp[s] = BF16_NAN
            vp[s] = BF16_NAN
        for b in range(B):
            L = int(min(max(seqlens[b], 0), max_kv_len))
            if L % PAGE and npages[b]:
                last = bt[b, npages[b] - 1]
                kp[last, L % PAGE :] = BF16_NAN
                vp[last, L % PAGE :] = BF16_NAN
    if name is None:
        name = f"decode_paged_b{B}h{Hq}x{Hkv}d{d}"
    return DecodeCase(name, B, Hq, Hkv, d, int(max_kv_len), 1.0 / math.sqrt(d), seqlens, q, kp, vp, bt)


def decode_contig_32k() -> DecodeCase:
    """Contiguous decode: B=4, Hq=32, Hkv=8, 32768 cached tokens each, d=128."""
    return decode_contiguous(4, 32, 8, 128, 32768, seed=1003, name="decode_contig_b4h32x8kv32768d128")


def paged_lengths(seed: int, B: int, lo: int, hi: int) -> np.ndarray:
    """Integer lengths uniform on [lo, hi], both ends inclusive."""
    return rng(seed, 4).integers(lo, hi + 1, size=B).astype(np.int32)


def decode_paged_mixed(poison=False) -> DecodeCase:
    """Paged decode: B=8, Hq=32, Hkv=8, d=128, lengths U{1024..16384}, page 16, shuffled pool."""
    lens = paged_lengths(1004, 8, 1024, 16384)
    return decode_paged(8, 32, 8, 128, lens, 16384, seed=1004, name="decode_paged_b8h32x8kv1k16kd128", poison=poison)


def decode_long_256k(poison=False) -> DecodeCase:
    """Long-context paged decode: B=1, Hq=16, Hkv=2, d=128, 262144 tokens, shuffled pages."""
    return decode_paged(1, 16, 2, 128, np.array([262144], dtype=np.int32), 262144, seed=1005,
                        name="decode_long_b1h16x2kv256kd128", poison=poison)


def decode_paged_d256(poison=False) -> DecodeCase:
    """Decode at head dim 256: B=4, Hq=16, Hkv=8, mixed lengths U{1024..16384},
    page 16, shuffled pool (GQA with two query heads per kv head)."""
    return decode_paged(4, 16, 8, 256, paged_lengths(1009, 4, 1024, 16384), 16384, seed=1009,
                        name="decode_paged_b4h16x8kv1k16kd256", poison=poison)


def decode_batch_short(poison=False) -> DecodeCase:
    """A serving batch of short contexts: B=64, Hq=32, Hkv=8, d=128, lengths
    U{256..1024}, capacity 1024, page 16, shuffled pool. 512 (sequence, kv
    head) pairs: the default split size gives one split per sequence, so
    decode runs in one launch."""
    lens = rng(1011, 21).integers(256, 1025, size=64).astype(np.int32)
    return decode_paged(64, 32, 8, 128, lens, 1024, seed=1011, name="decode_batch_b64h32x8kv256to1kd128",
                        poison=poison)


def decode_b1_chat(poison=False) -> DecodeCase:
    """One sequence of a chat-length context: B=1, Hq=32, Hkv=8, d=128, 4096
    cached tokens, page 16, shuffled pool (the latency case of decode)."""
    return decode_paged(1, 32, 8, 128, np.array([4096], np.int32), 4096, seed=1012,
                        name="decode_b1h32x8kv4kd128", poison=poison)


def decode_paged_hd(d: int, poison=False) -> DecodeCase:
    """Decode at a further head dim d (32 or 96): the head-dim-256 workload's
    shape and lengths (B=4, Hq=16, Hkv=8, lengths drawn U{1024..16384} with
    its seed), other values, page 16, shuffled pool."""
    return decode_paged(4, 16, 8, d, paged_lengths(1009, 4, 1024, 16384), 16384, seed=1010 + d,
                        name=f"decode_paged_b4h16x8kv1k16kd{d}", poison=poison)


def paged_from_contiguous(case: DecodeCase, seed: int = 99) -> DecodeCase:
    """Scatter a contiguous cache into a shuffled page pool (same values, same
    lengths): the paged view of exactly the same data."""
    assert not case.paged and case.max_kv_len % PAGE == 0
    B, L = case.B, case.max_kv_len
    pps = L // PAGE
    P = B * pps
    perm = rng(seed, 5).permutation(P).astype(np.int32)
    bt = perm.reshape(B, pps)
    kp = np.empty((P, PAGE, case.Hkv, case.d), dtype=case.kcache.dtype)
    vp = np.empty_like(kp)
    kp[bt.reshape(-1)] = case.kcache.reshape(B * pps, PAGE, case.Hkv, case.d)
    vp[bt.reshape(-1)] = case.vcache.reshape(B * pps, PAGE, case.Hkv, case.d)
    return DecodeCase(case.name + "_paged", case.B, case.Hq, case.Hkv, case.d, L, case.scale,
                      case.seqlens.copy(), case.q, kp, vp, bt, case.fp8, case.k_scale, case.v_scale, case.int8)


# --------------------------------------------------------------------------- chunked prefill over a KV cache


@dataclass
class PrefillCacheCase:
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    d: int
    max_kv_len: int
    scale: float
    causal: bool
    seqlens: np.ndarray  # int32 [B]: cached tokens, the Sq new ones included
    q: np.ndarray = field(repr=False)  # bf16 bits [B, Hq, Sq, d]
    kcache: np.ndarray = field(repr=False)  # decode layouts (contiguous or page pool)
    vcache: np.ndarray = field(repr=False)
    block_table: np.ndarray | None = field(default=None, repr=False)

    @property
    def paged(self) -> bool:
        return self.block_table is not None


def prefill_cache_case(B, Hq, Hkv, Sq, d, seqlens, max_kv_len, paged=True, causal=True, seed=13, name=None,
                       poison=False) -> PrefillCacheCase:
    """Sq new queries per sequence (N(0,1), bf16) over a cache built like the
    decode caches (same generators, same seed): contiguous [B, max_kv_len,
    Hkv, d] or a shuffled pool of 16-token pages. With poison, slots past each
    length and the slack pages hold NaN."""
    seqlens = np.asarray(seqlens, dtype=np.int32)
    if paged:
        dc = decode_paged(B, Hq, Hkv, d, seqlens, max_kv_len, seed=seed, poison=poison)
    else:
        dc = decode_contiguous(B, Hq, Hkv, d, max_kv_len, seqlens=seqlens, seed=seed, poison=poison)
    q = normal_bf16(seed, 8, (B, Hq, Sq, d))
    if name is None:
        name = f"prefill_cache_b{B}h{Hq}x{Hkv}sq{Sq}kv{max_kv_len}d{d}{'_paged' if paged else ''}"
    return PrefillCacheCase(name, B, Hq, Hkv, Sq, d, int(max_kv_len), 1.0 / math.sqrt(d), bool(causal), seqlens, q,
                            dc.kcache, dc.vcache, dc.block_table)


def prefill_cache_chunk512() -> PrefillCacheCase:
    """Chunked prefill: B=4, Hq=32, Hkv=8, d=128, a chunk of 512 new tokens per
    sequence, cached lengths (chunk included) U{2048..16384}, page 16, shuffled
    pool, causal."""
    lens = paged_lengths(1006, 4, 2048, 16384)
    return prefill_cache_case(4, 32, 8, 512, 128, lens, 16384, paged=True, causal=True, seed=1006,
                              name="prefill_cache_b4h32x8sq512kv2k16kd128")


# --------------------------------------------------------------------------- fp8 KV cache

FP8_NAN = 0x7F  # an OCP FP8 E4M3 NaN code


def fp8_codes(seed: int, stream: int, shape) -> np.ndarray:
    """Random OCP FP8 E4M3 codes (uint8), drawn as bit fields: sign uniform,
    biased exponent field 3..8 with weights 1:2:4:6:5:2 (magnitudes 1/16 ..
    3.75, most near 1/2 .. 2), mantissa field uniform 0..7, and 1 % zero codes.
    Never a NaN code (exponent field 15 is not drawn)."""
    g = rng(seed, stream)
    n = int(np.prod(shape))
    sign = g.integers(0, 2, size=n, dtype=np.uint8)
    w = np.array([1, 2, 4, 6, 5, 2], dtype=np.float64)
    expo = (3 + g.choice(6, size=n, p=w / w.sum())).astype(np.uint8)
    mant = g.integers(0, 8, size=n, dtype=np.uint8)
    codes = (sign << 7) | (expo << 3) | mant
    codes[g.random(n) < 0.01] = 0
    return codes.reshape(shape).astype(np.uint8)


def as_fp8(case: DecodeCase, k_scale: float = 0.35, v_scale: float = 0.6, seed: int | None = None) -> DecodeCase:
    """The same decode case (q, lengths, block table) over an FP8 E4M3 cache of
    random codes with per-tensor scales; slots that hold NaN in the bf16 cache
    (poisoned tails and pages) hold the NaN code."""
    sd = (zlib.crc32(case.name.encode()) % 100000) if seed is None else seed
    kc = fp8_codes(sd, 6, case.kcache.shape)
    vc = fp8_codes(sd, 7, case.vcache.shape)
    kc[case.kcache == BF16_NAN] = FP8_NAN
    vc[case.vcache == BF16_NAN] = FP8_NAN
    return DecodeCase(case.name + "_fp8", case.B, case.Hq, case.Hkv, case.d, case.max_kv_len, case.scale,
                      case.seqlens.copy(), case.q, kc, vc, case.block_table, True, float(k_scale), float(v_scale))


# Every finite OCP FP8 E4M3 code: all 256 but the two NaN codes 0x7F and 0xFF.
E4M3_FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def e4m3_codes_by_exponent(lo: int, hi: int) -> np.ndarray:
    """The finite E4M3 codes whose biased exponent field (bits 6..3) is in
    [lo, hi], both signs: field 0 holds the zeros and the subnormals, field 15
    the largest binade (up to 448)."""
    e = (E4M3_FINITE >> 3) & 0xF
    return E4M3_FINITE[(e >= lo) & (e <= hi)]


def fp8_every_code(case: DecodeCase, codes: np.ndarray, k_scale: float, v_scale: float, seed: int) -> DecodeCase:
    """The same contiguous decode case (q, lengths) over an FP8 E4M3 cache whose
    codes are drawn uniformly from ``codes``; every one of ``codes`` is also
    placed, in a random order, among the first valid tokens of sequence 0 of
    both K and V, so each appears where it is read. Slots past each length hold
    the NaN code."""
    assert not case.paged
    codes = np.asarray(codes, dtype=np.uint8)
    B, L, Hkv, d = case.kcache.shape
    per_tok = Hkv * d
    ntok = -(-len(codes) // per_tok)
    assert int(case.seqlens[0]) >= ntok, "sequence 0 must hold one copy of every code"
    out = []
    for stream in (6, 7):
        g = rng(seed, stream)
        c = codes[g.integers(0, len(codes), size=case.kcache.shape)]
        first = c[0, :ntok].reshape(-1)
        first[: len(codes)] = g.permutation(codes)
        c[0, :ntok] = first.reshape(ntok, Hkv, d)
        for b in range(B):
            c[b, max(0, min(int(case.seqlens[b]), L)):] = FP8_NAN
        out.append(c)
    return DecodeCase(case.name + "_fp8codes", case.B, case.Hq, case.Hkv, case.d, case.max_kv_len, case.scale,
                      case.seqlens.copy(), case.q, out[0], out[1], None, True, float(k_scale), float(v_scale))


# --------------------------------------------------------------------------- int8 KV cache

INT8_POISON = 0x7F  # the largest code (127): garbage of the largest magnitude in slots past a length


def int8_codes(seed: int, stream: int, shape) -> np.ndarray:
    """Random signed 8-bit codes, stored as uint8 bytes (two's complement):
    uniform over all 256 values, -128..127."""
    return rng(seed, stream).integers(0, 256, size=int(np.prod(shape)), dtype=np.uint8).reshape(shape)


def as_int8(case: DecodeCase, k_scale: float = 1.0 / 64, v_scale: float = 0.02, seed: int | None = None) -> DecodeCase:
    """The same decode case (q, lengths, block table) over an INT8 cache of
    random codes with per-tensor scales; slots that hold NaN in the bf16 cache
    (poisoned tails and pages) hold the code 127."""
    sd = (zlib.crc32(case.name.encode()) % 100000) if seed is None else seed
    kc = int8_codes(sd, 10, case.kcache.shape)
    vc = int8_codes(sd, 11, case.vcache.shape)
    kc[case.kcache == BF16_NAN] = INT8_POISON
    vc[case.vcache == BF16_NAN] = INT8_POISON
    return DecodeCase(case.name + "_int8", case.B, case.Hq, case.Hkv, case.d, case.max_kv_len, case.scale,
                      case.seqlens.copy(), case.q, kc, vc, case.block_table, False, float(k_scale), float(v_scale),
                      True)

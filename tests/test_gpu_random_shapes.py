"""Seeded random shapes through every entry point, each compared element by
element with the fp64 oracle: prefill (bf16 and fp32) at every head dim,
chunked prefill over a paged or contiguous cache, and decode over bf16, FP8
and INT8 caches. The shapes are drawn once from fixed seeds (so each case has
a stable id) over the ranges the kernels take: head groups up to 32 (two head
chunks in decode), Sq not a tile multiple, Sq < Skv and Sq > Skv, empty and
full sequences, explicit and default split sizes. They reach combinations of
grid size, tile count and split plan that the named cases do not.
"""
import numpy as np
import pytest

import attention_fa_prefill_amd as fa
import oracle
import workloads
from tests.gpu_util import assert_bf16_close, assert_f32_close, dev_bf16, dev_f32, dev_i32, host_f64, torch_gpu

pytestmark = pytest.mark.gpu

HEAD_DIMS = (32, 64, 96, 128, 256)


def draw_prefill(i, dtype):
    r = np.random.default_rng(7100 + i + (1000 if dtype == "f32" else 0))
    d = HEAD_DIMS[i % len(HEAD_DIMS)]
    B = int(r.integers(1, 4))
    Hkv = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 2, 3, 4, 8]))
    causal = bool(r.integers(0, 2))
    Sq = int(r.integers(1, 401))
    Skv = int(r.integers(Sq, Sq + 401)) if causal else int(r.integers(1, 701))
    return (B, G * Hkv, Hkv, Sq, Skv, d, causal)


PREFILL_BF16 = [draw_prefill(i, "bf16") for i in range(30)]
PREFILL_F32 = [draw_prefill(i, "f32") for i in range(10)]


def pid(s):
    return "b{}h{}x{}sq{}skv{}d{}{}".format(*s[:6], "c" if s[6] else "")


@pytest.mark.parametrize("shape", PREFILL_BF16, ids=pid)
def test_prefill_bf16_random(shape):
    B, Hq, Hkv, Sq, Skv, d, causal = shape
    torch_gpu()
    case = workloads.prefill_case(B, Hq, Hkv, Sq, Skv, d, causal, "bf16", seed=hash(shape) % 100000)
    print(f"case {case.name} causal={causal}", flush=True)
    o = fa.prefill(dev_bf16(case.q), dev_bf16(case.k), dev_bf16(case.v), causal=causal, scale=case.scale)
    ref, _ = oracle.attention(*case.as_f64(), case.scale, causal)
    assert_bf16_close(host_f64(o), ref, case.name)


@pytest.mark.parametrize("shape", PREFILL_F32, ids=pid)
def test_prefill_f32_random(shape):
    B, Hq, Hkv, Sq, Skv, d, causal = shape
    torch_gpu()
    case = workloads.prefill_case(B, Hq, Hkv, Sq, Skv, d, causal, "f32", seed=hash(shape) % 100000)
    print(f"case {case.name} causal={causal}", flush=True)
    o = fa.prefill(dev_f32(case.q), dev_f32(case.k), dev_f32(case.v), causal=causal, scale=case.scale)
    ref, _ = oracle.attention(*case.as_f64(), case.scale, causal)
    assert_f32_close(host_f64(o), ref, case.name)


def draw_cache(i):
    r = np.random.default_rng(7300 + i)
    d = HEAD_DIMS[i % len(HEAD_DIMS)]
    B = int(r.integers(1, 5))
    Hkv = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 2, 4, 8]))
    Sq = int(r.integers(1, 301))
    lens = r.integers(0, 1501, size=B)
    lens[r.integers(0, B)] = int(r.integers(Sq, 1501))  # at least one sequence holds all its queries
    mkl = int(lens.max()) + int(r.integers(0, 40))
    return (B, G * Hkv, Hkv, Sq, d, [int(x) for x in lens], max(mkl, 1), bool(r.integers(0, 2)),
            bool(r.integers(0, 2)))


CACHE = [draw_cache(i) for i in range(16)]


@pytest.mark.parametrize("shape", CACHE, ids=lambda s: "b{}h{}x{}sq{}d{}kv{}{}{}".format(
    *s[:5], s[6], "_paged" if s[7] else "", "c" if s[8] else ""))
def test_prefill_cache_random(shape):
    B, Hq, Hkv, Sq, d, lens, mkl, paged, causal = shape
    torch_gpu()
    case = workloads.prefill_cache_case(B, Hq, Hkv, Sq, d, lens, mkl, paged=paged, causal=causal,
                                        seed=hash(tuple(lens)) % 100000)
    print(f"case {case.name} causal={causal} lens={lens}", flush=True)
    o = fa.prefill_cache(dev_bf16(case.q), dev_bf16(case.kcache), dev_bf16(case.vcache), dev_i32(case.seqlens),
                         block_table=dev_i32(case.block_table) if paged else None, max_kv_len=mkl, causal=causal,
                         scale=case.scale)
    ref = oracle.prefill_cache(workloads.bf16_bits_to_f64(case.q), workloads.bf16_bits_to_f64(case.kcache),
                               workloads.bf16_bits_to_f64(case.vcache), case.seqlens, case.scale, causal,
                               block_table=case.block_table, max_kv_len=mkl)
    assert_bf16_close(host_f64(o), ref, case.name)


def draw_decode(i):
    r = np.random.default_rng(7500 + i)
    fmt = ("bf16", "fp8", "int8")[i % 3]
    d = HEAD_DIMS[(i // 3) % len(HEAD_DIMS)]
    B = int(r.integers(1, 41))
    Hkv = int(r.choice([1, 2, 4, 8]))
    G = int(r.choice([1, 2, 4, 5, 8, 16, 17, 32]))
    mkl = int(r.integers(1, 3001))
    # at most 2^24 cached elements per cache, so the host side stays quick
    mkl = max(1, min(mkl, (1 << 24) // (B * Hkv * d)))
    lens = r.integers(0, mkl + 1, size=B)
    if B > 2:
        lens[0], lens[1] = 0, mkl
    tps = int(r.choice([0, 0, 32, 64, 256, 1024]))
    return (fmt, B, G * Hkv, Hkv, d, mkl, [int(x) for x in lens], tps, bool(r.integers(0, 2)))


DECODE = [draw_decode(i) for i in range(36)]


@pytest.mark.parametrize("shape", DECODE, ids=lambda s: "{}_b{}h{}x{}d{}kv{}_tps{}{}".format(
    s[0], *s[1:6], s[7], "_paged" if s[8] else ""))
def test_decode_random(shape):
    fmt, B, Hq, Hkv, d, mkl, lens, tps, paged = shape
    torch = torch_gpu()
    seed = hash(tuple(lens)) % 100000
    if paged:
        case = workloads.decode_paged(B, Hq, Hkv, d, np.array(lens, np.int32), mkl, seed=seed)
    else:
        case = workloads.decode_contiguous(B, Hq, Hkv, d, mkl, seqlens=np.array(lens, np.int32), seed=seed)
    if fmt == "fp8":
        case = workloads.as_fp8(case)
    elif fmt == "int8":
        case = workloads.as_int8(case)
    print(f"case {fmt} {case.name} tps={tps} lens={lens[:8]}", flush=True)
    q = dev_bf16(case.q)
    bt = dev_i32(case.block_table) if paged else None
    seq = dev_i32(case.seqlens)
    if fmt == "bf16":
        o = fa.decode(q, dev_bf16(case.kcache), dev_bf16(case.vcache), seq, block_table=bt, max_kv_len=mkl,
                      scale=case.scale, tokens_per_split=tps)
        ref, _ = oracle.decode(*(workloads.bf16_bits_to_f64(x) for x in (case.q, case.kcache, case.vcache)),
                               case.seqlens, case.scale, block_table=case.block_table, max_kv_len=mkl)
    else:
        kc = torch.from_numpy(np.ascontiguousarray(case.kcache, dtype=np.uint8)).to("cuda")
        vc = torch.from_numpy(np.ascontiguousarray(case.vcache, dtype=np.uint8)).to("cuda")
        run = fa.decode_fp8 if fmt == "fp8" else fa.decode_int8
        o = run(q, kc, vc, seq, k_scale=case.k_scale, v_scale=case.v_scale, block_table=bt, max_kv_len=mkl,
                scale=case.scale, tokens_per_split=tps)
        ref_fn = oracle.decode_fp8 if fmt == "fp8" else oracle.decode_int8
        ref, _ = ref_fn(workloads.bf16_bits_to_f64(case.q), case.kcache, case.vcache, case.seqlens, case.scale,
                        case.k_scale, case.v_scale, block_table=case.block_table, max_kv_len=mkl)
    got = host_f64(o)
    empty = np.asarray(lens) == 0
    assert np.all(got[empty] == 0.0)
    assert_bf16_close(got, ref, case.name)

"""GPU parity of fa_prefill_cache (chunked prefill over a contiguous or paged
KV cache) against the fp64 oracle, every output element; bitwise checks
against fa_prefill and between the paged and contiguous caches."""
import dataclasses

import numpy as np
import pytest

import attention_fa_prefill_amd as fa
import oracle
import workloads
from tests.gpu_util import assert_bf16_close, dev_bf16, dev_i32, host_bits, host_f64, torch_gpu

pytestmark = pytest.mark.gpu


def run(case):
    torch_gpu()
    print(f"case {case.name} causal={case.causal} lens={case.seqlens.tolist()[:8]}", flush=True)
    return fa.prefill_cache(dev_bf16(case.q), dev_bf16(case.kcache), dev_bf16(case.vcache), dev_i32(case.seqlens),
                            block_table=dev_i32(case.block_table) if case.paged else None,
                            max_kv_len=case.max_kv_len, causal=case.causal, scale=case.scale)


def oracle_out(case):
    return oracle.prefill_cache(workloads.bf16_bits_to_f64(case.q), workloads.bf16_bits_to_f64(case.kcache),
                                workloads.bf16_bits_to_f64(case.vcache), case.seqlens, case.scale, case.causal,
                                block_table=case.block_table, max_kv_len=case.max_kv_len)


def test_chunk512_full_size():
    case = workloads.prefill_cache_chunk512()
    assert_bf16_close(host_f64(run(case)), oracle_out(case), case.name)


SHAPES = [
    # B, Hq, Hkv, Sq, d, lens, max_kv_len, paged, causal
    (2, 8, 2, 128, 128, [1000, 129], 1024, True, True),
    (3, 4, 1, 200, 128, [200, 1500, 333], 1536, True, True),     # MQA, Sq not a tile multiple
    (2, 4, 4, 300, 64, [700, 301], 704, False, True),
    (1, 16, 2, 640, 128, [4000], 4096, True, True),               # 5 query tiles
    (2, 2, 1, 256, 128, [100, 0], 256, True, True),               # L < Sq and L = 0: zero rows
    (2, 8, 2, 96, 128, [50, 1000], 1024, False, False),           # non-causal
    (4, 4, 2, 64, 64, [64, 65, 1, 17], 80, True, False),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b{}h{}x{}sq{}d{}kv{}{}{}".format(
    s[0], s[1], s[2], s[3], s[4], s[6], "p" if s[7] else "c", "c" if s[8] else "n"))
def test_shapes(shape):
    B, Hq, Hkv, Sq, d, lens, mkl, paged, causal = shape
    case = workloads.prefill_cache_case(B, Hq, Hkv, Sq, d, lens, mkl, paged=paged, causal=causal,
                                        seed=sum(lens) % 1000 + Sq)
    got = host_f64(run(case))
    ref = oracle_out(case)
    assert_bf16_close(got, ref, case.name)
    for b, L in enumerate(lens):  # rows that see no key are exactly zero
        if causal and L < Sq:
            assert np.all(got[b, :, : Sq - L] == 0.0)
        if L == 0:
            assert np.all(got[b] == 0.0)


@pytest.mark.parametrize("d", [128, 96, 32])
def test_full_cache_matches_prefill(d):
    """A contiguous cache holding exactly prefill's K and V (every length =
    max_kv_len = Skv): fa_prefill_cache agrees with fa_prefill. The two split
    a tile's keys differently between the halves of a work-group (one tile
    per work-group here, pairs of tiles there), so the agreement is to
    rounding, not bitwise; both are also held to the oracle."""
    torch = torch_gpu()
    case = workloads.prefill_cache_case(2, 8, 2, 700, d, [1100, 1100], 1100, paged=False, causal=True,
                                        seed={128: 71, 96: 75, 32: 77}[d])
    o_cache = host_f64(run(case))
    k = dev_bf16(case.kcache).permute(0, 2, 1, 3).contiguous()  # [B, Hkv, Skv, d]
    v = dev_bf16(case.vcache).permute(0, 2, 1, 3).contiguous()
    o_plain = host_f64(fa.prefill(dev_bf16(case.q), k, v, causal=True, scale=case.scale))
    torch.cuda.synchronize()
    ref = oracle_out(case)
    assert_bf16_close(o_cache, ref, "cache")
    assert_bf16_close(o_plain, ref, "plain")
    diff = np.abs(o_cache - o_plain)
    assert diff.max() <= 1e-2 and diff.mean() <= 1e-4


def test_paged_equals_contiguous_bitwise():
    case = workloads.prefill_cache_case(3, 8, 2, 300, 128, [2048, 777, 300], 2048, paged=False, causal=True, seed=72)
    B, L = case.B, case.max_kv_len
    perm = np.random.default_rng(9).permutation(B * (L // 16))
    bt = perm.reshape(B, L // 16).astype(np.int32)
    kp = np.empty((B * (L // 16), 16, case.Hkv, case.d), np.uint16)
    vp = np.empty_like(kp)
    kp[bt.reshape(-1)] = case.kcache.reshape(-1, 16, case.Hkv, case.d)
    vp[bt.reshape(-1)] = case.vcache.reshape(-1, 16, case.Hkv, case.d)
    paged = dataclasses.replace(case, kcache=kp, vcache=vp, block_table=bt, name=case.name + "_paged")
    assert np.array_equal(host_bits(run(case)), host_bits(run(paged)))


def test_poisoned_slots_do_not_leak():
    """NaN past every length and in the unused pages: same bits as clean."""
    lens = [1000, 17, 512]
    clean = workloads.prefill_cache_case(3, 4, 2, 256, 128, lens, 1024, paged=True, seed=73)
    dirty = workloads.prefill_cache_case(3, 4, 2, 256, 128, lens, 1024, paged=True, seed=73, poison=True)
    o_dirty = run(dirty)
    assert np.all(np.isfinite(host_f64(o_dirty)))
    assert np.array_equal(host_bits(o_dirty), host_bits(run(clean)))


@pytest.mark.parametrize("B", [37, 600])
def test_many_sequences_mixed_lengths(B):
    """Many short sequences with mixed lengths (zeros included): up to 512
    sequences the work-groups order them by length; beyond, by index. Either
    way every (tile, head, sequence) is computed once."""
    lens = np.random.default_rng(B).integers(0, 200, size=B).astype(np.int32)
    case = workloads.prefill_cache_case(B, 2, 1, 40, 64, lens, 208, paged=True, causal=True, seed=B)
    got = host_f64(run(case))
    assert_bf16_close(got, oracle_out(case), f"B={B}")
    assert np.all(got[lens == 0] == 0.0)


# ---------------------------------------------------------------- head dims 32, 96, 256
SHAPES_HD = [
    # B, Hq, Hkv, Sq, d, lens, max_kv_len, paged, causal
    (2, 8, 2, 128, 96, [1000, 129], 1024, True, True),
    (3, 4, 1, 200, 256, [200, 1500, 333], 1536, True, True),     # MQA, Sq not a tile multiple
    (2, 4, 4, 300, 32, [700, 301], 704, False, True),
    (1, 16, 8, 640, 256, [3000], 3008, True, True),
    (2, 2, 1, 256, 96, [100, 0], 256, True, True),                # L < Sq and L = 0: zero rows
    (2, 8, 2, 96, 256, [50, 1000], 1024, False, False),           # non-causal
    (4, 4, 2, 64, 32, [64, 65, 1, 17], 80, True, False),
    (2, 12, 12, 333, 96, [2000, 333], 2048, True, True),
]


@pytest.mark.parametrize("shape", SHAPES_HD, ids=lambda s: "b{}h{}x{}sq{}d{}kv{}{}{}".format(
    s[0], s[1], s[2], s[3], s[4], s[6], "p" if s[7] else "c", "c" if s[8] else "n"))
def test_head_dim_shapes(shape):
    B, Hq, Hkv, Sq, d, lens, mkl, paged, causal = shape
    case = workloads.prefill_cache_case(B, Hq, Hkv, Sq, d, lens, mkl, paged=paged, causal=causal,
                                        seed=sum(lens) % 1000 + Sq + d)
    got = host_f64(run(case))
    assert_bf16_close(got, oracle_out(case), case.name)
    for b, L in enumerate(lens):
        if causal and L < Sq:
            assert np.all(got[b, :, : Sq - L] == 0.0)
        if L == 0:
            assert np.all(got[b] == 0.0)


@pytest.mark.parametrize("d", [32, 96, 256])
def test_head_dim_paged_equals_contiguous_bitwise(d):
    case = workloads.prefill_cache_case(2, 8, 4, 200, d, [1024, 555], 1024, paged=False, causal=True, seed=80 + d)
    B, L = case.B, case.max_kv_len
    perm = np.random.default_rng(10).permutation(B * (L // 16))
    bt = perm.reshape(B, L // 16).astype(np.int32)
    kp = np.empty((B * (L // 16), 16, case.Hkv, case.d), np.uint16)
    vp = np.empty_like(kp)
    kp[bt.reshape(-1)] = case.kcache.reshape(-1, 16, case.Hkv, case.d)
    vp[bt.reshape(-1)] = case.vcache.reshape(-1, 16, case.Hkv, case.d)
    paged = dataclasses.replace(case, kcache=kp, vcache=vp, block_table=bt, name=case.name + "_paged")
    assert np.array_equal(host_bits(run(case)), host_bits(run(paged)))


@pytest.mark.parametrize("d", [96, 256])
def test_head_dim_poisoned_slots_do_not_leak(d):
    lens = [1000, 17, 512]
    clean = workloads.prefill_cache_case(3, 4, 2, 256, d, lens, 1024, paged=True, seed=74 + d)
    dirty = workloads.prefill_cache_case(3, 4, 2, 256, d, lens, 1024, paged=True, seed=74 + d, poison=True)
    o_dirty = run(dirty)
    assert np.all(np.isfinite(host_f64(o_dirty)))
    assert np.array_equal(host_bits(o_dirty), host_bits(run(clean)))

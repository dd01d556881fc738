"""GPU parity of fa_decode_int8: decode over a KV cache of signed 8-bit
integers with one scale per tensor (the INT8 KV cache of the FasterTransformer
walkthrough, section 3.3), through the C ABI, against the fp64 oracle
(oracle.decode_int8, pinned in test_oracle_int8.py).

With power-of-two scales every dequantised value is a bf16 value and the
scales fold exactly, so the int8 path must also equal fa_decode over the
dequantised bf16 cache bit for bit.
"""
import numpy as np
import pytest

import attention_fa_prefill_amd as fa
import oracle
import workloads
from tests.gpu_util import assert_bf16_close, dev_bf16, dev_i32, host_bits, host_f64, torch_gpu

pytestmark = pytest.mark.gpu


def dev_u8(codes):
    torch = torch_gpu()
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).to("cuda")


def run_int8(case, tps=0):
    torch_gpu()
    print(f"case {case.name} paged={case.paged} tps={tps} ks={case.k_scale} vs={case.v_scale}", flush=True)
    q, kc, vc = dev_bf16(case.q), dev_u8(case.kcache), dev_u8(case.vcache)
    bt = dev_i32(case.block_table) if case.paged else None
    return fa.decode_int8(q, kc, vc, dev_i32(case.seqlens), k_scale=case.k_scale, v_scale=case.v_scale,
                          block_table=bt, max_kv_len=case.max_kv_len, scale=case.scale, tokens_per_split=tps)


def oracle_out(case):
    q = workloads.bf16_bits_to_f64(case.q)
    o, _ = oracle.decode_int8(q, case.kcache, case.vcache, case.seqlens, case.scale, case.k_scale, case.v_scale,
                              block_table=case.block_table, max_kv_len=case.max_kv_len)
    return o


def bf16_path_on_dequantised(case):
    """fa_decode over the dequantised cache (exact in bf16 for power-of-two scales)."""
    deq_k = workloads.f32_to_bf16_bits((oracle.int8_to_f64(case.kcache) * case.k_scale).astype(np.float32))
    deq_v = workloads.f32_to_bf16_bits((oracle.int8_to_f64(case.vcache) * case.v_scale).astype(np.float32))
    bt = dev_i32(case.block_table) if case.paged else None
    return fa.decode(dev_bf16(case.q), dev_bf16(deq_k), dev_bf16(deq_v), dev_i32(case.seqlens), block_table=bt,
                     max_kv_len=case.max_kv_len, scale=case.scale)


@pytest.mark.parametrize("make", [workloads.decode_contig_32k, workloads.decode_paged_mixed,
                                  workloads.decode_long_256k])
def test_int8_full_size(make):
    case = workloads.as_int8(make())
    assert_bf16_close(host_f64(run_int8(case)), oracle_out(case), case.name)


def test_int8_equals_bf16_on_the_dequantised_cache():
    case = workloads.as_int8(workloads.decode_paged_mixed(), k_scale=2.0 ** -6, v_scale=2.0 ** -5)
    assert np.array_equal(host_bits(run_int8(case)), host_bits(bf16_path_on_dequantised(case)))


def test_int8_paged_equals_contiguous_bitwise():
    case = workloads.as_int8(workloads.decode_contiguous(4, 16, 4, 128, 4096, seed=62))
    paged = workloads.paged_from_contiguous(case)
    assert paged.int8
    assert np.array_equal(host_bits(run_int8(case)), host_bits(run_int8(paged)))


@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_int8_every_code(paged):
    """All 256 codes appear among the tokens read, in K and in V (uniform
    draws; the test asserts it), with scales that keep the scores of order 1."""
    base = workloads.decode_contiguous(4, 8, 2, 128, 2048, seqlens=np.array([700, 2048, 33, 1500], np.int32),
                                       seed=85)
    case = workloads.as_int8(base, k_scale=2.0 ** -6, v_scale=2.0 ** -6, seed=86)
    for cache in (case.kcache, case.vcache):
        seen = set()
        for b in range(case.B):
            seen |= set(np.unique(cache[b, : int(case.seqlens[b])]).tolist())
        assert seen == set(range(256))
    if paged:
        case = workloads.paged_from_contiguous(case)
    o = run_int8(case)
    assert_bf16_close(host_f64(o), oracle_out(case), f"{case.name} every code")
    assert np.array_equal(host_bits(o), host_bits(bf16_path_on_dequantised(case)))


@pytest.mark.parametrize("vs", [1.0, 2.0 ** -7])
def test_int8_single_token_gives_every_v_code_exactly(vs):
    """With one cached token its softmax weight is exactly 1, so each output row
    is v_scale * code of that token's V row; the two sequences' V rows hold all
    256 codes, checked value for value against two's complement."""
    base = workloads.decode_contiguous(2, 4, 1, 128, 16, seqlens=np.ones(2, np.int32), seed=87)
    case = workloads.as_int8(base, k_scale=0.5, v_scale=vs, seed=88)
    row_codes = workloads.rng(88, 9).permutation(np.arange(256)).astype(np.uint8)
    case.vcache[:, 0, 0, :] = row_codes.reshape(2, 128)
    got = host_f64(run_int8(case, 32))
    want = (row_codes.view(np.int8).astype(np.float64).reshape(2, 1, 128) * vs).repeat(4, axis=1)
    assert np.array_equal(got, want)
    assert np.array_equal(got, oracle_out(case))


@pytest.mark.parametrize("G,Hkv,d", [(1, 4, 128), (4, 2, 64), (8, 1, 128), (32, 1, 128), (2, 4, 256)])
@pytest.mark.parametrize("tps", [0, 32, 1024])
def test_int8_head_groups_and_split_sizes(G, Hkv, d, tps):
    lens = np.array([1, 16, 200, 1500], np.int32)
    case = workloads.as_int8(workloads.decode_paged(4, G * Hkv, Hkv, d, lens, 1536, seed=G * 100 + d + tps + 9))
    assert_bf16_close(host_f64(run_int8(case, tps)), oracle_out(case), f"{case.name} G={G} tps={tps}")


@pytest.mark.parametrize("ks,vs,scale", [(0.002, 0.05, None), (0.05, 0.002, None), (1.0 / 64, 0.02, -0.09),
                                         (1.0 / 64, 1.0 / 64, 0.0)])
def test_int8_scales(ks, vs, scale):
    """Small and large K and V scales (codes reach 127, so the scales keep V
    of the order of the bf16 bar's data), a negative softmax scale, and scale
    0 (uniform weights)."""
    base = workloads.decode_paged(3, 8, 2, 128, np.array([700, 33, 1], np.int32), 768, seed=72)
    case = workloads.as_int8(base, k_scale=ks, v_scale=vs)
    if scale is not None:
        case.scale = scale
    assert_bf16_close(host_f64(run_int8(case, 64)), oracle_out(case), f"ks={ks} vs={vs} scale={scale}")


def test_int8_poisoned_slots_do_not_leak():
    """Code 127 in every slot past each length and in the unused pages: the
    output equals the unpoisoned run bit for bit (those rows are never read)."""
    lens = np.array([1, 15, 16, 17, 31, 33, 100, 513], np.int32)
    clean = workloads.as_int8(workloads.decode_paged(8, 8, 2, 128, lens, 640, seed=22), seed=6)
    dirty = workloads.as_int8(workloads.decode_paged(8, 8, 2, 128, lens, 640, seed=22, poison=True), seed=6)
    assert np.sum(dirty.kcache == workloads.INT8_POISON) > np.sum(clean.kcache == workloads.INT8_POISON)
    assert np.array_equal(host_bits(run_int8(dirty)), host_bits(run_int8(clean)))

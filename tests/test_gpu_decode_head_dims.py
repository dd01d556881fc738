"""GPU parity of decode (bf16, FP8 and INT8 caches) and fa_merge_lse at head
dims 32 and 96, the further head dims of the FlashRT-HF-kernels usage
section beyond 64, 128 and 256. At d = 96 (12 chunks of 16 bytes per bf16
row) and d = 32 over one-byte caches the kernel pads its LDS rows to a power
of two; every element is compared with the fp64 oracle.
"""
import numpy as np
import pytest

import attention_fa_prefill_amd as fa
import oracle
import workloads
from tests.gpu_util import F32_MAX_ABS, assert_bf16_close, dev_bf16, dev_f32, dev_i32, host_bits, host_f64, torch_gpu
from tests.test_gpu_decode import oracle_out, oracle_out_fp8, run, run_fp8
from tests.test_gpu_decode_int8 import bf16_path_on_dequantised, oracle_out as oracle_out_int8, run_int8

pytestmark = pytest.mark.gpu

DIMS = [32, 96]


@pytest.mark.parametrize("d", DIMS)
def test_mixed_lengths_workload(d):
    """B=4, Hq=16, Hkv=8, lengths U{1024..16384}, shuffled pages."""
    case = workloads.decode_paged_hd(d)
    assert_bf16_close(host_f64(run(case)), oracle_out(case), case.name)


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("G,Hkv", [(1, 4), (4, 2), (8, 1), (32, 1), (5, 2)])
@pytest.mark.parametrize("tps", [0, 32, 1024])
def test_head_groups_and_split_sizes(d, G, Hkv, tps):
    lens = np.array([1, 16, 200, 1500], np.int32)
    case = workloads.decode_paged(4, G * Hkv, Hkv, d, lens, 1536, seed=G * 100 + d + tps + 11)
    assert_bf16_close(host_f64(run(case, tps)), oracle_out(case), f"{case.name} G={G} tps={tps}")


@pytest.mark.parametrize("d", DIMS)
def test_paged_equals_contiguous_bitwise(d):
    case = workloads.decode_contiguous(4, 16, 4, d, 4096, seqlens=np.array([4096, 1, 3000, 777], np.int32),
                                       seed=63 + d)
    paged = workloads.paged_from_contiguous(case)
    assert np.array_equal(host_bits(run(case)), host_bits(run(paged)))


@pytest.mark.parametrize("d", DIMS)
def test_poisoned_slots_do_not_leak(d):
    lens = np.array([1, 15, 16, 17, 31, 33, 100, 513], np.int32)
    clean = workloads.decode_paged(8, 8, 2, d, lens, 640, seed=23 + d)
    dirty = workloads.decode_paged(8, 8, 2, d, lens, 640, seed=23 + d, poison=True)
    o = run(dirty)
    assert np.all(np.isfinite(host_f64(o)))
    assert np.array_equal(host_bits(o), host_bits(run(clean)))


@pytest.mark.parametrize("d", DIMS)
def test_fp8_cache(d):
    base = workloads.decode_paged(4, 16, 4, d, np.array([1, 700, 2048, 33], np.int32), 2048, seed=64 + d)
    case = workloads.as_fp8(base)
    assert_bf16_close(host_f64(run_fp8(case)), oracle_out_fp8(case), case.name)
    exact = workloads.as_fp8(base, k_scale=0.5, v_scale=0.25)
    deq_k = workloads.f32_to_bf16_bits((oracle.e4m3_to_f64(exact.kcache) * 0.5).astype(np.float32))
    deq_v = workloads.f32_to_bf16_bits((oracle.e4m3_to_f64(exact.vcache) * 0.25).astype(np.float32))
    o16 = fa.decode(dev_bf16(exact.q), dev_bf16(deq_k), dev_bf16(deq_v), dev_i32(exact.seqlens),
                    block_table=dev_i32(exact.block_table), max_kv_len=exact.max_kv_len, scale=exact.scale)
    assert np.array_equal(host_bits(run_fp8(exact)), host_bits(o16))


@pytest.mark.parametrize("d", DIMS)
def test_int8_cache(d):
    base = workloads.decode_paged(4, 16, 4, d, np.array([1, 700, 2048, 33], np.int32), 2048, seed=65 + d)
    case = workloads.as_int8(base)
    assert_bf16_close(host_f64(run_int8(case)), oracle_out_int8(case), case.name)
    exact = workloads.as_int8(base, k_scale=2.0 ** -6, v_scale=2.0 ** -5)
    assert np.array_equal(host_bits(run_int8(exact)), host_bits(bf16_path_on_dequantised(exact)))


@pytest.mark.parametrize("d", DIMS)
def test_byte_caches_paged_equal_contiguous(d):
    base = workloads.decode_contiguous(3, 8, 2, d, 1024, seqlens=np.array([1024, 5, 600], np.int32), seed=66 + d)
    for make, runner in ((workloads.as_fp8, run_fp8), (workloads.as_int8, run_int8)):
        case = make(base)
        assert np.array_equal(host_bits(runner(case)), host_bits(runner(workloads.paged_from_contiguous(case))))


@pytest.mark.parametrize("d", DIMS)
def test_merge_lse(d):
    torch = torch_gpu()
    rng = np.random.default_rng(30 + d)
    R, S = 9, 40
    op = rng.standard_normal((R, S, d)).astype(np.float32)
    ls = (rng.standard_normal((R, S)) * 4).astype(np.float32)
    ls[2, ::3] = -np.inf
    op[2, ::3] = np.nan
    o, lse_out = fa.merge_lse(dev_f32(op), dev_f32(ls), out_dtype=torch.float32)
    ref_o, ref_l = oracle.merge(op.astype(np.float64), ls.astype(np.float64))
    assert np.max(np.abs(host_f64(o) - ref_o)) <= F32_MAX_ABS
    assert np.max(np.abs(host_f64(lse_out) - ref_l)) <= F32_MAX_ABS


@pytest.mark.parametrize("B", [300, 4100])
@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_d32_many_sequences_and_head_chunks(B, fmt):
    """d = 32 (row slices of 64 or 32 bytes: the work-groups of all kv heads
    and head chunks of a split on one XCD) with G = 32 (two head chunks per kv
    head), B above and below the batch that is scanned per work-group, short
    mixed lengths with zeros, poisoned slots."""
    lens = np.random.default_rng(B + 7).integers(0, 97, size=B).astype(np.int32)
    case = workloads.decode_contiguous(B, 64, 2, 32, 96, seqlens=lens, seed=37, poison=True)
    if fmt == "fp8":
        case = workloads.as_fp8(case)
        o, ref = run_fp8(case, 32), oracle_out_fp8(case)
    else:
        o, ref = run(case, 32), oracle_out(case)
    got = host_f64(o)
    assert np.all(got[lens == 0] == 0.0)
    assert np.all(np.isfinite(got))
    assert_bf16_close(got, ref, f"d=32 B={B} {fmt}")

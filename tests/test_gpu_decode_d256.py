"""GPU parity of fa_decode, fa_decode_fp8 and fa_merge_lse at head dim 256
against the fp64 oracle.

At d = 256 the split kernel holds 376 registers per lane and two 32-token V
stages of 16 KB per wave, so one work-group runs per CU; the same tests as at
d = 64 and 128 hold: full-size mixed-length paged workload, head groups and
split sizes, paged = contiguous bit for bit, poisoned slots, the FP8 cache
(against its oracle and against the bf16 path on the dequantised cache).
"""
import numpy as np
import pytest

import attention_fa_prefill_amd as fa
import oracle
import workloads
from tests.gpu_util import F32_MAX_ABS, assert_bf16_close, dev_bf16, dev_f32, dev_i32, host_bits, host_f64, torch_gpu
from tests.test_gpu_decode import oracle_out, oracle_out_fp8, run, run_fp8

pytestmark = pytest.mark.gpu


def test_paged_mixed_lengths_full_size():
    case = workloads.decode_paged_d256()
    assert_bf16_close(host_f64(run(case)), oracle_out(case), case.name)


def test_paged_equals_contiguous_bitwise():
    case = workloads.decode_contiguous(4, 16, 8, 256, 3008, seed=91)
    paged = workloads.paged_from_contiguous(case)
    assert np.array_equal(host_bits(run(case)), host_bits(run(paged)))


@pytest.mark.parametrize("G,Hkv", [(1, 2), (2, 8), (8, 1), (16, 1), (5, 2)])
@pytest.mark.parametrize("tps", [0, 32, 1024])
def test_head_groups_and_split_sizes(G, Hkv, tps):
    lens = np.array([1, 16, 200, 1500], np.int32)
    case = workloads.decode_paged(4, G * Hkv, Hkv, 256, lens, 1536, seed=G * 100 + 256 + tps)
    assert_bf16_close(host_f64(run(case, tps)), oracle_out(case), f"{case.name} G={G} tps={tps}")


def test_long_sequence_many_splits():
    case = workloads.decode_paged(1, 8, 4, 256, np.array([65536], np.int32), 65536, seed=93)
    assert_bf16_close(host_f64(run(case)), oracle_out(case), case.name)


def test_poisoned_slots_do_not_leak():
    lens = np.array([1, 15, 16, 17, 31, 33, 100, 513], np.int32)
    clean = workloads.decode_paged(8, 8, 2, 256, lens, 640, seed=94)
    dirty = workloads.decode_paged(8, 8, 2, 256, lens, 640, seed=94, poison=True)
    o_dirty = run(dirty)
    assert np.array_equal(host_bits(o_dirty), host_bits(run(clean)))
    assert_bf16_close(host_f64(o_dirty), oracle_out(clean), "poisoned d256")


def test_fp8_full_size():
    case = workloads.as_fp8(workloads.decode_paged_d256())
    assert_bf16_close(host_f64(run_fp8(case)), oracle_out_fp8(case), case.name)


@pytest.mark.parametrize("tps", [0, 32])
def test_fp8_head_groups(tps):
    case = workloads.as_fp8(workloads.decode_paged(4, 8, 4, 256, np.array([1, 16, 200, 1500], np.int32), 1536,
                                                   seed=95 + tps))
    assert_bf16_close(host_f64(run_fp8(case, tps)), oracle_out_fp8(case), f"{case.name} tps={tps}")


def test_fp8_equals_bf16_on_the_dequantised_cache():
    case = workloads.as_fp8(workloads.decode_paged(4, 16, 8, 256, np.array([700, 3000, 33, 1], np.int32), 3072,
                                                   seed=96), k_scale=0.5, v_scale=0.25)
    deq_k = workloads.f32_to_bf16_bits((oracle.e4m3_to_f64(case.kcache) * 0.5).astype(np.float32))
    deq_v = workloads.f32_to_bf16_bits((oracle.e4m3_to_f64(case.vcache) * 0.25).astype(np.float32))
    o16 = fa.decode(dev_bf16(case.q), dev_bf16(deq_k), dev_bf16(deq_v), dev_i32(case.seqlens),
                    block_table=dev_i32(case.block_table), max_kv_len=case.max_kv_len, scale=case.scale)
    assert np.array_equal(host_bits(run_fp8(case)), host_bits(o16))


def test_fp8_paged_equals_contiguous_bitwise():
    case = workloads.as_fp8(workloads.decode_contiguous(2, 8, 2, 256, 2048, seed=97))
    paged = workloads.paged_from_contiguous(case)
    assert np.array_equal(host_bits(run_fp8(case)), host_bits(run_fp8(paged)))


def test_merge_lse():
    torch = torch_gpu()
    rng = np.random.default_rng(98)
    R, S, d = 21, 37, 256
    op = rng.standard_normal((R, S, d)).astype(np.float32)
    ls = (rng.standard_normal((R, S)) * 4).astype(np.float32)
    ls[2, :5] = -np.inf
    op[2, :5] = np.nan  # empty splits are never read
    o, lse_out = fa.merge_lse(dev_f32(op), dev_f32(ls), out_dtype=torch.float32)
    ref_o, ref_l = oracle.merge(op.astype(np.float64), ls.astype(np.float64))
    assert np.max(np.abs(host_f64(o) - ref_o)) <= F32_MAX_ABS
    assert np.max(np.abs(host_f64(lse_out) - ref_l)) <= F32_MAX_ABS

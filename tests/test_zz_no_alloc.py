"""fa_decode_noalloc: decode with the split partials in the library's device
array instead of a caller's workspace (for callers that cannot allocate).

It runs the kernels of fa_decode with the same split plan, so its output must
equal fa_decode's bit for bit, and both must match the fp64 oracle at the
bf16 bar. Two calls in a row, the second smaller than the first, show that a
call does not depend on what the previous call left in the array.
"""
import ctypes

import numpy as np
import pytest

import attention_fa_prefill_amd as fa
import oracle
import workloads
from tests.gpu_util import assert_bf16_close, dev_bf16, dev_i32, host_bits, host_f64, torch_gpu

pytestmark = pytest.mark.gpu


def _inputs(case):
    q, kc, vc = dev_bf16(case.q), dev_bf16(case.kcache), dev_bf16(case.vcache)
    lens = dev_i32(case.seqlens)
    bt = dev_i32(case.block_table) if case.paged else None
    return q, kc, vc, lens, bt


def _noalloc(case, tps=0):
    torch = torch_gpu()
    print(f"fa_decode_noalloc {case.name} B={case.B} paged={case.paged} tps={tps}", flush=True)
    q, kc, vc, lens, bt = _inputs(case)
    o = torch.empty_like(q)
    P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
    st = fa.lib().fa_decode_noalloc(P(q), P(kc), P(vc), P(bt), P(lens), P(o), case.B, case.Hq, case.Hkv, case.d,
                                    case.max_kv_len, 16 if case.paged else 0, tps, case.scale,
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == fa.FA_OK, fa.status_string(st)
    torch.cuda.synchronize()
    return o


def _with_workspace(case, tps=0):
    q, kc, vc, lens, bt = _inputs(case)
    return fa.decode(q, kc, vc, lens, block_table=bt, max_kv_len=case.max_kv_len, scale=case.scale,
                     tokens_per_split=tps)


def _oracle(case):
    q, kc, vc = (workloads.bf16_bits_to_f64(x) for x in (case.q, case.kcache, case.vcache))
    o, _ = oracle.decode(q, kc, vc, case.seqlens, case.scale, block_table=case.block_table,
                         max_kv_len=case.max_kv_len)
    return o


def test_two_calls_in_a_row_equal_fa_decode():
    big = workloads.decode_paged_mixed()
    small = workloads.decode_paged(3, 8, 2, 128, np.array([1, 333, 1200], np.int32), 1280, seed=93)
    o_big = _noalloc(big)
    o_small = _noalloc(small)
    assert np.array_equal(host_bits(o_big), host_bits(_with_workspace(big)))
    assert np.array_equal(host_bits(o_small), host_bits(_with_workspace(small)))
    assert_bf16_close(host_f64(o_big), _oracle(big), "noalloc first call (B=8 mixed lengths)")
    assert_bf16_close(host_f64(o_small), _oracle(small), "noalloc second, smaller call")


def test_contiguous_cache_and_explicit_split_size():
    case = workloads.decode_contiguous(2, 16, 4, 64, 3000, seqlens=np.array([2999, 17], np.int32), seed=94)
    for tps in (64, 0):
        o = _noalloc(case, tps)
        assert np.array_equal(host_bits(o), host_bits(_with_workspace(case, tps)))
        assert_bf16_close(host_f64(o), _oracle(case), f"noalloc contiguous tps={tps}")


def test_binding_and_size_limit():
    torch = torch_gpu()
    case = workloads.decode_paged(2, 8, 2, 128, np.array([40, 500], np.int32), 512, seed=95)
    q, kc, vc, lens, bt = _inputs(case)
    o = torch.empty_like(q)
    fa.decode_noalloc(q, kc, vc, lens, o, block_table=bt, max_kv_len=case.max_kv_len, scale=case.scale)
    assert np.array_equal(host_bits(o), host_bits(_with_workspace(case)))
    # partials beyond the array: rejected on the host, nothing launched
    big = fa.lib().fa_decode_noalloc(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), None, lens.data_ptr(),
                                     o.data_ptr(), 64, 32, 8, 128, 32768, 0, 64, 0.1, None)
    assert big == 5  # FA_ERR_WORKSPACE

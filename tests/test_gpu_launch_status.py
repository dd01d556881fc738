"""A runtime error left pending by the caller is not reported as a failure of
the next library call, and the call still computes the right result.

The TensorRT page's plugin contract (answer queries or fail explicitly) makes
the status code the caller's only signal, so it must describe this call's own
launches: include/fa.h states that the library neither reads nor clears the
runtime's pending error. The error planted here is an invalid device ordinal
(hipSetDevice(-1)), which touches no device state.
"""
import ctypes
import os

import numpy as np
import pytest

import attention_fa_prefill_amd as fa
import oracle
import workloads
from tests.gpu_util import assert_bf16_close, dev_bf16, dev_i32, host_f64, torch_gpu

pytestmark = pytest.mark.gpu


def hip_runtime():
    """The HIP runtime already loaded in this process (the one torch and libfa.so share)."""
    return ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)


def plant_error(hip):
    rc = hip.hipSetDevice(ctypes.c_int(-1))
    assert rc != 0, "hipSetDevice(-1) should fail"
    return rc


def test_prefill_and_decode_ignore_a_pending_error():
    torch = torch_gpu()
    hip = hip_runtime()
    hip.hipGetLastError.restype = ctypes.c_int
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    pc = workloads.prefill_case(1, 8, 2, 300, 300, 128, True, "bf16", seed=91)
    q, k, v = dev_bf16(pc.q), dev_bf16(pc.k), dev_bf16(pc.v)
    o = torch.empty_like(q)
    dc = workloads.decode_paged(3, 8, 2, 128, np.array([1, 333, 1200], np.int32), 1280, seed=92)
    dq, dk, dv = dev_bf16(dc.q), dev_bf16(dc.kcache), dev_bf16(dc.vcache)
    lens, bt = dev_i32(dc.seqlens), dev_i32(dc.block_table)
    od = torch.empty_like(dq)
    need = fa.decode_workspace_bytes(dc.B, dc.Hq, dc.Hkv, dc.d, dc.max_kv_len, 0)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    assert hip.hipGetLastError() == 0
    L = fa.lib()
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731

    planted = plant_error(hip)
    st = L.fa_prefill(P(q), P(k), P(v), P(o), 1, 8, 2, 300, 300, 128, pc.scale, 1, stream)
    left = hip.hipGetLastError()  # collect (and clear) whatever is pending before torch runs again
    print(f"planted {planted}; fa_prefill -> {st}; pending afterwards {left}", flush=True)
    assert st == fa.FA_OK
    assert left == planted  # neither reported nor cleared by the call

    planted = plant_error(hip)
    st = L.fa_decode(P(dq), P(dk), P(dv), P(bt), P(lens), P(od), dc.B, dc.Hq, dc.Hkv, dc.d, dc.max_kv_len, 16, 0,
                     dc.scale, P(ws), need, stream)
    left = hip.hipGetLastError()
    print(f"planted {planted}; fa_decode -> {st}; pending afterwards {left}", flush=True)
    assert st == fa.FA_OK
    assert left == planted  # neither reported nor cleared by the call
    torch.cuda.synchronize()

    ref, _ = oracle.attention(*pc.as_f64(), pc.scale, True)
    assert_bf16_close(host_f64(o), ref, "prefill after a pending error")
    q64, k64, v64 = (workloads.bf16_bits_to_f64(x) for x in (dc.q, dc.kcache, dc.vcache))
    refd, _ = oracle.decode(q64, k64, v64, dc.seqlens, dc.scale, block_table=dc.block_table, max_kv_len=dc.max_kv_len)
    assert_bf16_close(host_f64(od), refd, "decode after a pending error")

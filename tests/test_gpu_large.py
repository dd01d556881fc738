"""Tensors past 2^31 elements (4 GiB and more of bf16 per tensor): the largest
offsets of q, o and the KV caches need 64-bit arithmetic. Inputs are drawn on
the device (seeded); sampled outputs are compared with the fp64 oracle, one
query row at a time (row i of causal attention is a single-query attention
over keys 0..i, which the oracle's decode computes).
"""
import math

import numpy as np
import pytest

import attention_fa_prefill_amd as fa
import oracle
import workloads
from tests.gpu_util import assert_bf16_close, torch_gpu

pytestmark = pytest.mark.gpu


def to_f64(t):
    """bf16 device tensor -> float64 host array (exact)."""
    return t.float().cpu().numpy().astype(np.float64)


def test_prefill_past_2_31_elements():
    """B = 4, Hq = 64, Hkv = 8, S = 70000, d = 128, causal: q and o hold
    2.29e9 elements; the last heads start past element 2^31."""
    torch = torch_gpu()
    B, Hq, Hkv, S, d = 4, 64, 8, 70000, 128
    assert B * Hq * S * d > 2**31
    scale = 1.0 / math.sqrt(d)
    print(f"large prefill B={B} Hq={Hq} Hkv={Hkv} S={S} d={d}", flush=True)
    q = workloads.device_normal_bf16((B, Hq, S, d), seed=2001)
    k = workloads.device_normal_bf16((B, Hkv, S, d), seed=2002)
    v = workloads.device_normal_bf16((B, Hkv, S, d), seed=2003)
    o = fa.prefill(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    G = Hq // Hkv
    for b, h in ((0, 0), (2, 17), (3, Hq - 1)):
        g = h // G
        rows = [0, 1, 4095, 65535, S - 1]
        kh, vh = to_f64(k[b, g]), to_f64(v[b, g])
        for i in rows:
            qi = to_f64(q[b, h, i]).reshape(1, 1, d)
            ref, _ = oracle.decode(qi, kh[: i + 1].reshape(1, i + 1, 1, d), vh[: i + 1].reshape(1, i + 1, 1, d),
                                   np.array([i + 1], np.int32), scale)
            got = to_f64(o[b, h, i]).reshape(1, 1, d)
            assert_bf16_close(got, ref, f"b={b} h={h} row={i}")


@pytest.mark.parametrize("paged", [True, False], ids=["paged", "contiguous"])
def test_decode_cache_past_2_31_elements(paged):
    """B = 4, Hq = 32, Hkv = 8, d = 128, capacity 540000 tokens: each cache
    holds 2.2e9 elements (the paged pool 135000 shuffled pages of 16)."""
    torch = torch_gpu()
    B, Hq, Hkv, d, cap = 4, 32, 8, 128, 540000
    lens = np.array([cap, cap - 1, 1, 300001], np.int32)
    scale = 1.0 / math.sqrt(d)
    pps = -(-cap // 16)
    print(f"large decode paged={paged} B={B} cap={cap}", flush=True)
    q = workloads.device_normal_bf16((B, Hq, d), seed=2011)
    if paged:
        P = B * pps
        assert P * 16 * Hkv * d > 2**31
        kc = workloads.device_normal_bf16((P, 16, Hkv, d), seed=2012)
        vc = workloads.device_normal_bf16((P, 16, Hkv, d), seed=2013)
        bt_host = workloads.rng(2014, 0).permutation(P).astype(np.int32).reshape(B, pps)
        bt = torch.from_numpy(bt_host).cuda()
    else:
        assert B * cap * Hkv * d > 2**31
        kc = workloads.device_normal_bf16((B, cap, Hkv, d), seed=2012)
        vc = workloads.device_normal_bf16((B, cap, Hkv, d), seed=2013)
        bt_host, bt = None, None
    seq = torch.from_numpy(lens).cuda()
    o = fa.decode(q, kc, vc, seq, block_table=bt, max_kv_len=cap, scale=scale)
    torch.cuda.synchronize()
    G = Hq // Hkv
    for b in range(B):
        L = int(lens[b])
        for h in (0, Hq - 1):
            g = h // G
            if paged:
                pages = torch.from_numpy(bt_host[b, : -(-L // 16)].astype(np.int64)).cuda()
                kh = to_f64(kc[pages][:, :, g].reshape(-1, d)[:L])
                vh = to_f64(vc[pages][:, :, g].reshape(-1, d)[:L])
            else:
                kh, vh = to_f64(kc[b, :L, g]), to_f64(vc[b, :L, g])
            ref, _ = oracle.decode(to_f64(q[b, h]).reshape(1, 1, d), kh.reshape(1, L, 1, d), vh.reshape(1, L, 1, d),
                                   np.array([L], np.int32), scale)
            assert_bf16_close(to_f64(o[b, h]).reshape(1, 1, d), ref, f"b={b} h={h} len={L}")

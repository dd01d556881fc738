"""GPU parity of fa_prefill / fa_prefill_f32 at head dims 32, 96 and 256
against the fp64 oracle, every output element.

These head dims run on their own bf16 kernel (one wave per 32 query rows,
64-key blocks double-buffered in LDS; d = 256 at one wave per SIMD). Shapes
span several 128-row query tiles and 64-key blocks with ragged tails,
MQA/GQA/MHA, causal and not, Sq != Skv; the full-size d = 256 and d = 96
workloads are compared whole.
"""
import dataclasses

import numpy as np
import pytest

import attention_fa_prefill_amd as fa
import oracle
import workloads
from tests.gpu_util import (assert_bf16_close, assert_f32_close, dev_bf16, dev_f32, dev_i32, host_bits, host_f64,
                            torch_gpu)

pytestmark = pytest.mark.gpu


def run_case(case, **kw):
    torch_gpu()
    if case.dtype == "bf16":
        q, k, v = dev_bf16(case.q), dev_bf16(case.k), dev_bf16(case.v)
    else:
        q, k, v = dev_f32(case.q), dev_f32(case.k), dev_f32(case.v)
    print(f"case {case.name} scale={case.scale:.4g}", flush=True)
    return fa.prefill(q, k, v, causal=case.causal, scale=case.scale, **kw)


def oracle_out(case):
    q, k, v = case.as_f64()
    o, _ = oracle.attention(q, k, v, case.scale, case.causal)
    return o


@pytest.mark.parametrize("make", [workloads.prefill_gqa_d256, workloads.prefill_mha_d96, workloads.prefill_gqa_d32],
                         ids=["gqa_b1h16x8s2048d256", "mha_b1h32s2048d96", "gqa_b1h32x8s2048d32"])
def test_full_size(make):
    case = make()
    assert_bf16_close(host_f64(run_case(case)), oracle_out(case), case.name)


SHAPES = [
    # B, Hq, Hkv, Sq, Skv, d, causal
    (1, 1, 1, 1, 1, 32, True),
    (1, 2, 1, 7, 7, 256, True),
    (2, 4, 2, 100, 100, 96, True),
    (1, 4, 1, 129, 129, 256, True),      # MQA, one row past a tile
    (1, 8, 8, 257, 257, 32, True),       # MHA, ragged
    (1, 4, 2, 300, 300, 96, False),
    (2, 2, 1, 64, 200, 256, True),       # Sq < Skv, bottom-right causal
    (1, 4, 4, 200, 64, 96, False),       # Sq > Skv non-causal
    (1, 2, 1, 640, 640, 256, True),
    (1, 2, 2, 1000, 1500, 32, True),
    (3, 6, 3, 383, 383, 96, True),
    (1, 2, 1, 128, 4096, 32, False),     # long KV
    (1, 2, 1, 33, 4000, 256, True),
    (1, 3, 1, 65, 191, 96, False),
    (2, 4, 1, 65, 300, 32, True),        # d = 32 (key-split kernel): MQA, Sq < Skv
    (1, 4, 2, 300, 100, 32, False),      # Sq > Skv non-causal
    (3, 6, 2, 191, 191, 32, True),
    (2, 64, 8, 1100, 1100, 32, True),    # a causal grid past two rounds: two key parts
    # d = 256 grids of at least two rounds of 128-row tiles (512 on 256 CUs)
    # take the one-group kernel, smaller ones the key-split kernel
    (4, 16, 8, 1024, 1024, 256, True),
    (2, 32, 4, 1000, 900, 256, False),
    (1, 8, 2, 1500, 1500, 256, True),
    (1, 2, 1, 2, 777, 256, False),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b{}h{}x{}sq{}skv{}d{}{}".format(*s[:6], "c" if s[6] else ""))
def test_bf16_shapes(shape):
    B, Hq, Hkv, Sq, Skv, d, causal = shape
    case = workloads.prefill_case(B, Hq, Hkv, Sq, Skv, d, causal, "bf16", seed=hash(shape) % 10000)
    assert_bf16_close(host_f64(run_case(case)), oracle_out(case), case.name)


@pytest.mark.parametrize("shape", [(1, 2, 1, 65, 65, 32, True), (2, 4, 2, 130, 260, 96, True),
                                   (1, 3, 3, 200, 150, 256, False), (1, 1, 1, 1, 300, 96, False),
                                   (1, 2, 1, 128, 128, 256, True)],
                         ids=lambda s: "b{}h{}x{}sq{}skv{}d{}{}".format(*s[:6], "c" if s[6] else ""))
def test_fp32_shapes(shape):
    B, Hq, Hkv, Sq, Skv, d, causal = shape
    case = workloads.prefill_case(B, Hq, Hkv, Sq, Skv, d, causal, "f32", seed=11 + Sq)
    assert_f32_close(host_f64(run_case(case)), oracle_out(case), case.name)


@pytest.mark.parametrize("d", [32, 96, 256])
@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.5])
def test_bf16_scale_sign_and_zero(d, scale):
    case = workloads.prefill_case(1, 4, 2, 150, 150, d, True, "bf16", seed=321 + d, scale=scale)
    assert_bf16_close(host_f64(run_case(case)), oracle_out(case), f"{case.name} scale={scale}")


@pytest.mark.parametrize("profile", ["rising", "falling"])
@pytest.mark.parametrize("d", [32, 96, 256])
def test_bf16_score_jumps_between_blocks(profile, d):
    """Key magnitudes ramp along the sequence, so row maxima jump between key
    blocks far beyond the lazy rescale threshold."""
    base = workloads.prefill_case(1, 2, 1, 700, 700, d, True, "bf16", seed=78 + d, scale=0.25)
    k = workloads.bf16_bits_to_f32(base.k).astype(np.float64)
    j = np.arange(700, dtype=np.float64)
    ramp = (0.2 + 6.0 * j / 699.0) if profile == "rising" else (6.2 - 6.0 * j / 699.0)
    k *= ramp[None, None, :, None]
    case = dataclasses.replace(base, k=workloads.f32_to_bf16_bits(k.astype(np.float32)), name=f"{base.name}_{profile}")
    assert_bf16_close(host_f64(run_case(case)), oracle_out(case), case.name)


@pytest.mark.parametrize("d", [32, 96, 256])
def test_bf16_exact_cases(d):
    """Causal row 0 sees one key (probability exactly 1): o = V[0] bit for bit.
    With Skv = 1 every row gives v_0 exactly."""
    case = workloads.prefill_case(2, 4, 2, 300, 300, d, True, "bf16", seed=5 + d)
    bits = host_bits(run_case(case))
    for h in range(4):
        assert np.array_equal(bits[:, h, 0, :], case.v[:, h // 2, 0, :])
    case1 = workloads.prefill_case(1, 4, 1, 70, 1, d, False, "bf16", seed=6 + d)
    assert np.array_equal(host_bits(run_case(case1)), np.broadcast_to(case1.v[:, :1, :1, :], (1, 4, 70, d)))


def test_bf16_deterministic():
    case = workloads.prefill_case(1, 8, 2, 700, 700, 256, True, "bf16", seed=8)
    assert np.array_equal(host_bits(run_case(case)), host_bits(run_case(case)))


@pytest.mark.parametrize("d", [32, 96, 256])
def test_output_canary_untouched(d):
    """Writes stay inside o: neighbours of the output buffer keep their bytes."""
    torch = torch_gpu()
    case = workloads.prefill_case(1, 2, 1, 130, 130, d, True, "bf16", seed=9 + d)
    q, k, v = dev_bf16(case.q), dev_bf16(case.k), dev_bf16(case.v)
    n = q.numel()
    buf = torch.full((n + 2048,), 1234.0, dtype=torch.bfloat16, device="cuda")
    o = buf[1024:1024 + n].view(q.shape)
    fa.prefill(q, k, v, o, causal=True, scale=case.scale)
    torch.cuda.synchronize()
    assert torch.all(buf[:1024] == 1234.0) and torch.all(buf[1024 + n:] == 1234.0)
    assert_bf16_close(host_f64(o), oracle_out(case), case.name)


@pytest.mark.parametrize("d,B", [(128, 1), (256, 1), (256, 4), (96, 1), (32, 1)])
def test_graph_capture_replays(d, B):
    """fa_prefill captured in a HIP graph (the ping-pong kernel at d = 128 and
    96, the key-split and one-group kernels at d = 256, the key-split kernel at
    d = 32):
    every replay, with eager work between replays and new q written in place,
    equals the eager call bit for bit."""
    torch = torch_gpu()
    case = workloads.prefill_case(B, 16, 8, 1024, 1024, d, True, "bf16", seed=500 + d + B)
    q, k, v = dev_bf16(case.q), dev_bf16(case.k), dev_bf16(case.v)
    o = torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fa.prefill(q, k, v, o, causal=True, scale=case.scale)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.prefill(q, k, v, o, causal=True, scale=case.scale)
    torch.cuda.synchronize()
    for rep in range(4):
        if rep % 2 == 1:
            q.copy_(torch.randn(q.shape, device="cuda").to(torch.bfloat16))
        x = torch.randn(1 << 20, device="cuda")
        (x * 2 + 1).sum().item()  # eager work between replays
        print(f"replay {rep} d={d} B={B}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        ref = fa.prefill(q, k, v, causal=True, scale=case.scale)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(o), host_bits(ref)), f"replay {rep}"


def test_graph_capture_replays_prefill_cache():
    """fa_prefill_cache (paged, d = 256 and 128) captured in a HIP graph: replays
    with new lengths written into seqlens equal the eager call bit for bit."""
    torch = torch_gpu()
    for d in (256, 128):
        case = workloads.prefill_cache_case(3, 8, 4, 300, d, [1200, 700, 300], 1216, paged=True, causal=True,
                                            seed=600 + d)
        q, kc, vc = dev_bf16(case.q), dev_bf16(case.kcache), dev_bf16(case.vcache)
        lens, bt = dev_i32(case.seqlens), dev_i32(case.block_table)
        o = torch.empty_like(q)

        def call(out=None):
            return fa.prefill_cache(q, kc, vc, lens, block_table=bt, max_kv_len=case.max_kv_len, causal=True,
                                    scale=case.scale, o=out)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call(o)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call(o)
        torch.cuda.synchronize()
        for rep, new in enumerate(([1200, 700, 300], [400, 1216, 301], [299, 1, 1000], [1200, 700, 300])):
            lens.copy_(torch.tensor(new, dtype=torch.int32))
            (torch.randn(1 << 20, device="cuda") * 2).sum().item()
            print(f"replay {rep} d={d} lens={new}", flush=True)
            g.replay()
            torch.cuda.synchronize()
            ref = call()
            torch.cuda.synchronize()
            assert np.array_equal(host_bits(o), host_bits(ref)), f"d={d} replay {rep}"

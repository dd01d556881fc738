"""GPU parity of fa_prefill / fa_prefill_f32 against the fp64 oracle.

Inputs are the seeded synthetic workloads of ``workloads.py``; every output
element is compared with the oracle (it finishes the full-size GQA prefill in
seconds). Shapes span several 128-row query tiles and 64-key blocks with
ragged tails, MQA/GQA/MHA, d = 64 and 128, causal and not, Sq != Skv.
"""
import math

import numpy as np
import pytest

import attention_fa_prefill_amd as fa
import oracle
import workloads
from tests.gpu_util import (assert_bf16_close, assert_f32_close, dev_bf16, dev_f32, host_bits, host_f64,
                            torch_gpu)

pytestmark = pytest.mark.gpu


def run_case(case, **kw):
    torch_gpu()
    if case.dtype == "bf16":
        q, k, v = dev_bf16(case.q), dev_bf16(case.k), dev_bf16(case.v)
    else:
        q, k, v = dev_f32(case.q), dev_f32(case.k), dev_f32(case.v)
    print(f"case {case.name} scale={case.scale:.4g}", flush=True)
    o = fa.prefill(q, k, v, causal=case.causal, scale=case.scale, **kw)
    return o, (q, k, v)


def oracle_out(case):
    q, k, v = case.as_f64()
    o, _ = oracle.attention(q, k, v, case.scale, case.causal)
    return o


def test_fp32_single_head_causal_s128_d64():
    case = workloads.prefill_f32_small()
    o, _ = run_case(case)
    assert_f32_close(host_f64(o), oracle_out(case), case.name)


def test_gqa_causal_prefill_s2048_full_size():
    case = workloads.prefill_gqa_2k()
    o, _ = run_case(case)
    assert_bf16_close(host_f64(o), oracle_out(case), case.name)


SHAPES = [
    # B, Hq, Hkv, Sq, Skv, d, causal
    (1, 1, 1, 1, 1, 128, True),
    (1, 2, 1, 7, 7, 64, True),
    (2, 4, 2, 100, 100, 128, True),
    (1, 4, 1, 129, 129, 128, True),      # MQA, one row past a tile
    (1, 8, 8, 257, 257, 64, True),       # MHA, ragged
    (1, 4, 2, 300, 300, 128, False),
    (2, 2, 1, 64, 200, 128, True),       # Sq < Skv, bottom-right causal
    (1, 4, 4, 200, 64, 128, False),      # Sq > Skv non-causal
    (1, 2, 1, 640, 640, 128, True),      # 5 query tiles: odd count, middle tile split
    (1, 2, 2, 1000, 1500, 64, True),
    (3, 6, 3, 383, 383, 128, True),
    (1, 16, 2, 1024, 1024, 128, True),
    (1, 2, 1, 128, 4096, 128, False),    # long KV
    (1, 2, 1, 33, 4000, 128, True),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b{}h{}x{}sq{}skv{}d{}{}".format(*s[:6], "c" if s[6] else ""))
def test_bf16_shapes(shape):
    B, Hq, Hkv, Sq, Skv, d, causal = shape
    case = workloads.prefill_case(B, Hq, Hkv, Sq, Skv, d, causal, "bf16", seed=hash(shape) % 10000)
    o, _ = run_case(case)
    assert_bf16_close(host_f64(o), oracle_out(case), case.name)


@pytest.mark.parametrize("shape", [(1, 2, 1, 65, 65, 128, True), (2, 4, 2, 130, 260, 64, True),
                                   (1, 3, 3, 200, 150, 64, False), (1, 1, 1, 1, 300, 128, False)],
                         ids=lambda s: "b{}h{}x{}sq{}skv{}d{}{}".format(*s[:6], "c" if s[6] else ""))
def test_fp32_shapes(shape):
    B, Hq, Hkv, Sq, Skv, d, causal = shape
    case = workloads.prefill_case(B, Hq, Hkv, Sq, Skv, d, causal, "f32", seed=7 + Sq)
    o, _ = run_case(case)
    assert_f32_close(host_f64(o), oracle_out(case), case.name)


CROSS = [
    # cross-attention: the queries of one sequence over the keys and values of
    # another (an encoder's output), non-causal, Sq != Skv
    # B, Hq, Hkv, Sq, Skv, d
    (2, 8, 8, 77, 1500, 64),     # decoder tokens over a long encoder output
    (1, 16, 16, 448, 1500, 64),
    (3, 4, 4, 1024, 77, 128),    # many queries over a short context
    (1, 12, 12, 333, 257, 96),
    (2, 8, 4, 150, 600, 256),
]


@pytest.mark.parametrize("shape", CROSS, ids=lambda s: "b{}h{}x{}sq{}skv{}d{}".format(*s))
def test_bf16_cross_attention(shape):
    B, Hq, Hkv, Sq, Skv, d = shape
    case = workloads.prefill_case(B, Hq, Hkv, Sq, Skv, d, False, "bf16", seed=4000 + Sq + Skv + d,
                                  name=f"cross_b{B}h{Hq}x{Hkv}sq{Sq}skv{Skv}d{d}")
    o, _ = run_case(case)
    assert_bf16_close(host_f64(o), oracle_out(case), case.name)


@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.5])
def test_bf16_scale_sign_and_zero(scale):
    case = workloads.prefill_case(1, 4, 2, 150, 150, 128, True, "bf16", seed=321, scale=scale)
    o, _ = run_case(case)
    assert_bf16_close(host_f64(o), oracle_out(case), f"{case.name} scale={scale}")


def _ramped_case(profile, causal, seed):
    """Keys whose magnitude follows a profile along the sequence, so that the
    row maxima jump between key blocks (rising, falling, or one spike late),
    far beyond the range the kernel's exponent reference tolerates without
    being raised."""
    import dataclasses

    base = workloads.prefill_case(1, 2, 1, 700, 700, 128, causal, "bf16", seed=seed, scale=0.25)
    k = workloads.bf16_bits_to_f32(base.k).astype(np.float64)
    j = np.arange(700, dtype=np.float64)
    if profile == "rising":
        k *= (0.2 + 6.0 * j / 699.0)[None, None, :, None]
    elif profile == "falling":
        k *= (6.2 - 6.0 * j / 699.0)[None, None, :, None]
    else:  # spike: one late key aligned with every query row's sum direction
        q = workloads.bf16_bits_to_f32(base.q).astype(np.float64)
        k[0, 0, 650, :] = 4.0 * np.sign(q[0, 0].sum(axis=0))
    kb = workloads.f32_to_bf16_bits(k.astype(np.float32))
    return dataclasses.replace(base, k=kb, name=f"{base.name}_{profile}")


@pytest.mark.parametrize("profile", ["rising", "falling", "spike"])
@pytest.mark.parametrize("causal", [True, False])
def test_bf16_score_jumps_between_blocks(profile, causal):
    case = _ramped_case(profile, causal, seed=77)
    o, _ = run_case(case)
    assert_bf16_close(host_f64(o), oracle_out(case), case.name)


def test_bf16_exact_cases():
    """Causal row 0 sees one key (probability exactly 1): o = V[0] bit for bit.
    With Skv = 1 every row gives v_0 exactly."""
    case = workloads.prefill_case(2, 4, 2, 300, 300, 128, True, "bf16", seed=5)
    o, _ = run_case(case)
    bits = host_bits(o)
    G = 2
    for h in range(4):
        assert np.array_equal(bits[:, h, 0, :], case.v[:, h // G, 0, :])
    case1 = workloads.prefill_case(1, 4, 1, 70, 1, 64, False, "bf16", seed=6)
    o1, _ = run_case(case1)
    assert np.array_equal(host_bits(o1), np.broadcast_to(case1.v[:, :1, :1, :], (1, 4, 70, 64)))


def test_bf16_deterministic():
    case = workloads.prefill_case(1, 8, 2, 700, 700, 128, True, "bf16", seed=8)
    o1, _ = run_case(case)
    o2, _ = run_case(case)
    assert np.array_equal(host_bits(o1), host_bits(o2))


def test_output_canary_untouched():
    """Writes stay inside o: neighbours of the output buffer keep their bytes."""
    torch = torch_gpu()
    case = workloads.prefill_case(1, 2, 1, 130, 130, 64, True, "bf16", seed=9)
    q, k, v = dev_bf16(case.q), dev_bf16(case.k), dev_bf16(case.v)
    n = q.numel()
    buf = torch.full((n + 2048,), 1234.0, dtype=torch.bfloat16, device="cuda")
    o = buf[1024:1024 + n].view(q.shape)
    fa.prefill(q, k, v, o, causal=True, scale=case.scale)
    torch.cuda.synchronize()
    assert torch.all(buf[:1024] == 1234.0) and torch.all(buf[1024 + n:] == 1234.0)
    assert_bf16_close(host_f64(o), oracle_out(case), case.name)

"""GPU parity of fa_prefill_f32 on grids large enough for its matrix-core
kernel (v_mfma_f32_32x32x2_f32, at least 64 query tiles of 128 rows over
heads and batch; d = 32, 64, 96, 128), every output element against the fp64
oracle to the fp32 bound. Smaller shapes (the vector kernel) are covered in
test_gpu_prefill.py and test_gpu_prefill_hd.py.
"""
import pytest

import attention_fa_prefill_amd as fa
import oracle
import workloads
from tests.gpu_util import assert_f32_close, dev_f32, host_f64, torch_gpu

pytestmark = pytest.mark.gpu


def run_and_check(case):
    torch_gpu()
    assert -(-case.Sq // 128) * case.Hq * case.B >= 64  # the matrix-core kernel
    print(f"case {case.name} scale={case.scale:.4g}", flush=True)
    o = fa.prefill(dev_f32(case.q), dev_f32(case.k), dev_f32(case.v), causal=case.causal, scale=case.scale)
    q, k, v = case.as_f64()
    ref, _ = oracle.attention(q, k, v, case.scale, case.causal)
    assert_f32_close(host_f64(o), ref, case.name)


SHAPES = [
    # B, Hq, Hkv, Sq, Skv, d, causal
    (1, 16, 8, 1024, 1024, 128, True),
    (2, 16, 16, 700, 1500, 64, False),   # Sq != Skv, non-causal
    (1, 32, 8, 1000, 1000, 96, True),    # GQA, Sq not a tile multiple
    (1, 64, 64, 513, 513, 32, True),     # MHA, one row past 4 tiles
    (2, 32, 32, 300, 2000, 128, True),   # Sq < Skv, bottom-right causal
    (1, 32, 4, 1500, 383, 128, False),   # MQA-like, Sq > Skv
    (3, 16, 8, 383, 1031, 64, True),
    # causal grids of one round at two work-groups per CU (256 < tiles <= 512:
    # costly and cheap tiles paired per CU), with Sq < Skv and a ragged last tile
    (3, 16, 8, 900, 1200, 64, True),
    (1, 48, 16, 1000, 1000, 128, True),
    # the smallest grids on the matrix cores (64 tiles)
    (1, 8, 8, 1024, 1024, 64, True),
    (1, 4, 2, 2048, 2048, 128, False),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b{}h{}x{}sq{}skv{}d{}{}".format(*s[:6], "c" if s[6] else ""))
def test_f32_mfma_shapes(shape):
    B, Hq, Hkv, Sq, Skv, d, causal = shape
    run_and_check(workloads.prefill_case(B, Hq, Hkv, Sq, Skv, d, causal, "f32", seed=900 + Sq + Skv + d))


@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.5])
def test_f32_mfma_scales(scale):
    run_and_check(workloads.prefill_case(1, 16, 8, 1024, 1024, 128, True, "f32", seed=950, scale=scale))


def test_f32_mfma_full_size_gqa_s2048():
    """The C2 shape (B = 1, Hq = 32, Hkv = 8, S = 2048, d = 128, causal) in fp32."""
    run_and_check(workloads.prefill_case(1, 32, 8, 2048, 2048, 128, True, "f32", seed=1002, scale=128 ** -0.5))

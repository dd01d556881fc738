"""Fixtures under tests/golden/ (CPU only)."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.cpu
HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_oracle_reproduces_tiny_fixture():
    with open(os.path.join(HERE, "oracle_tiny.json")) as f:
        data = json.load(f)
    for c in data["cases"]:
        shp_q = (c["B"], c["Hq"], c["Sq"], c["d"])
        shp_kv = (c["B"], c["Hkv"], c["Skv"], c["d"])
        q = workloads.bf16_bits_to_f64(np.array(c["q_bits"], np.uint16).reshape(shp_q))
        k = workloads.bf16_bits_to_f64(np.array(c["k_bits"], np.uint16).reshape(shp_kv))
        v = workloads.bf16_bits_to_f64(np.array(c["v_bits"], np.uint16).reshape(shp_kv))
        o, lse = oracle.attention(q, k, v, c["scale"], c["causal"])
        assert np.max(np.abs(o.reshape(-1) - np.array(c["o"]))) < 1e-15
        assert np.max(np.abs(lse.reshape(-1) - np.array(c["lse"]))) < 1e-14


def test_workloads_use_the_pages_facts():
    with open(os.path.join(HERE, "pages_facts.json")) as f:
        facts = json.load(f)
    assert workloads.PAGE == facts["page_size_tokens"]["value"]
    case = workloads.prefill_case(1, 32, 8, 16, 16, 128, True, "bf16", seed=1)
    assert case.Hq == facts["usage_example_heads"]["value"]
    assert case.d == facts["usage_example_head_dim"]["value"]


def test_bf16_rounding_is_nearest_even():
    # exact halfway cases round to the even neighbour; others to nearest
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, np.inf, -np.inf, np.nan], np.float32)
    b = workloads.f32_to_bf16_bits(x)
    back = workloads.bf16_bits_to_f32(b)
    assert back[0] == 1.0
    assert back[1] == 1.0                 # halfway, 1.0 is even
    assert back[2] == 1.0 + 4 * 2**-8     # halfway, rounds up to even
    assert back[3] == 1.0                 # below halfway
    assert back[4] == -2.5
    assert np.isposinf(back[5]) and np.isneginf(back[6]) and np.isnan(back[7])
    # widening is exact and round-trips
    r = workloads.normal_bf16(3, 0, (1000,))
    assert np.array_equal(workloads.f32_to_bf16_bits(workloads.bf16_bits_to_f32(r)), r)

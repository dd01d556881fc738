"""Pins of the oracle's INT8 KV-cache path (two's-complement dequantisation,
then the same decode definition), and a mutation test of those pins. CPU only.

The 8-bit integer KV cache is the one the FasterTransformer source
walkthrough lists among its quantisation steps (section 3.3), here with one
scale per tensor, as for the FP8 cache.
"""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.cpu

CODES = np.arange(256, dtype=np.uint8)


def pin_library_routines(f):
    """All 256 bytes agree with numpy's int8 view and with Python's signed
    int.from_bytes, two independent implementations of two's complement."""
    got = f(CODES)
    assert np.array_equal(got, CODES.view(np.int8).astype(np.float64))
    assert [int(x) for x in got] == [int.from_bytes(bytes([c]), "little", signed=True) for c in range(256)]


def pin_values_of_the_definition(f):
    """0x00 = 0, 0x01 = 1, 0x7F = 127 (largest), 0x80 = -128 (smallest),
    0x81 = -127, 0xFF = -1."""
    v = f(np.array([0x00, 0x01, 0x7F, 0x80, 0x81, 0xFF], np.uint8))
    assert list(v) == [0.0, 1.0, 127.0, -128.0, -127.0, -1.0]


def pin_order_and_negation(f):
    """Read as signed bytes, 0x80..0xFF then 0x00..0x7F is the increasing run
    -128..127, and the byte of -x is 256 - x for x = 1..127."""
    order = np.concatenate([CODES[128:], CODES[:128]])
    assert np.array_equal(f(order), np.arange(-128, 128, dtype=np.float64))
    x = np.arange(1, 128)
    assert np.array_equal(f((256 - x).astype(np.uint8)), -f(x.astype(np.uint8)))


def pin_decode_closed_forms(f):
    """Through the int8 decode: every V code equal gives o = v_scale * value
    for every row (the weights sum to 1), and a single cached token gives
    o = its dequantised V row."""
    case = workloads.as_int8(workloads.decode_paged(3, 4, 2, 64, np.array([1, 40, 17], np.int32), 48, seed=3))
    vc = np.full_like(case.vcache, 0xF9)  # -7
    q = workloads.bf16_bits_to_f64(case.q)
    o, _ = oracle.decode_int8(q, case.kcache, vc, case.seqlens, case.scale, case.k_scale, case.v_scale,
                              block_table=case.block_table, max_kv_len=48)
    assert np.max(np.abs(o - case.v_scale * -7.0)) < 1e-13
    o, _ = oracle.decode_int8(q, case.kcache, case.vcache, case.seqlens, case.scale, case.k_scale, case.v_scale,
                              block_table=case.block_table, max_kv_len=48)
    page0 = case.block_table[0, 0]
    v0 = f(case.vcache[page0, 0]) * case.v_scale  # [Hkv, d]
    for h in range(4):
        assert np.max(np.abs(o[0, h] - v0[h // 2])) < 1e-13


PINS = [pin_library_routines, pin_values_of_the_definition, pin_order_and_negation, pin_decode_closed_forms]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle.int8_to_f64)


def _as(f):
    return lambda codes: f(np.asarray(codes, dtype=np.uint8).astype(np.int64)).astype(np.float64)


# Plausible mistakes in an int8 decoder; each must fail at least one pin.
MUTANTS = {
    "unsigned": _as(lambda c: c),
    "offset_binary": _as(lambda c: c - 128),
    "sign_magnitude": _as(lambda c: np.where(c >= 128, -(c - 128), c)),
    "ones_complement": _as(lambda c: np.where(c >= 128, c - 255, c)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    f = MUTANTS[name]
    monkeypatch.setattr(oracle, "int8_to_f64", f)  # the int8 decode dequantises through it
    caught = 0
    for pin in PINS:
        try:
            pin(f)
        except AssertionError:
            caught += 1
    assert caught > 0, f"mutant {name} passes every pin"

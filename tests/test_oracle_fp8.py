"""Pins of the oracle's FP8 KV-cache path (E4M3 dequantisation, then the same
decode definition), and a mutation test of those pins. CPU only.

The format is OCP 8-bit floating point E4M3 ("FN": no infinities), with one
scale per tensor: the 8-bit KV cache of the FasterTransformer source
walkthrough (section 3.3) in the FP8 form of the FlashRT project summary.
"""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.cpu

CODES = np.arange(256, dtype=np.uint8)


def pin_library_routine(f):
    """All 256 codes agree with PyTorch's float8_e4m3fn, an independent
    implementation of the same format (NaN codes included)."""
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch has no float8_e4m3fn")
    ref = torch.from_numpy(CODES.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = f(CODES)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def pin_values_of_the_definition(f):
    """Values fixed by the bit layout: 1.0 is exponent field 7, mantissa 0;
    the smallest subnormal is 2^-9; the smallest normal 2^-6; the largest
    finite value 448 = 1.75 * 2^8; sign bit 7; 0x7F and 0xFF are NaN."""
    v = f(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x3C, 0x40, 0x7E, 0x80, 0xB8, 0xFE, 0x7F, 0xFF], np.uint8))
    assert v[0] == 0.0 and not np.signbit(v[0])
    assert v[1] == 2.0 ** -9 and v[2] == 7 * 2.0 ** -9 and v[3] == 2.0 ** -6
    assert v[4] == 1.0 and v[5] == 1.5 and v[6] == 2.0 and v[7] == 448.0
    assert v[8] == 0.0 and np.signbit(v[8])
    assert v[9] == -1.0 and v[10] == -448.0
    assert np.isnan(v[11]) and np.isnan(v[12])


def pin_order_and_symmetry(f):
    """Codes 0x00..0x7E are strictly increasing (the format orders like its
    unsigned bit patterns), and code c | 0x80 is the negative of code c."""
    pos = f(CODES[:0x7F])
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(f(CODES[:0x7F] | 0x80), -pos)


def pin_decode_closed_forms(f):
    """Through the fp8 decode: every V code equal gives o = v_scale * value
    for every row (the weights sum to 1), and a single cached token gives
    o = its dequantised V row."""
    case = workloads.as_fp8(workloads.decode_paged(3, 4, 2, 64, np.array([1, 40, 17], np.int32), 48, seed=3))
    vc = np.full_like(case.vcache, 0x3C)  # 1.5
    q = workloads.bf16_bits_to_f64(case.q)
    o, _ = oracle.decode_fp8(q, case.kcache, vc, case.seqlens, case.scale, case.k_scale, case.v_scale,
                             block_table=case.block_table, max_kv_len=48)
    assert np.max(np.abs(o - case.v_scale * 1.5)) < 1e-14
    o, _ = oracle.decode_fp8(q, case.kcache, case.vcache, case.seqlens, case.scale, case.k_scale, case.v_scale,
                             block_table=case.block_table, max_kv_len=48)
    page0 = case.block_table[0, 0]
    v0 = f(case.vcache[page0, 0]) * case.v_scale  # [Hkv, d]
    for h in range(4):
        assert np.max(np.abs(o[0, h] - v0[h // 2])) < 1e-15


PINS = [pin_library_routine, pin_values_of_the_definition, pin_order_and_symmetry, pin_decode_closed_forms]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle.e4m3_to_f64)


def _mutant(bias=7, sub_exp=-6, sign=True, nan=True, sub_as_normal=False):
    def f(codes):
        c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
        e, m = (c >> 3) & 15, (c & 7).astype(np.float64)
        norm = (1.0 + m / 8.0) * np.exp2((e - bias).astype(np.float64))
        sub = norm if sub_as_normal else (m / 8.0) * 2.0 ** sub_exp
        mag = np.where(e == 0, sub, norm)
        if nan:
            mag = np.where((e == 15) & (m == 7), np.nan, mag)
        return np.where(c >> 7, -1.0, 1.0) * mag if sign else mag
    return f


# Plausible mistakes in an E4M3 decoder; each must fail at least one pin.
MUTANTS = {
    "bias_8": _mutant(bias=8),
    "subnormal_exponent_-7": _mutant(sub_exp=-7),
    "subnormals_as_normals": _mutant(sub_as_normal=True),
    "sign_ignored": _mutant(sign=False),
    "no_nan": _mutant(nan=False),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    f = MUTANTS[name]
    monkeypatch.setattr(oracle, "e4m3_to_f64", f)  # the fp8 decode dequantises through it
    caught = 0
    for pin in PINS:
        try:
            pin(f)
        except AssertionError:
            caught += 1
    assert caught > 0, f"mutant {name} passes every pin"

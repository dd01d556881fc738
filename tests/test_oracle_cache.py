"""Pins of the oracle's chunked prefill over a KV cache (``oracle.prefill_cache``)
and a mutation test of those pins. CPU only.

Context and generation phases with a KV cache are the FasterTransformer
walkthrough's sections 3.1-3.2; the cache layouts and the page size 16 are the
paged sketch of the "Real-time inference optimisation" page.
"""
import inspect

import numpy as np
import pytest

import oracle
import workloads
from oracle import brute

pytestmark = pytest.mark.cpu


def _gather(case, b):
    """Sequence b's first L cached tokens as [Hkv][L][d] lists, read slot by slot."""
    kc = workloads.bf16_bits_to_f64(case.kcache)
    vc = workloads.bf16_bits_to_f64(case.vcache)
    L = int(min(max(int(case.seqlens[b]), 0), case.max_kv_len))
    ks, vs = [], []
    for g in range(case.Hkv):
        kr, vr = [], []
        for t in range(L):
            if case.paged:
                pg, sl = int(case.block_table[b][t // 16]), t % 16
                kr.append(list(kc[pg, sl, g])); vr.append(list(vc[pg, sl, g]))
            else:
                kr.append(list(kc[b, t, g])); vr.append(list(vc[b, t, g]))
        ks.append(kr); vs.append(vr)
    return ks, vs


def _oracle(case, f=None):
    f = f or oracle.prefill_cache
    return f(workloads.bf16_bits_to_f64(case.q), workloads.bf16_bits_to_f64(case.kcache),
             workloads.bf16_bits_to_f64(case.vcache), case.seqlens, case.scale, case.causal,
             block_table=case.block_table, max_kv_len=case.max_kv_len)


TINY = [
    # B, Hq, Hkv, Sq, d, lens, max_kv_len, paged, causal
    (3, 2, 1, 5, 4, [9, 3, 0], 20, True, True),      # L < Sq (rows without keys), L = 0
    (2, 4, 2, 4, 3, [17, 4], 17, False, True),
    (2, 2, 2, 3, 4, [1, 33], 40, True, False),
    (1, 3, 1, 6, 2, [6], 6, False, True),             # L = Sq: the plain causal square
]


def pin_brute_force(f=None):
    """Every element against the pure-Python formulation (exact sums, no max
    subtraction, empty rows zero) on sequence-by-sequence gathered K/V."""
    for i, (B, Hq, Hkv, Sq, d, lens, mkl, paged, causal) in enumerate(TINY):
        case = workloads.prefill_cache_case(B, Hq, Hkv, Sq, d, lens, mkl, paged=paged, causal=causal, seed=40 + i)
        o = _oracle(case, f)
        q = workloads.bf16_bits_to_f64(case.q)
        for b in range(B):
            ks, vs = _gather(case, b)
            if not ks[0]:
                assert np.all(o[b] == 0.0)
                continue
            ref = np.array(brute.attention([q[b].tolist()], [ks], [vs], case.scale, causal)[0])
            assert np.max(np.abs(o[b] - ref)) < 1e-12, (i, b)


def pin_paged_equals_contiguous(f=None):
    """The same tokens scattered into a shuffled page pool give the same output."""
    case = workloads.prefill_cache_case(2, 4, 2, 7, 8, [48, 29], 48, paged=False, causal=True, seed=51)
    B, L = case.B, case.max_kv_len
    perm = np.random.default_rng(5).permutation(B * (L // 16))
    bt = perm.reshape(B, L // 16).astype(np.int32)
    kp = np.empty((B * (L // 16), 16, case.Hkv, case.d), np.uint16)
    vp = np.empty_like(kp)
    kp[bt.reshape(-1)] = case.kcache.reshape(-1, 16, case.Hkv, case.d)
    vp[bt.reshape(-1)] = case.vcache.reshape(-1, 16, case.Hkv, case.d)
    import dataclasses
    paged = dataclasses.replace(case, kcache=kp, vcache=vp, block_table=bt)
    assert np.array_equal(_oracle(case, f), _oracle(paged, f))


def pin_full_cache_is_prefill(f=None):
    """A contiguous cache holding exactly the K and V of a plain prefill
    (max_kv_len = Skv = every length) gives the plain prefill."""
    case = workloads.prefill_cache_case(2, 4, 2, 9, 8, [12, 12], 12, paged=False, causal=True, seed=61)
    q = workloads.bf16_bits_to_f64(case.q)
    k = workloads.bf16_bits_to_f64(case.kcache).transpose(0, 2, 1, 3)
    v = workloads.bf16_bits_to_f64(case.vcache).transpose(0, 2, 1, 3)
    ref, _ = oracle.attention(q, np.ascontiguousarray(k), np.ascontiguousarray(v), case.scale, True)
    assert np.max(np.abs(_oracle(case, f) - ref)) < 1e-15


PINS = [pin_brute_force, pin_paged_equals_contiguous, pin_full_cache_is_prefill]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin()


# Plausible mistakes planted in a copy of the function; each must fail a pin.
MUTANTS = {
    "page_slot": ("rows = bt[b, t // page_size], t % page_size", "rows = bt[b, t % page_size], t // page_size"),
    "top_left_causal": ("ob, _ = attention(q[b:b + 1, :, Sq - L:], kb, vb, scale, True, lib=lib)",
                        "ob, _ = attention(q[b:b + 1, :, :L], kb, vb, scale, True, lib=lib)"),
    "length_unclamped": ("L = int(min(max(lens[b], 0), mkl))", "L = int(max(lens[b], 0)) + 1"),
    "keys_from_other_sequence": ("kb, vb = kc[b, :L], vc[b, :L]", "kb, vb = kc[0, :L], vc[0, :L]"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    src = inspect.getsource(oracle.prefill_cache)
    a, b = MUTANTS[name]
    assert a in src
    ns = dict(vars(oracle))
    exec(src.replace(a, b), ns)
    mutant = ns["prefill_cache"]
    caught = 0
    for pin in PINS:
        try:
            pin(mutant)
        except (AssertionError, IndexError, ValueError):
            caught += 1
    assert caught > 0, f"mutant {name} passes every pin"

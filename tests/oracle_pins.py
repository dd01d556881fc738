"""Pins of the fp64 oracle to facts other than itself.

Each ``pin_*`` function checks the oracle (optionally a library built from a
modified copy of its source, ``lib``) against something the pages or the
mathematics fix: closed forms, invariances, special cases that reduce to a
library routine, and a brute-force formulation. They raise AssertionError on
failure. ``test_oracle.py`` runs them on the real oracle and, as a mutation
test, on copies with plausible mistakes planted in them, each of which must
fail at least one pin.

Page references: the definition is the softmax attention that the tiled kernel
of the "Real-time inference optimisation" page (section "Flash Attention
optimisation") computes; the causal mask and MQA/GQA come from the
FlashRT-HF-kernels page (section "attention optimisation"); page size 16 and
the per-page sum that the merge replaces come from the paged sketch of the
real-time inference page.
"""
from __future__ import annotations

import math

import numpy as np

import oracle
from oracle import brute


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def pin_single_key(lib=None):
    """Skv = 1: the only probability is exp(0)/exp(0) = 1, so o = v_0 exactly."""
    q, k, v = _rand((2, 4, 3, 8), 1), _rand((2, 2, 1, 8), 2), _rand((2, 2, 1, 8), 3)
    for causal in (False,):
        o, lse = oracle.attention(q, k, v, 0.37, causal, lib=lib)
        for h in range(4):
            g = h * 2 // 4
            assert np.array_equal(o[:, h], np.broadcast_to(v[:, g, 0:1, :], o[:, h].shape))
        # log-sum-exp of a single score is the score itself
        s = 0.37 * np.einsum("bhid,bhd->bhi", q, np.repeat(k[:, :, 0, :], 2, axis=1))
        assert np.allclose(lse, s, rtol=0, atol=1e-13)


def pin_constant_v(lib=None):
    """All value rows equal to u: o = u * sum_j p_j = u (rows of P sum to 1)."""
    q, k = _rand((1, 2, 9, 16), 4), _rand((1, 1, 13, 16), 5)
    u = _rand((16,), 6)
    v = np.broadcast_to(u, (1, 1, 13, 16)).copy()
    for causal in (False, True):
        o, _ = oracle.attention(q, k, v, 0.8, causal, lib=lib)
        assert np.max(np.abs(o - u)) < 1e-14


def pin_causal_first_row(lib=None):
    """Causal, Sq = Skv: row 0 sees only key 0, so o[...,0,:] = v[...,0,:] exactly."""
    q, k, v = _rand((2, 2, 7, 8), 7), _rand((2, 2, 7, 8), 8), _rand((2, 2, 7, 8), 9)
    o, _ = oracle.attention(q, k, v, 0.5, True, lib=lib)
    assert np.array_equal(o[:, :, 0, :], v[:, :, 0, :])


def pin_scale_zero_mean(lib=None):
    """scale = 0: all visible scores are equal, so o_i = mean of the visible value
    rows: all Skv rows (non-causal), rows 0..i (causal)."""
    q, k, v = _rand((1, 1, 6, 4), 10), _rand((1, 1, 6, 4), 11), _rand((1, 1, 6, 4), 12)
    o, lse = oracle.attention(q, k, v, 0.0, False, lib=lib)
    assert np.max(np.abs(o[0, 0] - v[0, 0].mean(axis=0))) < 1e-14
    assert np.allclose(lse, math.log(6), atol=1e-14)
    o, lse = oracle.attention(q, k, v, 0.0, True, lib=lib)
    for i in range(6):
        assert np.max(np.abs(o[0, 0, i] - v[0, 0, : i + 1].mean(axis=0))) < 1e-14
        assert abs(lse[0, 0, i] - math.log(i + 1)) < 1e-14


def pin_two_keys_logistic(lib=None):
    """Two keys: the weights are logistic functions of the score difference,
    p_0 = 1 / (1 + exp(s_1 - s_0)). Hand-built scores: q = (a, 0), k_0 = (1, 0),
    k_1 = (0, 1) gives s_0 = scale*a, s_1 = 0."""
    for a, scale in ((1.0, 1.0), (-2.5, 0.5), (3.0, 2.0)):
        q = np.array([a, 0.0]).reshape(1, 1, 1, 2)
        k = np.array([[1.0, 0.0], [0.0, 1.0]]).reshape(1, 1, 2, 2)
        v = np.array([[1.0, 0.0], [0.0, 1.0]]).reshape(1, 1, 2, 2)
        o, lse = oracle.attention(q, k, v, scale, False, lib=lib)
        p0 = 1.0 / (1.0 + math.exp(-scale * a))
        assert abs(o[0, 0, 0, 0] - p0) < 1e-15 and abs(o[0, 0, 0, 1] - (1 - p0)) < 1e-15
        assert abs(lse[0, 0, 0] - math.log(math.exp(scale * a) + 1.0)) < 1e-14


def pin_dominant_key(lib=None):
    """One score far above the rest: o is that key's value row to within exp(-gap)."""
    d = 8
    k = np.eye(d).reshape(1, 1, d, d)
    v = _rand((1, 1, d, d), 13)
    for target in (0, 5):
        q = np.zeros((1, 1, 1, d))
        q[0, 0, 0, target] = 60.0
        o, _ = oracle.attention(q, k, v, 1.0, False, lib=lib)
        assert np.max(np.abs(o[0, 0, 0] - v[0, 0, target])) < 1e-20


def pin_probability_rows(lib=None):
    """With V = identity (one-hot value rows) the output row is the probability
    row itself: entries >= 0, summing to 1 within 1e-14, and zero on masked keys."""
    S = 10
    q, k = _rand((1, 1, S, 5), 14), _rand((1, 1, S, 5), 15)
    v = np.eye(S).reshape(1, 1, S, S)
    # head dim of v must equal that of q/k for the oracle: embed into a common d
    d = S
    qq = np.zeros((1, 1, S, d)); qq[..., :5] = q
    kk = np.zeros((1, 1, S, d)); kk[..., :5] = k
    for causal in (False, True):
        P, _ = oracle.attention(qq, kk, v, 0.9, causal, lib=lib)
        P = P[0, 0]
        assert np.all(P >= 0)
        assert np.max(np.abs(P.sum(axis=1) - 1.0)) < 1e-14
        if causal:
            assert np.all(np.triu(P, 1) == 0.0)
            assert np.all(np.diag(P) > 0)


def pin_shift_invariance(lib=None):
    """Adding the same constant to every score of a row leaves the softmax, and o,
    unchanged: append a coordinate with q = c_i, k = 1 (score shift scale*c_i)."""
    q, k, v = _rand((1, 2, 5, 6), 16), _rand((1, 1, 7, 6), 17), _rand((1, 1, 7, 6), 18)
    c = _rand((1, 2, 5, 1), 19) * 5
    q2 = np.concatenate([q, c], axis=-1)
    k2 = np.concatenate([k, np.ones((1, 1, 7, 1))], axis=-1)
    v2 = np.concatenate([v, np.zeros((1, 1, 7, 1))], axis=-1)
    for causal in (False, True):
        o1, l1 = oracle.attention(q, k, v, 0.7, causal, lib=lib)
        o2, l2 = oracle.attention(q2, k2, v2, 0.7, causal, lib=lib)
        assert np.max(np.abs(o1 - o2[..., :6])) < 1e-13
        assert np.max(np.abs((l2 - l1) - 0.7 * c[..., 0])) < 1e-12


def pin_key_permutation(lib=None):
    """Non-causal attention is a sum over keys: permuting K and V rows together
    leaves o unchanged."""
    q, k, v = _rand((2, 2, 4, 8), 20), _rand((2, 1, 11, 8), 21), _rand((2, 1, 11, 8), 22)
    perm = np.random.default_rng(23).permutation(11)
    o1, _ = oracle.attention(q, k, v, 0.4, False, lib=lib)
    o2, _ = oracle.attention(q, k[:, :, perm], v[:, :, perm], 0.4, False, lib=lib)
    assert np.max(np.abs(o1 - o2)) < 1e-13


def pin_convex_hull(lib=None):
    """Each output coordinate is a convex combination of the visible value rows."""
    q, k, v = _rand((1, 2, 9, 8), 24) * 3, _rand((1, 2, 9, 8), 25), _rand((1, 2, 9, 8), 26)
    o, _ = oracle.attention(q, k, v, 1.0, True, lib=lib)
    for h in range(2):
        for i in range(9):
            lo = v[0, h, : i + 1].min(axis=0) - 1e-14
            hi = v[0, h, : i + 1].max(axis=0) + 1e-14
            assert np.all(o[0, h, i] >= lo) and np.all(o[0, h, i] <= hi)


def pin_gqa_is_repeated_mha(lib=None):
    """GQA with G = Hq/Hkv equals MHA on K/V whose kv head g is repeated G times
    (query head h uses kv head floor(h*Hkv/Hq))."""
    q, k, v = _rand((2, 8, 5, 8), 27), _rand((2, 2, 6, 8), 28), _rand((2, 2, 6, 8), 29)
    for causal in (False, True):
        o1, _ = oracle.attention(q, k, v, 0.6, causal, lib=lib)
        o2, _ = oracle.attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), 0.6, causal, lib=lib)
        assert np.array_equal(o1, o2)
    # and head h really reads kv head h // 4: changing kv head 1 only moves heads 4..7
    k3 = k.copy(); k3[:, 1] += _rand((2, 6, 8), 60)
    o3, _ = oracle.attention(q, k3, v, 0.6, False, lib=lib)
    o1, _ = oracle.attention(q, k, v, 0.6, False, lib=lib)
    assert np.array_equal(o1[:, :4], o3[:, :4]) and not np.allclose(o1[:, 4:], o3[:, 4:])


def pin_brute_force(lib=None):
    """Agreement with the pure-Python fsum formulation on a grid of tiny shapes."""
    rng = np.random.default_rng(30)
    for B in (1, 2):
        for Hq, Hkv in ((1, 1), (2, 1), (2, 2), (4, 2), (4, 1)):
            for Skv in (1, 2, 5):
                for Sq in sorted({1, min(3, Skv), Skv}):
                    for d in (1, 4):
                        for causal in (False, True):
                            q = rng.standard_normal((B, Hq, Sq, d))
                            k = rng.standard_normal((B, Hkv, Skv, d))
                            v = rng.standard_normal((B, Hkv, Skv, d))
                            o, _ = oracle.attention(q, k, v, 0.75, causal, lib=lib)
                            ob = np.array(brute.attention(q.tolist(), k.tolist(), v.tolist(), 0.75, causal))
                            assert np.max(np.abs(o - ob)) < 1e-12, (B, Hq, Hkv, Sq, Skv, d, causal)


def pin_torch_sdpa(lib=None):
    """Library special case: torch's scaled_dot_product_attention on the CPU in
    float64. Its causal mask is top-left aligned, which equals the bottom-right
    reading when Sq == Skv; non-causal is compared for Sq != Skv too."""
    import torch

    for (B, Hq, Hkv, Sq, Skv, d, causal) in ((1, 1, 1, 128, 128, 64, True), (2, 4, 2, 33, 33, 16, True),
                                             (1, 4, 1, 7, 19, 8, False), (2, 2, 2, 16, 16, 32, False),
                                             (1, 2, 1, 40, 40, 96, True), (1, 2, 2, 9, 70, 256, False)):
        q, k, v = _rand((B, Hq, Sq, d), 31), _rand((B, Hkv, Skv, d), 32), _rand((B, Hkv, Skv, d), 33)
        o, _ = oracle.attention(q, k, v, 1.0 / math.sqrt(d), causal, lib=lib)
        G = Hq // Hkv
        tq = torch.from_numpy(q)
        tk = torch.from_numpy(np.repeat(k, G, axis=1))
        tv = torch.from_numpy(np.repeat(v, G, axis=1))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                               scale=1.0 / math.sqrt(d)).numpy()
        assert np.max(np.abs(o - ref)) < 1e-12


def pin_bottom_right_suffix(lib=None):
    """Bottom-right causal alignment (a reading: the pages are silent for
    Sq < Skv) is the one under which the last Sq queries of a causal pass over
    Skv queries give the same rows when run on their own against all Skv keys
    (chunked prefill). Checked here, so the reading is at least self-consistent."""
    Skv, Sq = 12, 5
    qf, k, v = _rand((1, 2, Skv, 8), 34), _rand((1, 1, Skv, 8), 35), _rand((1, 1, Skv, 8), 36)
    of, _ = oracle.attention(qf, k, v, 0.5, True, lib=lib)
    os_, _ = oracle.attention(qf[:, :, Skv - Sq:], k, v, 0.5, True, lib=lib)
    assert np.array_equal(os_, of[:, :, Skv - Sq:])


def pin_decode_is_last_causal_row(lib=None):
    """Decode of the last token equals the last row of causal prefill over the
    same keys (and non-causal attention of that single query)."""
    B, Hq, Hkv, L, d = 2, 4, 2, 9, 8
    q, k, v = _rand((B, Hq, L, d), 37), _rand((B, Hkv, L, d), 38), _rand((B, Hkv, L, d), 39)
    of, lf = oracle.attention(q, k, v, 0.3, True, lib=lib)
    kc = np.ascontiguousarray(k.transpose(0, 2, 1, 3))  # [B, L, Hkv, d]
    vc = np.ascontiguousarray(v.transpose(0, 2, 1, 3))
    od, ld = oracle.decode(q[:, :, -1], kc, vc, np.full((B,), L, np.int32), 0.3, lib=lib)
    assert np.max(np.abs(od - of[:, :, -1])) < 1e-15
    assert np.max(np.abs(ld - lf[:, :, -1])) < 1e-14


def pin_paged_equals_contiguous(lib=None):
    """A shuffled page pool read through the block table gives exactly the
    contiguous-cache result (identical arithmetic, different addresses); the
    per-sequence length cuts the last page."""
    B, Hq, Hkv, d, page = 3, 4, 2, 8, 16
    lens = np.array([37, 16, 1], np.int32)
    Lmax = 48
    q = _rand((B, Hq, d), 40)
    kc, vc = _rand((B, Lmax, Hkv, d), 41), _rand((B, Lmax, Hkv, d), 42)
    pps = Lmax // page
    perm = np.random.default_rng(43).permutation(B * pps).astype(np.int32)
    bt = perm.reshape(B, pps)
    kp = np.empty((B * pps, page, Hkv, d)); vp = np.empty_like(kp)
    kp[bt.reshape(-1)] = kc.reshape(B * pps, page, Hkv, d)
    vp[bt.reshape(-1)] = vc.reshape(B * pps, page, Hkv, d)
    o1, l1 = oracle.decode(q, kc, vc, lens, 0.35, lib=lib)
    o2, l2 = oracle.decode(q, kp, vp, lens, 0.35, block_table=bt, page_size=page, max_kv_len=Lmax, lib=lib)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # the length is honoured: tokens past len_b do not matter
    kc2 = kc.copy(); kc2[0, 37:] = 1e3; vc2 = vc.copy(); vc2[0, 37:] = -1e3
    o3, _ = oracle.decode(q, kc2, vc2, lens, 0.35, lib=lib)
    assert np.array_equal(o1, o3)


def pin_empty_and_clamped_decode(lib=None):
    """A sequence of length 0 has no visible key: output 0 and lse -inf.
    Lengths above max_kv_len are clamped."""
    q = _rand((2, 2, 4), 44)
    kc, vc = _rand((2, 5, 1, 4), 45), _rand((2, 5, 1, 4), 46)
    o, l = oracle.decode(q, kc, vc, np.array([0, 99], np.int32), 1.0, max_kv_len=5, lib=lib)
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(l[0]))
    o5, l5 = oracle.decode(q, kc, vc, np.array([0, 5], np.int32), 1.0, max_kv_len=5, lib=lib)
    assert np.array_equal(o[1], o5[1])


def pin_merge_of_splits(lib=None):
    """Splitting the keys into disjoint chunks, attending to each, and merging by
    log-sum-exp reproduces attention over all keys (within 1e-12), for any split.
    The per-page plain sum of the paged sketch does not."""
    q, k, v = _rand((1, 3, 2, 8), 47), _rand((1, 3, 50, 8), 48), _rand((1, 3, 50, 8), 49)
    o_full, l_full = oracle.attention(q, k, v, 0.6, False, lib=lib)
    rng = np.random.default_rng(50)
    for _ in range(4):
        cuts = np.sort(rng.choice(np.arange(1, 50), size=rng.integers(1, 8), replace=False))
        bounds = [0, *cuts.tolist(), 50]
        parts_o, parts_l = [], []
        for a, b in zip(bounds[:-1], bounds[1:]):
            o_s, l_s = oracle.attention(q, k[:, :, a:b], v[:, :, a:b], 0.6, False, lib=lib)
            parts_o.append(o_s); parts_l.append(l_s)
        S = len(parts_o)
        op = np.stack(parts_o, axis=3).reshape(3 * 2, S, 8)  # [R, S, d] with R = B*H*Sq
        lp = np.stack(parts_l, axis=3).reshape(3 * 2, S)
        om, lm = oracle.merge(op, lp, lib=lib)
        assert np.max(np.abs(om - o_full.reshape(6, 8))) < 1e-12
        assert np.max(np.abs(lm - l_full.reshape(6))) < 1e-12
    # an empty part (lse = -inf) contributes nothing, even with garbage values
    op2 = np.concatenate([op, np.full((6, 1, 8), np.nan)], axis=1)
    lp2 = np.concatenate([lp, np.full((6, 1), -np.inf)], axis=1)
    om2, _ = oracle.merge(op2, lp2, lib=lib)
    assert np.max(np.abs(om2 - o_full.reshape(6, 8))) < 1e-12
    om3, lm3 = oracle.merge(np.zeros((1, 2, 8)), np.full((1, 2), -np.inf), lib=lib)
    assert np.all(om3 == 0) and np.isneginf(lm3[0])


def pin_page_sum_counterexample(lib=None):
    """The paged sketch adds per-page outputs. With the same value row u in every
    one of n pages each page's output is u, so the sum is n*u; the true result
    (and the log-sum-exp merge) is u."""
    n, page, d = 5, 16, 8
    q = _rand((1, 1, 1, d), 51)
    k = _rand((1, 1, n * page, d), 52)
    u = _rand((d,), 53)
    v = np.broadcast_to(u, (1, 1, n * page, d)).copy()
    o_full, _ = oracle.attention(q, k, v, 0.5, False, lib=lib)
    parts = [oracle.attention(q, k[:, :, p * page:(p + 1) * page], v[:, :, p * page:(p + 1) * page], 0.5, False,
                              lib=lib) for p in range(n)]
    page_sum = sum(o for o, _ in parts)
    assert np.max(np.abs(page_sum[0, 0, 0] - n * u)) < 1e-13
    assert np.max(np.abs(o_full[0, 0, 0] - u)) < 1e-14
    om, _ = oracle.merge(np.stack([o for o, _ in parts], axis=3).reshape(1, n, d),
                         np.stack([l for _, l in parts], axis=3).reshape(1, n), lib=lib)
    assert np.max(np.abs(om[0] - u)) < 1e-14


ALL_PINS = [
    pin_single_key, pin_constant_v, pin_causal_first_row, pin_scale_zero_mean, pin_two_keys_logistic,
    pin_dominant_key, pin_probability_rows, pin_shift_invariance, pin_key_permutation, pin_convex_hull,
    pin_gqa_is_repeated_mha, pin_brute_force, pin_torch_sdpa, pin_bottom_right_suffix,
    pin_decode_is_last_causal_row, pin_paged_equals_contiguous, pin_empty_and_clamped_decode,
    pin_merge_of_splits, pin_page_sum_counterexample,
]

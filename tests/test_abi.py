"""The C-ABI library loads, exports every symbol include/fa.h declares, and
rejects invalid calls on the host with the documented status codes.

CPU only: every call below is invalid in exactly one way, so the library
returns before any launch and no GPU is touched.
"""
import os
import re

import pytest

import attention_fa_prefill_amd as fa

pytestmark = pytest.mark.cpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, NULL, SHAPE, UNSUP, ALIGN, WS, HIP, ARG = range(8)
A = 0x10000  # a 16-byte aligned, never dereferenced address


def header_symbols():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    return sorted(set(re.findall(r"^\S.*?\b(fa_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    L = fa.lib()
    declared = header_symbols()
    assert declared, "no declarations found in include/fa.h"
    assert set(declared) == set(fa.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings_and_version():
    for code, name in fa.STATUS_NAMES.items():
        assert fa.status_string(code).startswith(name)
    assert fa.status_string(99) == "FA_ERR_UNKNOWN"
    assert fa.lib().fa_version() == 200


def prefill(fn="fa_prefill", q=A, k=A, v=A, o=A, B=1, Hq=4, Hkv=2, Sq=8, Skv=8, d=128, scale=0.125, causal=1):
    return getattr(fa.lib(), fn)(q, k, v, o, B, Hq, Hkv, Sq, Skv, d, scale, causal, None)


@pytest.mark.parametrize("fn", ["fa_prefill", "fa_prefill_f32"])
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL), (dict(o=None), NULL),
    (dict(B=0), SHAPE), (dict(Hq=0), SHAPE), (dict(Hkv=0), SHAPE), (dict(Sq=0), SHAPE), (dict(Skv=-1), SHAPE),
    (dict(Hq=6, Hkv=4), SHAPE), (dict(Sq=9, Skv=8, causal=1), SHAPE), (dict(B=70000), SHAPE),
    (dict(d=48), UNSUP), (dict(d=80), UNSUP), (dict(d=512), UNSUP), (dict(d=0), SHAPE),
    (dict(scale=float("inf")), ARG), (dict(scale=float("nan")), ARG), (dict(causal=2), ARG),
    (dict(q=A + 8), ALIGN), (dict(k=A + 4), ALIGN), (dict(v=A + 2), ALIGN), (dict(o=A + 1), ALIGN),
])
def test_prefill_rejects(fn, kw, code):
    assert prefill(fn, **kw) == code


def prefill_cache(q=A, kc=A, vc=A, bt=None, lens=A, o=A, B=2, Hq=4, Hkv=2, Sq=8, d=128, L=64, page=16, scale=0.1,
                  causal=1):
    return fa.lib().fa_prefill_cache(q, kc, vc, bt, lens, o, B, Hq, Hkv, Sq, d, L, page, scale, causal, None)


@pytest.mark.parametrize("kw,code", [
    (dict(lens=None), NULL), (dict(q=None), NULL), (dict(Sq=0), SHAPE), (dict(Hq=6, Hkv=4), SHAPE),
    (dict(d=48), UNSUP), (dict(d=80), UNSUP), (dict(d=512), UNSUP), (dict(bt=A, page=32), UNSUP),
    (dict(causal=2), ARG), (dict(scale=float("nan")), ARG), (dict(lens=A + 2), ALIGN), (dict(bt=A + 1), ALIGN),
])
def test_prefill_cache_rejects(kw, code):
    """Host-side checks of fa_prefill_cache."""
    assert prefill_cache(**kw) == code


def decode(q=A, k=A, v=A, bt=None, lens=A, o=A, B=2, Hq=8, Hkv=2, d=128, L=64, page=16, tps=0, scale=0.1,
           ws=A, wsb=None):
    if wsb is None:
        wsb = fa.decode_workspace_bytes(B, Hq, Hkv, d, L, tps) if B > 0 else 0
    return fa.lib().fa_decode(q, k, v, bt, lens, o, B, Hq, Hkv, d, L, page, tps, scale, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL), (dict(lens=None), NULL), (dict(o=None), NULL),
    (dict(B=0, wsb=1 << 20), SHAPE), (dict(Hq=6, Hkv=4), SHAPE), (dict(L=0, wsb=1 << 20), SHAPE),
    (dict(Hkv=0), SHAPE),
    (dict(d=80), UNSUP), (dict(d=48), UNSUP), (dict(d=16), UNSUP), (dict(d=512), UNSUP),
    (dict(bt=A, page=32), UNSUP), (dict(bt=A, page=8), UNSUP),
    (dict(tps=48), ARG), (dict(tps=-32), ARG), (dict(tps=4096), ARG), (dict(scale=float("nan")), ARG),
    (dict(q=A + 2), ALIGN), (dict(k=A + 8), ALIGN), (dict(o=A + 4), ALIGN), (dict(lens=A + 2), ALIGN),
    (dict(bt=A + 1), ALIGN), (dict(ws=A + 8), ALIGN),
    (dict(ws=None), WS), (dict(wsb=16), WS),
])
def test_decode_rejects(kw, code):
    assert decode(**kw) == code


def decode_fp8(ks=0.5, vs=0.5, fn="fa_decode_fp8", **kw):
    a = dict(q=A, k=A, v=A, bt=None, lens=A, o=A, B=2, Hq=8, Hkv=2, d=128, L=64, page=16, tps=0, scale=0.1, ws=A,
             wsb=None)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = fa.decode_workspace_bytes(a["B"], a["Hq"], a["Hkv"], a["d"], a["L"], a["tps"]) if a["B"] > 0 else 0
    return getattr(fa.lib(), fn)(a["q"], a["k"], a["v"], a["bt"], a["lens"], a["o"], a["B"], a["Hq"], a["Hkv"],
                                 a["d"], a["L"], a["page"], a["tps"], a["scale"], ks, vs, a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(ks=0.0), ARG), (dict(ks=-1.0), ARG), (dict(ks=float("nan")), ARG), (dict(ks=float("inf")), ARG),
    (dict(vs=0.0), ARG), (dict(vs=-0.5), ARG), (dict(vs=float("nan")), ARG), (dict(vs=float("inf")), ARG),
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(d=48), UNSUP), (dict(Hq=6, Hkv=4), SHAPE),
    (dict(tps=48), ARG), (dict(k=A + 8), ALIGN), (dict(wsb=16), WS),
])
@pytest.mark.parametrize("fn", ["fa_decode_fp8", "fa_decode_int8"])
def test_decode_byte_cache_rejects(fn, kw, code):
    """The fp8 and int8 entry points check what fa_decode checks, and their
    scales (finite, > 0)."""
    assert decode_fp8(fn=fn, **kw) == code


def noalloc(q=A, k=A, v=A, bt=None, lens=A, o=A, B=2, Hq=8, Hkv=2, d=128, L=64, page=16, tps=0, scale=0.1):
    return fa.lib().fa_decode_noalloc(q, k, v, bt, lens, o, B, Hq, Hkv, d, L, page, tps, scale, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(lens=None), NULL), (dict(B=0), SHAPE), (dict(Hq=6, Hkv=4), SHAPE),
    (dict(d=48), UNSUP), (dict(bt=A, page=32), UNSUP), (dict(tps=48), ARG), (dict(scale=float("inf")), ARG),
    (dict(k=A + 8), ALIGN),
    # partials beyond the 16 MiB device array
    (dict(B=64, Hq=32, Hkv=8, L=32768, tps=64), WS), (dict(B=2, Hq=64, Hkv=8, d=256, L=65536, tps=256), WS),
])
def test_decode_noalloc_rejects(kw, code):
    """fa_decode_noalloc checks what fa_decode checks (without a workspace),
    and rejects sizes whose partials do not fit its device array."""
    assert noalloc(**kw) == code


def test_decode_noalloc_limit_is_16_mib():
    """Every size whose partials need more than 16 MiB is rejected on the host
    (sizes that fit are not called here: they would launch)."""
    lim = 16 << 20
    over = 0
    for B in (1, 2, 4, 8, 16, 32):
        for L, tps in ((32768, 64), (65536, 128), (262144, 256), (16384, 32)):
            need = fa.decode_workspace_bytes(B, 32, 8, 128, L, tps)
            if need > lim:
                assert noalloc(B=B, Hq=32, Hkv=8, L=L, tps=tps) == WS, (B, L, tps, need)
                over += 1
    assert over > 5
    # the boundary: 16 MiB is 2^24 bytes; rows * (128 + 1) * 4 + rounding + 256 crosses it between these two
    assert fa.decode_workspace_bytes(1, 32, 8, 128, 32 * 1016, 32) <= lim
    assert noalloc(B=1, Hq=32, Hkv=8, L=32 * 1017, tps=32) == WS


def test_decode_split_tokens():
    # explicit sizes are returned unchanged, invalid ones give 0
    assert fa.decode_split_tokens(4, 32, 8, 32768, 256) == 256
    assert fa.decode_split_tokens(4, 32, 8, 32768, 2048) == 2048
    for bad in (48, -32, 4096):
        assert fa.decode_split_tokens(4, 32, 8, 32768, bad) == 0
    assert fa.decode_split_tokens(4, 32, 6, 32768, 0) == 0  # Hq % Hkv != 0
    assert fa.decode_split_tokens(0, 32, 8, 32768, 0) == 0
    # default: one split per sequence (max_kv_len rounded up to 32) for
    # max_kv_len <= 512, or for max_kv_len <= 2048 with 8 * streams >= max_kv_len;
    # else the smallest power of two in [64, 1024] with
    # B * Hkv * ceil(G / 16) * ceil(max_kv_len / tps) <= 256 work-groups
    cases = [(4, 32, 8, 32768), (8, 32, 8, 16384), (1, 16, 2, 262144), (1, 8, 8, 1024), (1, 1, 1, 1),
             (2, 64, 2, 4096), (3, 40, 8, 777), (1, 1, 1, 512), (1, 1, 1, 513), (64, 32, 8, 1024),
             (16, 32, 8, 1024), (8, 32, 8, 1024), (32, 32, 8, 2048), (16, 32, 8, 2048), (64, 32, 8, 2049),
             (4, 64, 2, 100), (128, 8, 8, 4096)]
    for B, Hq, Hkv, L in cases:
        t = fa.decode_split_tokens(B, Hq, Hkv, L, 0)
        streams = B * Hkv * (-(-(Hq // Hkv) // 16))
        if L <= 512 or (L <= 2048 and 8 * streams >= L):
            assert t == -(-L // 32) * 32 and t >= L, (B, Hq, Hkv, L, t)
            continue
        fits = [x for x in (64, 128, 256, 512, 1024) if streams * L <= 256 * x]
        assert t == (fits[0] if fits else 1024), (B, Hq, Hkv, L, t)
    assert fa.decode_split_tokens(16, 32, 8, 1024, 0) == 1024   # 128 streams: one launch
    assert fa.decode_split_tokens(8, 32, 8, 1024, 0) == 256     # 64 streams: 4 splits
    # the long-context workload keeps at least 256 splits
    t5 = fa.decode_split_tokens(1, 16, 2, 262144, 0)
    assert -(-262144 // t5) >= 256


def test_decode_workspace_bytes():
    # [B, Hq, nsplit, d] fp32 partials + [B, Hq, nsplit] fp32 lse, each rounded up to 256 bytes,
    # + 256 bytes for the split size the call used
    n = 32768 // 512
    assert fa.decode_workspace_bytes(4, 32, 8, 128, 32768, 512) == 4 * 32 * n * 128 * 4 + 4 * 32 * n * 4 + 256
    t = fa.decode_split_tokens(4, 32, 8, 32768, 0)
    n = -(-32768 // t)
    assert fa.decode_workspace_bytes(4, 32, 8, 128, 32768, 0) == 4 * 32 * n * 128 * 4 + 4 * 32 * n * 4 + 256
    assert fa.decode_workspace_bytes(1, 1, 1, 64, 1, 32) == 256 + 256 + 256
    assert fa.decode_workspace_bytes(0, 1, 1, 64, 1, 32) == 0
    assert fa.decode_workspace_bytes(1, 8, 3, 64, 64, 32) == 0
    n5 = -(-262144 // fa.decode_split_tokens(1, 16, 2, 262144, 0))
    assert fa.decode_workspace_bytes(1, 16, 2, 128, 262144, 0) == 16 * n5 * 128 * 4 + 16 * n5 * 4 + 256


@pytest.mark.parametrize("kw,code", [
    (dict(op=None), NULL), (dict(lse=None), NULL), (dict(o=None), NULL),
    (dict(R=0), SHAPE), (dict(S=0), SHAPE), (dict(d=16), UNSUP), (dict(d=48), UNSUP), (dict(d=512), UNSUP),
    (dict(op=A + 4), ALIGN), (dict(o=A + 8), ALIGN), (dict(lse=A + 2), ALIGN), (dict(lo=A + 1), ALIGN),
])
def test_merge_rejects(kw, code):
    a = dict(op=A, lse=A, o=A, lo=None, R=4, S=3, d=128)
    a.update(kw)
    assert fa.lib().fa_merge_lse(a["op"], a["lse"], a["o"], a["lo"], a["R"], a["S"], a["d"], 1, None) == code


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.prefill(q, q, q)
    with pytest.raises(ValueError):
        fa.decode(torch.zeros(1, 1, 64, dtype=torch.bfloat16), torch.zeros(1, 16, 1, 64, dtype=torch.bfloat16),
                  torch.zeros(1, 16, 1, 64, dtype=torch.bfloat16), torch.zeros(1, dtype=torch.int32))


def test_product_code_does_not_touch_the_oracle():
    """The HIP library and its binding never import, link or run oracle/."""
    pkg = os.path.join(ROOT, "attention_fa_prefill_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text and "liboracle" not in text, f

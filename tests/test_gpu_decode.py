"""GPU parity of fa_decode (split-KV + log-sum-exp merge) and fa_merge_lse.

Full-size contiguous, paged and long-context workloads are compared element by
element with the fp64 oracle; the paged path is checked to reproduce the
contiguous path bit for bit on the same data; poisoned cache slots (NaN past
each sequence's length and in unused pages) must not reach the output.
"""
import dataclasses
import math

import numpy as np
import pytest

import attention_fa_prefill_amd as fa
import oracle
import workloads
from tests.gpu_util import (F32_MAX_ABS, assert_bf16_close, dev_bf16, dev_f32, dev_i32, host_bits, host_f64,
                            torch_gpu)

pytestmark = pytest.mark.gpu


def run(case, tps=0):
    torch_gpu()
    print(f"case {case.name} paged={case.paged} tps={tps}", flush=True)
    q, kc, vc = dev_bf16(case.q), dev_bf16(case.kcache), dev_bf16(case.vcache)
    lens = dev_i32(case.seqlens)
    bt = dev_i32(case.block_table) if case.paged else None
    return fa.decode(q, kc, vc, lens, block_table=bt, max_kv_len=case.max_kv_len, scale=case.scale,
                     tokens_per_split=tps)


def oracle_out(case):
    q, kc, vc = (workloads.bf16_bits_to_f64(x) for x in (case.q, case.kcache, case.vcache))
    o, _ = oracle.decode(q, kc, vc, case.seqlens, case.scale, block_table=case.block_table,
                         max_kv_len=case.max_kv_len)
    return o


def test_contiguous_decode_32k_full_size():
    case = workloads.decode_contig_32k()
    o = run(case)
    assert_bf16_close(host_f64(o), oracle_out(case), case.name)


def test_paged_decode_mixed_lengths_full_size():
    case = workloads.decode_paged_mixed()
    o = run(case)
    assert_bf16_close(host_f64(o), oracle_out(case), case.name)


def test_long_context_paged_decode_256k_full_size():
    """256k tokens in shuffled pages, split into at least 256 chunks merged by
    log-sum-exp: the number of chunks is read back from the split size the
    kernel reports in the workspace (the size it chose on the device)."""
    torch = torch_gpu()
    case = workloads.decode_long_256k()
    t0 = fa.decode_split_tokens(case.B, case.Hq, case.Hkv, case.max_kv_len, 0)
    need = fa.decode_workspace_bytes(case.B, case.Hq, case.Hkv, case.d, case.max_kv_len, 0)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    print(f"case {case.name} default split size, t0={t0}", flush=True)
    o = fa.decode(dev_bf16(case.q), dev_bf16(case.kcache), dev_bf16(case.vcache), dev_i32(case.seqlens),
                  block_table=dev_i32(case.block_table), max_kv_len=case.max_kv_len, scale=case.scale, workspace=ws)
    torch.cuda.synchronize()
    used = int(ws[_split_size_offset(case, t0):][:4].view(torch.int32).item())
    chunks = -(-int(case.seqlens[0]) // used)
    print(f"split size used {used}: {chunks} chunks per kv head", flush=True)
    assert chunks >= 256
    assert_bf16_close(host_f64(o), oracle_out(case), case.name)


def test_paged_equals_contiguous_bitwise_32k():
    """The contiguous 32k cache scattered into a shuffled page pool: same bits out."""
    case = workloads.decode_contig_32k()
    paged = workloads.paged_from_contiguous(case)
    o1 = run(case)
    o2 = run(paged)
    assert np.array_equal(host_bits(o1), host_bits(o2))


def test_contiguous_equals_paged_bitwise_mixed():
    """The mixed-length page pool gathered into a padded contiguous cache (on the
    device, by plain indexing): same bits out, for two split sizes."""
    torch = torch_gpu()
    case = workloads.decode_paged_mixed()
    B, L = case.B, case.max_kv_len
    pool_k, pool_v = dev_bf16(case.kcache), dev_bf16(case.vcache)
    bt = dev_i32(case.block_table).long()
    kc = pool_k[bt.reshape(-1)].reshape(B, L, case.Hkv, case.d).contiguous()
    vc = pool_v[bt.reshape(-1)].reshape(B, L, case.Hkv, case.d).contiguous()
    q, lens = dev_bf16(case.q), dev_i32(case.seqlens)
    for tps in (0, 256):
        o_paged = run(case, tps)
        o_contig = fa.decode(q, kc, vc, lens, max_kv_len=L, scale=case.scale, tokens_per_split=tps)
        assert np.array_equal(host_bits(o_paged), host_bits(o_contig))


def test_poisoned_slots_do_not_leak():
    """NaN in tail slots past each length and in unused pages: output finite and
    bitwise equal to the unpoisoned run; canaries around o unchanged."""
    torch = torch_gpu()
    lens = np.array([1, 15, 16, 17, 31, 33, 100, 513], np.int32)
    clean = workloads.decode_paged(8, 8, 2, 128, lens, 640, seed=21)
    dirty = workloads.decode_paged(8, 8, 2, 128, lens, 640, seed=21, poison=True)
    o_clean = run(clean)
    q, kc, vc = dev_bf16(dirty.q), dev_bf16(dirty.kcache), dev_bf16(dirty.vcache)
    n = q.numel()
    buf = torch.full((n + 512,), -77.0, dtype=torch.bfloat16, device="cuda")
    o = buf[256:256 + n].view(q.shape)
    fa.decode(q, kc, vc, dev_i32(dirty.seqlens), block_table=dev_i32(dirty.block_table), max_kv_len=640,
              scale=dirty.scale, o=o)
    torch.cuda.synchronize()
    assert torch.all(buf[:256] == -77.0) and torch.all(buf[256 + n:] == -77.0)
    assert np.array_equal(host_bits(o), host_bits(o_clean))
    assert_bf16_close(host_f64(o), oracle_out(clean), "poisoned")


def test_contiguous_poisoned_tail():
    lens = np.array([0, 1, 47, 64], np.int32)
    case = workloads.decode_contiguous(4, 4, 4, 64, 64, seqlens=lens, seed=22, poison=True)
    o = run(case)
    got = host_f64(o)
    assert np.all(got[0] == 0.0)  # length 0: empty sum
    assert_bf16_close(got, oracle_out(case), case.name)


@pytest.mark.parametrize("G,Hkv,d", [(1, 4, 128), (4, 2, 64), (8, 1, 128), (16, 1, 128), (32, 1, 128), (5, 2, 64)])
@pytest.mark.parametrize("tps", [0, 32, 1024])
def test_head_groups_and_split_sizes(G, Hkv, d, tps):
    lens = np.array([1, 16, 200, 1500], np.int32)
    case = workloads.decode_paged(4, G * Hkv, Hkv, d, lens, 1536, seed=G * 100 + d + tps)
    o = run(case, tps)
    assert_bf16_close(host_f64(o), oracle_out(case), f"{case.name} G={G} tps={tps}")


@pytest.mark.parametrize("B", [300, 4096, 4100])
def test_many_short_sequences(B):
    """Large batches of short mixed-length sequences (zeros included). Up to
    4096 sequences the live splits are numbered densely by a scan over all
    lengths in every work-group (16 sequences per thread at 4096); above that
    the plain numbering is used. Either way every split must be covered once."""
    lens = np.random.default_rng(B).integers(0, 97, size=B).astype(np.int32)
    case = workloads.decode_contiguous(B, 2, 1, 64, 96, seqlens=lens, seed=31, poison=True)
    o = run(case, 32)
    got = host_f64(o)
    assert np.all(got[lens == 0] == 0.0)
    assert_bf16_close(got, oracle_out(case), f"B={B}")


def test_b1_chat_length_workload():
    """The bench's latency case: one sequence of 4096 cached tokens (B = 1,
    Hq = 32, Hkv = 8, paged), every element against the oracle."""
    case = workloads.decode_b1_chat()
    assert_bf16_close(host_f64(run(case)), oracle_out(case), case.name)


@pytest.mark.parametrize("lens,cap", [([1000], 8192), ([4000], 4096), ([1000, 1, 0, 3000], 4096), ([200, 17], 512)],
                         ids=["one_sequence_short", "one_sequence_full", "batch", "one_launch"])
def test_table_entries_past_the_last_page_are_not_used(lens, cap):
    """Block-table entries at or past ceil(len / 16) may hold anything (one
    sequence: they are read, within the row, before the length): with page
    numbers far out of range there, the output is bit for bit the output with
    the generator's entries, and matches the oracle."""
    case = workloads.decode_paged(len(lens), 16, 4, 128, np.array(lens, np.int32), cap, seed=53)
    ref = host_bits(run(case))
    bt = case.block_table.copy()
    for b, L in enumerate(lens):
        n = -(-L // 16)
        bt[b, n:] = np.where(np.arange(bt.shape[1] - n) % 2 == 0, np.int32(2**31 - 1), np.int32(-(2**31)))
    junk = dataclasses.replace(case, block_table=bt)
    got = run(junk)
    assert np.array_equal(host_bits(got), ref)
    assert_bf16_close(host_f64(got), oracle_out(case), case.name)


def test_seqlens_clamped_to_capacity():
    lens = np.array([5000, -3], np.int32)  # above capacity and negative
    case = workloads.decode_contiguous(2, 4, 2, 128, 96, seqlens=lens, seed=23)
    o = run(case)
    got = host_f64(o)
    assert np.all(got[1] == 0.0)
    assert_bf16_close(got, oracle_out(case), "clamped")


def test_decode_equals_last_row_of_causal_prefill():
    """One decode step over L cached tokens equals row L-1 of a causal prefill
    over the same keys (both against the oracle and with each other)."""
    torch = torch_gpu()
    L, Hq, Hkv, d = 700, 8, 2, 128
    pc = workloads.prefill_case(1, Hq, Hkv, L, L, d, True, "bf16", seed=24)
    o_pre = fa.prefill(dev_bf16(pc.q), dev_bf16(pc.k), dev_bf16(pc.v), causal=True, scale=pc.scale)
    kc = np.ascontiguousarray(pc.k.transpose(0, 2, 1, 3))
    vc = np.ascontiguousarray(pc.v.transpose(0, 2, 1, 3))
    o_dec = fa.decode(dev_bf16(np.ascontiguousarray(pc.q[:, :, -1])), dev_bf16(kc), dev_bf16(vc),
                      dev_i32(np.array([L], np.int32)), scale=pc.scale)
    ref, _ = oracle.attention(*pc.as_f64(), pc.scale, True)
    assert_bf16_close(host_f64(o_dec), ref[:, :, -1], "decode")
    assert np.max(np.abs(host_f64(o_dec) - host_f64(o_pre)[:, :, -1])) <= 2e-2


def test_decode_deterministic():
    case = workloads.decode_paged(2, 16, 2, 128, np.array([3000, 777], np.int32), 4096, seed=25)
    assert np.array_equal(host_bits(run(case)), host_bits(run(case)))


def test_merge_lse_against_oracle():
    torch = torch_gpu()
    rng = np.random.default_rng(26)
    R, S, d = 37, 19, 128
    op = rng.standard_normal((R, S, d)).astype(np.float32)
    ls = (rng.standard_normal((R, S)) * 4).astype(np.float32)
    ls[3, :5] = -np.inf
    op[3, :5] = np.nan  # empty splits are never read
    ls[7, :] = -np.inf  # all-empty row
    o, lse_out = fa.merge_lse(dev_f32(op), dev_f32(ls), out_dtype=torch.float32)
    ref_o, ref_l = oracle.merge(op.astype(np.float64), ls.astype(np.float64))
    got = host_f64(o)
    assert np.all(got[7] == 0.0) and np.isneginf(host_f64(lse_out)[7])
    ok = np.arange(R) != 7
    assert np.max(np.abs(got[ok] - ref_o[ok])) <= F32_MAX_ABS
    assert np.max(np.abs(host_f64(lse_out)[ok] - ref_l[ok])) <= F32_MAX_ABS
    ob, _ = fa.merge_lse(dev_f32(op), dev_f32(ls))
    assert_bf16_close(host_f64(ob)[ok], ref_o[ok], "merge bf16")


def test_merge_lse_many_splits():
    """More splits than one round of the merge covers, with the maximum rising
    across rounds (so partial sums are rescaled) and scattered empty splits."""
    torch = torch_gpu()
    rng = np.random.default_rng(29)
    R, S, d = 5, 600, 64
    op = rng.standard_normal((R, S, d)).astype(np.float32)
    ls = (np.linspace(-40.0, 40.0, S)[None, :] + rng.standard_normal((R, S)) * 3).astype(np.float32)
    ls[1] = ls[1][::-1]  # maximum first
    ls[2, ::7] = -np.inf
    op[2, ::7] = np.nan
    o, lse_out = fa.merge_lse(dev_f32(op), dev_f32(ls), out_dtype=torch.float32)
    ref_o, ref_l = oracle.merge(op.astype(np.float64), ls.astype(np.float64))
    assert np.max(np.abs(host_f64(o) - ref_o)) <= F32_MAX_ABS
    assert np.max(np.abs(host_f64(lse_out) - ref_l)) <= F32_MAX_ABS


def test_merge_rejects_page_sum():
    """Constant value rows over many splits: the merge returns that row (the
    paged sketch's per-page sum would return it times the split count)."""
    torch = torch_gpu()
    u = np.random.default_rng(27).standard_normal(64).astype(np.float32)
    S = 9
    op = np.broadcast_to(u, (2, S, 64)).copy()
    ls = np.random.default_rng(28).standard_normal((2, S)).astype(np.float32)
    o, _ = fa.merge_lse(dev_f32(op), dev_f32(ls), out_dtype=torch.float32)
    assert np.max(np.abs(host_f64(o) - u)) < 1e-6


def _split_size_offset(case, t0):
    """Byte offset of the split-size slot in the workspace: after the fp32
    partials [B, Hq, n, d] and their lse [B, Hq, n], each rounded up to 256."""
    r = lambda x: -(-x // 256) * 256
    rows = case.B * case.Hq * -(-case.max_kv_len // t0)
    return r(rows * case.d * 4) + r(rows * 4)


def _default_split_size(case, t0, cap):
    """The split size fa_decode picks on the device with tokens_per_split = 0:
    of t0 * {1, 5/4, 3/2, 2} (multiples of 32, at most 2048), the one with the
    fewest tokens per resident work-group slot over the rounds the live splits
    need, the smallest on a tie."""
    G = case.Hq // case.Hkv
    gh = case.Hkv * -(-G // 16)
    lens = np.clip(np.asarray(case.seqlens, dtype=np.int64), 0, case.max_kv_len)
    best = None
    for q4 in (4, 5, 6, 8):
        t = min(2048, -(-(t0 * q4 // 4) // 32) * 32)
        n = gh * int(np.sum(-(-lens // t)))
        cost = -(-n // cap) * t
        if best is None or cost < best[0]:
            best = (cost, t)
    return best[1]


def _one_sequence_72k():
    """B = 1 with 8 kv heads and 72k tokens: 576 splits of the default 1024
    tokens overrun one round of resident work-groups; 1280 fit one."""
    return workloads.decode_paged(1, 32, 8, 128, np.array([73728], np.int32), 73728, seed=47,
                                  name="decode_b1h32x8kv72kd128")


@pytest.mark.parametrize("make", [workloads.decode_contig_32k, workloads.decode_paged_mixed,
                                  workloads.decode_long_256k, _one_sequence_72k])
def test_default_split_size_chosen_on_device(make):
    """With the default split size the kernel picks its split size from seqlens;
    the size it reports in the workspace follows the documented rule, and the
    output is bit for bit the output of an explicit call with that size."""
    torch = torch_gpu()
    case = make()
    q, kc, vc = dev_bf16(case.q), dev_bf16(case.kcache), dev_bf16(case.vcache)
    lens = dev_i32(case.seqlens)
    bt = dev_i32(case.block_table) if case.paged else None
    t0 = fa.decode_split_tokens(case.B, case.Hq, case.Hkv, case.max_kv_len, 0)
    need = fa.decode_workspace_bytes(case.B, case.Hq, case.Hkv, case.d, case.max_kv_len, 0)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    print(f"case {case.name} default split size, t0={t0}", flush=True)
    o_auto = fa.decode(q, kc, vc, lens, block_table=bt, max_kv_len=case.max_kv_len, scale=case.scale, workspace=ws)
    torch.cuda.synchronize()
    used = int(ws[_split_size_offset(case, t0):][:4].view(torch.int32).item())
    cap = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    assert used == _default_split_size(case, t0, cap)
    o_explicit = fa.decode(q, kc, vc, lens, block_table=bt, max_kv_len=case.max_kv_len, scale=case.scale,
                           tokens_per_split=used)
    assert np.array_equal(host_bits(o_auto), host_bits(o_explicit))


def test_many_splits_and_empty_sequence():
    """66, 22, 0 and 2 splits of 32 tokens in one batch (an empty sequence
    gives o = 0)."""
    lens = np.array([2100, 700, 0, 33], np.int32)
    case = workloads.decode_paged(4, 8, 2, 128, lens, 2112, seed=41)
    o = run(case, 32)
    got = host_f64(o)
    assert np.all(got[2] == 0.0)
    assert_bf16_close(got, oracle_out(case), "many splits")


def test_workspace_needs_no_initialisation():
    """A workspace of random bytes works, and calls with other lengths on the
    same workspace follow."""
    torch = torch_gpu()
    L = 1536
    need = fa.decode_workspace_bytes(4, 8, 2, 128, L, 32)
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda")
    for i, lens in enumerate(([1500, 1, 700, 64], [33, 1536, 0, 900], [1500, 1, 700, 64])):
        case = workloads.decode_paged(4, 8, 2, 128, np.array(lens, np.int32), L, seed=50 + i)
        print(f"call {i} lens={lens}", flush=True)
        o = fa.decode(dev_bf16(case.q), dev_bf16(case.kcache), dev_bf16(case.vcache), dev_i32(case.seqlens),
                      block_table=dev_i32(case.block_table), max_kv_len=L, scale=case.scale, tokens_per_split=32,
                      workspace=ws)
        assert_bf16_close(host_f64(o), oracle_out(case), f"call {i}")


def test_graph_capture_replays():
    """fa_decode (split kernel, then merge kernel) captured in a HIP graph:
    every replay, with eager work and synchronisations between replays and new
    lengths written into seqlens in place, equals the eager call on the same
    inputs bit for bit."""
    torch = torch_gpu()
    case = workloads.decode_paged_mixed()
    q, kc, vc = dev_bf16(case.q), dev_bf16(case.kcache), dev_bf16(case.vcache)
    lens = dev_i32(case.seqlens)
    bt = dev_i32(case.block_table)
    L = case.max_kv_len
    need = fa.decode_workspace_bytes(case.B, case.Hq, case.Hkv, case.d, L, 0)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream, as graph capture asks
        fa.decode(q, kc, vc, lens, block_table=bt, max_kv_len=L, scale=case.scale, o=o, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.decode(q, kc, vc, lens, block_table=bt, max_kv_len=L, scale=case.scale, o=o, workspace=ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for rep in range(4):
        new_lens = case.seqlens if rep % 2 == 0 else rng.integers(0, L + 1, size=case.B).astype(np.int32)
        lens.copy_(torch.from_numpy(np.ascontiguousarray(new_lens, dtype=np.int32)))
        x = torch.randn(1 << 20, device="cuda")
        (x * 2 + 1).sum().item()  # eager work between replays
        print(f"replay {rep} lens={new_lens.tolist()}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        ref = fa.decode(q, kc, vc, lens, block_table=bt, max_kv_len=L, scale=case.scale)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(o), host_bits(ref)), f"replay {rep}"


# --------------------------------------------------------------------------- FP8 E4M3 cache


def dev_u8(codes):
    torch = torch_gpu()
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).to("cuda")


def run_fp8(case, tps=0):
    torch_gpu()
    print(f"case {case.name} paged={case.paged} tps={tps} ks={case.k_scale} vs={case.v_scale}", flush=True)
    q, kc, vc = dev_bf16(case.q), dev_u8(case.kcache), dev_u8(case.vcache)
    lens = dev_i32(case.seqlens)
    bt = dev_i32(case.block_table) if case.paged else None
    return fa.decode_fp8(q, kc, vc, lens, k_scale=case.k_scale, v_scale=case.v_scale, block_table=bt,
                         max_kv_len=case.max_kv_len, scale=case.scale, tokens_per_split=tps)


def oracle_out_fp8(case):
    q = workloads.bf16_bits_to_f64(case.q)
    o, _ = oracle.decode_fp8(q, case.kcache, case.vcache, case.seqlens, case.scale, case.k_scale, case.v_scale,
                             block_table=case.block_table, max_kv_len=case.max_kv_len)
    return o


@pytest.mark.parametrize("make", [workloads.decode_contig_32k, workloads.decode_paged_mixed,
                                  workloads.decode_long_256k])
def test_fp8_full_size(make):
    case = workloads.as_fp8(make())
    o = run_fp8(case)
    assert_bf16_close(host_f64(o), oracle_out_fp8(case), case.name)


def test_fp8_paged_equals_contiguous_bitwise():
    case = workloads.as_fp8(workloads.decode_contiguous(4, 16, 4, 128, 4096, seed=61))
    paged = workloads.paged_from_contiguous(case)
    assert paged.fp8
    assert np.array_equal(host_bits(run_fp8(case)), host_bits(run_fp8(paged)))


def test_fp8_equals_bf16_on_the_dequantised_cache():
    """With power-of-two scales the dequantised cache is exact in bf16, the K
    scale folds exactly into the softmax factor and the V scale into the
    output: the fp8 path must give the bf16 path's result bit for bit."""
    case = workloads.as_fp8(workloads.decode_paged_mixed(), k_scale=0.5, v_scale=0.25)
    deq_k = workloads.f32_to_bf16_bits((oracle.e4m3_to_f64(case.kcache) * 0.5).astype(np.float32))
    deq_v = workloads.f32_to_bf16_bits((oracle.e4m3_to_f64(case.vcache) * 0.25).astype(np.float32))
    o8 = run_fp8(case)
    o16 = fa.decode(dev_bf16(case.q), dev_bf16(deq_k), dev_bf16(deq_v), dev_i32(case.seqlens),
                    block_table=dev_i32(case.block_table), max_kv_len=case.max_kv_len, scale=case.scale)
    assert np.array_equal(host_bits(o8), host_bits(o16))


@pytest.mark.parametrize("G,Hkv,d", [(1, 4, 128), (4, 2, 64), (8, 1, 128), (32, 1, 128), (5, 2, 64)])
@pytest.mark.parametrize("tps", [0, 32, 1024])
def test_fp8_head_groups_and_split_sizes(G, Hkv, d, tps):
    lens = np.array([1, 16, 200, 1500], np.int32)
    case = workloads.as_fp8(workloads.decode_paged(4, G * Hkv, Hkv, d, lens, 1536, seed=G * 100 + d + tps + 7))
    o = run_fp8(case, tps)
    assert_bf16_close(host_f64(o), oracle_out_fp8(case), f"{case.name} G={G} tps={tps}")


@pytest.mark.parametrize("ks,vs,scale", [(0.02, 3.0, None), (4.0, 0.01, None), (0.35, 0.6, -0.09), (1.0, 1.0, 0.0)])
def test_fp8_scales(ks, vs, scale):
    base = workloads.decode_paged(3, 8, 2, 128, np.array([700, 33, 1], np.int32), 768, seed=71)
    case = workloads.as_fp8(base, k_scale=ks, v_scale=vs)
    if scale is not None:
        case.scale = scale
    o = run_fp8(case, 64)
    assert_bf16_close(host_f64(o), oracle_out_fp8(case), f"ks={ks} vs={vs} scale={scale}")


def test_fp8_poisoned_slots_do_not_leak():
    """NaN codes in tail slots past each length and in unused pages: output
    finite and equal to the unpoisoned run bit for bit."""
    lens = np.array([1, 15, 16, 17, 31, 33, 100, 513], np.int32)
    clean = workloads.as_fp8(workloads.decode_paged(8, 8, 2, 128, lens, 640, seed=21), seed=5)
    dirty = workloads.as_fp8(workloads.decode_paged(8, 8, 2, 128, lens, 640, seed=21, poison=True), seed=5)
    assert np.sum(dirty.kcache == workloads.FP8_NAN) > 0
    o_clean, o_dirty = run_fp8(clean), run_fp8(dirty)
    assert np.all(np.isfinite(host_f64(o_dirty)))
    assert np.array_equal(host_bits(o_dirty), host_bits(o_clean))
    assert_bf16_close(host_f64(o_dirty), oracle_out_fp8(clean), "fp8 poisoned")


# Code classes for the every-code tests, each with power-of-two scales (so that
# every dequantised value is a bf16 value) sized to keep the scores of order 1:
# every finite code; the zeros, subnormals and two smallest binades (exponent
# fields 0..2, where a subnormal decoded as a normal or as zero would move K
# and V by up to their own size); the largest binades (fields 9..15, up to 448).
FP8_CODE_CLASSES = {
    "every_finite_code": (workloads.E4M3_FINITE, 2.0 ** -6, 2.0 ** -6),
    "subnormals_and_fields_0_to_2": (workloads.e4m3_codes_by_exponent(0, 2), 2.0 ** 5, 2.0 ** 5),
    "fields_9_to_15_up_to_448": (workloads.e4m3_codes_by_exponent(9, 15), 2.0 ** -7, 2.0 ** -7),
}


@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
@pytest.mark.parametrize("cls", list(FP8_CODE_CLASSES))
def test_fp8_every_code(cls, paged):
    """Every code of the class appears among the tokens read, in K and in V. The
    result matches the oracle (which decodes by the format's definition) at the
    bf16 bar, and equals bit for bit fa_decode over the dequantised bf16 cache."""
    codes, ks, vs = FP8_CODE_CLASSES[cls]
    base = workloads.decode_contiguous(4, 8, 2, 128, 2048, seqlens=np.array([700, 2048, 33, 1500], np.int32),
                                       seed=81)
    case = workloads.fp8_every_code(base, codes, ks, vs, seed=82)
    for cache in (case.kcache, case.vcache):
        seen = set()
        for b in range(case.B):
            seen |= set(np.unique(cache[b, : int(case.seqlens[b])]).tolist())
        assert seen == set(codes.tolist())
    if paged:
        case = workloads.paged_from_contiguous(case)
    o = run_fp8(case)
    assert_bf16_close(host_f64(o), oracle_out_fp8(case), f"{case.name} {cls}")
    deq_k = workloads.f32_to_bf16_bits((oracle.e4m3_to_f64(case.kcache) * ks).astype(np.float32))
    deq_v = workloads.f32_to_bf16_bits((oracle.e4m3_to_f64(case.vcache) * vs).astype(np.float32))
    bt = dev_i32(case.block_table) if case.paged else None
    o16 = fa.decode(dev_bf16(case.q), dev_bf16(deq_k), dev_bf16(deq_v), dev_i32(case.seqlens), block_table=bt,
                    max_kv_len=case.max_kv_len, scale=case.scale)
    assert np.array_equal(host_bits(o), host_bits(o16))


@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
@pytest.mark.parametrize("vs", [1.0, 2.0 ** -3])
def test_fp8_single_token_gives_every_v_code_exactly(paged, vs):
    """With one cached token its softmax weight is exactly 1, so each output row
    is that token's V row, v_scale * E4M3(code), exactly. The two sequences' V
    rows hold every finite code (and two zeros): the V decoding is checked value
    for value against the format's definition, subnormals and +-448 included."""
    base = workloads.decode_contiguous(2, 4, 1, 128, 16, seqlens=np.ones(2, np.int32), seed=83)
    case = workloads.as_fp8(base, k_scale=0.5, v_scale=vs, seed=84)
    row_codes = workloads.rng(84, 9).permutation(np.concatenate([workloads.E4M3_FINITE, [0x00, 0x80]]))
    case.vcache[:, 0, 0, :] = row_codes.astype(np.uint8).reshape(2, 128)
    if paged:
        case = workloads.paged_from_contiguous(case)
    got = host_f64(run_fp8(case, 32))
    want = (oracle.e4m3_to_f64(row_codes).reshape(2, 1, 128) * vs).repeat(4, axis=1)
    assert np.array_equal(got, want)
    assert np.array_equal(got, oracle_out_fp8(case))

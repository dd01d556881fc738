"""GPU tests of decode in one launch. When every sequence fits one split
(max_kv_len <= the split size: the default gives this for batches of 512 or
more (sequence, kv head) pairs with max_kv_len <= 1024, or an explicit
tokens_per_split >= max_kv_len), the split kernel writes o itself and no
merge kernel runs: per-call launch overhead is what bounds small and
short-context decode (FlashRT summary, per-call overhead and graph replay).

The one-launch result must equal, bit for bit, the two-kernel path on the
same sequences (a capacity twice as large makes two splits per row, the
second always empty, so the merge runs with a single live split of weight
exactly 1), and the oracle to the bf16 bar.
"""
import dataclasses

import numpy as np
import pytest

import attention_fa_prefill_amd as fa
import workloads
from tests.gpu_util import assert_bf16_close, dev_bf16, dev_i32, host_bits, host_f64, torch_gpu
from tests.test_gpu_decode import oracle_out, oracle_out_fp8, run, run_fp8
from tests.test_gpu_decode_int8 import oracle_out as oracle_out_int8, run_int8

pytestmark = pytest.mark.gpu

FORMATS = {
    "bf16": (lambda c: c, run, oracle_out),
    "fp8": (workloads.as_fp8, run_fp8, oracle_out_fp8),
    "int8": (workloads.as_int8, run_int8, oracle_out_int8),
}


def widened(case, max_kv_len):
    """The same paged case at a larger capacity: the block table gains
    columns (pointing at page 0; never read, since no length exceeds the old
    capacity)."""
    bt = np.zeros((case.B, -(-max_kv_len // 16)), np.int32)
    bt[:, : case.block_table.shape[1]] = case.block_table
    return dataclasses.replace(case, max_kv_len=max_kv_len, block_table=bt, name=case.name + f"_cap{max_kv_len}")


def short_lengths(seed, B, hi):
    lens = workloads.rng(seed, 20).integers(0, hi + 1, size=B).astype(np.int32)
    lens[:6] = [0, 1, 16, 17, hi, hi - 1]
    return lens


@pytest.mark.parametrize("fmt", sorted(FORMATS))
def test_one_launch_equals_two_kernel_path(fmt):
    """B = 64, Hq = 32, Hkv = 8, d = 128, lengths 0..1024: the default split
    size gives one split per sequence."""
    make, runner, ref = FORMATS[fmt]
    B, Hq, Hkv, d, cap = 64, 32, 8, 128, 1024
    assert fa.decode_split_tokens(B, Hq, Hkv, cap, 0) >= cap  # one split: one launch
    case = make(workloads.decode_paged(B, Hq, Hkv, d, short_lengths(70, B, cap), cap, seed=70))
    o1 = runner(case)
    wide = widened(case, 2 * cap)
    o2 = runner(wide, cap)  # two splits per row: split kernel + merge
    assert np.array_equal(host_bits(o1), host_bits(o2))
    got = host_f64(o1)
    assert np.all(got[case.seqlens == 0] == 0.0)
    assert_bf16_close(got, ref(case), case.name)


@pytest.mark.parametrize("d", [32, 64, 96, 256])
def test_one_launch_head_dims(d):
    B, Hq, Hkv, cap = 24, 16, 4, 512
    case = workloads.decode_paged(B, Hq, Hkv, d, short_lengths(71 + d, B, cap), cap, seed=71 + d)
    o1 = run(case, cap)  # explicit split size = capacity: one launch
    o2 = run(widened(case, 2 * cap), cap)
    assert np.array_equal(host_bits(o1), host_bits(o2))
    assert_bf16_close(host_f64(o1), oracle_out(case), case.name)


@pytest.mark.parametrize("G,Hkv", [(1, 4), (5, 2), (16, 1), (32, 1)])
def test_one_launch_head_groups(G, Hkv):
    B, cap = 16, 256
    case = workloads.decode_paged(B, G * Hkv, Hkv, 128, short_lengths(80 + G, B, cap), cap, seed=80 + G)
    o1 = run(case, cap)
    assert np.array_equal(host_bits(o1), host_bits(run(widened(case, 2 * cap), cap)))
    assert_bf16_close(host_f64(o1), oracle_out(case), case.name)


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_one_launch_byte_cache_d64(fmt):
    """d = 64 over a one-byte cache: 64-byte row slices, the work-groups of
    neighbouring kv heads grouped on one XCD."""
    make, runner, ref = FORMATS[fmt]
    B, cap = 24, 512
    case = make(workloads.decode_paged(B, 16, 4, 64, short_lengths(85, B, cap), cap, seed=85))
    o1 = runner(case, cap)
    assert np.array_equal(host_bits(o1), host_bits(runner(widened(case, 2 * cap), cap)))
    assert_bf16_close(host_f64(o1), ref(case), case.name)


def test_one_launch_contiguous_equals_paged():
    lens = short_lengths(90, 32, 512)
    case = workloads.decode_contiguous(32, 16, 4, 128, 512, seqlens=lens, seed=90)
    paged = workloads.paged_from_contiguous(case)
    o = run(case, 512)
    assert np.array_equal(host_bits(o), host_bits(run(paged, 512)))
    assert_bf16_close(host_f64(o), oracle_out(case), case.name)


def test_one_launch_poisoned_slots_do_not_leak():
    lens = short_lengths(91, 32, 256)
    clean = workloads.decode_paged(32, 8, 2, 128, lens, 256, seed=91)
    dirty = workloads.decode_paged(32, 8, 2, 128, lens, 256, seed=91, poison=True)
    o = run(dirty, 256)
    assert np.all(np.isfinite(host_f64(o)))
    assert np.array_equal(host_bits(o), host_bits(run(clean, 256)))


def test_one_launch_overwrites_stale_output():
    """An empty sequence's rows are written (zeros), whatever o held."""
    torch = torch_gpu()
    lens = np.array([0, 5, 0, 300], np.int32)
    case = workloads.decode_paged(4, 8, 2, 128, lens, 320, seed=92)
    o = torch.full((4, 8, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    fa.decode(dev_bf16(case.q), dev_bf16(case.kcache), dev_bf16(case.vcache), dev_i32(case.seqlens),
              block_table=dev_i32(case.block_table), max_kv_len=320, scale=case.scale, tokens_per_split=320,
              o=o)
    got = host_f64(o)
    assert np.all(got[[0, 2]] == 0.0)
    assert_bf16_close(got, oracle_out(case), case.name)


def test_one_launch_noalloc_equals_decode():
    lens = short_lengths(93, 64, 1024)
    case = workloads.decode_paged(64, 32, 8, 128, lens, 1024, seed=93)
    args = (dev_bf16(case.q), dev_bf16(case.kcache), dev_bf16(case.vcache), dev_i32(case.seqlens))
    kw = dict(block_table=dev_i32(case.block_table), max_kv_len=1024, scale=case.scale)
    o = torch_gpu().empty_like(args[0])
    assert np.array_equal(host_bits(fa.decode_noalloc(*args, o, **kw)), host_bits(fa.decode(*args, **kw)))


def test_one_launch_graph_capture_replays():
    """The one-launch call captured in a HIP graph: every replay, with eager
    work between replays and new lengths written into seqlens in place, equals
    the eager call bit for bit."""
    torch = torch_gpu()
    cap = 512
    case = workloads.decode_paged(32, 16, 4, 128, short_lengths(94, 32, cap), cap, seed=94)
    q, kc, vc = dev_bf16(case.q), dev_bf16(case.kcache), dev_bf16(case.vcache)
    lens, bt = dev_i32(case.seqlens), dev_i32(case.block_table)
    need = fa.decode_workspace_bytes(32, 16, 4, 128, cap, cap)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    kw = dict(block_table=bt, max_kv_len=cap, scale=case.scale, tokens_per_split=cap)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream, as graph capture asks
        fa.decode(q, kc, vc, lens, o=o, workspace=ws, **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.decode(q, kc, vc, lens, o=o, workspace=ws, **kw)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    for rep in range(4):
        new_lens = case.seqlens if rep % 2 == 0 else rng.integers(0, cap + 1, size=case.B).astype(np.int32)
        lens.copy_(torch.from_numpy(np.ascontiguousarray(new_lens, dtype=np.int32)))
        x = torch.randn(1 << 20, device="cuda")
        (x * 2 + 1).sum().item()  # eager work between replays
        print(f"replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        ref = fa.decode(q, kc, vc, lens, **kw)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(o), host_bits(ref)), f"replay {rep}"


def test_short_context_batch_workload():
    """The bench's short-context batch (B = 64, lengths U{256..1024}): one
    launch, every element against the oracle; poisoned slots change nothing."""
    case = workloads.decode_batch_short()
    assert fa.decode_split_tokens(case.B, case.Hq, case.Hkv, case.max_kv_len, 0) >= case.max_kv_len
    o = run(case)
    assert_bf16_close(host_f64(o), oracle_out(case), case.name)
    assert np.array_equal(host_bits(o), host_bits(run(workloads.decode_batch_short(poison=True))))


def test_one_launch_at_the_largest_split():
    """max_kv_len 2048 with 256 split streams: the default is one split of
    2048 tokens (the largest) per sequence, 128 pages per work-group."""
    B, Hq, Hkv, d, cap = 32, 32, 8, 64, 2048
    assert fa.decode_split_tokens(B, Hq, Hkv, cap, 0) == cap
    lens = short_lengths(95, B, cap)
    case = workloads.decode_paged(B, Hq, Hkv, d, lens, cap, seed=95)
    o1 = run(case)
    assert np.array_equal(host_bits(o1), host_bits(run(widened(case, 2 * cap), cap)))
    assert_bf16_close(host_f64(o1), oracle_out(case), case.name)

"""The Python binding rejects inconsistent tensors before the C ABI is called.

The kernels take sizes, not shapes: a contiguous cache's max_kv_len is its
per-sequence row stride, B lengths and B block-table rows are read, and the
output is written as [rows, d] of the output dtype. A mismatch between those
sizes and the tensors would read or write outside them on the GPU, so the
binding checks shapes and dtypes first (these tests run on CPU tensors and
never reach the library), and only then that the tensors are on the GPU.
"""
import pytest

torch = pytest.importorskip("torch")

import attention_fa_prefill_amd as fa  # noqa: E402

pytestmark = pytest.mark.cpu

bf16, f32, i32 = torch.bfloat16, torch.float32, torch.int32


def z(*shape, dtype=bf16):
    return torch.zeros(shape, dtype=dtype)


def decode_args(B=2, Hq=8, Hkv=2, d=64, L=32, paged=False):
    q = z(B, Hq, d)
    if paged:
        kc, vc = z(9, 16, Hkv, d), z(9, 16, Hkv, d)
        bt = torch.zeros((B, (L + 15) // 16), dtype=i32)
    else:
        kc, vc, bt = z(B, L, Hkv, d), z(B, L, Hkv, d), None
    return q, kc, vc, torch.zeros(B, dtype=i32), bt


def test_decode_contiguous_max_len_must_equal_cache_length():
    q, kc, vc, lens, _ = decode_args()
    for bad in (16, 31, 33, 64):
        with pytest.raises(ValueError, match="max_kv_len"):
            fa.decode(q, kc, vc, lens, max_kv_len=bad)


def test_decode_seqlens_must_have_b_entries():
    q, kc, vc, lens, _ = decode_args()
    for bad in (torch.zeros(1, dtype=i32), torch.zeros(3, dtype=i32), torch.zeros((2, 1), dtype=i32)):
        with pytest.raises(ValueError, match="seqlens"):
            fa.decode(q, kc, vc, bad)


@pytest.mark.parametrize("o", [z(2, 8, 32), z(2, 4, 64), z(2, 8, 64, dtype=f32), z(16, 64)])
def test_decode_output_must_match_q(o):
    q, kc, vc, lens, _ = decode_args()
    with pytest.raises(ValueError, match="o must match q"):
        fa.decode(q, kc, vc, lens, o=o)


def test_decode_paged_table_rows_and_columns():
    q, kc, vc, lens, bt = decode_args(paged=True)
    with pytest.raises(ValueError, match="block_table"):
        fa.decode(q, kc, vc, lens, block_table=torch.zeros((3, 2), dtype=i32))
    with pytest.raises(ValueError, match="ceil"):
        fa.decode(q, kc, vc, lens, block_table=bt, max_kv_len=48)


def test_decode_fp8_checks_the_same_geometry():
    q, kc, vc, lens, _ = decode_args()
    k8, v8 = kc.view(torch.int16).to(torch.uint8), vc.view(torch.int16).to(torch.uint8)
    with pytest.raises(ValueError, match="max_kv_len"):
        fa.decode_fp8(q, k8, v8, lens, k_scale=1.0, v_scale=1.0, max_kv_len=16)
    with pytest.raises(ValueError, match="o must match q"):
        fa.decode_fp8(q, k8, v8, lens, k_scale=1.0, v_scale=1.0, o=z(2, 8, 63))


def test_prefill_cache_checks():
    B, Hq, Hkv, Sq, d, L = 2, 4, 2, 8, 64, 40
    q = z(B, Hq, Sq, d)
    kc, vc = z(B, L, Hkv, d), z(B, L, Hkv, d)
    lens = torch.zeros(B, dtype=i32)
    with pytest.raises(ValueError, match="max_kv_len"):
        fa.prefill_cache(q, kc, vc, lens, max_kv_len=32)
    with pytest.raises(ValueError, match="seqlens"):
        fa.prefill_cache(q, kc, vc, torch.zeros(B + 1, dtype=i32))
    with pytest.raises(ValueError, match="o must match q"):
        fa.prefill_cache(q, kc, vc, lens, o=z(B, Hq, Sq + 1, d))
    with pytest.raises(ValueError, match="o must match q"):
        fa.prefill_cache(q, kc, vc, lens, o=z(B, Hq, Sq, d, dtype=f32))


def test_prefill_output_must_match_q():
    q, k = z(1, 4, 8, 64), z(1, 2, 8, 64)
    with pytest.raises(ValueError, match="o must match q"):
        fa.prefill(q, k, k, o=z(1, 4, 8, 32))


@pytest.mark.parametrize("out_dtype", [torch.float16, torch.float64, torch.int32])
def test_merge_output_dtype_is_bf16_or_f32(out_dtype):
    with pytest.raises(ValueError, match="bfloat16 or float32"):
        fa.merge_lse(z(3, 5, 64, dtype=f32), z(3, 5, dtype=f32), out_dtype=out_dtype)
    with pytest.raises(ValueError, match="bfloat16 or float32"):
        fa.merge_lse(z(3, 5, 64, dtype=f32), z(3, 5, dtype=f32), o=z(3, 64, dtype=out_dtype))


def test_merge_shapes():
    op, ls = z(3, 5, 64, dtype=f32), z(3, 5, dtype=f32)
    with pytest.raises(ValueError, match="lse must be"):
        fa.merge_lse(op, z(3, 4, dtype=f32))
    with pytest.raises(ValueError, match="lse must be"):
        fa.merge_lse(op, z(15, dtype=f32))
    with pytest.raises(ValueError, match="o must be"):
        fa.merge_lse(op, ls, o=z(3, 32))
    with pytest.raises(ValueError, match="o must be"):
        fa.merge_lse(op, ls, o=z(4, 64, dtype=f32), out_dtype=f32)
    with pytest.raises(ValueError, match="lse_out"):
        fa.merge_lse(op, ls, lse_out=z(4, dtype=f32))
    with pytest.raises(ValueError, match="lse_out"):
        fa.merge_lse(op, ls, lse_out=z(3))


def test_consistent_cpu_tensors_are_refused_for_the_device():
    q, kc, vc, lens, _ = decode_args()
    with pytest.raises(ValueError, match="GPU only"):
        fa.decode(q, kc, vc, lens)
    with pytest.raises(ValueError, match="GPU only"):
        fa.merge_lse(z(3, 5, 64, dtype=f32), z(3, 5, dtype=f32))

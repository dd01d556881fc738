"""Helpers shared by the GPU parity tests: moving seeded host inputs to the
device and comparing device outputs with the fp64 oracle."""
from __future__ import annotations

import numpy as np
import pytest

# Tolerances of the parity bar: bf16 inputs with fp32 accumulation against the
# fp64 oracle, over every output element; fp32 path max-abs.
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
F32_MAX_ABS = 1e-5


def torch_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch


def dev_bf16(bits: np.ndarray):
    torch = torch_gpu()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def dev_f32(x: np.ndarray):
    torch = torch_gpu()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")


def dev_i32(x: np.ndarray):
    torch = torch_gpu()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to("cuda")


def host_f64(t) -> np.ndarray:
    torch = torch_gpu()
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def host_bits(t) -> np.ndarray:
    torch = torch_gpu()
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def err_stats(got: np.ndarray, ref: np.ndarray):
    diff = np.abs(got - ref)
    return float(diff.max()), float(diff.mean())


def assert_bf16_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mx, mean = err_stats(got, ref)
    print(f"{what}: max_abs={mx:.3e} mean_abs={mean:.3e}", flush=True)
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, f"{what}: max_abs={mx:.3e} mean_abs={mean:.3e}"


def assert_f32_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mx, mean = err_stats(got, ref)
    print(f"{what}: max_abs={mx:.3e} mean_abs={mean:.3e}", flush=True)
    assert mx <= F32_MAX_ABS, f"{what}: max_abs={mx:.3e}"

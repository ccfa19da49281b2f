"""Helpers shared by the GPU parity tests (host <-> device conversion, tolerances)."""
import numpy as np
import torch

import oracle as orc

# Tolerances stated for the hot path: bf16 outputs pass element-wise when
# |gpu - ref| <= BF16_ATOL + BF16_RTOL * |ref|; fp32 outputs within F32_ATOL.
BF16_ATOL, BF16_RTOL = 2e-2, 1e-2
F32_ATOL = 1e-5


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).cuda().view(torch.bfloat16)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bits(t: torch.Tensor) -> np.ndarray:
    assert t.dtype == torch.bfloat16
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return orc.bf16_bits_to_f64(bits(t))
    return t.detach().cpu().numpy().astype(np.float64)


def assert_bf16_close(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    excess = err - (BF16_ATOL + BF16_RTOL * np.abs(ref))
    i = int(np.argmax(excess))
    assert excess.flat[i] <= 0, (
        f"{what}: element {np.unravel_index(i, got.shape)} got {got.flat[i]} ref {ref.flat[i]} "
        f"(max abs err {err.max():.3e})")
    return float(err.max())


def assert_f32_close(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape
    err = np.abs(got - ref)
    assert err.max() <= F32_ATOL, f"{what}: max abs err {err.max():.3e}"
    return float(err.max())


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))

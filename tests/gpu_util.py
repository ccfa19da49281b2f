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


# A stricter self-check on top of the element-wise bound: the relative L2 error
# of a bf16 result is dominated by its own rounding (about 0.1-0.2 %), so a
# kernel bug worth a few percent on small outputs cannot hide below the
# absolute tolerance.
REL_L2_MAX = 5e-3


def assert_bf16_close(got, ref, what="", rel_l2_max=REL_L2_MAX, magnitude=None):
    """Element-wise |got - ref| <= BF16_ATOL + BF16_RTOL * magnitude, where the
    magnitude is |ref| unless given (for a sum y = x + n the relative part of
    the bound belongs to the magnitude of the rounded summand, see the
    sub-layer test)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    mag = np.abs(ref) if magnitude is None else np.asarray(magnitude, np.float64)
    excess = err - (BF16_ATOL + BF16_RTOL * mag)
    i = int(np.argmax(excess))
    assert excess.flat[i] <= 0, (
        f"{what}: element {np.unravel_index(i, got.shape)} got {got.flat[i]} ref {ref.flat[i]} "
        f"(max abs err {err.max():.3e}, rel L2 {rel_l2(got, ref):.2e})")
    if rel_l2_max is not None:
        r = rel_l2(got, ref)
        assert r <= rel_l2_max, f"{what}: relative L2 error {r:.3e} > {rel_l2_max}"
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

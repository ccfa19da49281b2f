"""Helpers shared by the GPU parity tests (host <-> device conversion, tolerances)."""
import numpy as np
import torch

import oracle as orc
from gqa_inputs.device import dev, dev_bf16  # noqa: F401  (re-exported for the tests)

# Tolerances stated for the hot path: bf16 outputs pass element-wise when
# |gpu - ref| <= BF16_ATOL + BF16_RTOL * |ref|; fp32 outputs within F32_ATOL.
BF16_ATOL, BF16_RTOL = 2e-2, 1e-2
F32_ATOL = 1e-5


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
    magnitude is |ref| unless given. For a residual output y = x + n the tests
    pass max(|y|, |n|): n = norm(o) is rounded to bf16 before the add, as the
    sandwich norm hands it on, so y carries one bf16 rounding of n, up to
    2**-9 |n| (0.031 at |n| = 4 to 8), which exceeds 2e-2 + 1e-2 |y| where x
    and n cancel. Where |n| <= |y| the bound is the unwidened one; the number
    of elements that need the widening is printed."""
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
    if magnitude is not None:
        # elements that pass only because of the widened magnitude
        n_wide = int(np.count_nonzero(err > BF16_ATOL + BF16_RTOL * np.abs(ref)))
        print(f"{what}: {n_wide} of {err.size} elements within the bound only through max(|y|, |n|)")
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

"""Shared helpers for the GPU tests: moving seeded inputs to the device and the
parity bar (bit-exact on integer inputs; on Gaussian inputs
max|err| <= 1e-2 * (|ref| + 1) element-wise and relative Frobenius error
<= 1e-3 against the fp64 oracle)."""
from __future__ import annotations

import sys

import numpy as np

MAX_REL = 1e-2
FROB_REL = 1e-3


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev_f32(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (device output) for comparison."""
    u = bits.astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def check_tolerance(got: np.ndarray, ref: np.ndarray, frob_ref: np.ndarray | None = None,
                    what: str = "") -> tuple[float, float]:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = MAX_REL * (np.abs(ref) + 1.0)
    worst = float(np.max(err / bound)) if err.size else 0.0
    fr = ref if frob_ref is None else np.asarray(frob_ref, dtype=np.float64)
    denom = float(np.linalg.norm(fr))
    frob = float(np.linalg.norm(got - fr) / denom) if denom > 0 else float(np.linalg.norm(got - fr))
    assert worst <= 1.0, f"{what}: element-wise bound exceeded ({worst:.3g} of bound)"
    assert frob <= FROB_REL, f"{what}: relative Frobenius error {frob:.3g} > {FROB_REL}"
    return worst, frob


def check_exact(got: np.ndarray, ref: np.ndarray, what: str = "") -> None:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    bad = np.nonzero(got != ref)
    assert bad[0].size == 0, (f"{what}: {bad[0].size} mismatches, first at "
                              f"{tuple(int(b[0]) for b in bad)}: got {got[tuple(b[0] for b in bad)]}, "
                              f"want {ref[tuple(b[0] for b in bad)]}")

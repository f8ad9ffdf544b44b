"""Shared test helpers: tolerances and host <-> device transfers of bf16 bits."""
import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def fp32_tol(oracle: np.ndarray) -> np.ndarray:
    """Per-element bound for fp32-accumulated outputs: 1e-3 * ||oracle row||_2 / sqrt(N) + 1e-5."""
    n = oracle.shape[-1]
    return 1e-3 * np.linalg.norm(oracle, axis=-1, keepdims=True) / np.sqrt(n) + 1e-5


def bf16_tol(oracle: np.ndarray) -> np.ndarray:
    """Per-element bound for bf16-stored outputs: 8e-3 * |oracle| + 1e-2."""
    return 8e-3 * np.abs(oracle) + 1e-2


def assert_within(got: np.ndarray, want: np.ndarray, tol: np.ndarray, what: str = "") -> None:
    err = np.abs(got - want)
    tol = np.broadcast_to(tol, err.shape)
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        ratio = float(np.max(err / tol))
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance; first at {tuple(i)}: "
                             f"got {got[tuple(i)]!r} want {want[tuple(i)]!r} tol {tol[tuple(i)]!r}; "
                             f"max err/tol {ratio:.3g}")


def max_ratio(got, want, tol) -> float:
    return float(np.max(np.abs(got - want) / tol))


def to_dev(bits: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_bits(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

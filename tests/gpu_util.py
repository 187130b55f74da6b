"""Helpers shared by the GPU tests: moving seeded inputs to the device and
comparing with the oracle under the stated tolerances."""

import sys

import numpy as np
import pytest
import torch


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")


def announce(*parts):
    """Name the case before any GPU work (a fault then still says which one)."""
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def to_dev_bf16(bits: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def to_dev_f32(a, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def u32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def gemm_close(y_gpu: np.ndarray, y_ref: np.ndarray, tol: float = 1e-3):
    """GEMM tolerance: |d| <= tol * max(|y|, rms(Y)) elementwise and
    ||d||_F / ||Y||_F <= tol."""
    y_gpu = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    d = np.abs(y_gpu - y_ref)
    rms = np.sqrt(np.mean(y_ref ** 2)) if y_ref.size else 0.0
    bound = tol * np.maximum(np.abs(y_ref), rms)
    worst = float(np.max(d / np.maximum(bound, 1e-300))) if d.size else 0.0
    fro = float(np.linalg.norm(d) / max(np.linalg.norm(y_ref), 1e-300)) if d.size else 0.0
    assert np.all(d <= bound), f"elementwise GEMM error {worst:.3g} x tolerance"
    assert fro <= tol, f"relative Frobenius error {fro:.3g}"
    return worst, fro


def ulp_distance_f32(a, b) -> np.ndarray:
    ai = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    bi = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(ai - bi)

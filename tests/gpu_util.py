"""Helpers for the GPU parity tests: device copies of the seeded inputs, the
oracle comparison and its tolerances, and a progress line per case that
bypasses pytest's capture (so a run that dies still names its last case)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import fagen

# Tolerances on |O_gpu - O_oracle| and |LSE_gpu - LSE_oracle|.  bf16/fp16 with
# fp32 accumulation: max-abs 2e-2, mean-abs 2e-3, LSE 1e-3; fp32: 1e-5.
TOL = {
    "bf16": dict(max_abs=2e-2, mean_abs=2e-3, lse=1e-3),
    "f16": dict(max_abs=2e-2, mean_abs=2e-3, lse=1e-3),
    "f32": dict(max_abs=1e-5, mean_abs=1e-5, lse=1e-5),
}

TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def announce(msg: str) -> None:
    sys.__stdout__.write(f"[gpu-case] {msg}\n")
    sys.__stdout__.flush()


def to_dev(a: np.ndarray, dt: str) -> torch.Tensor:
    """Storage array (fagen.to_storage layout) -> contiguous device tensor."""
    if dt == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to("cuda")


def widen(a: np.ndarray, dt: str) -> np.ndarray:
    return fagen.storage_to_f32(a, dt)


def compare(o_gpu: torch.Tensor, lse_gpu, o_ref: np.ndarray, lse_ref, dt: str, what: str = ""):
    """Check GPU outputs against oracle outputs; returns the metrics."""
    og = o_gpu.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(og)), f"{what}: non-finite output"
    err = np.abs(og - o_ref)
    m = dict(max_abs=float(err.max()) if err.size else 0.0,
             mean_abs=float(err.mean()) if err.size else 0.0,
             rel=float(err.max() / max(np.abs(o_ref).max(), 1e-30)) if err.size else 0.0)
    if lse_gpu is not None:
        lg = lse_gpu.cpu().numpy().astype(np.float64)
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lg), fin), f"{what}: -inf pattern of LSE differs"
        m["lse"] = float(np.abs(lg[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    t = TOL[dt]
    assert m["max_abs"] <= t["max_abs"], (what, m)
    assert m["mean_abs"] <= t["mean_abs"], (what, m)
    if "lse" in m:
        assert m["lse"] <= t["lse"], (what, m)
    return m

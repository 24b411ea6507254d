"""Host <-> device marshalling for the GPU tests (no attention arithmetic here)."""
from __future__ import annotations

import numpy as np
import torch

import oracle

BF16_TOL = 2e-2   # max abs error against the fp64 oracle, bf16 in/out with fp32 accumulation
F32_TOL = 1e-4    # max abs error against the fp64 oracle, fp32 in/out


def to_dev(x: np.ndarray) -> torch.Tensor:
    """uint16 arrays are bf16 bit patterns; float32 stays float32."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def to_host_f64(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return oracle.widen(t.view(torch.int16).numpy().view(np.uint16))
    return t.numpy().astype(np.float64)


def nan_like(t: torch.Tensor) -> torch.Tensor:
    return torch.full_like(t, float("nan"))


def report(got: np.ndarray, want: np.ndarray) -> dict:
    err = np.abs(got - want)
    rms = np.sqrt(np.mean((got - want) ** 2)) / max(np.sqrt(np.mean(want ** 2)), 1e-30)
    return {"max_abs": float(err.max()), "p99_abs": float(np.quantile(err, 0.99)),
            "p50_abs": float(np.quantile(err, 0.5)), "rel_rms": float(rms)}


def assert_close(got: np.ndarray, want: np.ndarray, tol: float, what: str):
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    r = report(got, want)
    print(f"{what}: {r}", flush=True)
    assert r["max_abs"] <= tol, f"{what}: max abs err {r['max_abs']:.3e} > {tol:.1e} ({r})"
    return r


def diff_params_dev(params):
    a, g, b, lm = params
    return to_dev(a), to_dev(g), to_dev(b), to_dev(lm)

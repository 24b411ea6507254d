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


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> its uint16 bit patterns on the host."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns, rounded once to nearest (ties to even).  Spacing of bf16
    values in [2^(e-1), 2^e) is 2^(e-8); below 2^-126 it is 2^-133 (subnormals)."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.round(x / q) * q                      # exact scaling; np.round is half-to-even
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bf16_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 steps between bit patterns (sign-magnitude mapped onto one ordered line)."""
    def ordered(u):
        u = np.asarray(u, dtype=np.uint16).astype(np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(ordered(a) - ordered(b))


def nan_like(t: torch.Tensor) -> torch.Tensor:
    return torch.full_like(t, float("nan"))


def report(got: np.ndarray, want: np.ndarray, got_bits: np.ndarray | None = None) -> dict:
    """Max, p99, p50 abs error and relative RMS against the oracle.  With the output's bf16 bits, the
    error is also split against the oracle rounded once to bf16 (RNE), the best a bf16 output can do:
    rounding_only = max |RNE(oracle) - oracle|, vs_rne = max |gpu - RNE(oracle)| (the kernel's own
    compute error, in absolute terms), and the distance in bf16 steps where |oracle| >= 1/16 (near
    zero a count of steps says nothing: the spacing there is far below the computation's error)."""
    err = np.abs(got - want)
    rms = np.sqrt(np.mean((got - want) ** 2)) / max(np.sqrt(np.mean(want ** 2)), 1e-30)
    r = {"n": int(got.size), "max_abs": float(err.max()), "p99_abs": float(np.quantile(err, 0.99)),
         "p50_abs": float(np.quantile(err, 0.5)), "rel_rms": float(rms), "max_abs_out": float(np.abs(want).max())}
    if got_bits is not None:
        rb = bf16_rne_bits(want).reshape(-1)
        rv = (rb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        gb = got_bits.reshape(-1)
        big = np.abs(want.reshape(-1)) >= 1.0 / 16
        u = bf16_ulp_distance(gb[big], rb[big])
        r.update({"rounding_only_max_abs": float(np.abs(rv - want.reshape(-1)).max()),
                  "vs_rne_max_abs": float(np.abs(got.reshape(-1) - rv).max()),
                  "frac_eq_rne": float(np.mean(gb == rb)),
                  "max_steps_vs_rne_o_ge_1_16": int(u.max()) if u.size else 0})
    return r


def assert_close(got: np.ndarray, want: np.ndarray, tol: float, what: str, got_bits: np.ndarray | None = None):
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    r = report(got, want, got_bits)
    print(f"{what}: {r}", flush=True)
    assert r["max_abs"] <= tol, f"{what}: max abs err {r['max_abs']:.3e} > {tol:.1e} ({r})"
    return r


def diff_params_dev(params):
    a, g, b, lm = params
    return to_dev(a), to_dev(g), to_dev(b), to_dev(lm)

"""Seeded synthetic inputs, shared by the parity tests, the smoke check and the bench.

This module holds no attention arithmetic: it draws numbers and stores them in
the dtypes the library consumes.  bf16 tensors are returned as uint16 bit
patterns (rounded from float32 with round-to-nearest-even), fp32 tensors as
float32, all in the [B, H, S, D] layout, C-contiguous.

Recipe (the same for every workload): numpy Generator(PCG64(seed)); activations
~ N(0, 1) drawn in float64, narrowed to float32, then (for bf16) to bf16.  DyT
gains gamma ~ U[2, 8] per tensor and channel, alpha = 0.5, beta = 0; lambda = 0.8
per head; rope base 10000; scale 1/8.  Seeds are 1000*workload + tensor index
(q/q1 = 0, k/k1 = 1, v = 2, q2 = 3, k2 = 4, gamma = 5, RMSNorm weight = 6).

Model forms of the differential workloads: RMSNorm weights ~ U[0.5, 1.5] per
tensor and channel, eps 1e-6; V padding flags mark the last `pad` tokens of batch
element b (pad + b of them) as padding, the layout of latents padded at the end.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

D = 64


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal(seed: int, shape, dtype: str) -> np.ndarray:
    x = np.random.Generator(np.random.PCG64(seed)).standard_normal(shape).astype(np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def uniform(seed: int, shape, lo: float, hi: float) -> np.ndarray:
    return np.random.Generator(np.random.PCG64(seed)).uniform(lo, hi, shape).astype(np.float32)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, dtype and the parameters of its form."""
    key: str
    form: str            # "dense" | "cross" | "diff"
    dtype: str           # "f32" | "bf16"
    B: int
    H: int
    Sq: int
    Sk: int
    scale: float = 0.125
    window: int = -1     # diff only: >= 0 band half-width, < 0 every key
    index: int = 0       # seed namespace
    desc: str = ""
    extra: dict = field(default_factory=dict)
    D: int = D           # head dim


WORKLOADS = {
    "dense_f32_b1h2s256": Workload("dense_f32_b1h2s256", "dense", "f32", 1, 2, 256, 256, index=1,
                                   desc="dense non-causal, fp32, B=1 H=2 S=256"),
    "sdxl_l1_self_b2h10s4096": Workload("sdxl_l1_self_b2h10s4096", "dense", "bf16", 2, 10, 4096, 4096, index=2,
                                        desc="SDXL level-1 self-attention (64x64 latent), bf16, B=2 H=10 S=4096"),
    "sdxl_l2_cross_b2h20q1024k77": Workload("sdxl_l2_cross_b2h20q1024k77", "cross", "bf16", 2, 20, 1024, 77, index=3,
                                            desc="SDXL level-2 cross-attention, bf16, B=2 H=20 Sq=1024 Sk=77"),
    "sdxl_l1_cross_b2h10q4096k77": Workload("sdxl_l1_cross_b2h10q4096k77", "cross", "bf16", 2, 10, 4096, 77, index=6,
                                            desc="SDXL level-1 cross-attention, bf16, B=2 H=10 Sq=4096 Sk=77"),
    "sa3_dit_cross_h24q1422k257": Workload("sa3_dit_cross_h24q1422k257", "cross", "bf16", 1, 24, 1422, 257, index=7,
                                           desc="cross-attention to 257 conditioning tokens, DiT-shaped, bf16, "
                                                "B=1 H=24 Sq=1422 Sk=257"),
    "sdxl_vae_mid_b1h1s16384d512": Workload("sdxl_vae_mid_b1h1s16384d512", "dense", "bf16", 1, 1, 16384, 16384,
                                            scale=512 ** -0.5, index=8, D=512,
                                            desc="SDXL VAE mid-block attention (128x128 latent, one head of 512 "
                                                 "channels), bf16, B=1 H=1 S=16384 D=512"),
    "sa3_decoder_banddiff_h8s23086w17": Workload("sa3_decoder_banddiff_h8s23086w17", "diff", "bf16", 1, 8, 23086,
                                                 23086, window=17, index=4,
                                                 desc="banded differential attention, decoder-shaped, bf16, "
                                                      "B=1 H=8 S=23086, window +-17"),
    "sa3_dit_fulldiff_h16s1422": Workload("sa3_dit_fulldiff_h16s1422", "diff", "bf16", 1, 16, 1422, 1422, window=-1,
                                          index=5, desc="full differential attention, DiT-shaped, bf16, "
                                                        "B=1 H=16 S=1422"),
}


def make_dense(wl: Workload, seed_base: int | None = None, Sq: int | None = None, Sk: int | None = None,
               B: int | None = None, H: int | None = None):
    """q [B,H,Sq,D], k, v [B,H,Sk,D] for the dense / cross forms."""
    base = 1000 * wl.index if seed_base is None else seed_base
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    Sq = wl.Sq if Sq is None else Sq
    Sk = wl.Sk if Sk is None else Sk
    q = normal(base + 0, (B, H, Sq, wl.D), wl.dtype)
    k = normal(base + 1, (B, H, Sk, wl.D), wl.dtype)
    v = normal(base + 2, (B, H, Sk, wl.D), wl.dtype)
    return q, k, v


def make_diff_params(H: int, seed: int, alpha: float = 0.5, gamma_lo: float = 2.0, gamma_hi: float = 8.0,
                     lam: float = 0.8):
    """alpha [4], gamma [4, D], beta [4, D], lambda [H] as float32 (set order q1, k1, q2, k2)."""
    a = np.full(4, alpha, dtype=np.float32)
    g = uniform(seed, (4, D), gamma_lo, gamma_hi)
    b = np.zeros((4, D), dtype=np.float32)
    lm = np.full(H, lam, dtype=np.float32)
    return a, g, b, lm


def make_diff_params_varied(H: int, seed: int):
    """Parameters that tell the four sets and the heads apart: alpha ~ U[0.3, 0.9] per set, gamma ~
    U[2, 8] and beta ~ N(0, 0.3) per set and channel, lambda ~ U[0.2, 0.9] per head (float32)."""
    r = np.random.Generator(np.random.PCG64(seed))
    a = r.uniform(0.3, 0.9, 4).astype(np.float32)
    g = r.uniform(2.0, 8.0, (4, D)).astype(np.float32)
    b = r.normal(0.0, 0.3, (4, D)).astype(np.float32)
    lm = r.uniform(0.2, 0.9, H).astype(np.float32)
    return a, g, b, lm


def make_diff(wl: Workload, seed_base: int | None = None, S: int | None = None, B: int | None = None,
              H: int | None = None):
    """q1, k1, q2, k2, v [B,H,S,D] bf16 bits and (alpha, gamma, beta, lambda)."""
    base = 1000 * wl.index if seed_base is None else seed_base
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    S = wl.Sq if S is None else S
    shape = (B, H, S, D)
    q1 = normal(base + 0, shape, "bf16")
    k1 = normal(base + 1, shape, "bf16")
    v = normal(base + 2, shape, "bf16")
    q2 = normal(base + 3, shape, "bf16")
    k2 = normal(base + 4, shape, "bf16")
    params = make_diff_params(H, base + 5)
    return (q1, k1, q2, k2, v), params


def make_model_params(H: int, seed: int, lam: float = 0.8):
    """RMSNorm weights [4, D] (set order q1, k1, q2, k2) and lambda [H], float32."""
    return uniform(seed, (4, D), 0.5, 1.5), np.full(H, lam, dtype=np.float32)


def make_v_keep(B: int, S: int, pad: int) -> np.ndarray:
    """[B, S] uint8 flags: 1 = real token, 0 = padding (the last pad + b tokens of batch element b)."""
    keep = np.ones((B, S), dtype=np.uint8)
    for b in range(B):
        n = min(S, pad + b)
        if n > 0:
            keep[b, S - n:] = 0
    return keep

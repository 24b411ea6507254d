"""Algorithmic work of each form: the FLOP and byte counts that rooflines divide by.

Counting rules (the "fused traffic" model):
  * FLOPs: 2 flops per multiply-add; the scores cost B*H*Sq*Sk*D multiply-adds and the
    weighted sum the same again ("SDXL as a requirements inventory", s2.1), so
    4*D flops per (query, key) pair.  A differential call pays that per branch,
    and a banded call counts only the in-band pairs.
  * Bytes: every input element read once and every output element written once;
    scores never leave the chip ("401 -> 163 ms: Stable Audio 3 medium on one TPU
    v6e chip", appendix "Roofline after E1": attention is charged its fused traffic).
Peaks are AMD's published MI355X figures.
"""
from __future__ import annotations

MFMA_BF16_PEAK = 2.5e15      # dense bf16/fp16 matrix FLOP/s
MFMA_FP32_PEAK = 157.3e12    # fp32 matrix FLOP/s
HBM_PEAK = 8.0e12            # HBM3E bytes/s

DTYPE_BYTES = {"f32": 4, "bf16": 2}


def attn_flops(B: int, H: int, Sq: int, Sk: int, D: int = 64) -> int:
    return 4 * B * H * Sq * Sk * D


def band_pairs(S: int, window: int) -> int:
    """Number of (query, key) pairs with |i - j| <= window inside [0, S); window < 0 means all."""
    if window < 0 or window >= S - 1:
        return S * S
    w = window
    # every query sees 2w+1 keys, minus the keys that fall off either end
    return S * (2 * w + 1) - w * (w + 1)


def diff_flops(B: int, H: int, S: int, window: int, D: int = 64) -> int:
    return 2 * 4 * D * B * H * band_pairs(S, window)


def dense_bytes(B: int, H: int, Sq: int, Sk: int, D: int = 64, dtype: str = "bf16") -> int:
    e = DTYPE_BYTES[dtype]
    return e * B * H * D * (2 * Sq + 2 * Sk)          # q and o, k and v


def diff_bytes(B: int, H: int, S: int, D: int = 64, dtype: str = "bf16") -> int:
    return DTYPE_BYTES[dtype] * B * H * S * D * 6      # q1 k1 q2 k2 v read, o written

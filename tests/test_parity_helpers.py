"""CPU checks of the parity report's bf16 helpers (the reference rounding and the ulp distance)."""
import numpy as np

from gpu_util import bf16_rne_bits, bf16_ulp_distance, report

ALL = np.arange(0, 0x7F80, dtype=np.uint32).astype(np.uint16)          # every finite non-negative bf16
VALS = (ALL.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _nearest_brute(x):
    ax = np.abs(x)
    i = np.searchsorted(VALS, ax)
    lo, hi = np.clip(i - 1, 0, len(VALS) - 1), np.clip(i, 0, len(VALS) - 1)
    dlo, dhi = ax - VALS[lo], VALS[hi] - ax
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(ALL[lo] % 2 == 0, lo, hi)))
    return ALL[pick] | np.where(np.signbit(x), 0x8000, 0).astype(np.uint16)


def test_rne_matches_brute_force_nearest():
    r = np.random.default_rng(3)
    x = np.concatenate([r.standard_normal(30000) * r.choice([1e-40, 1e-3, 1.0, 1e5], 30000),
                        VALS[::97], (VALS[1:] + VALS[:-1])[::101] / 2,       # exact values and exact ties
                        -VALS[::89]])
    assert np.array_equal(bf16_rne_bits(x), _nearest_brute(x))


def test_ulp_distance():
    a = np.array([0x3F80, 0x8001, 0x0001, 0x7F7F, 0xBF80], dtype=np.uint16)
    b = np.array([0x3F81, 0x0001, 0x8000, 0x7F7F, 0xBF82], dtype=np.uint16)
    assert bf16_ulp_distance(a, b).tolist() == [1, 2, 1, 0, 2]


def test_report_counts_ulps_against_the_rounded_oracle():
    want = np.array([1.0 + 2 ** -9, 3.0, -0.5])            # first value rounds to 1.0 (a tie, even)
    got_bits = np.array([0x3F80, 0x4041, 0xBF00], dtype=np.uint16)   # 1.0, 3.0 + one step, -0.5
    got = (got_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    r = report(got, want, got_bits)
    assert r["max_steps_vs_rne_o_ge_1_16"] == 1 and abs(r["frac_eq_rne"] - 2 / 3) < 1e-12
    assert r["max_abs"] == 2 ** -6 and r["vs_rne_max_abs"] == 2 ** -6 and r["rounding_only_max_abs"] == 2 ** -9

"""Pins for the fp64 oracle: checks against facts that do not come from the oracle.

Each pin takes an `ora` namespace (the oracle module bound to one compiled
library, so the mutant test can run the same pins against deliberately broken
builds) and raises AssertionError on failure.  The kinds of pin:

  * library routine: torch's float64 scaled_dot_product_attention (dense), and a
    complex-number formulation of the rotation fed through it (differential);
  * closed forms: uniform weights, constant V, one-hot V (the output row is the
    softmax row), single key, the DyT identity tanh = (e^2y - 1)/(e^2y + 1), the
    rotation of a basis vector;
  * invariants: linearity in V, joint permutation of keys and values, the
    relative-position property of the rotation, norm preservation, branch
    cancellation at lambda = 1, window >= S-1 equals the full window;
  * brute force: a long-double log-sum-exp implementation on tiny inputs.

Definitions follow "SDXL as a requirements inventory" s1.3 (softmax(q k^T/8) v per
head) and "401 -> 163 ms: Stable Audio 3 medium on one TPU v6e chip" s3 / appendix
E1-E2 (DyT, rotate-half rotary embedding, two softmax branches over a +-17 band
masked by position, subtraction) with the readings stated in ka_oracle.c.  The
same page's model forms (appendix D1, D3, D4, E1: per-head RMSNorm, rotary on 32
of the 64 dims, V zeroed for padded tokens whose keys stay) are pinned against
torch's rms_norm and SDPA, closed forms and a long-double brute force.
"""
from __future__ import annotations

import types

import numpy as np
import torch

D = 64
TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _params(H, seed, alpha=0.5, lam=None):
    r = _rng(seed)
    a = np.full(4, alpha)
    g = r.uniform(2.0, 8.0, (4, D))
    b = r.normal(0.0, 0.3, (4, D))
    lm = r.uniform(0.2, 0.9, H) if lam is None else np.full(H, lam)
    return a, g, b, lm


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.max(np.abs(a - b) / (1.0 + np.abs(b))) if a.size else 0.0
    assert err <= tol, f"{what}: max rel err {err:.3e} > {tol:.1e}"


# ------------------------------------------------------------------ dense / cross

def pin_dense_vs_torch_sdpa(ora):
    """Dense and cross definitions equal torch's float64 SDPA (a library routine)."""
    r = _rng(1)
    for (B, H, Sq, Sk, scale) in [(2, 3, 9, 13, 0.125), (1, 2, 5, 77, 0.125), (1, 1, 4, 4, 0.37)]:
        q, k, v = (r.standard_normal((B, H, s, D)) for s in (Sq, Sk, Sk))
        q *= 3.0  # peakier softmax
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k).contiguous(), torch.from_numpy(v), scale=scale).numpy()
        _close(ora.attn(q, k, v, scale), ref, 1e-12, "sdpa")


def pin_dense_d512_vs_torch_sdpa(ora):
    """Head dim 512 (the SDXL VAE's single-head AttnBlock, "SDXL as a requirements inventory" s1.5, s5.10):
    the same definition, against torch's float64 SDPA at scale 512^-1/2."""
    r = _rng(3)
    for (B, H, Sq, Sk) in [(1, 1, 37, 53), (2, 1, 16, 100)]:
        q, k, v = (r.standard_normal((B, H, s, 512)) for s in (Sq, Sk, Sk))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k).contiguous(), torch.from_numpy(v), scale=512 ** -0.5).numpy()
        _close(ora.attn(q, k, v, 512 ** -0.5), ref, 1e-12, "sdpa d512")


def pin_onehot_v_gives_softmax_rows(ora):
    """V = identity rows: output row i is the softmax row (sums to 1, >= 0, zero past Sk)."""
    r = _rng(2)
    Sq, Sk = 11, 23
    q, k = r.standard_normal((1, 1, Sq, D)) * 2, r.standard_normal((1, 1, Sk, D))
    v = np.zeros((1, 1, Sk, D))
    v[0, 0, np.arange(Sk), np.arange(Sk)] = 1.0
    o = ora.attn(q, k, v, 0.125)[0, 0]
    assert np.all(o[:, :Sk] >= 0.0)
    assert np.all(o[:, Sk:] == 0.0)
    _close(o.sum(axis=1), np.ones(Sq), 1e-13, "row sums")
    # and the row is exactly the textbook softmax of the scores
    s = 0.125 * q[0, 0] @ k[0, 0].T
    p = np.exp(s - s.max(axis=1, keepdims=True))
    _close(o[:, :Sk], p / p.sum(axis=1, keepdims=True), 1e-13, "softmax row")


def pin_constant_v(ora):
    r = _rng(3)
    q, k = r.standard_normal((2, 2, 7, D)), r.standard_normal((2, 2, 19, D))
    c = r.standard_normal(D)
    v = np.broadcast_to(c, (2, 2, 19, D)).copy()
    _close(ora.attn(q, k, v, 0.125), np.broadcast_to(c, (2, 2, 7, D)), 1e-13, "constant V")


def pin_uniform_when_q_zero(ora):
    r = _rng(4)
    k, v = r.standard_normal((1, 3, 29, D)), r.standard_normal((1, 3, 29, D))
    q = np.zeros((1, 3, 5, D))
    ref = np.broadcast_to(v.mean(axis=2, keepdims=True), (1, 3, 5, D))
    _close(ora.attn(q, k, v, 0.125), ref, 1e-13, "uniform")


def pin_single_key(ora):
    r = _rng(5)
    q, k, v = r.standard_normal((2, 2, 6, D)), r.standard_normal((2, 2, 1, D)), r.standard_normal((2, 2, 1, D))
    _close(ora.attn(q, k, v, 0.125), np.broadcast_to(v, (2, 2, 6, D)), 1e-15, "single key")


def pin_dominant_key(ora):
    """One key with a score margin of >= 60 takes all the weight (error < e^-60)."""
    r = _rng(6)
    Sk = 12
    k = r.standard_normal((1, 1, Sk, D))
    v = r.standard_normal((1, 1, Sk, D))
    star = 7
    # q along key `star`, sized so that key's score is 800: past exp()'s double range unless the
    # row maximum is subtracted first, and far ahead of every other key
    q = k[:, :, star:star + 1, :] * (800.0 / (0.125 * np.sum(k[0, 0, star] ** 2)))
    s = 0.125 * (q[0, 0] @ k[0, 0].T)[0]
    assert s[star] - np.max(np.delete(s, star)) >= 60.0 and s[star] > 750.0
    _close(ora.attn(q, k, v, 0.125)[0, 0, 0], v[0, 0, star], 1e-14, "dominant key")


def pin_linear_in_v(ora):
    r = _rng(7)
    q, k = r.standard_normal((1, 2, 8, D)), r.standard_normal((1, 2, 15, D))
    v1, v2 = r.standard_normal((1, 2, 15, D)), r.standard_normal((1, 2, 15, D))
    lhs = ora.attn(q, k, 2.5 * v1 - 0.75 * v2, 0.125)
    rhs = 2.5 * ora.attn(q, k, v1, 0.125) - 0.75 * ora.attn(q, k, v2, 0.125)
    _close(lhs, rhs, 1e-13, "linearity")


def pin_joint_permutation(ora):
    r = _rng(8)
    q, k, v = r.standard_normal((1, 2, 9, D)), r.standard_normal((1, 2, 21, D)), r.standard_normal((1, 2, 21, D))
    pk = r.permutation(21)
    pq = r.permutation(9)
    base = ora.attn(q, k, v, 0.125)
    _close(ora.attn(q, k[:, :, pk], v[:, :, pk], 0.125), base, 1e-13, "key permutation")
    _close(ora.attn(q[:, :, pq], k, v, 0.125), base[:, :, pq], 1e-15, "query permutation")


def pin_rows_subset_matches_full(ora):
    """The sampled-row mode returns exactly the rows of the full computation."""
    r = _rng(9)
    q, k, v = r.standard_normal((2, 3, 10, D)), r.standard_normal((2, 3, 14, D)), r.standard_normal((2, 3, 14, D))
    full = ora.attn(q, k, v, 0.125).reshape(-1, D)
    rows = np.array([0, 5, 17, 59, 33])
    assert np.array_equal(ora.attn(q, k, v, 0.125, rows=rows), full[rows])


# ------------------------------------------------------------------ DyT and RoPE

def pin_dyt_closed_form(ora):
    """gamma*tanh(alpha x)+beta against the exponential form of tanh in long double."""
    r = _rng(10)
    x = r.standard_normal(D) * 4
    g, b = r.uniform(2, 8, D), r.normal(0, 1, D)
    for alpha in (0.5, 1.7, -0.3):
        y = ora.dyt_row(x, alpha, g, b)
        e = np.exp(np.longdouble(2 * alpha) * x.astype(np.longdouble))
        ref = g.astype(np.longdouble) * (e - 1) / (e + 1) + b.astype(np.longdouble)
        _close(y, ref.astype(np.float64), 1e-14, f"dyt alpha={alpha}")
    # tanh(0) = 0: the output is beta
    _close(ora.dyt_row(np.zeros(D), 0.5, g, b), b, 0.0, "dyt at 0")
    # small-alpha limit: gamma*alpha*x + beta to O(alpha^3)
    a = 1e-6
    _close(ora.dyt_row(x, a, g, b), g * a * x + b, 4e-15, "dyt small alpha")


def pin_rope_basis_vectors(ora):
    """R_p e_i = cos t e_i + sin t e_{i+32};  R_p e_{i+32} = -sin t e_i + cos t e_{i+32};  t = p*base^(-i/32)."""
    for p in (0, 1, 5, 23085):
        for i in (0, 1, 13, 31):
            t = p * 10000.0 ** (-i / 32.0)
            e = np.zeros(D)
            e[i] = 1.0
            ref = np.zeros(D)
            ref[i], ref[i + 32] = np.cos(t), np.sin(t)
            _close(ora.rope_row(e, p, 10000.0), ref, 1e-13, f"rope e_{i} p={p}")
            e = np.zeros(D)
            e[i + 32] = 1.0
            ref = np.zeros(D)
            ref[i], ref[i + 32] = -np.sin(t), np.cos(t)
            _close(ora.rope_row(e, p, 10000.0), ref, 1e-13, f"rope e_{i + 32} p={p}")


def pin_rope_invariants(ora):
    r = _rng(11)
    x, y = r.standard_normal(D), r.standard_normal(D)
    # identity at position 0
    _close(ora.rope_row(x, 0, 10000.0), x, 0.0, "rope p=0")
    # each (i, i+32) pair keeps its length
    for p in (3, 777, 23000):
        z = ora.rope_row(x, p, 10000.0)
        _close(np.hypot(z[:32], z[32:]), np.hypot(x[:32], x[32:]), 1e-14, "pair norms")
    # relative position: <R_p x, R_j y> depends only on p - j
    for (p, j, t) in [(10, 3, 100), (0, 50, 7), (2000, 1999, 12345)]:
        a = ora.rope_row(x, p, 10000.0) @ ora.rope_row(y, j, 10000.0)
        b = ora.rope_row(x, p + t, 10000.0) @ ora.rope_row(y, j + t, 10000.0)
        assert abs(a - b) <= 1e-9 * (1 + abs(a)), f"relative position {a} vs {b}"
    # base matters: a different base changes the rotation of pair 1 at p=1
    assert not np.allclose(ora.rope_row(x, 1, 10000.0), ora.rope_row(x, 1, 500.0))


# ------------------------------------------------------------------ differential attention

def _torch_diff(q1, k1, q2, k2, v, scale, window, a, g, b, base, lam):
    """Differential attention through torch: tanh, complex rotation, SDPA with a boolean band mask."""
    B, H, S, _ = q1.shape
    pos = torch.arange(S, dtype=torch.float64)
    freq = float(base) ** (-torch.arange(32, dtype=torch.float64) / 32.0)
    rot = torch.polar(torch.ones(S, 32, dtype=torch.float64), pos[:, None] * freq[None, :])

    def prep(x, t):
        y = torch.from_numpy(g[t]) * torch.tanh(float(a[t]) * torch.from_numpy(x)) + torch.from_numpy(b[t])
        z = torch.complex(y[..., :32], y[..., 32:]) * rot
        return torch.cat([z.real, z.imag], dim=-1).contiguous()

    mask = None
    if window >= 0:
        idx = torch.arange(S)
        mask = (idx[:, None] - idx[None, :]).abs() <= window
    vt = torch.from_numpy(v)
    o1 = torch.nn.functional.scaled_dot_product_attention(prep(q1, 0), prep(k1, 1), vt, attn_mask=mask, scale=scale)
    o2 = torch.nn.functional.scaled_dot_product_attention(prep(q2, 2), prep(k2, 3), vt, attn_mask=mask, scale=scale)
    return (o1 - torch.from_numpy(lam)[None, :, None, None] * o2).numpy()


def _diff_inputs(B, H, S, seed, qk_scale=1.0):
    r = _rng(seed)
    return [r.standard_normal((B, H, S, D)) * (qk_scale if i != 4 else 1.0) for i in range(5)]


def pin_diff_vs_torch(ora):
    for (B, H, S, w, seed) in [(1, 2, 40, 5, 20), (2, 1, 33, -1, 21), (1, 3, 64, 17, 22), (1, 1, 9, 0, 23)]:
        q1, k1, q2, k2, v = _diff_inputs(B, H, S, seed)
        a, g, b, lm = _params(H, seed + 100)
        out = ora.diffattn(q1, k1, q2, k2, v, 0.125, w, a, g, b, 10000.0, lm)
        ref = _torch_diff(q1, k1, q2, k2, v, 0.125, w, a, g, b, 10000.0, lm)
        _close(out, ref, 1e-11, f"diff vs torch S={S} w={w}")


def pin_band_uniform_closed_form(ora):
    """q1 = q2 = 0 and beta = 0: DyT(0) = 0, all scores 0, so each branch is the mean of V over the
    clipped window W(p) = [max(0, p-w), min(S-1, p+w)] and the output is (1 - lambda_h) times it."""
    B, H, S, w = 1, 3, 41, 6
    r = _rng(30)
    k1, k2, v = (r.standard_normal((B, H, S, D)) for _ in range(3))
    z = np.zeros((B, H, S, D))
    a, g, _, lm = _params(H, 31)
    b = np.zeros((4, D))
    out = ora.diffattn(z, k1, z, k2, v, 0.125, w, a, g, b, 10000.0, lm)
    ref = np.empty_like(out)
    for p in range(S):
        lo, hi = max(0, p - w), min(S - 1, p + w)
        ref[:, :, p] = (1.0 - lm)[None, :, None] * v[:, :, lo:hi + 1].mean(axis=2)
    _close(out, ref, 1e-13, "band uniform")


def pin_band_onehot_counts(ora):
    """One-hot V: branch weights sit exactly on the in-window keys (zero outside, row sums 1 - lambda)."""
    S, w = 40, 4
    r = _rng(32)
    q1, k1, q2, k2, _ = _diff_inputs(1, 1, S, 33)
    v = np.zeros((1, 1, S, D))
    v[0, 0, np.arange(S), np.arange(S) % D] = 1.0  # S <= D: key j -> column j
    a, g, b, lm = _params(1, 34)
    out = ora.diffattn(q1, k1, q2, k2, v, 0.125, w, a, g, b, 10000.0, lm)[0, 0]
    for p in range(S):
        lo, hi = max(0, p - w), min(S - 1, p + w)
        outside = np.ones(D, dtype=bool)
        outside[lo:hi + 1] = False
        assert np.all(out[p, outside] == 0.0), f"weight outside window at p={p}"
        _close(out[p].sum(), 1.0 - lm[0], 1e-13, "band row sum")
    del r


def pin_window_full_equivalence(ora):
    """A window of S-1 or more is the full window; window 0 sees only the query's own position."""
    B, H, S = 1, 2, 19
    q1, k1, q2, k2, v = _diff_inputs(B, H, S, 40)
    a, g, b, lm = _params(H, 41)
    full = ora.diffattn(q1, k1, q2, k2, v, 0.125, -1, a, g, b, 10000.0, lm)
    for w in (S - 1, S, 10 * S):
        assert np.array_equal(ora.diffattn(q1, k1, q2, k2, v, 0.125, w, a, g, b, 10000.0, lm), full)
    own = ora.diffattn(q1, k1, q2, k2, v, 0.125, 0, a, g, b, 10000.0, lm)
    _close(own, (1.0 - lm)[None, :, None, None] * v, 1e-15, "window 0")


def pin_branch_cancellation(ora):
    """Identical branches and lambda = 1 give exactly zero."""
    B, H, S = 1, 2, 23
    q, k, _, _, v = _diff_inputs(B, H, S, 50)
    a, g, b, _ = _params(H, 51)
    a[2], g[2], b[2] = a[0], g[0], b[0]
    a[3], g[3], b[3] = a[1], g[1], b[1]
    for w in (-1, 3):
        out = ora.diffattn(q, k, q, k, v, 0.125, w, a, g, b, 10000.0, np.ones(H))
        assert np.all(out == 0.0), f"cancellation w={w}: max {np.abs(out).max()}"


def pin_diff_constant_v(ora):
    B, H, S = 2, 3, 17
    q1, k1, q2, k2, _ = _diff_inputs(B, H, S, 60)
    c = _rng(61).standard_normal(D)
    v = np.broadcast_to(c, (B, H, S, D)).copy()
    a, g, b, lm = _params(H, 62)
    for w in (-1, 2):
        out = ora.diffattn(q1, k1, q2, k2, v, 0.125, w, a, g, b, 10000.0, lm)
        ref = (1.0 - lm)[None, :, None, None] * c[None, None, None, :]
        _close(out, np.broadcast_to(ref, out.shape), 1e-13, f"diff constant V w={w}")


def pin_diff_single_token(ora):
    q1, k1, q2, k2, v = _diff_inputs(1, 2, 1, 70)
    a, g, b, lm = _params(2, 71)
    out = ora.diffattn(q1, k1, q2, k2, v, 0.125, 17, a, g, b, 10000.0, lm)
    _close(out, (1.0 - lm)[None, :, None, None] * v, 1e-15, "S=1")


def pin_diff_composes_from_dense(ora):
    """Row p of the differential output equals dense attention of the prepared rows over W(p),
    branch 1 minus lambda times branch 2, built from the oracle's own DyT / RoPE / dense pieces."""
    B, H, S, w = 1, 2, 30, 5
    q1, k1, q2, k2, v = _diff_inputs(B, H, S, 80)
    a, g, b, lm = _params(H, 81)
    out = ora.diffattn(q1, k1, q2, k2, v, 0.125, w, a, g, b, 10000.0, lm)

    def prep(x, t, p):
        return ora.rope_row(ora.dyt_row(x, a[t], g[t], b[t]), p, 10000.0)

    for h in range(H):
        for p in (0, 1, 5, 14, 28, 29):
            lo, hi = max(0, p - w), min(S - 1, p + w)
            js = range(lo, hi + 1)
            res = 0.0
            for (qt, kt, tq, tk, sign) in ((q1, k1, 0, 1, 1.0), (q2, k2, 2, 3, -lm[h])):
                qq = prep(qt[0, h, p], tq, p)[None, None, None, :]
                kk = np.stack([prep(kt[0, h, j], tk, j) for j in js])[None, None]
                vv = v[0, h, lo:hi + 1][None, None]
                res = res + sign * ora.attn(qq, kk, vv, 0.125)[0, 0, 0]
            _close(out[0, h, p], res, 1e-13, f"composition h={h} p={p}")


def pin_diff_rows_subset(ora):
    B, H, S = 2, 2, 25
    q1, k1, q2, k2, v = _diff_inputs(B, H, S, 90)
    a, g, b, lm = _params(H, 91)
    full = ora.diffattn(q1, k1, q2, k2, v, 0.125, 4, a, g, b, 10000.0, lm).reshape(-1, D)
    rows = np.array([0, 24, 25, 77, 99, 51])
    assert np.array_equal(ora.diffattn(q1, k1, q2, k2, v, 0.125, 4, a, g, b, 10000.0, lm, rows=rows), full[rows])


def _ld_attn(q, k, v, scale, keymask=None):
    """Long-double brute force in log-sum-exp form, keys in the outer loop."""
    q, k, v = (np.asarray(t, dtype=np.longdouble) for t in (q, k, v))
    Sq, Sk = q.shape[0], k.shape[0]
    s = np.full((Sq, Sk), -np.inf, dtype=np.longdouble)
    for j in range(Sk):
        for i in range(Sq):
            if keymask is None or keymask[i, j]:
                s[i, j] = scale * np.sum(q[i] * k[j])
    lse = np.array([np.log(np.sum(np.exp(row[np.isfinite(row)] - row.max()))) + row.max() for row in s],
                   dtype=np.longdouble)
    out = np.zeros((Sq, v.shape[1]), dtype=np.longdouble)
    for j in range(Sk):
        w = np.where(np.isfinite(s[:, j]), np.exp(s[:, j] - lse), 0)
        out += w[:, None] * v[j][None, :]
    return out


def pin_brute_force_long_double(ora):
    r = _rng(100)
    for (Sq, Sk) in [(1, 1), (3, 5), (6, 6), (2, 4)]:
        q, k, v = r.standard_normal((Sq, D)) * 3, r.standard_normal((Sk, D)), r.standard_normal((Sk, D))
        out = ora.attn(q[None, None], k[None, None], v[None, None], 0.125)[0, 0]
        _close(out, _ld_attn(q, k, v, 0.125).astype(np.float64), 1e-14, "dense brute force")
    # differential, tiny: prepare with long-double DyT (exp form) and a 2x2 rotation matrix per pair
    S, w = 6, 2
    q1, k1, q2, k2, v = (t[0, 0] for t in _diff_inputs(1, 1, S, 101))
    a, g, b, lm = _params(1, 102)

    def prep(x, t, p):
        x = np.asarray(x, dtype=np.longdouble)
        e = np.exp(np.longdouble(2 * a[t]) * x)
        y = g[t].astype(np.longdouble) * (e - 1) / (e + 1) + b[t].astype(np.longdouble)
        out = np.empty(D, dtype=np.longdouble)
        for i in range(32):
            th = np.longdouble(p) * np.longdouble(10000.0) ** (-np.longdouble(i) / 32)
            m = np.array([[np.cos(th), -np.sin(th)], [np.sin(th), np.cos(th)]], dtype=np.longdouble)
            out[i], out[i + 32] = m @ np.array([y[i], y[i + 32]], dtype=np.longdouble)
        return out

    mask = np.abs(np.arange(S)[:, None] - np.arange(S)[None, :]) <= w
    o1 = _ld_attn(np.stack([prep(q1[p], 0, p) for p in range(S)]), np.stack([prep(k1[j], 1, j) for j in range(S)]),
                  v, 0.125, mask)
    o2 = _ld_attn(np.stack([prep(q2[p], 2, p) for p in range(S)]), np.stack([prep(k2[j], 3, j) for j in range(S)]),
                  v, 0.125, mask)
    ref = (o1 - np.longdouble(lm[0]) * o2).astype(np.float64)
    out = ora.diffattn(q1[None, None], k1[None, None], q2[None, None], k2[None, None], v[None, None], 0.125, w, a, g,
                       b, 10000.0, lm)[0, 0]
    _close(out, ref, 1e-13, "diff brute force")


# ------------------------------------------------------------------ model forms: RMSNorm, partial rotary, V mask

def pin_rmsnorm_closed_forms(ora):
    """A constant row c gives w c / sqrt(c^2 + eps); with eps = 0 and unit weights the output has mean
    square exactly 1, is unchanged by positive scaling of x, and is odd in x."""
    r = _rng(200)
    w = r.uniform(0.5, 2.0, D)
    for c in (0.3, -2.5, 7.0):
        for eps in (0.0, 1e-6, 0.25):
            _close(ora.rmsnorm_row(np.full(D, c), eps, w), w * c / np.sqrt(c * c + eps), 1e-15,
                   f"rms constant c={c} eps={eps}")
    x = r.standard_normal(D) * 3
    y = ora.rmsnorm_row(x, 0.0, np.ones(D))
    _close(np.mean(y * y), 1.0, 1e-15, "rms unit mean square")
    _close(ora.rmsnorm_row(5.5 * x, 0.0, w), ora.rmsnorm_row(x, 0.0, w), 1e-15, "rms scale invariance")
    _close(ora.rmsnorm_row(-x, 1e-3, w), -ora.rmsnorm_row(x, 1e-3, w), 0.0, "rms odd")


def pin_rope_partial_basis_vectors(ora):
    """Width 32: e_i -> cos t e_i + sin t e_{i+16}, e_{i+16} -> -sin t e_i + cos t e_{i+16} with
    t = p base^(-2i/32); e_d for d >= 32 passes through.  Width 64 is the full rotation."""
    for p in (0, 1, 7, 23085):
        for i in (0, 1, 9, 15):
            t = p * 10000.0 ** (-2.0 * i / 32.0)
            e = np.zeros(D)
            e[i] = 1.0
            ref = np.zeros(D)
            ref[i], ref[i + 16] = np.cos(t), np.sin(t)
            _close(ora.rope_row_partial(e, 32, p, 10000.0), ref, 1e-13, f"rope32 e_{i} p={p}")
            e = np.zeros(D)
            e[i + 16] = 1.0
            ref = np.zeros(D)
            ref[i], ref[i + 16] = -np.sin(t), np.cos(t)
            _close(ora.rope_row_partial(e, 32, p, 10000.0), ref, 1e-13, f"rope32 e_{i + 16} p={p}")
        for d in (32, 41, 63):
            e = np.zeros(D)
            e[d] = 1.0
            _close(ora.rope_row_partial(e, 32, p, 10000.0), e, 0.0, f"rope32 pass-through e_{d} p={p}")
    x = _rng(201).standard_normal(D)
    for p in (0, 3, 999):
        _close(ora.rope_row_partial(x, 64, p, 10000.0), ora.rope_row(x, p, 10000.0), 1e-15, "rope width 64")


def _torch_diff_model(q1, k1, q2, k2, v, scale, window, w, eps, base, lam, keep):
    """The model form through torch: rms_norm (a library routine), complex rotation of pairs (i, i+16)
    for i < 16 with dims 32..63 appended unrotated, SDPA with a boolean band mask, V times the flags."""
    B, H, S, _ = q1.shape
    pos = torch.arange(S, dtype=torch.float64)
    freq = float(base) ** (-torch.arange(16, dtype=torch.float64) / 16.0)
    rot = torch.polar(torch.ones(S, 16, dtype=torch.float64), pos[:, None] * freq[None, :])

    def prep(x, t):
        y = torch.nn.functional.rms_norm(torch.from_numpy(x), (D,), weight=torch.from_numpy(w[t]), eps=eps)
        z = torch.complex(y[..., :16], y[..., 16:32]) * rot
        return torch.cat([z.real, z.imag, y[..., 32:]], dim=-1).contiguous()

    mask = None
    if window >= 0:
        idx = torch.arange(S)
        mask = (idx[:, None] - idx[None, :]).abs() <= window
    vt = (torch.from_numpy(v) * torch.from_numpy(keep.astype(np.float64))[:, None, :, None]).contiguous()
    o1 = torch.nn.functional.scaled_dot_product_attention(prep(q1, 0), prep(k1, 1), vt, attn_mask=mask, scale=scale)
    o2 = torch.nn.functional.scaled_dot_product_attention(prep(q2, 2), prep(k2, 3), vt, attn_mask=mask, scale=scale)
    return (o1 - torch.from_numpy(lam)[None, :, None, None] * o2).numpy()


def _model_params(H, seed):
    r = _rng(seed)
    return r.uniform(0.5, 2.0, (4, D)), r.uniform(0.2, 0.9, H)


def pin_diff_model_form_vs_torch(ora):
    for (B, H, S, win, eps, seed) in [(1, 2, 40, 5, 1e-6, 210), (2, 1, 33, -1, 1e-5, 211), (1, 3, 64, 17, 0.1, 212)]:
        q1, k1, q2, k2, v = _diff_inputs(B, H, S, seed, qk_scale=2.0)
        w, lm = _model_params(H, seed + 1)
        keep = (_rng(seed + 2).random((B, S)) > 0.25).astype(np.uint8)
        out = ora.diffattn(q1, k1, q2, k2, v, 0.125, win, None, None, None, 10000.0, lm, norm="rms", rms_weight=w,
                           rms_eps=eps, rotary_dims=32, v_keep=keep)
        ref = _torch_diff_model(q1, k1, q2, k2, v, 0.125, win, w, eps, 10000.0, lm, keep)
        _close(out, ref, 1e-11, f"model form vs torch S={S} w={win}")


def pin_v_keep_semantics(ora):
    """All flags set is the unmasked result bit for bit; none set gives exactly 0.  With one-hot V the
    columns of kept tokens equal the unmasked output (masked keys stay in the softmax, so the kept
    weights do not change) and the columns of padded tokens are exactly 0.  Flags index (b, token)."""
    S, win = 40, 6
    q1, k1, q2, k2, _ = _diff_inputs(2, 1, S, 220)
    v = np.zeros((2, 1, S, D))
    v[:, 0, np.arange(S), np.arange(S)] = 1.0  # key j -> column j (S <= D)
    a, g, b, lm = _params(1, 221)
    base = ora.diffattn(q1, k1, q2, k2, v, 0.125, win, a, g, b, 10000.0, lm)
    ones = np.ones((2, S), dtype=np.uint8)
    assert np.array_equal(ora.diffattn(q1, k1, q2, k2, v, 0.125, win, a, g, b, 10000.0, lm, v_keep=ones), base)
    assert np.all(ora.diffattn(q1, k1, q2, k2, v, 0.125, win, a, g, b, 10000.0, lm, v_keep=0 * ones) == 0.0)
    keep = (_rng(222).random((2, S)) > 0.4).astype(np.uint8)
    keep[0, :5] = 0
    keep[1, :5] = 1  # the two batches differ
    out = ora.diffattn(q1, k1, q2, k2, v, 0.125, win, a, g, b, 10000.0, lm, v_keep=keep)
    for bb in range(2):
        kept = keep[bb].astype(bool)
        _close(out[bb, 0][:, :S][:, kept], base[bb, 0][:, :S][:, kept], 1e-15, f"kept columns b={bb}")
        assert np.all(out[bb, 0][:, :S][:, ~kept] == 0.0), f"padded columns b={bb}"
    for win2 in (-1, 3):
        one = ora.diffattn(q1[1:], k1[1:], q2[1:], k2[1:], v[1:], 0.125, win2, a, g, b, 10000.0, lm, v_keep=keep[1:])
        both = ora.diffattn(q1, k1, q2, k2, v, 0.125, win2, a, g, b, 10000.0, lm, v_keep=keep)
        assert np.array_equal(both[1:], one), f"flags follow the batch index (w={win2})"


def pin_brute_force_model_form(ora):
    """Long-double brute force of the model form on a tiny input: RMSNorm, a 2x2 rotation per pair
    (i, i+16) for i < 16, dims 32..63 untouched, V rows of padded tokens zero, band mask."""
    S, win, eps = 7, 2, 1e-3
    q1, k1, q2, k2, v = (t[0, 0] for t in _diff_inputs(1, 1, S, 230, qk_scale=2.0))
    w, lm = _model_params(1, 231)
    keep = np.array([1, 0, 1, 1, 0, 1, 1], dtype=np.uint8)

    def prep(x, t, p):
        x = np.asarray(x, dtype=np.longdouble)
        y = w[t].astype(np.longdouble) * x / np.sqrt(np.mean(x * x) + np.longdouble(eps))
        out = y.copy()
        for i in range(16):
            th = np.longdouble(p) * np.longdouble(10000.0) ** (-np.longdouble(2 * i) / 32)
            m = np.array([[np.cos(th), -np.sin(th)], [np.sin(th), np.cos(th)]], dtype=np.longdouble)
            out[i], out[i + 16] = m @ np.array([y[i], y[i + 16]], dtype=np.longdouble)
        return out

    mask = np.abs(np.arange(S)[:, None] - np.arange(S)[None, :]) <= win
    vk = v * keep[:, None]
    o1 = _ld_attn(np.stack([prep(q1[p], 0, p) for p in range(S)]), np.stack([prep(k1[j], 1, j) for j in range(S)]),
                  vk, 0.125, mask)
    o2 = _ld_attn(np.stack([prep(q2[p], 2, p) for p in range(S)]), np.stack([prep(k2[j], 3, j) for j in range(S)]),
                  vk, 0.125, mask)
    ref = (o1 - np.longdouble(lm[0]) * o2).astype(np.float64)
    out = ora.diffattn(q1[None, None], k1[None, None], q2[None, None], k2[None, None], v[None, None], 0.125, win,
                       None, None, None, 10000.0, lm, norm="rms", rms_weight=w, rms_eps=eps, rotary_dims=32,
                       v_keep=keep[None])[0, 0]
    _close(out, ref, 1e-13, "model form brute force")


ALL_PINS = [obj for name, obj in sorted(globals().items()) if name.startswith("pin_") and callable(obj)]


def bound_oracle(lib):
    """The oracle module's functions bound to one compiled library."""
    import oracle
    ns = types.SimpleNamespace()
    ns.attn = lambda *a, **kw: oracle.attn(*a, lib=lib, **kw)
    ns.diffattn = lambda *a, **kw: oracle.diffattn(*a, lib=lib, **kw)
    ns.dyt_row = lambda *a, **kw: oracle.dyt_row(*a, lib=lib, **kw)
    ns.rope_row = lambda *a, **kw: oracle.rope_row(*a, lib=lib, **kw)
    ns.rmsnorm_row = lambda *a, **kw: oracle.rmsnorm_row(*a, lib=lib, **kw)
    ns.rope_row_partial = lambda *a, **kw: oracle.rope_row_partial(*a, lib=lib, **kw)
    return ns

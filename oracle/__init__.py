"""fp64 CPU oracle for fused head-dim-64 attention -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check in __graft_entry__.py and the cpu_baseline leg of
bench.py may import this package.  The library in head_attention_flash_amd/ never
does, and this package never imports the library: the two share no code.

The arithmetic lives in ka_oracle.c (plain C, double precision, OpenMP over rows).
This module only widens stored values to float64 (exactly: a bf16 or fp32 element
is representable in a double), hands them to the C code through ctypes and
returns float64 results.  Definitions and citations are in ka_oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ka_oracle.c")
_LIB = os.path.join(_HERE, "libka_oracle.so")
_lock = threading.Lock()
_lib = None


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, strict IEEE double: no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
           "-Wall", "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: str | None = None):
    """Load (building first if absent or stale) and return the ctypes handle."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if (not os.path.exists(_LIB)) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int64)
    lib.ora_attn.argtypes = [dp, dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                             ctypes.c_double, ip, ctypes.c_int64]
    lib.ora_attn.restype = ctypes.c_int
    lib.ora_diffattn.argtypes = [dp, dp, dp, dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_double, ctypes.c_int, dp, dp, dp, ctypes.c_double, dp, ip, ctypes.c_int64]
    lib.ora_diffattn.restype = ctypes.c_int
    u8p = ctypes.POINTER(ctypes.c_ubyte)
    lib.ora_diffattn_ex.argtypes = [dp, dp, dp, dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_double, ctypes.c_int, ctypes.c_int, dp, dp, dp, ctypes.c_double, dp,
                                    ctypes.c_int, ctypes.c_double, dp, u8p, ip, ctypes.c_int64]
    lib.ora_diffattn_ex.restype = ctypes.c_int
    lib.ora_rmsnorm_row.argtypes = [dp, ctypes.c_int, ctypes.c_double, dp, dp]
    lib.ora_rmsnorm_row.restype = None
    lib.ora_rope_row_partial.argtypes = [dp, ctypes.c_int, ctypes.c_int, ctypes.c_long, ctypes.c_double, dp]
    lib.ora_rope_row_partial.restype = None
    lib.ora_dyt_row.argtypes = [dp, ctypes.c_int, ctypes.c_double, dp, dp, dp]
    lib.ora_dyt_row.restype = None
    lib.ora_rope_row.argtypes = [dp, ctypes.c_int, ctypes.c_long, ctypes.c_double, dp]
    lib.ora_rope_row.restype = None
    lib.ora_num_threads.argtypes = []
    lib.ora_num_threads.restype = ctypes.c_int
    return lib


# ------------------------------------------------------------------ marshalling

def widen(x) -> np.ndarray:
    """Exact float64 view of stored values.  uint16 arrays are bf16 bit patterns."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"unsupported storage dtype {x.dtype}")


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _c64(a) -> np.ndarray:
    return np.ascontiguousarray(widen(a), dtype=np.float64)


def _rows(rows):
    if rows is None:
        return None, None, 0
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    return r, r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), int(r.size)


def attn(q, k, v, scale: float, rows=None, lib=None) -> np.ndarray:
    """softmax(scale * q k^T) v per (b, h); q [B,H,Sq,D], k/v [B,H,Sk,D].

    rows: optional flat row indices (b*H + h)*Sq + i; then the result is [len(rows), D].
    """
    lib = lib or load()
    q, k, v = _c64(q), _c64(k), _c64(v)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    assert k.shape == (B, H, Sk, D) and v.shape == (B, H, Sk, D)
    out = np.full((B, H, Sq, D), np.nan)
    r, rp, nr = _rows(rows)
    rc = lib.ora_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, Sq, Sk, D, float(scale), rp, nr)
    if rc != 0:
        raise RuntimeError(f"ora_attn failed ({rc})")
    return out if r is None else out.reshape(-1, D)[r]


def diffattn(q1, k1, q2, k2, v, scale: float, window: int, alpha, gamma, beta, base: float, lam, rows=None,
             lib=None, norm: str = "dyt", rms_weight=None, rms_eps: float = 0.0, rotary_dims: int | None = None,
             v_keep=None) -> np.ndarray:
    """Differential attention: O = softmax(q1^ k1^T) V' - lam_h softmax(q2^ k2^T) V'.

    q^/k^ = RoPE(Norm(.)); window >= 0 keeps keys with |i - j| <= window, window < 0 keeps all.
    norm "dyt": alpha [4], gamma/beta [4, D] for (q1, k1, q2, k2).  norm "rms": rms_weight [4, D]
    and rms_eps (alpha, gamma, beta may be None).  rotary_dims: the rotated width (default D).
    v_keep: optional [B, S] flags; V' zeroes the V rows of tokens whose flag is 0 (their keys stay).
    lam [H].  With the defaults this is the DyT form over all D dims ("ora_diffattn").
    """
    lib = lib or load()
    q1, k1, q2, k2, v = (_c64(t) for t in (q1, k1, q2, k2, v))
    B, H, S, D = q1.shape
    for t in (k1, q2, k2, v):
        assert t.shape == (B, H, S, D)
    lm = np.ascontiguousarray(np.asarray(lam, dtype=np.float64).reshape(H))
    out = np.full((B, H, S, D), np.nan)
    r, rp, nr = _rows(rows)
    if norm == "dyt" and rotary_dims in (None, D) and v_keep is None:
        a = np.ascontiguousarray(np.asarray(alpha, dtype=np.float64).reshape(4))
        g = np.ascontiguousarray(np.asarray(gamma, dtype=np.float64).reshape(4, D))
        b_ = np.ascontiguousarray(np.asarray(beta, dtype=np.float64).reshape(4, D))
        rc = lib.ora_diffattn(_ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(v), _ptr(out), B, H, S, D, float(scale),
                              int(window), _ptr(a), _ptr(g), _ptr(b_), float(base), _ptr(lm), rp, nr)
    else:
        null = ctypes.POINTER(ctypes.c_double)()
        if norm == "dyt":
            a = np.ascontiguousarray(np.asarray(alpha, dtype=np.float64).reshape(4))
            g = np.ascontiguousarray(np.asarray(gamma, dtype=np.float64).reshape(4, D))
            b_ = np.ascontiguousarray(np.asarray(beta, dtype=np.float64).reshape(4, D))
            pa, pg, pb, pw, nid = _ptr(a), _ptr(g), _ptr(b_), null, 0
        elif norm == "rms":
            w = np.ascontiguousarray(np.asarray(rms_weight, dtype=np.float64).reshape(4, D))
            pa, pg, pb, pw, nid = null, null, null, _ptr(w), 1
        else:
            raise ValueError(f"unknown norm {norm!r}")
        keep = None
        pk = ctypes.POINTER(ctypes.c_ubyte)()
        if v_keep is not None:
            keep = np.ascontiguousarray((np.asarray(v_keep).reshape(B, S) != 0).astype(np.uint8))
            pk = keep.ctypes.data_as(ctypes.POINTER(ctypes.c_ubyte))
        rot = D if rotary_dims is None else int(rotary_dims)
        rc = lib.ora_diffattn_ex(_ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(v), _ptr(out), B, H, S, D, float(scale),
                                 int(window), nid, pa, pg, pb, float(rms_eps), pw, rot, float(base), _ptr(lm), pk, rp,
                                 nr)
    if rc != 0:
        raise RuntimeError(f"ora_diffattn failed ({rc})")
    return out if r is None else out.reshape(-1, D)[r]


def dyt_row(x, alpha: float, gamma, beta, lib=None) -> np.ndarray:
    lib = lib or load()
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    D = x.size
    g = np.ascontiguousarray(np.asarray(gamma, dtype=np.float64).reshape(D))
    b_ = np.ascontiguousarray(np.asarray(beta, dtype=np.float64).reshape(D))
    y = np.empty(D)
    lib.ora_dyt_row(_ptr(x), D, float(alpha), _ptr(g), _ptr(b_), _ptr(y))
    return y


def rope_row(x, p: int, base: float, lib=None) -> np.ndarray:
    lib = lib or load()
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    y = np.empty(x.size)
    lib.ora_rope_row(_ptr(x), x.size, int(p), float(base), _ptr(y))
    return y


def rmsnorm_row(x, eps: float, weight, lib=None) -> np.ndarray:
    lib = lib or load()
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    w = np.ascontiguousarray(np.asarray(weight, dtype=np.float64).reshape(x.size))
    y = np.empty(x.size)
    lib.ora_rmsnorm_row(_ptr(x), x.size, float(eps), _ptr(w), _ptr(y))
    return y


def rope_row_partial(x, rot: int, p: int, base: float, lib=None) -> np.ndarray:
    lib = lib or load()
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    y = np.empty(x.size)
    lib.ora_rope_row_partial(_ptr(x), x.size, int(rot), int(p), float(base), _ptr(y))
    return y


def num_threads(lib=None) -> int:
    return int((lib or load()).ora_num_threads())

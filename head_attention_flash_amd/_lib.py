"""Thin ctypes binding of libka_attn.so: argument marshalling only.

The functions carry the C names.  They take torch tensors that already live on
the GPU (torch only allocates memory and supplies the stream), pass their data
pointers and the current HIP stream to the C ABI, and raise KaError on any
non-OK status.  Every step of the computation runs in the library's HIP kernels;
there is no fallback: if the library is not built, the first call raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libka_attn.so")

KA_OK, KA_ERR_NULL, KA_ERR_SHAPE, KA_ERR_UNSUPPORTED, KA_ERR_PARAM, KA_ERR_ALIGN, KA_ERR_ALIAS, \
    KA_ERR_WORKSPACE, KA_ERR_HIP = range(9)
KA_F32, KA_BF16 = 0, 1
KA_QKNORM_DYT, KA_QKNORM_RMS = 0, 1
KA_XATTN_MAX_SK = 512

# every symbol include/ka_attn.h declares
EXPORTS = ("ka_attn_fwd", "ka_xattn_fwd", "ka_diffattn_fwd", "ka_diffattn_fwd_ex", "ka_diffattn_fwd_noalloc",
           "ka_diffattn_workspace_bytes", "ka_attn_kernel_name", "ka_status_string", "ka_last_hip_error", "ka_version")
KA_STATIC_WORKSPACE_BYTES = 32 << 20


class KaError(RuntimeError):
    def __init__(self, status: int, where: str, lib=None):
        msg = lib.ka_status_string(status).decode() if lib is not None else str(status)
        extra = f" (hipError {lib.ka_last_hip_error()})" if (lib is not None and status == KA_ERR_HIP) else ""
        super().__init__(f"{where}: {msg}{extra}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load libka_attn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    fp = ctypes.POINTER(ctypes.c_float)
    lib.ka_attn_fwd.argtypes = [i, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    lib.ka_attn_fwd.restype = i
    lib.ka_xattn_fwd.argtypes = [i, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    lib.ka_xattn_fwd.restype = i
    lib.ka_diffattn_fwd.argtypes = [i, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, vp, vp, f, vp, vp, sz, vp]
    lib.ka_diffattn_fwd.restype = i
    lib.ka_diffattn_fwd_ex.argtypes = [i, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, vp, vp, vp, f, i, f, vp,
                                       vp, vp, vp, sz, vp]
    lib.ka_diffattn_fwd_ex.restype = i
    lib.ka_diffattn_fwd_noalloc.argtypes = [i, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, vp, vp, vp, f, i, f,
                                            vp, vp, vp, vp]
    lib.ka_diffattn_fwd_noalloc.restype = i
    lib.ka_diffattn_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.ka_diffattn_workspace_bytes.restype = sz
    lib.ka_attn_kernel_name.argtypes = [i, i, i, i, i, i]
    lib.ka_attn_kernel_name.restype = ctypes.c_char_p
    lib.ka_status_string.argtypes = [i]
    lib.ka_status_string.restype = ctypes.c_char_p
    lib.ka_last_hip_error.argtypes = []
    lib.ka_last_hip_error.restype = i
    lib.ka_version.argtypes = []
    lib.ka_version.restype = ctypes.c_char_p
    del fp
    if path == LIB_PATH:
        _lib = lib
    return lib


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return KA_F32
    if t.dtype == torch.bfloat16:
        return KA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _expect(t, name: str, shape, dtype, device):
    """Check a tensor argument's shape, dtype and device before any pointer reaches the C ABI (which
    sees raw pointers only and cannot tell a short or mistyped buffer from a good one)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device} (the device of the first operand)")


def _check_qkv(q, k, v, o):
    """q [B,H,Sq,D], k and v [B,H,Sk,D], o like q: one dtype (fp32 or bf16), one device."""
    if q.dim() != 4:
        raise ValueError(f"q must be [B, H, Sq, D], got shape {tuple(q.shape)}")
    _dtype_code(q)
    if k.dim() != 4:
        raise ValueError(f"k must be [B, H, Sk, D], got shape {tuple(k.shape)}")
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    _expect(k, "k", (B, H, Sk, D), q.dtype, q.device)
    _expect(v, "v", (B, H, Sk, D), q.dtype, q.device)
    if o is not None:
        _expect(o, "o", (B, H, Sq, D), q.dtype, q.device)


def _check_diff(q1, k1, q2, k2, v, o, lam, params, v_keep=None, workspace=None):
    """q1, k1, q2, k2, v, o [B,H,S,64] bf16; lam [H] fp32; params: (name, tensor, shape) of the fp32
    parameter arrays in use; v_keep [B,S] uint8; workspace a uint8 tensor.  One device."""
    torch = _torch()
    if q1.dim() != 4:
        raise ValueError(f"q1 must be [B, H, S, 64], got shape {tuple(q1.shape)}")
    B, H, S, D = q1.shape
    dev = q1.device
    for t, name in ((q1, "q1"), (k1, "k1"), (q2, "q2"), (k2, "k2"), (v, "v"), (o, "o")):
        if t is not None:
            _expect(t, name, (B, H, S, D), torch.bfloat16, dev)
    _expect(lam, "lambda", (H,), torch.float32, dev)
    for name, t, shape in params:
        _expect(t, name, shape, torch.float32, dev)
    if v_keep is not None:
        _expect(v_keep, "v_keep", (B, S), torch.uint8, dev)
    if workspace is not None:
        if workspace.dtype != torch.uint8 or workspace.dim() != 1:
            raise ValueError("workspace must be a 1-D uint8 tensor")
        if workspace.device != dev:
            raise ValueError(f"workspace is on {workspace.device}, expected {dev}")


def _dev(t, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous [B, H, S, D]")
    return ctypes.c_void_p(t.data_ptr())


class KaLayout(ctypes.Structure):
    """ka_layout: element strides (batch, head, token) of a [B][H][S][64] view."""
    _fields_ = [("batch", ctypes.c_int64), ("head", ctypes.c_int64), ("token", ctypes.c_int64)]


def _dev_view(t, name: str):
    """A [B, H, S, 64] GPU view whose last dim is contiguous; returns (pointer, ka_layout)."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dim() != 4 or t.stride(-1) != 1:
        raise ValueError(f"{name} must be a [B, H, S, D] view with contiguous D")
    return ctypes.c_void_p(t.data_ptr()), KaLayout(t.stride(0), t.stride(1), t.stride(2))


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(lib, st: int, where: str):
    if st != KA_OK:
        raise KaError(st, where, lib)


def ka_attn_fwd(q, k, v, o=None, scale: float = 0.125, stream=None):
    """Dense attention; q [B,H,Sq,64], k/v [B,H,Sk,64] (fp32 or bf16, same dtype). Returns o."""
    lib = load()
    _check_qkv(q, k, v, o)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    if o is None:
        o = _torch().empty_like(q)
    st = lib.ka_attn_fwd(_dtype_code(q), _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), B, H, Sq, Sk, D,
                         float(scale), _stream(stream))
    _check(lib, st, "ka_attn_fwd")
    return o


def ka_xattn_fwd(q, k, v, o=None, scale: float = 0.125, stream=None):
    """Cross-attention: key sets up to 256 held on chip, longer ones streamed. Returns o."""
    lib = load()
    _check_qkv(q, k, v, o)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    if o is None:
        o = _torch().empty_like(q)
    st = lib.ka_xattn_fwd(_dtype_code(q), _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), B, H, Sq, Sk, D,
                          float(scale), _stream(stream))
    _check(lib, st, "ka_xattn_fwd")
    return o


def ka_diffattn_workspace_bytes(B: int, H: int, S: int, D: int = 64, window: int = -1) -> int:
    return int(load().ka_diffattn_workspace_bytes(B, H, S, D, window))


def ka_attn_kernel_name(B: int, H: int, Sq: int, Sk: int, D: int = 64, dtype: int = KA_BF16):
    """Name and layout of the kernel ka_attn_fwd runs for this shape on the current device, or None."""
    r = load().ka_attn_kernel_name(dtype, B, H, Sq, Sk, D)
    return r.decode() if r is not None else None


def ka_diffattn_fwd(q1, k1, q2, k2, v, alpha, gamma, beta, lam, o=None, scale: float = 0.125, window: int = -1,
                    rope_base: float = 10000.0, workspace=None, stream=None):
    """Differential attention (bf16). alpha [4], gamma/beta [4,64], lam [H]: fp32 GPU tensors.

    workspace: a GPU uint8 tensor of at least ka_diffattn_workspace_bytes(...) bytes, or None to
    have torch allocate one for this call.
    """
    lib = load()
    _check_diff(q1, k1, q2, k2, v, o, lam, (("alpha", alpha, (4,)), ("gamma", gamma, (4, 64)), ("beta", beta, (4, 64))),
                workspace=workspace)
    B, H, S, D = q1.shape
    if o is None:
        o = _torch().empty_like(q1)
    need = int(lib.ka_diffattn_workspace_bytes(B, H, S, D, window))
    if workspace is None and need:
        workspace = _torch().empty(need, dtype=_torch().uint8, device=q1.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.ka_diffattn_fwd(_dtype_code(q1), _dev(q1, "q1"), _dev(k1, "k1"), _dev(q2, "q2"), _dev(k2, "k2"),
                             _dev(v, "v"), _dev(o, "o"), B, H, S, S, D, float(scale), int(window),
                             _dev(alpha, "alpha"), _dev(gamma, "gamma"), _dev(beta, "beta"), float(rope_base),
                             _dev(lam, "lambda"), ws_ptr, ws_bytes, _stream(stream))
    _check(lib, st, "ka_diffattn_fwd")
    return o


def ka_diffattn_fwd_ex(q1, k1, q2, k2, v, lam, o=None, scale: float = 0.125, window: int = -1, qk_norm: str = "dyt",
                       alpha=None, gamma=None, beta=None, rms_weight=None, rms_eps: float = 1e-6,
                       rotary_dims: int = 64, rope_base: float = 10000.0, v_keep=None, workspace=None, stream=None):
    """Differential attention (bf16) in the model forms: qk_norm "dyt" (alpha [4], gamma/beta [4,64]) or
    "rms" (rms_weight [4,64], rms_eps); rotary_dims 64 or 32; v_keep: optional [B,S] uint8 GPU tensor
    (0 = that token's V row is zero, its key stays).  All parameter tensors are fp32 GPU tensors.
    q1, k1, q2, k2, v and o may be strided [B, H, S, 64] views (e.g. slices of a fused projection);
    their strides are passed as ka_layout views.
    """
    lib = load()
    if qk_norm not in ("dyt", "rms"):
        raise ValueError(f"qk_norm must be 'dyt' or 'rms', got {qk_norm!r}")
    prm = ((("alpha", alpha, (4,)), ("gamma", gamma, (4, 64)), ("beta", beta, (4, 64))) if qk_norm == "dyt"
           else (("rms_weight", rms_weight, (4, 64)),))
    _check_diff(q1, k1, q2, k2, v, o, lam, prm, v_keep=v_keep, workspace=workspace)
    B, H, S, D = q1.shape
    if o is None:
        o = _torch().empty_like(q1)
    need = int(lib.ka_diffattn_workspace_bytes(B, H, S, D, window))
    if workspace is None and need:
        workspace = _torch().empty(need, dtype=_torch().uint8, device=q1.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    norm = {"dyt": KA_QKNORM_DYT, "rms": KA_QKNORM_RMS}[qk_norm]
    opt = lambda t, name: _dev(t, name) if t is not None else ctypes.c_void_p(0)  # noqa: E731
    views = [_dev_view(t, n) for t, n in ((q1, "q1"), (k1, "k1"), (q2, "q2"), (k2, "k2"), (v, "v"), (o, "o"))]
    layouts = None
    if not all(t.is_contiguous() for t in (q1, k1, q2, k2, v, o)):
        layouts = (KaLayout * 6)(*[lay for _, lay in views])
    st = lib.ka_diffattn_fwd_ex(_dtype_code(q1), *[ptr for ptr, _ in views], B, H, S, S, D, float(scale), int(window),
                                norm, opt(alpha, "alpha"), opt(gamma, "gamma"), opt(beta, "beta"),
                                opt(rms_weight, "rms_weight"), float(rms_eps), int(rotary_dims), float(rope_base),
                                _dev(lam, "lambda"), opt(v_keep, "v_keep"),
                                ctypes.cast(layouts, ctypes.c_void_p) if layouts is not None else None, ws_ptr,
                                ws_bytes, _stream(stream))
    _check(lib, st, "ka_diffattn_fwd_ex")
    return o


def ka_diffattn_fwd_noalloc(q1, k1, q2, k2, v, lam, o=None, scale: float = 0.125, window: int = -1,
                            qk_norm: str = "dyt", alpha=None, gamma=None, beta=None, rms_weight=None,
                            rms_eps: float = 1e-6, rotary_dims: int = 64, rope_base: float = 10000.0, v_keep=None,
                            stream=None):
    """ka_diffattn_fwd_ex without a workspace: the library's per-GPU scratch array (KA_STATIC_WORKSPACE_BYTES)
    serves the full path, and the call allocates nothing (pass o to avoid torch allocating the output).
    Calls that overlap in time on one GPU share that array and race."""
    lib = load()
    if qk_norm not in ("dyt", "rms"):
        raise ValueError(f"qk_norm must be 'dyt' or 'rms', got {qk_norm!r}")
    prm = ((("alpha", alpha, (4,)), ("gamma", gamma, (4, 64)), ("beta", beta, (4, 64))) if qk_norm == "dyt"
           else (("rms_weight", rms_weight, (4, 64)),))
    _check_diff(q1, k1, q2, k2, v, o, lam, prm, v_keep=v_keep)
    B, H, S, D = q1.shape
    if o is None:
        o = _torch().empty_like(q1)
    norm = {"dyt": KA_QKNORM_DYT, "rms": KA_QKNORM_RMS}[qk_norm]
    opt = lambda t, name: _dev(t, name) if t is not None else ctypes.c_void_p(0)  # noqa: E731
    views = [_dev_view(t, n) for t, n in ((q1, "q1"), (k1, "k1"), (q2, "q2"), (k2, "k2"), (v, "v"), (o, "o"))]
    layouts = None
    if not all(t.is_contiguous() for t in (q1, k1, q2, k2, v, o)):
        layouts = (KaLayout * 6)(*[lay for _, lay in views])
    st = lib.ka_diffattn_fwd_noalloc(_dtype_code(q1), *[ptr for ptr, _ in views], B, H, S, S, D, float(scale),
                                     int(window), norm, opt(alpha, "alpha"), opt(gamma, "gamma"), opt(beta, "beta"),
                                     opt(rms_weight, "rms_weight"), float(rms_eps), int(rotary_dims),
                                     float(rope_base), _dev(lam, "lambda"), opt(v_keep, "v_keep"),
                                     ctypes.cast(layouts, ctypes.c_void_p) if layouts is not None else None,
                                     _stream(stream))
    _check(lib, st, "ka_diffattn_fwd_noalloc")
    return o

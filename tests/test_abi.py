"""The C ABI on the CPU: the library loads, exports what the header declares, and rejects bad
arguments with the documented status codes before touching HIP (no compute call is made here)."""
import ctypes
import math
import os
import re

import pytest

import head_attention_flash_amd as ka
from head_attention_flash_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ka_attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return _lib.load()


def declared_symbols():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ka_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_three_operations():
    syms = declared_symbols()
    for s in ("ka_attn_fwd", "ka_xattn_fwd", "ka_diffattn_fwd", "ka_diffattn_fwd_ex"):
        assert s in syms


def test_library_exports_every_declared_symbol(lib):
    for s in declared_symbols():
        assert hasattr(lib, s), f"{s} declared in ka_attn.h but not exported"
    assert set(declared_symbols()) == set(_lib.EXPORTS)


def test_version_and_status_strings(lib):
    assert re.match(rb"^\d+\.\d+\.\d+$", lib.ka_version())
    for st in range(9):
        assert lib.ka_status_string(st)
    assert lib.ka_status_string(99) == b"unknown status"
    assert lib.ka_last_hip_error() == 0


# fake, distinct, 16-byte aligned device addresses: only validation runs on them
Q, K, V, O, O2, A, G, BT, L, W = (0x100000 * (i + 1) for i in range(10))


def dense(lib, fn, dt=ka.KA_BF16, q=Q, k=K, v=V, o=O, B=1, H=1, Sq=4, Sk=4, D=64, scale=0.125):
    f = getattr(lib, fn)
    return f(dt, q, k, v, o, B, H, Sq, Sk, D, ctypes.c_float(scale), None)


@pytest.mark.parametrize("fn", ["ka_attn_fwd", "ka_xattn_fwd"])
def test_dense_validation(lib, fn):
    assert dense(lib, fn, q=0) == _lib.KA_ERR_NULL
    assert dense(lib, fn, o=0) == _lib.KA_ERR_NULL
    assert dense(lib, fn, B=0) == _lib.KA_ERR_SHAPE
    assert dense(lib, fn, H=-1) == _lib.KA_ERR_SHAPE
    assert dense(lib, fn, Sq=0) == _lib.KA_ERR_SHAPE
    assert dense(lib, fn, Sk=0) == _lib.KA_ERR_SHAPE
    assert dense(lib, fn, D=128) == _lib.KA_ERR_UNSUPPORTED
    assert dense(lib, fn, D=512, dt=ka.KA_F32) == _lib.KA_ERR_UNSUPPORTED
    assert dense(lib, fn, dt=7) == _lib.KA_ERR_UNSUPPORTED
    assert dense(lib, fn, scale=float("nan")) == _lib.KA_ERR_PARAM
    assert dense(lib, fn, scale=math.inf) == _lib.KA_ERR_PARAM
    assert dense(lib, fn, scale=0.0) == _lib.KA_ERR_PARAM
    assert dense(lib, fn, q=Q + 8) == _lib.KA_ERR_ALIGN
    assert dense(lib, fn, o=O + 2) == _lib.KA_ERR_ALIGN
    assert dense(lib, fn, o=Q) == _lib.KA_ERR_ALIAS
    assert dense(lib, fn, o=K + 256) == _lib.KA_ERR_ALIAS
    assert dense(lib, fn, B=1 << 20, H=1 << 20, Sq=1 << 20) == _lib.KA_ERR_SHAPE  # bytes overflow
    assert lib.ka_last_hip_error() == 0


def test_head_dim_512(lib):
    # ka_attn_fwd takes D = 512 in bf16 (validation runs in full: here it stops at the alias check)
    assert dense(lib, "ka_attn_fwd", D=512, o=Q) == _lib.KA_ERR_ALIAS
    assert dense(lib, "ka_xattn_fwd", D=512) == _lib.KA_ERR_UNSUPPORTED


def test_xattn_takes_long_key_sets(lib):
    # past the on-chip limit the keys stream: the only shape limits left are the dense ones
    assert dense(lib, "ka_xattn_fwd", Sk=ka.KA_XATTN_MAX_SK + 1, o=Q) == _lib.KA_ERR_ALIAS
    assert dense(lib, "ka_xattn_fwd", Sk=(1 << 31) - 1) == _lib.KA_ERR_SHAPE  # 32-bit buffer offsets


def diff(lib, dt=ka.KA_BF16, q1=Q, k1=K, q2=V, k2=O2, v=A, o=O, B=1, H=2, Sq=8, Sk=8, D=64, scale=0.125, window=2,
         alpha=A + 0x80000, gamma=G, beta=BT, base=10000.0, lam=L, ws=0, ws_bytes=0):
    return lib.ka_diffattn_fwd(dt, q1, k1, q2, k2, v, o, B, H, Sq, Sk, D, ctypes.c_float(scale), window, alpha, gamma,
                               beta, ctypes.c_float(base), lam, ws, ws_bytes, None)


def test_diff_validation(lib):
    for name in ("q1", "k1", "q2", "k2", "v", "o", "alpha", "gamma", "beta", "lam"):
        assert diff(lib, **{name: 0}) == _lib.KA_ERR_NULL, name
    assert diff(lib, Sk=9) == _lib.KA_ERR_SHAPE
    assert diff(lib, B=0) == _lib.KA_ERR_SHAPE
    assert diff(lib, D=32) == _lib.KA_ERR_UNSUPPORTED
    assert diff(lib, dt=ka.KA_F32) == _lib.KA_ERR_UNSUPPORTED
    assert diff(lib, base=1.0) == _lib.KA_ERR_PARAM
    assert diff(lib, base=float("inf")) == _lib.KA_ERR_PARAM
    assert diff(lib, scale=-1.0) == _lib.KA_ERR_PARAM
    assert diff(lib, v=A + 4) == _lib.KA_ERR_ALIGN
    assert diff(lib, o=Q + 64) == _lib.KA_ERR_ALIAS
    # the full path needs a workspace: the prepared keys and V, three fp16 planes
    assert lib.ka_diffattn_workspace_bytes(1, 2, 8, 64, -1) == 3 * 1 * 2 * 8 * 64 * 2
    need = 3 * 1 * 2 * 8 * 64 * 2
    assert diff(lib, window=-1) == _lib.KA_ERR_NULL
    assert diff(lib, window=-1, ws=W, ws_bytes=need - 1) == _lib.KA_ERR_WORKSPACE
    assert diff(lib, window=-1, ws=W + 8, ws_bytes=need) == _lib.KA_ERR_ALIGN
    assert diff(lib, window=-1, ws=O, ws_bytes=need) == _lib.KA_ERR_ALIAS
    assert diff(lib, window=-1, ws=K, ws_bytes=need) == _lib.KA_ERR_ALIAS
    assert lib.ka_last_hip_error() == 0


KEEP = 0x100000 * 12


def diff_ex(lib, dt=ka.KA_BF16, q1=Q, k1=K, q2=V, k2=O2, v=A, o=O, B=1, H=2, Sq=8, Sk=8, D=64, scale=0.125,
            window=2, norm=ka.KA_QKNORM_RMS, alpha=0, gamma=0, beta=0, rms_w=G, eps=1e-6, rot=32, base=10000.0,
            lam=L, keep=KEEP, layouts=None, ws=0, ws_bytes=0):
    return lib.ka_diffattn_fwd_ex(dt, q1, k1, q2, k2, v, o, B, H, Sq, Sk, D, ctypes.c_float(scale), window, norm,
                                  alpha, gamma, beta, rms_w, ctypes.c_float(eps), rot, ctypes.c_float(base), lam,
                                  keep, layouts, ws, ws_bytes, None)


def test_diff_ex_validation(lib):
    # every case fails before any HIP call
    assert diff_ex(lib, norm=7) == _lib.KA_ERR_UNSUPPORTED
    assert diff_ex(lib, rms_w=0) == _lib.KA_ERR_NULL
    assert diff_ex(lib, norm=ka.KA_QKNORM_DYT) == _lib.KA_ERR_NULL  # DyT parameters missing
    assert diff_ex(lib, norm=ka.KA_QKNORM_DYT, alpha=A + 0x80000, gamma=G, beta=BT, o=Q) == _lib.KA_ERR_ALIAS
    for name in ("q1", "k1", "q2", "k2", "v", "o", "lam"):
        assert diff_ex(lib, **{name: 0}) == _lib.KA_ERR_NULL, name
    assert diff_ex(lib, rot=48) == _lib.KA_ERR_PARAM
    assert diff_ex(lib, rot=0) == _lib.KA_ERR_PARAM
    assert diff_ex(lib, eps=0.0) == _lib.KA_ERR_PARAM
    assert diff_ex(lib, eps=float("nan")) == _lib.KA_ERR_PARAM
    assert diff_ex(lib, Sk=9) == _lib.KA_ERR_SHAPE
    assert diff_ex(lib, D=128) == _lib.KA_ERR_UNSUPPORTED
    assert diff_ex(lib, o=KEEP) == _lib.KA_ERR_ALIAS  # o over the V flags
    # the full path's workspace, with or without V flags
    need3 = lib.ka_diffattn_workspace_bytes(1, 2, 8, 64, -1)
    assert diff_ex(lib, window=-1, ws=W, ws_bytes=need3 - 1) == _lib.KA_ERR_WORKSPACE
    assert diff_ex(lib, window=-1, ws=KEEP - need3 + 16, ws_bytes=need3) == _lib.KA_ERR_ALIAS
    assert lib.ka_last_hip_error() == 0


def _views(**over):
    """Six ka_layout views (q1, k1, q2, k2, v, o) for B=1, H=2, S=8, contiguous unless overridden."""
    base = (2 * 8 * 64, 8 * 64, 64)
    arr = (_lib.KaLayout * 6)(*[_lib.KaLayout(*over.get(n, base)) for n in ("q1", "k1", "q2", "k2", "v", "o")])
    return ctypes.cast(arr, ctypes.c_void_p), arr


def test_diff_ex_layout_validation(lib):
    # a fused projection [B][S][5][H][64]: token stride 5*H*64, head stride 64; merged output [B][S][H][64]
    fused = (8 * 5 * 2 * 64, 64, 5 * 2 * 64)
    ok = dict(q1=fused, k1=fused, q2=fused, k2=fused, v=fused, o=(8 * 2 * 64, 64, 2 * 64))
    p, keep_alive = _views(**ok)
    assert diff_ex(lib, layouts=p, o=Q) == _lib.KA_ERR_ALIAS  # o inside q1's extent
    for bad in ((0, 0, 32), (512, 64, 60), (512, 4, 64), (-8, 64, 64)):
        p, keep_alive = _views(**dict(ok, k2=bad))
        assert diff_ex(lib, layouts=p) == _lib.KA_ERR_SHAPE, bad
    p, keep_alive = _views(**dict(ok, o=(1024, 0, 64)))  # the two heads of o on the same rows
    assert diff_ex(lib, layouts=p) == _lib.KA_ERR_SHAPE
    p, keep_alive = _views(**dict(ok, v=(1024, 512, 1 << 28)))  # one slice past 32-bit offsets
    assert diff_ex(lib, layouts=p) == _lib.KA_ERR_SHAPE
    del keep_alive
    assert lib.ka_last_hip_error() == 0


def test_workspace_sizes(lib):
    # banded windows the one-pass kernel takes need no workspace
    assert lib.ka_diffattn_workspace_bytes(1, 8, 23086, 64, 17) == 0
    assert lib.ka_diffattn_workspace_bytes(1, 8, 23086, 64, 40) == 0
    # wide windows and the full window prepare keys once into the workspace
    assert lib.ka_diffattn_workspace_bytes(1, 16, 1422, 64, -1) == 3 * 16 * 1422 * 64 * 2
    assert lib.ka_diffattn_workspace_bytes(1, 8, 100, 64, 41) == 3 * 8 * 100 * 64 * 2
    assert lib.ka_diffattn_workspace_bytes(1, 8, 30, 64, 29) == 3 * 8 * 30 * 64 * 2  # window >= S-1: full
    assert lib.ka_diffattn_workspace_bytes(0, 8, 100, 64, -1) == 0
    assert lib.ka_diffattn_workspace_bytes(1, 8, 100, 32, -1) == 0


def test_binding_refuses_cpu_tensors(lib):
    import torch
    x = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):
        ka.ka_attn_fwd(x, x, x, o=torch.zeros_like(x))


def test_grid_limit_is_a_shape_error(lib):
    # B*H*ceil(Sq/64) must stay below 2^23 (one-dimensional grids, 32-bit work-item counts)
    assert dense(lib, "ka_attn_fwd", H=1 << 23, Sq=1, Sk=1) == _lib.KA_ERR_SHAPE
    assert dense(lib, "ka_attn_fwd", H=1 << 22, Sq=65, Sk=1) == _lib.KA_ERR_SHAPE
    assert dense(lib, "ka_attn_fwd", H=(1 << 23) - 1, Sq=64, Sk=1, o=Q) == _lib.KA_ERR_ALIAS  # accepted shape
    assert dense(lib, "ka_xattn_fwd", B=2, H=1 << 22, Sq=1, Sk=77) == _lib.KA_ERR_SHAPE
    assert diff(lib, B=1, H=1 << 23, Sq=1, Sk=1) == _lib.KA_ERR_SHAPE
    assert diff_ex(lib, B=1, H=1 << 22, Sq=100, Sk=100) == _lib.KA_ERR_SHAPE
    assert lib.ka_last_hip_error() == 0


def test_parameter_arrays_may_not_overlap_outputs(lib):
    # o over alpha, gamma, beta or lambda (DyT); over rms_weight (RMSNorm)
    assert diff(lib, o=0x7000000, alpha=0x7000000 + 64) == _lib.KA_ERR_ALIAS
    assert diff(lib, gamma=O + 512) == _lib.KA_ERR_ALIAS
    assert diff(lib, beta=O + 16) == _lib.KA_ERR_ALIAS
    assert diff(lib, lam=O + 1024) == _lib.KA_ERR_ALIAS
    assert diff_ex(lib, rms_w=O + 32) == _lib.KA_ERR_ALIAS
    # ... and the workspace over any of them (the full path)
    need = lib.ka_diffattn_workspace_bytes(1, 2, 8, 64, -1)
    assert diff(lib, window=-1, ws=G - 64, ws_bytes=need) == _lib.KA_ERR_ALIAS
    assert diff(lib, window=-1, ws=L - need + 16, ws_bytes=need) == _lib.KA_ERR_ALIAS
    assert diff_ex(lib, window=-1, ws=G - 16, ws_bytes=need) == _lib.KA_ERR_ALIAS
    assert lib.ka_last_hip_error() == 0


def test_kernel_name_introspection(lib):
    # no GPU here: the launch plan assumes 256 CUs, MI355X's count
    name = lambda *a: lib.ka_attn_kernel_name(*a)  # noqa: E731
    assert name(ka.KA_BF16, 2, 10, 4096, 4096, 64).startswith(b"attn_bf16_quad")
    assert name(ka.KA_BF16, 1, 1, 100, 100, 64) == b"attn_bf16_pipe"
    assert name(ka.KA_BF16, 1, 256, 370, 333, 64) == b"attn_bf16_duo 3+3"
    assert name(ka.KA_F32, 1, 2, 256, 256, 64) == b"attn_f32"
    assert name(ka.KA_BF16, 1, 1, 16384, 16384, 512) == b"attn512_pair"
    assert name(ka.KA_F32, 1, 1, 16, 16, 512) is None
    assert name(ka.KA_BF16, 0, 1, 16, 16, 64) is None
    assert name(ka.KA_BF16, 1, 1 << 23, 1, 1, 64) is None


def _cpu(*shape, dtype=None):
    import torch
    return torch.zeros(*shape, dtype=dtype or torch.bfloat16)


def test_binding_checks_shapes_dtypes_before_any_call(lib):
    import torch
    q, k, v = _cpu(1, 2, 8, 64), _cpu(1, 2, 5, 64), _cpu(1, 2, 5, 64)
    bad = [dict(k=_cpu(1, 1, 5, 64)), dict(v=_cpu(1, 2, 6, 64)), dict(k=_cpu(1, 2, 5, 64, dtype=torch.float32)),
           dict(o=_cpu(1, 2, 7, 64)), dict(o=_cpu(1, 2, 8, 64, dtype=torch.float32)), dict(q=_cpu(2, 8, 64))]
    for fn in (ka.ka_attn_fwd, ka.ka_xattn_fwd):
        for over in bad:
            args = dict(q=q, k=k, v=v, o=None)
            args.update(over)
            with pytest.raises(ValueError):
                fn(args["q"], args["k"], args["v"], o=args["o"])
    with pytest.raises(TypeError):  # dtype the library does not take
        ka.ka_attn_fwd(_cpu(1, 1, 4, 64, dtype=torch.float16), _cpu(1, 1, 4, 64, dtype=torch.float16),
                       _cpu(1, 1, 4, 64, dtype=torch.float16))


def test_binding_checks_differential_arguments(lib):
    import torch
    f32 = torch.float32
    x = [_cpu(2, 3, 10, 64) for _ in range(5)]
    a, g, b, lm = _cpu(4, dtype=f32), _cpu(4, 64, dtype=f32), _cpu(4, 64, dtype=f32), _cpu(3, dtype=f32)
    good = dict(alpha=a, gamma=g, beta=b)
    cases = [(dict(x=[x[0], _cpu(2, 3, 9, 64)] + x[2:]), good, lm),   # k1 rows
             (dict(x=x[:4] + [_cpu(2, 2, 10, 64)]), good, lm),         # v heads
             (dict(x=x), dict(good, gamma=_cpu(4, 32, dtype=f32)), lm),
             (dict(x=x), dict(good, alpha=_cpu(4)), lm),               # bf16 alpha
             (dict(x=x), good, _cpu(2, dtype=f32))]                    # lambda per head
    for c, prm, lam in cases:
        with pytest.raises(ValueError):
            ka.ka_diffattn_fwd(*c["x"], prm["alpha"], prm["gamma"], prm["beta"], lam)
    with pytest.raises(ValueError):  # o of the wrong shape
        ka.ka_diffattn_fwd(*x, a, g, b, lm, o=_cpu(2, 3, 10, 32))
    with pytest.raises(ValueError):  # V flags [B, S] uint8
        ka.ka_diffattn_fwd_ex(*x, lm, qk_norm="rms", rms_weight=g, v_keep=_cpu(2, 11, dtype=torch.uint8))
    with pytest.raises(ValueError):
        ka.ka_diffattn_fwd_ex(*x, lm, qk_norm="rms", rms_weight=g, v_keep=_cpu(2, 10, dtype=torch.int32))
    with pytest.raises(ValueError):  # RMSNorm needs its weights
        ka.ka_diffattn_fwd_ex(*x, lm, qk_norm="rms")
    with pytest.raises(ValueError):
        ka.ka_diffattn_fwd_ex(*x, lm, qk_norm="layer")
    with pytest.raises(ValueError):  # a workspace must be bytes
        ka.ka_diffattn_fwd(*x, a, g, b, lm, workspace=_cpu(100, dtype=f32))
    # well-formed CPU tensors pass every shape check and stop at the device check
    with pytest.raises(ValueError, match="GPU"):
        ka.ka_diffattn_fwd(*x, a, g, b, lm, window=17)


def diff_na(lib, dt=ka.KA_BF16, q1=Q, k1=K, q2=V, k2=O2, v=A, o=O, B=1, H=2, Sq=8, Sk=8, D=64, scale=0.125,
            window=-1, norm=ka.KA_QKNORM_RMS, alpha=0, gamma=0, beta=0, rms_w=G, eps=1e-6, rot=32, base=10000.0,
            lam=L, keep=KEEP, layouts=None):
    return lib.ka_diffattn_fwd_noalloc(dt, q1, k1, q2, k2, v, o, B, H, Sq, Sk, D, ctypes.c_float(scale), window,
                                       norm, alpha, gamma, beta, rms_w, ctypes.c_float(eps), rot,
                                       ctypes.c_float(base), lam, keep, layouts, None)


def test_noalloc_validation(lib):
    # the same argument checks as ka_diffattn_fwd_ex, all before any HIP call
    assert diff_na(lib, norm=7) == _lib.KA_ERR_UNSUPPORTED
    assert diff_na(lib, rms_w=0) == _lib.KA_ERR_NULL
    assert diff_na(lib, q2=0) == _lib.KA_ERR_NULL
    assert diff_na(lib, Sk=9) == _lib.KA_ERR_SHAPE
    assert diff_na(lib, rot=48) == _lib.KA_ERR_PARAM
    assert diff_na(lib, o=Q) == _lib.KA_ERR_ALIAS
    assert diff_na(lib, v=A + 4) == _lib.KA_ERR_ALIGN
    # a shape whose full-path scratch exceeds the static array is refused before any HIP call
    rows = _lib.KA_STATIC_WORKSPACE_BYTES // (3 * 64 * 2) + 1
    big = dict(q1=0x10000000, k1=0x20000000, q2=0x30000000, k2=0x40000000, v=0x50000000, o=0x60000000,
               keep=0x70000000)
    assert diff_na(lib, B=1, H=1, Sq=rows, Sk=rows, **big) == _lib.KA_ERR_WORKSPACE
    assert lib.ka_last_hip_error() == 0

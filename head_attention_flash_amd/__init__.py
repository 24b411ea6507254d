"""Fused head-dim-64 attention for AMD MI355X (gfx950).

The compute lives in libka_attn.so (hand-written HIP kernels behind a C ABI,
include/ka_attn.h); this package is its ctypes binding.  Importing it does not
load the library; the first call does, and raises if it has not been built.
"""
from ._lib import (KA_BF16, KA_F32, KA_QKNORM_DYT, KA_QKNORM_RMS, KA_XATTN_MAX_SK, KaError,  # noqa: F401
                   ka_attn_fwd, ka_attn_kernel_name, ka_diffattn_fwd, ka_diffattn_fwd_ex, ka_diffattn_fwd_noalloc,
                   ka_diffattn_workspace_bytes, ka_xattn_fwd, load)

__all__ = ["ka_attn_fwd", "ka_attn_kernel_name", "ka_xattn_fwd", "ka_diffattn_fwd", "ka_diffattn_fwd_ex",
           "ka_diffattn_fwd_noalloc", "ka_diffattn_workspace_bytes", "load", "KaError", "KA_F32", "KA_BF16", "KA_QKNORM_DYT", "KA_QKNORM_RMS", "KA_XATTN_MAX_SK"]

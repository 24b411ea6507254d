"""The allocation-free differential entry point (the library's per-GPU scratch array in place of a
caller workspace), through the C ABI, against the entry point that takes a workspace: the same
kernels, so the same bits; and against the fp64 oracle.  Two calls in a row, the second smaller."""
import numpy as np
import pytest
import torch

import head_attention_flash_amd as ka
import oracle
from gpu_util import BF16_TOL, assert_close, nan_like, to_dev, to_host_bits, to_host_f64
from head_attention_flash_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ka.load()


def _case(B, H, S, seed, norm):
    wl = synth.WORKLOADS["sa3_dit_fulldiff_h16s1422"]
    inputs, params = synth.make_diff(wl, seed_base=seed, S=S, H=H, B=B)
    if norm == "rms":
        w, lm = synth.make_model_params(H, seed + 6)
        return inputs, dict(qk_norm="rms", rms_weight=w, rms_eps=1e-6), lm
    a, g, b, lm = synth.make_diff_params_varied(H, seed + 7)
    return inputs, dict(qk_norm="dyt", alpha=a, gamma=g, beta=b), lm


def _both(inputs, prm, lm, window, rot, keep):
    ins = [to_dev(x) for x in inputs]
    dprm = {k: (to_dev(v) if isinstance(v, np.ndarray) else v) for k, v in prm.items()}
    kw = dict(window=window, rotary_dims=rot, **dprm)
    if keep is not None:
        kw["v_keep"] = to_dev(keep)
    o_ws, o_na = nan_like(ins[0]), nan_like(ins[0])
    ka.ka_diffattn_fwd_ex(*ins, to_dev(lm), o=o_ws, **kw)
    ka.ka_diffattn_fwd_noalloc(*ins, to_dev(lm), o=o_na, **kw)
    torch.cuda.synchronize()
    return o_ws, o_na


@pytest.mark.parametrize("norm", ["dyt", "rms"])
def test_noalloc_matches_workspace_entry_point(norm):
    # the DiT shape (16 heads x 1422 tokens), then a smaller one on the same scratch array
    for (B, H, S), window, rot, pad in (((1, 16, 1422), -1, 64, 0), ((2, 3, 500), -1, 32, 37),
                                        ((1, 2, 300), 100, 64, 0), ((2, 3, 400), 17, 32, 11)):
        inputs, prm, lm = _case(B, H, S, 3000 + S + H, norm)
        keep = synth.make_v_keep(B, S, pad) if pad else None
        o_ws, o_na = _both(inputs, prm, lm, window, rot, keep)
        assert torch.equal(o_ws.view(torch.int16), o_na.view(torch.int16)), f"{B}x{H}x{S} w={window}"
        if norm == "rms":
            want = oracle.diffattn(*inputs, 0.125, window, None, None, None, 10000.0, lm, norm="rms",
                                   rms_weight=prm["rms_weight"], rms_eps=1e-6, rotary_dims=rot, v_keep=keep)
        else:
            want = oracle.diffattn(*inputs, 0.125, window, prm["alpha"], prm["gamma"], prm["beta"], 10000.0, lm,
                                   rotary_dims=rot, v_keep=keep)
        assert_close(to_host_f64(o_na), want, BF16_TOL, f"noalloc {norm} {B}x{H}x{S} w={window}",
                     got_bits=to_host_bits(o_na))


def test_noalloc_refuses_shapes_past_its_scratch():
    lib = ka.load()
    # with V flags the full path needs three planes of B*H*S rows; one row more than the array holds
    rows = ka._lib.KA_STATIC_WORKSPACE_BYTES // (3 * 64 * 2) + 1
    assert ka.ka_diffattn_workspace_bytes(1, 1, rows) > ka._lib.KA_STATIC_WORKSPACE_BYTES
    x = torch.empty(1, 1, rows, 64, dtype=torch.bfloat16, device="cuda")
    lm = torch.ones(1, dtype=torch.float32, device="cuda")
    w = torch.ones(4, 64, dtype=torch.float32, device="cuda")
    keep = torch.ones(1, rows, dtype=torch.uint8, device="cuda")
    with pytest.raises(ka.KaError) as e:
        ka.ka_diffattn_fwd_noalloc(x, x, x, x, x, lm, o=torch.empty_like(x), qk_norm="rms", rms_weight=w,
                                   v_keep=keep)
    assert e.value.status == ka._lib.KA_ERR_WORKSPACE
    assert lib.ka_last_hip_error() == 0

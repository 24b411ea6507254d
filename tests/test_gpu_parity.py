"""GPU parity: every form of the library, through the C ABI, against the fp64 oracle.

Every case, the full-size workloads the bench times included (in the same launch
configuration), is compared element by element on every output.  Tolerances: max
abs error 2e-2 for bf16 in/out (fp32 accumulation) and 1e-4 for fp32.  The full-size
cases also report p99, p50, relative RMS and the distance in bf16 steps from the
oracle rounded once to bf16 (lines starting "PARITY").
"""
import json
import os

import numpy as np
import pytest
import torch

import head_attention_flash_amd as ka
import oracle
from gpu_util import (BF16_TOL, F32_TOL, assert_close, bf16_ulp_distance, diff_params_dev, nan_like, to_dev,
                      to_host_bits, to_host_f64)

to_f64 = oracle.widen
from head_attention_flash_amd import synth

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
D = 64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ka.load()


def _parity(got, want, bits, what, tol=BF16_TOL):
    """Whole-output comparison with the full report, printed as one PARITY line (and appended to the
    file KA_PARITY_LOG names, if set)."""
    r = assert_close(got, want, tol, what, got_bits=bits)
    line = "PARITY " + json.dumps({"case": what, **r})
    print(line, flush=True)
    if os.environ.get("KA_PARITY_LOG"):
        with open(os.environ["KA_PARITY_LOG"], "a") as f:
            f.write(line + "\n")
    return r


# ------------------------------------------------------------------ dense

def _run_dense(fn, q, k, v, scale=0.125, bits=False):
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o = nan_like(qd)  # every output element must be written exactly once
    fn(qd, kd, vd, o=o, scale=scale)
    torch.cuda.synchronize()
    return (to_host_f64(o), to_host_bits(o)) if bits else to_host_f64(o)


def test_dense_f32_workload():
    wl = W["dense_f32_b1h2s256"]
    q, k, v = synth.make_dense(wl)
    got = _run_dense(ka.ka_attn_fwd, q, k, v, wl.scale)
    assert_close(got, oracle.attn(q, k, v, wl.scale), F32_TOL, wl.key)


@pytest.mark.parametrize("B,H,Sq,Sk", [(1, 1, 1, 1), (1, 3, 77, 130), (2, 1, 129, 33), (1, 1, 300, 1000)])
def test_dense_f32_ragged(B, H, Sq, Sk):
    wl = W["dense_f32_b1h2s256"]
    q, k, v = synth.make_dense(wl, seed_base=Sq * 7 + Sk, B=B, H=H, Sq=Sq, Sk=Sk)
    got = _run_dense(ka.ka_attn_fwd, q, k, v)
    assert_close(got, oracle.attn(q, k, v, 0.125), F32_TOL, f"f32 {B}x{H}x{Sq}x{Sk}")


@pytest.mark.parametrize("B,H,Sq,Sk", [(1, 2, 200, 333), (1, 1, 1, 1), (1, 1, 16, 64), (1, 1, 65, 65),
                                       (2, 3, 129, 257), (1, 1, 64, 4096), (1, 2, 1000, 1000)])
def test_dense_bf16_shapes(B, H, Sq, Sk):
    wl = W["sdxl_l1_self_b2h10s4096"]
    q, k, v = synth.make_dense(wl, seed_base=100 + Sq + Sk, B=B, H=H, Sq=Sq, Sk=Sk)
    got = _run_dense(ka.ka_attn_fwd, q, k, v)
    assert_close(got, oracle.attn(q, k, v, 0.125), BF16_TOL, f"bf16 {B}x{H}x{Sq}x{Sk}")


@pytest.mark.parametrize("Sq,Sk", [(370, 333), (300, 97), (250, 301), (16, 33)])
def test_dense_bf16_eight_wave_blocks(Sq, Sk):
    """256 (b, h) slices fill a 256-CU chip with 8-wave blocks; the query counts then select the
    3+3 (370), 3+2 (300) and 2+2 (250, 16) block layouts, each with a ragged last query block and a
    ragged last key tile (16 queries: most waves of the block own no valid query)."""
    wl = W["sdxl_l1_self_b2h10s4096"]
    q, k, v = synth.make_dense(wl, seed_base=300 + Sq + Sk, B=1, H=256, Sq=Sq, Sk=Sk)
    got = _run_dense(ka.ka_attn_fwd, q, k, v)
    assert_close(got, oracle.attn(q, k, v, 0.125), BF16_TOL, f"bf16 1x256x{Sq}x{Sk}")


@pytest.mark.parametrize("B,H,Sq,Sk", [(1, 13, 4900, 333), (2, 10, 4000, 1000), (2, 12, 3900, 77), (2, 10, 4000, 20)])
def test_dense_bf16_four_wave_blocks(B, H, Sq, Sk):
    """Grids whose 8-wave layouts leave CUs idle go to 4-wave blocks, two per CU, with the heads split
    into 2- and 3-unit items (a unit: 64 queries).  On a 256-CU chip these shapes select the 2+2
    (4900), 3+2 (4000) and 3+3 (3900) unit plans, with ragged last items and key tiles, idle blocks
    (fewer items than CUs in a round) and a single key tile (Sk = 20)."""
    wl = W["sdxl_l1_self_b2h10s4096"]
    q, k, v = synth.make_dense(wl, seed_base=500 + H + Sq + Sk, B=B, H=H, Sq=Sq, Sk=Sk)
    got = _run_dense(ka.ka_attn_fwd, q, k, v)
    assert_close(got, oracle.attn(q, k, v, 0.125), BF16_TOL, f"bf16 {B}x{H}x{Sq}x{Sk}")


def test_dense_bf16_peaked():
    """q scaled by 8: a peaked softmax, where a dropped or duplicated key tile is visible."""
    B, H, Sq, Sk = 1, 2, 256, 700
    r = np.random.default_rng(5)
    q = synth.f32_to_bf16_bits((8 * r.standard_normal((B, H, Sq, D))).astype(np.float32))
    k = synth.f32_to_bf16_bits(r.standard_normal((B, H, Sk, D)).astype(np.float32))
    v = synth.f32_to_bf16_bits(r.standard_normal((B, H, Sk, D)).astype(np.float32))
    got = _run_dense(ka.ka_attn_fwd, q, k, v)
    assert_close(got, oracle.attn(q, k, v, 0.125), BF16_TOL, "bf16 peaked")


def test_dense_bf16_workload_full():
    """SDXL level-1 self-attention (B=2, H=10, S=4096), the bench's launch, every output element."""
    wl = W["sdxl_l1_self_b2h10s4096"]
    q, k, v = synth.make_dense(wl)
    got, bits = _run_dense(ka.ka_attn_fwd, q, k, v, wl.scale, bits=True)
    r = _parity(got, oracle.attn(q, k, v, wl.scale), bits, wl.key)
    assert r["rel_rms"] < 1e-2


@pytest.mark.parametrize("B,H,Sq,Sk,qscale", [(1, 20, 4096, 128, 1), (1, 20, 4096, 256, 8), (4, 5, 4096, 384, 1),
                                             (1, 10, 8192, 640, 8), (2, 10, 4096, 4096, 8)])
def test_dense_bf16_peaked_large(B, H, Sq, Sk, qscale):
    """Peaked softmaxes (q scaled by 8: logits with a standard deviation of 8), every output element:
    the score scale has to be applied in fp32 (bf16(scale log2(e) q) moved scores by up to 2^-9 of
    sum |c q_d k_d| and failed the 2e-2 gate here).  Sk = 128, 256, 384 give one, two and three key
    tiles per 128 keys; the grids select the 4-wave unit plans."""
    wl = W["sdxl_l1_self_b2h10s4096"]
    r = np.random.default_rng(900 + Sk + qscale)
    q = synth.f32_to_bf16_bits((qscale * r.standard_normal((B, H, Sq, D))).astype(np.float32))
    k = synth.f32_to_bf16_bits(r.standard_normal((B, H, Sk, D)).astype(np.float32))
    v = synth.f32_to_bf16_bits(r.standard_normal((B, H, Sk, D)).astype(np.float32))
    got, bits = _run_dense(ka.ka_attn_fwd, q, k, v, wl.scale, bits=True)
    _parity(got, oracle.attn(q, k, v, wl.scale), bits, f"bf16 peaked x{qscale} {B}x{H}x{Sq}x{Sk}")


@pytest.mark.parametrize("B,H,Sq,Sk,Dh,step", [(1, 2, 256, 1024, 64, 9.0), (1, 2, 256, 1024, 64, -9.0),
                                              (2, 10, 4096, 512, 64, 9.0), (1, 1, 200, 512, 512, 9.0)])
def test_dense_score_ramp(B, H, Sq, Sk, Dh, step):
    """Scores that rise by `step` (in the exp2 domain) from each 32-key tile to the next: every tile's
    maximum passes the running one by more than the lazy threshold (8), so the kernels raise their
    reference and rescale O and l on every tile; a falling ramp raises only on the first.  Keys are
    a per-tile multiple of q plus noise; every output element against the oracle."""
    scale = Dh ** -0.5
    c = scale * np.log2(np.e)
    r = np.random.default_rng(4100 + Sk + Dh + int(step))
    tile = np.arange(Sk) // 32
    a = step * (tile - (tile.max() if step < 0 else 0)) / (c * Dh)  # c q.k = step * tile (+ const)
    qf = np.ones((B, H, Sq, Dh), np.float32) + 0.05 * r.standard_normal((B, H, Sq, Dh)).astype(np.float32)
    kf = a[None, None, :, None] + 0.05 * r.standard_normal((B, H, Sk, Dh))
    q = synth.f32_to_bf16_bits(qf)
    k = synth.f32_to_bf16_bits(kf.astype(np.float32))
    v = synth.f32_to_bf16_bits(r.standard_normal((B, H, Sk, Dh)).astype(np.float32))
    got = _run_dense(ka.ka_attn_fwd, q, k, v, scale)
    assert_close(got, oracle.attn(q, k, v, scale), BF16_TOL, f"ramp {step:+} {B}x{H}x{Sq}x{Sk} d{Dh}")


@pytest.mark.parametrize("Sq", [370, 2000])
def test_dense_layouts_agree(Sq):
    """Tile independence: one (b, h) slice copied into batches whose size selects each dense layout
    (the 4-wave unit plans, the 8-wave 3+3 / 3+2 / 2+2 blocks, the small-grid kernel).  The 4- and
    8-wave layouts run the same per-query arithmetic on the same 32-key tiles, and a query raises its
    running maximum from its own scores only, so they agree bit for bit, on every copy; the small-
    grid kernel (64-key tiles, its own maximum) agrees within a bf16 step or two.  q is scaled by 4
    so that maxima rise inside the loop."""
    Sk = 333
    q1, k1, v1 = _peaked((1, 1, Sq, D), (1, 1, Sk, D), 4, 2600 + Sq)
    plans = {}
    for H in range(1, 700):
        plans.setdefault(ka.ka_attn_kernel_name(1, H, Sq, Sk), H)
    print(f"Sq={Sq}: layouts {plans}", flush=True)
    assert "attn_bf16_pipe" in plans and sum(n.startswith("attn_bf16_quad") for n in plans) >= 2
    want = oracle.attn(q1, k1, v1, 0.125)
    outs = {}
    for name, H in plans.items():
        rep = lambda x: np.ascontiguousarray(np.broadcast_to(x, (1, H) + x.shape[2:]))  # noqa: E731
        got, bits = _run_dense(ka.ka_attn_fwd, rep(q1), rep(k1), rep(v1), bits=True)
        assert_close(got[:, :1], want, BF16_TOL, f"{name} (H={H})")
        same = (bits == bits[:, :1]).all()
        assert same, f"{name}: copies of one slice differ within a launch"
        outs[name] = bits[0, 0]
    ref = outs["attn_bf16_pipe"]
    tiled = [n for n in outs if n != "attn_bf16_pipe"]
    for n in tiled:
        assert np.array_equal(outs[n], outs[tiled[0]]), f"{n} differs from {tiled[0]}"
    a, b = (to_f64(x) for x in (outs[tiled[0]], ref))
    big = np.maximum(np.abs(a), np.abs(b)) >= 1.0 / 16
    u = bf16_ulp_distance(outs[tiled[0]][big], ref[big])
    dmax = float(np.abs(a - b).max())
    print(f"Sq={Sq}: tiled layouts bit-identical; small-grid kernel: {float(np.mean(a == b)):.4f} identical, "
          f"max abs difference {dmax:.2e}, max {int(u.max())} bf16 steps where |o| >= 1/16", flush=True)
    assert dmax <= BF16_TOL


@pytest.mark.parametrize("shape", [(1, 3, 1000, 900), None])
def test_dense_bf16_deterministic(shape):
    """Repeated calls give the same bits (no atomics, no order-dependent reductions), also at the
    workload's size, where two blocks share each CU."""
    wl = W["sdxl_l1_self_b2h10s4096"]
    kw = {} if shape is None else dict(zip(("B", "H", "Sq", "Sk"), shape))
    q, k, v = (to_dev(x) for x in synth.make_dense(wl, **kw))
    a = ka.ka_attn_fwd(q, k, v)
    b = ka.ka_attn_fwd(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ------------------------------------------------------------------ cross

def test_xattn_workload_full():
    wl = W["sdxl_l2_cross_b2h20q1024k77"]
    q, k, v = synth.make_dense(wl)
    got, bits = _run_dense(ka.ka_xattn_fwd, q, k, v, wl.scale, bits=True)
    _parity(got, oracle.attn(q, k, v, wl.scale), bits, wl.key)


@pytest.mark.parametrize("Sk", [1, 13, 32, 33, 77, 96, 97, 128, 129, 200, 256])
@pytest.mark.parametrize("Sq", [1, 50])
def test_xattn_key_counts(Sq, Sk):
    wl = W["sdxl_l2_cross_b2h20q1024k77"]
    q, k, v = synth.make_dense(wl, seed_base=300 + Sk, B=1, H=2, Sq=Sq, Sk=Sk)
    got = _run_dense(ka.ka_xattn_fwd, q, k, v)
    assert_close(got, oracle.attn(q, k, v, 0.125), BF16_TOL, f"xattn Sq={Sq} Sk={Sk}")


def test_xattn_f32_routes_to_fp32_kernel():
    wl = W["dense_f32_b1h2s256"]
    q, k, v = synth.make_dense(wl, B=1, H=2, Sq=100, Sk=77)
    got = _run_dense(ka.ka_xattn_fwd, q, k, v)
    assert_close(got, oracle.attn(q, k, v, 0.125), F32_TOL, "xattn f32")


def test_xattn_matches_dense_kernel():
    """Consistency (not parity: both sides are this library): the LDS-resident cross kernel and the
    flash kernel compute the same definition."""
    wl = W["sdxl_l2_cross_b2h20q1024k77"]
    q, k, v = (to_dev(x) for x in synth.make_dense(wl, B=1, H=4))
    a = ka.ka_xattn_fwd(q, k, v).float()
    b = ka.ka_attn_fwd(q, k, v).float()
    torch.cuda.synchronize()
    assert (a - b).abs().max().item() <= 2e-2


# ------------------------------------------------------------------ differential

def _run_diff(inputs, params, window, scale=0.125, base=10000.0, bits=False):
    q1, k1, q2, k2, v = (to_dev(x) for x in inputs)
    a, g, b, lm = diff_params_dev(params)
    o = nan_like(q1)
    ka.ka_diffattn_fwd(q1, k1, q2, k2, v, a, g, b, lm, o=o, scale=scale, window=window, rope_base=base)
    torch.cuda.synchronize()
    return (to_host_f64(o), to_host_bits(o)) if bits else to_host_f64(o)


def _oracle_diff(inputs, params, window, rows=None, scale=0.125, base=10000.0):
    a, g, b, lm = params
    return oracle.diffattn(*inputs, scale, window, a, g, b, base, lm, rows=rows)


@pytest.mark.parametrize("S", [1, 2, 17, 18, 35, 36, 127, 128, 129, 391])
def test_diff_band_lengths(S):
    wl = W["sa3_decoder_banddiff_h8s23086w17"]
    inputs, params = synth.make_diff(wl, seed_base=500 + S, S=S, H=2)
    got = _run_diff(inputs, params, 17)
    assert_close(got, _oracle_diff(inputs, params, 17), BF16_TOL, f"band S={S}")


@pytest.mark.parametrize("window", [17, 30])
def test_diff_band_strips(window):
    """Enough (b, h) slices that each workgroup walks several 64-row blocks through its key ring."""
    wl = W["sa3_decoder_banddiff_h8s23086w17"]
    inputs, params = synth.make_diff(wl, seed_base=800 + window, S=700, H=96, B=2)
    got = _run_diff(inputs, params, window)
    assert_close(got, _oracle_diff(inputs, params, window), BF16_TOL, f"band strips w={window}")


@pytest.mark.parametrize("window", [0, 1, 5, 16, 24, 25, 40, 41, 100, 298, 299, 1000, -1])
def test_diff_windows(window):
    wl = W["sa3_decoder_banddiff_h8s23086w17"]
    S = 300
    inputs, params = synth.make_diff(wl, seed_base=700 + max(window, 0), S=S, H=2, B=2)
    got = _run_diff(inputs, params, window)
    assert_close(got, _oracle_diff(inputs, params, window), BF16_TOL, f"window={window}")


def test_diff_band_workload_full():
    """Banded differential attention at the decoder's size (H=8, S=23086, +-17), every output element."""
    wl = W["sa3_decoder_banddiff_h8s23086w17"]
    inputs, params = synth.make_diff(wl)
    got, bits = _run_diff(inputs, params, wl.window, wl.scale, bits=True)
    _parity(got, _oracle_diff(inputs, params, wl.window, scale=wl.scale), bits, wl.key)


def test_diff_full_workload_full():
    """Full differential attention at the DiT's size (H=16, S=1422), every output element."""
    wl = W["sa3_dit_fulldiff_h16s1422"]
    inputs, params = synth.make_diff(wl)
    got, bits = _run_diff(inputs, params, wl.window, wl.scale, bits=True)
    _parity(got, _oracle_diff(inputs, params, wl.window, scale=wl.scale), bits, wl.key)


@pytest.mark.parametrize("window", [17, 30, 100, -1])
def test_diff_varied_parameters(window):
    """A different alpha per parameter set, beta ~ N(0, 0.3) per set and channel, lambda ~ U[0.2, 0.9]
    per head, B = 2: a dropped beta, a swapped set or a wrong head index for lambda shows here (the
    workload recipe's alpha, beta and lambda are the same everywhere)."""
    wl = W["sa3_decoder_banddiff_h8s23086w17"]
    B, H, S = 2, 5, 700
    inputs, _ = synth.make_diff(wl, seed_base=2300 + max(window, 0), S=S, H=H, B=B)
    params = synth.make_diff_params_varied(H, 2350 + max(window, 0))
    got, bits = _run_diff(inputs, params, window, bits=True)
    _parity(got, _oracle_diff(inputs, params, window), bits, f"varied params w={window}")


@pytest.mark.parametrize("window", [17, -1])
def test_diff_branch_cancellation(window):
    """Identical branches (same inputs, same parameter sets) and lambda = 1 give exactly zero."""
    wl = W["sa3_decoder_banddiff_h8s23086w17"]
    (q1, k1, _, _, v), (a, g, b, lm) = synth.make_diff(wl, seed_base=900, S=200, H=2)
    g[2], g[3], b[2], b[3] = g[0], g[1], b[0], b[1]
    got = _run_diff((q1, k1, q1, k1, v), (a, g, b, np.ones_like(lm)), window)
    assert np.all(got == 0.0)


@pytest.mark.parametrize("window", [17, -1])
def test_diff_constant_v(window):
    wl = W["sa3_decoder_banddiff_h8s23086w17"]
    (q1, k1, q2, k2, _), params = synth.make_diff(wl, seed_base=910, S=150, H=3)
    c = synth.f32_to_bf16_bits(np.linspace(-2, 2, D).astype(np.float32))
    v = np.ascontiguousarray(np.broadcast_to(c, q1.shape))
    got = _run_diff((q1, k1, q2, k2, v), params, window)
    want = (1.0 - params[3].astype(np.float64))[None, :, None, None] * oracle.widen(c)[None, None, None, :]
    assert_close(got, np.broadcast_to(want, got.shape), 1e-2, f"constant V w={window}")


@pytest.mark.parametrize("key,small", [("sa3_decoder_banddiff_h8s23086w17", True),
                                       ("sa3_decoder_banddiff_h8s23086w17", False),
                                       ("sa3_dit_fulldiff_h16s1422", False)])
def test_diff_deterministic(key, small):
    """Repeated calls give the same bits, also at the workloads' sizes, where several workgroups
    share each CU (and set their wave priorities by the work they have left)."""
    wl = W[key]
    inputs, params = synth.make_diff(wl, seed_base=920, **(dict(S=1000, H=2) if small else {}))
    a = _run_diff(inputs, params, wl.window, bits=True)[1]
    b = _run_diff(inputs, params, wl.window, bits=True)[1]
    assert np.array_equal(a, b)


# ------------------------------------------------------------------ graph capture

def test_graph_capture_replays_match_eager():
    """All three entry points captured into one HIP graph; every replay, with eager work and
    synchronisation in between, reproduces the eager results bit for bit."""
    wl = W["sdxl_l1_self_b2h10s4096"]
    q, k, v = (to_dev(x) for x in synth.make_dense(wl, B=1, H=2, Sq=500, Sk=700))
    xl = W["sdxl_l2_cross_b2h20q1024k77"]
    xq, xk, xv = (to_dev(x) for x in synth.make_dense(xl, B=1, H=3, Sq=300))
    dl = W["sa3_decoder_banddiff_h8s23086w17"]
    ins, prm = synth.make_diff(dl, S=400, H=2)
    ins = [to_dev(x) for x in ins]
    prm = [to_dev(x) for x in prm]
    ws = torch.empty(ka.ka_diffattn_workspace_bytes(1, 2, 400, 64, -1), dtype=torch.uint8, device="cuda")
    outs = [torch.empty_like(q), torch.empty_like(xq), torch.empty_like(ins[0]), torch.empty_like(ins[0])]

    def work():
        ka.ka_attn_fwd(q, k, v, o=outs[0])
        ka.ka_xattn_fwd(xq, xk, xv, o=outs[1])
        ka.ka_diffattn_fwd(*ins, *prm, o=outs[2], window=17)
        ka.ka_diffattn_fwd(*ins, *prm, o=outs[3], window=-1, workspace=ws)

    work()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            work()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.zero_()
        junk = (torch.randn(1 << 20, device="cuda") * 2).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        del junk
        for a, b in zip(outs, eager):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {rep} differs"


# ------------------------------------------------------------------ differential, model forms

def _run_diff_ex(inputs, params, window, norm, rot, keep, scale=0.125, base=10000.0, eps=1e-6, bits=False):
    q1, k1, q2, k2, v = (to_dev(x) for x in inputs)
    o = nan_like(q1)
    kw = dict(o=o, scale=scale, window=window, qk_norm=norm, rotary_dims=rot, rope_base=base)
    if norm == "rms":
        w, lm = params
        kw.update(rms_weight=to_dev(w), rms_eps=eps)
    else:
        a, g, b, lm = params
        kw.update(alpha=to_dev(a), gamma=to_dev(g), beta=to_dev(b))
    if keep is not None:
        kw["v_keep"] = to_dev(keep)
    ka.ka_diffattn_fwd_ex(q1, k1, q2, k2, v, to_dev(lm), **kw)
    torch.cuda.synchronize()
    return (to_host_f64(o), to_host_bits(o)) if bits else to_host_f64(o)


def _oracle_diff_ex(inputs, params, window, norm, rot, keep, rows=None, scale=0.125, base=10000.0, eps=1e-6):
    if norm == "rms":
        w, lm = params
        return oracle.diffattn(*inputs, scale, window, None, None, None, base, lm, rows=rows, norm="rms",
                               rms_weight=w, rms_eps=eps, rotary_dims=rot, v_keep=keep)
    a, g, b, lm = params
    return oracle.diffattn(*inputs, scale, window, a, g, b, base, lm, rows=rows, rotary_dims=rot, v_keep=keep)


def _model_case(norm, S, H, B, seed):
    wl = W["sa3_dit_fulldiff_h16s1422"]
    inputs, params = synth.make_diff(wl, seed_base=seed, S=S, H=H, B=B)
    if norm == "rms":
        params = synth.make_model_params(H, seed + 6)
    return inputs, params


@pytest.mark.parametrize("norm", ["dyt", "rms"])
@pytest.mark.parametrize("rot", [64, 32])
@pytest.mark.parametrize("padded", [False, True])
@pytest.mark.parametrize("window", [17, 100, -1])
def test_diff_model_forms(norm, rot, padded, window):
    """Every combination of normaliser, rotary width and V flags on the banded, wide-window and full paths."""
    S, H, B = 300, 2, 2
    inputs, params = _model_case(norm, S, H, B, 1200 + 10 * rot + (5 if padded else 0) + max(window, 0))
    keep = synth.make_v_keep(B, S, 37) if padded else None
    got = _run_diff_ex(inputs, params, window, norm, rot, keep)
    want = _oracle_diff_ex(inputs, params, window, norm, rot, keep)
    assert_close(got, want, BF16_TOL, f"model form norm={norm} rot={rot} padded={padded} w={window}")


@pytest.mark.parametrize("window", [-1, 200])
@pytest.mark.parametrize("step", [16.4, -16.4])
def test_diff_score_ramp(window, step):
    """Branch-1 scores that rise by `step` (in the exp2 domain) from each 32-key tile to the next,
    past the full path's lazy threshold (15), so its weights are rescaled on every tile (a falling
    ramp: only on the first).  Built without the rotation's mixing: rotary on dims 0-31 only, the
    signal in the unrotated dims 32-63; DyT with beta = 0 and gamma = 4 saturates the queries to +4
    and maps each key tile to one level of 4 tanh(k).  Every output element against the oracle."""
    S, H, B = 384, 2, 1
    c = 0.125 * np.log2(np.e)
    r = np.random.default_rng(5100 + int(step) + max(window, 0))
    tile = np.arange(S) // 32
    ntile = tile.max()
    lev = (-0.975 + 1.95 * tile / ntile) if step > 0 else (0.975 - 1.95 * tile / ntile)
    assert abs(c * 32 * 16 * 1.95 / ntile - abs(step)) < 0.05  # c q^.k^ moves by `step` per tile
    q1 = np.zeros((B, H, S, D), np.float32)
    q1[..., 32:] = 10.0
    k1 = np.zeros((B, H, S, D), np.float32)
    k1[..., 32:] = np.arctanh(lev)[None, None, :, None] + 0.01 * r.standard_normal((B, H, S, 32))
    q2, k2, v = (r.standard_normal((B, H, S, D)).astype(np.float32) for _ in range(3))
    inputs = tuple(synth.f32_to_bf16_bits(x.astype(np.float32)) for x in (q1, k1, q2, k2, v))
    alpha = np.array([1.0, 1.0, 0.5, 0.5], np.float32)
    gamma = np.ones((4, D), np.float32)
    gamma[:2] = 4.0
    beta = np.zeros((4, D), np.float32)
    lam = np.full(H, 0.8, np.float32)
    params = (alpha, gamma, beta, lam)
    got = _run_diff_ex(inputs, params, window, "dyt", 32, None)
    want = _oracle_diff_ex(inputs, params, window, "dyt", 32, None)
    assert_close(got, want, BF16_TOL, f"diff ramp {step:+} w={window}")


@pytest.mark.parametrize("norm", ["dyt", "rms"])
def test_diff_model_band_strips(norm):
    """RMSNorm's row reductions in the key ring fill and the per-block staging, many strips."""
    S, H, B = 700, 48, 2
    inputs, params = _model_case(norm, S, H, B, 1300)
    keep = synth.make_v_keep(B, S, 60)
    got = _run_diff_ex(inputs, params, 17, norm, 32, keep)
    assert_close(got, _oracle_diff_ex(inputs, params, 17, norm, 32, keep), BF16_TOL, f"model strips {norm}")


def test_diff_model_all_padded_is_zero():
    inputs, params = _model_case("rms", 200, 2, 1, 1400)
    keep = np.zeros((1, 200), dtype=np.uint8)
    for window in (17, -1):
        assert np.all(_run_diff_ex(inputs, params, window, "rms", 32, keep) == 0.0)


def test_diff_model_dit_workload_full():
    """The DiT's own form at the full-differential workload's size: RMSNorm, 32 rotary dims, the last
    142 tokens padded; every output element."""
    wl = W["sa3_dit_fulldiff_h16s1422"]
    inputs, _ = synth.make_diff(wl)
    params = synth.make_model_params(wl.H, 1000 * wl.index + 6)
    keep = synth.make_v_keep(wl.B, wl.Sq, 142)
    got, bits = _run_diff_ex(inputs, params, wl.window, "rms", 32, keep, wl.scale, bits=True)
    want = _oracle_diff_ex(inputs, params, wl.window, "rms", 32, keep, scale=wl.scale)
    _parity(got, want, bits, "dit model form")


def test_diff_model_decoder_workload_full():
    """The decoder's own form at the banded workload's size: DyT, 32 rotary dims; every output element."""
    wl = W["sa3_decoder_banddiff_h8s23086w17"]
    inputs, params = synth.make_diff(wl)
    got, bits = _run_diff_ex(inputs, params, wl.window, "dyt", 32, None, wl.scale, bits=True)
    want = _oracle_diff_ex(inputs, params, wl.window, "dyt", 32, None, scale=wl.scale)
    _parity(got, want, bits, "decoder model form")


# ------------------------------------------------------------------ cross-attention shapes

@pytest.mark.parametrize("key", ["sdxl_l1_cross_b2h10q4096k77", "sa3_dit_cross_h24q1422k257"])
def test_xattn_conditioning_workloads(key):
    """SDXL level-1 cross-attention (77 keys) and the DiT's 257 conditioning tokens, both on chip,
    every output element against the oracle."""
    wl = W[key]
    q, k, v = synth.make_dense(wl)
    got, bits = _run_dense(ka.ka_xattn_fwd, q, k, v, wl.scale, bits=True)
    _parity(got, oracle.attn(q, k, v, wl.scale), bits, wl.key)


@pytest.mark.parametrize("Sk", [129, 192, 193, 255, 256, 257, 300, 384, 449, 500, 511, 512, 513, 1000])
def test_xattn_around_the_on_chip_limit(Sk):
    """Key sets from 129 to 512 sit in LDS (64-key chunks, online softmax; 8-wave blocks past 256);
    513 and more stream through the dense kernels."""
    assert ka.KA_XATTN_MAX_SK == 512
    wl = W["sdxl_l2_cross_b2h20q1024k77"]
    q, k, v = synth.make_dense(wl, seed_base=1500 + Sk, B=1, H=3, Sq=333, Sk=Sk)
    got = _run_dense(ka.ka_xattn_fwd, q, k, v)
    assert_close(got, oracle.attn(q, k, v, 0.125), BF16_TOL, f"xattn Sk={Sk}")


@pytest.mark.parametrize("B,H,Sq,Sk", [(2, 20, 1024, 77), (1, 7, 5000, 100), (3, 1, 40, 300), (1, 64, 1000, 500)])
def test_xattn_query_chunks(B, H, Sq, Sk):
    """Grids where a wave serves several 16-query blocks (the next block's rows fetched during the
    current one) and the last chunk of a (b, h) is ragged, for the one-pass and the chunked forms."""
    wl = W["sdxl_l2_cross_b2h20q1024k77"]
    q, k, v = synth.make_dense(wl, seed_base=1900 + Sq + Sk, B=B, H=H, Sq=Sq, Sk=Sk)
    got = _run_dense(ka.ka_xattn_fwd, q, k, v)
    assert_close(got, oracle.attn(q, k, v, 0.125), BF16_TOL, f"xattn {B}x{H}x{Sq}x{Sk}")


# ------------------------------------------------------------------ strided views (fused projection in, merged out)

def _fused_views(inputs):
    """The five [B,H,S,64] inputs laid out as one [B, S, 5, H, 64] projection (sections q1, k1, v, q2,
    k2, the order of the pages' to_qkv), returned as strided [B,H,S,64] views, and a merged
    [B, S, H, 64] output viewed as [B,H,S,64]."""
    q1, k1, q2, k2, v = (to_dev(x) for x in inputs)
    B, H, S, _ = q1.shape
    X = torch.stack([t.permute(0, 2, 1, 3) for t in (q1, k1, v, q2, k2)], dim=2).contiguous()  # [B,S,5,H,64]
    views = [X[:, :, i].permute(0, 2, 1, 3) for i in (0, 1, 3, 4, 2)]  # q1, k1, q2, k2, v
    out = torch.full((B, S, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    return views, out, out.permute(0, 2, 1, 3)


@pytest.mark.parametrize("form", ["dyt64", "rms32_padded", "dyt64_varied"])
@pytest.mark.parametrize("window", [17, 100, -1])
def test_diff_strided_fused_projection(form, window):
    S, H, B = 300, 3, 2
    norm = "rms" if form.startswith("rms") else "dyt"
    rot = 32 if "32" in form else 64
    inputs, params = _model_case(norm, S, H, B, 1600 + max(window, 0))
    if form.endswith("varied"):  # a different alpha per set, beta per set and channel, lambda per head
        params = synth.make_diff_params_varied(H, 1650 + max(window, 0))
    keep = synth.make_v_keep(B, S, 29) if "padded" in form else None
    views, out, o = _fused_views(inputs)
    assert not views[0].is_contiguous() and not o.is_contiguous()
    kw = dict(o=o, scale=0.125, window=window, qk_norm=norm, rotary_dims=rot)
    if norm == "rms":
        kw.update(rms_weight=to_dev(params[0]), rms_eps=1e-6)
    else:
        kw.update(alpha=to_dev(params[0]), gamma=to_dev(params[1]), beta=to_dev(params[2]))
    if keep is not None:
        kw["v_keep"] = to_dev(keep)
    ka.ka_diffattn_fwd_ex(*views, to_dev(params[-1]), **kw)
    torch.cuda.synchronize()
    got = to_host_f64(o.contiguous())
    want = _oracle_diff_ex(inputs, params, window, norm, rot, keep)
    assert_close(got, want, BF16_TOL, f"strided {form} w={window}")
    # the same call on contiguous copies gives the same bits
    assert np.array_equal(got, _run_diff_ex(inputs, params, window, norm, rot, keep))


def test_diff_strided_decoder_workload_full():
    """The decoder form reading the fused projection at the banded workload's size; every output element."""
    wl = W["sa3_decoder_banddiff_h8s23086w17"]
    inputs, params = synth.make_diff(wl)
    views, out, o = _fused_views(inputs)
    a, g, b, lm = (to_dev(x) for x in params)
    ka.ka_diffattn_fwd_ex(*views, lm, o=o, scale=wl.scale, window=wl.window, qk_norm="dyt", alpha=a, gamma=g,
                          beta=b, rotary_dims=32)
    torch.cuda.synchronize()
    oc = o.contiguous()
    want = _oracle_diff_ex(inputs, params, wl.window, "dyt", 32, None, scale=wl.scale)
    _parity(to_host_f64(oc), want, to_host_bits(oc), "strided decoder form")


# ------------------------------------------------------------------ head dim 512 (SDXL VAE mid-block attention)

@pytest.mark.parametrize("B,H,Sq,Sk", [(1, 1, 300, 333), (2, 2, 64, 31), (1, 1, 1, 1), (1, 3, 130, 64),
                                       (1, 1, 65, 1000)])
def test_dense_d512_shapes(B, H, Sq, Sk):
    wl = W["sdxl_vae_mid_b1h1s16384d512"]
    q, k, v = synth.make_dense(wl, seed_base=1700 + Sq + Sk, B=B, H=H, Sq=Sq, Sk=Sk)
    got = _run_dense(ka.ka_attn_fwd, q, k, v, wl.scale)
    assert_close(got, oracle.attn(q, k, v, wl.scale), BF16_TOL, f"d512 {B}x{H}x{Sq}x{Sk}")


def _peaked(shape_q, shape_kv, qscale, seed):
    r = np.random.default_rng(seed)
    q = synth.f32_to_bf16_bits((qscale * r.standard_normal(shape_q)).astype(np.float32))
    k = synth.f32_to_bf16_bits(r.standard_normal(shape_kv).astype(np.float32))
    v = synth.f32_to_bf16_bits(r.standard_normal(shape_kv).astype(np.float32))
    return q, k, v


@pytest.mark.parametrize("Sk", [77, 256, 300, 512, 600])
def test_xattn_peaked(Sk):
    """Cross-attention with q scaled by 8 (logit std 8): LDS-resident keys (77 in one pass; 256, 300,
    512 in chunks) and streamed (600)."""
    q, k, v = _peaked((2, 4, 700, D), (2, 4, Sk, D), 8, 2100 + Sk)
    got = _run_dense(ka.ka_xattn_fwd, q, k, v)
    assert_close(got, oracle.attn(q, k, v, 0.125), BF16_TOL, f"xattn peaked Sk={Sk}")


def test_dense_d512_peaked():
    """Head dim 512 with q scaled by 4 (logit std 4 at scale 512^-1/2)."""
    wl = W["sdxl_vae_mid_b1h1s16384d512"]
    q, k, v = _peaked((1, 1, 300, 512), (1, 1, 700, 512), 4, 2200)
    got = _run_dense(ka.ka_attn_fwd, q, k, v, wl.scale)
    assert_close(got, oracle.attn(q, k, v, wl.scale), BF16_TOL, "d512 peaked")


def test_dense_d512_vae_workload_full():
    wl = W["sdxl_vae_mid_b1h1s16384d512"]
    q, k, v = synth.make_dense(wl)
    got, bits = _run_dense(ka.ka_attn_fwd, q, k, v, wl.scale, bits=True)
    _parity(got, oracle.attn(q, k, v, wl.scale), bits, wl.key)

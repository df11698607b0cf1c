"""GPU parity of the residual add + RMSNorm before the layer
(moe_add_rmsnorm), the fp32-input router that consumes its output, and the
combine fused with the norm (moe_combine_add_rmsnorm), against the oracle
(oracle/norm.py, oracle/moe.py) and against the separate calls, through the C
ABI.

Bars: the residual output z rounded to bf16 is bit-exact (the fp32 sum of
two bf16 values is exact); the fp32 output within 1e-5 relative (the
kernel's fp32 sum of squares over at most 8 * ceil(H / 2048) + 8 sequential
additions per path, a root in fp64 and two fp32 products stay below 1e-6);
the bf16 output is the round-to-nearest-even of the kernel's own fp32 output
and within one bf16 step of the oracle's; the MXFP8 codes and scales equal
the oracle's quantiser applied to the kernel's fp32 output (the block
exponent is an integer decided in the kernel's precision)."""
import numpy as np
import pytest
import torch

from expert_routing_grouped_gate_amd import binding as B
from expert_routing_grouped_gate_amd import workloads as W
from oracle import mx, norm

pytestmark = pytest.mark.gpu

RTOL_F32 = 1e-5


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    B.load()
    yield
    torch.cuda.synchronize()


def _bf16_step(v):
    """Distance between neighbouring bf16 values around |v| (v > 0 normal)."""
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -126)))
    return np.exp2(e - 7)


# (T, H): one 32-block; 12 chunks; the decode and prefill hidden size; a
# width that leaves some threads with one chunk fewer; the largest width; the
# prefill layer's input as the bench times it
CASES = [(1, 32), (7, 96), (16, 4096), (333, 4096), (5, 2080), (64, 16384), (4096, 4096)]


@pytest.mark.parametrize("with_residual", [True, False])
@pytest.mark.parametrize("T,H", CASES)
def test_add_rmsnorm_parity(T, H, with_residual):
    eps = 1e-6
    x, r, w = W.draw_norm_inputs(T, H, seed=100 + T + H)
    res = r if with_residual else None
    out = B.add_rmsnorm(x.cuda(), w.cuda(), eps, None if res is None else res.cuda(), mx=True)
    torch.cuda.synchronize()
    z, y = norm.add_rmsnorm(x.double().numpy(), None if res is None else res.double().numpy(),
                            w.double().numpy(), eps)
    # residual: bit-exact
    np.testing.assert_array_equal(out["residual"].double().cpu().numpy(), mx.bf16_round(z))
    # fp32 y
    yf = out["f32"].double().cpu().numpy()
    err = np.abs(yf - y)
    assert np.all(err <= RTOL_F32 * np.abs(y)), f"max rel err {np.max(err / np.maximum(np.abs(y), 1e-30))}"
    # bf16 y: RNE of the kernel's fp32 y, one bf16 step from the oracle's
    yb = out["bf16"].double().cpu().numpy()
    np.testing.assert_array_equal(yb, mx.bf16_round(yf))
    assert np.all(np.abs(yb - mx.bf16_round(y)) <= _bf16_step(y))
    # MXFP8: the oracle's quantiser on the kernel's fp32 y, bit for bit
    codes, scales = mx.mxfp8_quantize(yf)
    np.testing.assert_array_equal(out["mx"][0].cpu().numpy(), codes)
    np.testing.assert_array_equal(out["mx"][1].cpu().numpy(), scales)
    # and against the exact y the scales agree except where a block's amax
    # sits within the fp32 error of a power of two
    _, s_exact = mx.mxfp8_quantize(y)
    assert np.mean(s_exact == scales) > 0.999


def test_each_output_alone_equals_all_together():
    T, H = 40, 4096
    x, r, w = (t.cuda() for t in W.draw_norm_inputs(T, H, seed=7))
    full = B.add_rmsnorm(x, w, 1e-5, r, mx=True)
    only_bf16 = B.add_rmsnorm(x, w, 1e-5, r, f32=False, residual_out=False)
    only_res = B.add_rmsnorm(x, w, 1e-5, r, f32=False, bf16=False)
    only_mx = B.add_rmsnorm(x, w, 1e-5, r, f32=False, bf16=False, residual_out=False, mx=True)
    torch.cuda.synchronize()
    assert torch.equal(full["bf16"], only_bf16["bf16"])
    assert torch.equal(full["residual"], only_res["residual"])
    assert torch.equal(full["mx"][0], only_mx["mx"][0]) and torch.equal(full["mx"][1], only_mx["mx"][1])


def test_zero_row_and_large_eps():
    """A zero row normalises to zeros (eps > 0); a large eps shrinks y by
    sqrt(ms / (ms + eps))."""
    T, H = 3, 256
    x, r, w = W.draw_norm_inputs(T, H, seed=9)
    x[1] = 0
    r[1] = 0
    for eps in (1e-6, 4.0):
        out = B.add_rmsnorm(x.cuda(), w.cuda(), eps, r.cuda())
        torch.cuda.synchronize()
        _, y = norm.add_rmsnorm(x.double().numpy(), r.double().numpy(), w.double().numpy(), eps)
        yf = out["f32"].double().cpu().numpy()
        assert np.all(yf[1] == 0.0)
        assert np.all(np.abs(yf - y) <= RTOL_F32 * np.abs(y))


def test_zero_tokens():
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(256, dtype=torch.bfloat16, device="cuda")
    out = B.add_rmsnorm(x, w, 1e-6)
    assert out["f32"].shape == (0, 256)


def test_mx_output_dequantises_to_y():
    """The MXFP8 output dequantises to the fp32 output within the format's
    bound: half an E4M3 step (2^-4 of the element, or 2^-10 of the block
    scale in the subnormal range); elements beyond 448 x scale (the rule
    saturates scaled values in [448, 512)) lose exactly the clipped part."""
    T, H = 16, 4096
    x, r, w = (t.cuda() for t in W.draw_norm_inputs(T, H, seed=21))
    out = B.add_rmsnorm(x, w, 1e-6, r, mx=True)
    torch.cuda.synchronize()
    yf = out["f32"].double().cpu().numpy()
    deq = mx.mxfp8_dequant(out["mx"][0].cpu().numpy(), out["mx"][1].cpu().numpy())
    scale = np.repeat(mx.e8m0_decode(out["mx"][1].cpu().numpy()), 32, axis=-1)
    sat = np.abs(yf) > 448 * scale
    bound = np.where(sat, np.abs(yf) - 448 * scale, np.maximum(2.0 ** -4 * np.abs(yf), 2.0 ** -10 * scale))
    assert np.all(np.abs(deq - yf) <= bound * (1 + 1e-12))
    assert np.all(np.abs(deq[sat]) == 448 * scale[sat])


# ------------------------------------------- the gate's fp32 input: S1 ----
# moe_router_logits_f32: products and per-slice sums in fp64, 16 slice sums
# (H = 4096) rounded to fp32 and added in fp32: at most ~20 fp32 roundings of
# values of the logits' size (|L| < 3 here), so 2e-5 is a tenfold margin.
ATOL_LOGITS = 2e-5


@pytest.mark.parametrize("T,H,E", [(1, 256, 8), (16, 4096, 128), (333, 4096, 192), (70, 512, 256),
                                   (4096, 4096, 128)])
def test_router_logits_f32(T, H, E):
    g = torch.Generator().manual_seed(T * 7 + H + E)
    x = torch.randn((T, H), generator=g, dtype=torch.float32)
    wr = torch.randn((E, H), generator=g, dtype=torch.float32) * 0.02
    got = B.router_logits_f32(x.cuda(), wr.cuda())
    torch.cuda.synchronize()
    ref = x.double().numpy() @ wr.double().numpy().T
    np.testing.assert_allclose(got.double().cpu().numpy(), ref, atol=ATOL_LOGITS, rtol=0)


def test_router_logits_f32_exact_on_small_integers():
    """Integer inputs whose every partial sum is an integer below 2^24: the
    logits are exact."""
    g = torch.Generator().manual_seed(5)
    x = torch.randint(-4, 5, (40, 1024), generator=g).float()
    wr = torch.randint(-3, 4, (24, 1024), generator=g).float()
    got = B.router_logits_f32(x.cuda(), wr.cuda())
    torch.cuda.synchronize()
    want = (x.double() @ wr.double().T).numpy()
    np.testing.assert_array_equal(got.double().cpu().numpy(), want)


def test_norm_feeds_the_gate_in_fp32():
    """The step before the layer and the layer's S1/S2 chained on the device:
    add + RMSNorm -> fp32 y -> router logits -> top-k.  Logits against the
    oracle's fp64 logits of the same fp32 y; the selection against the
    oracle's gate on the GPU's logits (ids bit-exact)."""
    from oracle import moe
    T, H, E, k = 64, 4096, 128, 8
    x, r, w = (t.cuda() for t in W.draw_norm_inputs(T, H, seed=33))
    wr = (torch.randn((E, H), generator=torch.Generator().manual_seed(34)) * 0.02).cuda()
    y = B.add_rmsnorm(x, w, 1e-6, r, bf16=False, residual_out=False)["f32"]
    logits = B.router_logits_f32(y, wr)
    ids, wts = B.gate_topk(logits, k, B.GATE_SOFTMAX)
    torch.cuda.synchronize()
    gl = logits.cpu().numpy()
    ref = y.double().cpu().numpy() @ wr.double().cpu().numpy().T
    np.testing.assert_allclose(gl.astype(np.float64), ref, atol=ATOL_LOGITS, rtol=0)
    want_ids, want_w = moe.gate_topk_softmax(gl, k)
    np.testing.assert_array_equal(ids.cpu().numpy(), want_ids)
    np.testing.assert_allclose(wts.cpu().numpy(), want_w, rtol=1e-6, atol=1e-7)


# ------------------------- S7 fused with the next layer's add + RMSNorm ----

def _norm_bars(out, z, y, what):
    """The norm's bars (module docstring) for every output of a call against
    the oracle's z and y of the same combined rows."""
    np.testing.assert_array_equal(out["residual"].double().cpu().numpy(), mx.bf16_round(z))
    yf = out["f32"].double().cpu().numpy()
    err = np.abs(yf - y)
    assert np.all(err <= RTOL_F32 * np.abs(y)), f"{what}: f32 max rel err {np.max(err / np.maximum(np.abs(y), 1e-30))}"
    yb = out["bf16"].double().cpu().numpy()
    np.testing.assert_array_equal(yb, mx.bf16_round(yf))
    assert np.all(np.abs(yb - mx.bf16_round(y)) <= _bf16_step(y)), what
    codes, scales = mx.mxfp8_quantize(yf)
    np.testing.assert_array_equal(out["mx"][0].cpu().numpy(), codes)
    np.testing.assert_array_equal(out["mx"][1].cpu().numpy(), scales)


def _combine_bound(y64, pp_np, w_np, sh64, ref_out):
    """Largest distance between the kernel's combined row (fp32 slot sums
    rounded to bf16) and the oracle's (fp64 sums rounded to bf16): the fp32
    sum of k (+1 shared) products is within (k + 2) 2^-24 of the sum of
    their magnitudes, and the two roundings to bf16 add at most one bf16
    step of the larger value."""
    T, k = w_np.shape
    mag = np.zeros_like(ref_out)
    pos = pp_np.reshape(T, k)
    for j in range(k):
        mag += np.abs(w_np[:, j:j + 1].astype(np.float64)) * np.abs(y64[pos[:, j]])
    if sh64 is not None:
        mag += np.abs(sh64)
    e = (k + 2) * 2.0 ** -24 * mag
    return e + _bf16_step(np.abs(ref_out) + e) + 1e-30


def _fused_vs_oracle(fused, y, pp, w, shared, weight, eps, res):
    """Every output of moe_combine_add_rmsnorm against the oracle.

    (1) oracle/norm.add_rmsnorm of the call's own combined rows (its `out`
    output): the norm's bars, bit for bit where they are exact.
    (2) The oracle's whole chain: oracle/moe.combine of the same expert
    rows, then oracle/norm.add_rmsnorm.  The combined rows may differ by
    the bound of _combine_bound (fp32 against fp64 slot sums, then bf16
    roundings), and such a difference dz_i
    carries through the norm: y_i changes by |w_i| r dz_i directly and every
    y_j by |y_j| |dr / r| through the row's root, |dr / r| <= |d mean(z^2)| /
    (2 (mean(z^2) + eps)).  The f32 output must lie within that plus the
    norm's own 1e-5; bf16 and the residual within it plus one bf16 step; the
    MXFP8 output (dequantised) within it plus the format's rounding bound."""
    from oracle import moe
    y64, pp_np, w_np = y.double().cpu().numpy(), pp.cpu().numpy(), w.cpu().numpy()
    sh64 = None if shared is None else shared.double().cpu().numpy()
    res64 = None if res is None else res.double().cpu().numpy()
    g64 = weight.double().cpu().numpy()
    got_out = fused["out"].double().cpu().numpy()
    ref_out = moe.combine(y64, pp_np, w_np, sh64)
    dz = np.abs(got_out - ref_out)
    assert np.all(dz <= _combine_bound(y64, pp_np, w_np, sh64, ref_out)), "combined rows"
    z1, y1 = norm.add_rmsnorm(got_out, res64, g64, eps)            # (1)
    _norm_bars(fused, z1, y1, "fused vs oracle norm of its own rows")
    z2, y2 = norm.add_rmsnorm(ref_out, res64, g64, eps)            # (2)
    H = z2.shape[1]
    ms2 = np.sum(z2 * z2, axis=1, keepdims=True) / H
    r2 = 1.0 / np.sqrt(ms2 + eps)
    dms = np.abs(np.sum(z1 * z1 - z2 * z2, axis=1, keepdims=True)) / H
    drel = 0.5 * dms / (ms2 + eps) * 1.01
    prop = np.abs(g64)[None] * r2 * dz * 1.01 + np.abs(y2) * drel
    bound = RTOL_F32 * np.abs(y2) + prop + 1e-30
    yf = fused["f32"].double().cpu().numpy()
    assert np.all(np.abs(yf - y2) <= bound), "f32 vs the oracle's chain"
    yb = fused["bf16"].double().cpu().numpy()
    assert np.all(np.abs(yb - y2) <= bound + _bf16_step(y2)), "bf16 vs the oracle's chain"
    rz = fused["residual"].double().cpu().numpy()
    assert np.all(np.abs(rz - z2) <= dz + _bf16_step(z2) + 1e-30), "residual vs the oracle's chain"
    scale = np.repeat(mx.e8m0_decode(fused["mx"][1].cpu().numpy()), 32, axis=-1)
    deq = mx.mxfp8_dequant(fused["mx"][0].cpu().numpy(), fused["mx"][1].cpu().numpy())
    q_err = np.where(np.abs(yf) > 448 * scale, np.abs(yf) - 448 * scale,
                     np.maximum(2.0 ** -4 * np.abs(yf), 2.0 ** -10 * scale))
    assert np.all(np.abs(deq - y2) <= bound + q_err * (1 + 1e-12)), "MXFP8 vs the oracle's chain"
    rows_same = np.mean(np.all(dz == 0, axis=1))
    print(f"fused vs oracle chain: {rows_same:.3f} of rows combine identically", flush=True)

def _separate(y, pp, w, shared, weight, eps, res):
    out = B.combine(y, pp, w, shared)
    n = B.add_rmsnorm(out, weight, eps, res, mx=True)
    return out, n


@pytest.mark.parametrize("with_shared,with_residual", [(True, True), (False, True), (False, False)])
def test_combine_add_rmsnorm_equals_separate_calls_on_a_layer(with_shared, with_residual):
    """The expert rows of a real layer (the LDS-tiled GEMM path,
    sigmoid gating, shared expert): every output of the fused call equals
    moe_combine then moe_add_rmsnorm bit for bit; the combined rows match the
    oracle's combine of the same expert rows."""
    from oracle import moe
    from tests.layer_fixtures import get_layer
    cfg = W.CONFIGS["hy3"].with_(name="fuse_hy3", T=300, H=512, E=16, k=4, I=384, shared_I=384,
                                 x_seed=41, family_seed=1041)
    L = get_layer(cfg)
    layer = L.layer()
    layer.forward(L.dev["x"])
    b = layer.buf
    shared = b["shared_y"] if with_shared else None
    g = torch.Generator().manual_seed(42)
    res = torch.randn((cfg.T, cfg.H), generator=g).to(torch.bfloat16).cuda() if with_residual else None
    weight = (1 + 0.1 * torch.randn(cfg.H, generator=g)).to(torch.bfloat16).cuda()
    fused = B.combine_add_rmsnorm(b["y"], b["pair_pos"], b["topk_w"], shared, weight, 1e-6, res,
                                  out=True, mx=True)
    out, n = _separate(b["y"], b["pair_pos"], b["topk_w"], shared, weight, 1e-6, res)
    torch.cuda.synchronize()
    assert torch.equal(fused["out"], out)
    for key in ("f32", "bf16", "residual"):
        assert torch.equal(fused[key], n[key]), key
    assert torch.equal(fused["mx"][0], n["mx"][0]) and torch.equal(fused["mx"][1], n["mx"][1])
    ref = moe.combine(b["y"].double().cpu().numpy(), b["pair_pos"].cpu().numpy(),
                      b["topk_w"].cpu().numpy(), None if shared is None else shared.double().cpu().numpy())
    got = out.double().cpu().numpy()
    assert np.all(np.abs(got - ref) <= _combine_bound(b["y"].double().cpu().numpy(), b["pair_pos"].cpu().numpy(),
                                                      b["topk_w"].cpu().numpy(),
                                                      None if shared is None else shared.double().cpu().numpy(), ref))
    _fused_vs_oracle(fused, b["y"], b["pair_pos"], b["topk_w"], shared, weight, 1e-6, res)


@pytest.mark.parametrize("T,k,H", [(4096, 8, 4096), (16, 8, 4096), (3, 32, 256), (7, 1, 16384)])
def test_combine_add_rmsnorm_equals_separate_calls(T, k, H):
    """Synthetic expert rows at the prefill layer's full size and at the
    limits (k = 32, the widest H): the fused call equals the separate ones."""
    y, pp, w = W.draw_combine_inputs(T, k, H, seed=T + k + H)
    x, r, g = W.draw_norm_inputs(T, H, seed=7 * T + H)
    y, pp, w, r, g = y.cuda(), pp.cuda(), w.cuda(), r.cuda(), g.cuda()
    fused = B.combine_add_rmsnorm(y, pp, w, None, g, 1e-6, r, out=True, mx=True)
    out, n = _separate(y, pp, w, None, g, 1e-6, r)
    torch.cuda.synchronize()
    assert torch.equal(fused["out"], out)
    for key in ("f32", "bf16", "residual"):
        assert torch.equal(fused[key], n[key]), key
    assert torch.equal(fused["mx"][0], n["mx"][0]) and torch.equal(fused["mx"][1], n["mx"][1])
    _fused_vs_oracle(fused, y, pp, w, None, g, 1e-6, r)

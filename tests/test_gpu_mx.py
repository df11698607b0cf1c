"""GPU parity of the W4A8 path (MXFP4 weights, MXFP8 activations): the
dynamic MX quantiser bit for bit, each scaled-MFMA GEMM against the oracle on
the GPU's own inputs, and the whole layer within |d| <= 3e-2 + 3e-2*|ref|."""
import numpy as np
import pytest
import torch

from expert_routing_grouped_gate_amd import binding as B
from expert_routing_grouped_gate_amd import workloads as W
from oracle import moe, mx
from tests.layer_fixtures import (assert_close_bf16, check_ids_on_oracle_logits, expert_rows_to_check,
                                  get_layer, log)

pytestmark = pytest.mark.gpu

ATOL = RTOL = 3e-2
CFG = W.CONFIGS
SMALL = {
    "mx_tiny": CFG["qwen3_decode_w4a8"].with_(name="mx_tiny", T=16, H=256, E=8, k=2, I=128,
                                              family_seed=1105, x_seed=21),
    "mx_mid": CFG["qwen3_decode_w4a8"].with_(name="mx_mid", T=37, H=1024, E=16, k=4, I=256,
                                             family_seed=1106, x_seed=22),
    "mx_decode_shape": CFG["qwen3_decode_w4a8"].with_(name="mx_decode_shape", T=5, x_seed=23),
    # more tiles than the grid has waves: every wave streams several tiles
    # back to back (its next tile's first loads overlap the current tile)
    "mx_many_tiles": CFG["qwen3_decode_w4a8"].with_(name="mx_many_tiles", T=1024, H=256, E=8, k=4,
                                                    I=512, family_seed=1107, x_seed=24),
    # Hy3-style gate with an always-on W4A8 shared expert
    "mx_shared": CFG["hy3"].with_(name="mx_shared", T=40, H=512, E=16, k=4, I=256, shared_I=384,
                                  fmt="w4a8", family_seed=1108, x_seed=25),
    # more than 8 rows per expert on average and K a multiple of 512, at least 1024:
    # the LDS-tiled kernels; two quads of K-steps per tile ...
    "mx_tiled": CFG["qwen3_decode_w4a8"].with_(name="mx_tiled", T=512, H=1024, E=8, k=2, I=1024,
                                               family_seed=1109, x_seed=26),
    # ... several quads, ragged 128-row m-tiles, 8 n-tiles in each GEMM
    "mx_tiled_deep": CFG["qwen3_decode_w4a8"].with_(name="mx_tiled_deep", T=300, H=2048, E=4, k=2,
                                                    I=1024, family_seed=1110, x_seed=27),
    # shared expert (one identity group of T rows) on the tiled GEMM1; GEMM2
    # has K = 512 (streaming kernels)
    "mx_tiled_shared": CFG["hy3"].with_(name="mx_tiled_shared", T=200, H=1024, E=8, k=4, I=512,
                                        shared_I=512, fmt="w4a8", family_seed=1111, x_seed=28),
    # more tiles than resident blocks: blocks stream from one tile into the
    # next (the next tile's first steps load during the current one's last)
    "mx_tiled_stream": CFG["qwen3_decode_w4a8"].with_(name="mx_tiled_stream", T=1024, H=2048, E=4,
                                                      k=4, I=2048, family_seed=1112, x_seed=29),
    # GEMM2 with 6 K-steps (I = 768, a multiple of 3: the three-batch
    # rotation) and ~8,200 tiles of 16 rows x 64 columns for ~3,000 resident
    # waves: each wave streams several tiles, so both the in-tile batch loads
    # and the next tile's first two batches are used
    "mx_d3_stream": CFG["qwen3_decode_w4a8"].with_(name="mx_d3_stream", T=1024, H=2048, E=8, k=4,
                                                   I=768, family_seed=1113, x_seed=30),
    # 8 rows per expert on average (the streaming kernels although the tiled
    # ones would fit), the Zipf router bias putting most tokens on the first
    # experts: several 16-row tiles per group
    "mx_skew_stream": CFG["qwen3_decode_w4a8"].with_(name="mx_skew_stream", T=64, H=1024, E=16, k=2,
                                                     I=256, family_seed=1114, x_seed=31),
}

# The GEMM-level configs again with block scales spread over 2^-27 .. 2^13
# (E8M0 codes 100..140) instead of mostly 2^-7, so that the scaled MFMAs see
# every scale lane carry a different exponent.
WIDE = {f"{n}_wide": c.with_(name=f"{n}_wide", mx_scales="wide", family_seed=c.family_seed + 100)
        for n, c in SMALL.items()
        if n in ("mx_tiny", "mx_mid", "mx_decode_shape", "mx_shared", "mx_tiled_deep", "mx_tiled_shared",
                 "mx_d3_stream")}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    B.load()


def np_(t):
    return t.detach().cpu().numpy()


@pytest.mark.parametrize("rows,cols,scale", [(16, 4096, 1.0), (3, 256, 1e-3), (1, 32, 300.0), (7, 96, 1e-30)])
def test_mx_quantize_bit_exact(rows, cols, scale):
    g = torch.Generator().manual_seed(rows * 7 + cols)
    x = (torch.randn((rows, cols), generator=g) * scale)
    x[0, :32] = 0.0                                   # an all-zero block
    if cols >= 64:
        x[0, 32:64] = torch.linspace(-448, 448, 32)   # saturating values
    x = x.to(torch.bfloat16)
    codes, scales = B.mx_quantize(x.cuda())
    rc, rs = mx.mxfp8_quantize(x.to(torch.float64).numpy())
    assert np.array_equal(np_(scales), rs)
    assert np.array_equal(np_(codes), rc)


def _quant_codes_close(gpu_codes, gpu_scales, ref_vals, what, da=None):
    """The GPU quantises fp32 values, the oracle the fp64 ones; allow a code
    to differ by one E4M3 step on a small fraction of elements (values that
    sit next to a rounding boundary).  The value quantised is SiLU(g) * u of
    two fp32 dot products over K, whose rounding error is absolute: relative
    to the largest value of its 32-block, about 2^-14 covers it, so elements
    that cancel to almost zero are held to that instead of one E4M3 step.

    The block exponent is an integer decided by the block's amax, which the
    GPU takes from its fp32 values: a block whose exact amax lies within
    2^-12 (relative) of the power of two between two exponents may take the
    other one.  Such blocks (and only such) may differ by one in the scale;
    every block's codes are compared with the exact values quantised with the
    GPU's exponent (the oracle's own codes wherever the exponents agree).

    da (optional, per element): a bound on the error of the GPU's value
    before quantisation (widely spread block scales, where the scaled MFMA's
    block accumulation dominates; see _mfma_step_bound).  Then a block may
    take the other exponent when its amax lies within its largest da of the
    power of two, and each dequantised code must lie within da plus one
    E4M3 rounding (and any saturation) of the exact value."""
    rows, cols = ref_vals.shape
    rc, rs = mx.mxfp8_quantize(ref_vals)
    gs, rsi = gpu_scales.astype(np.int64), rs.astype(np.int64)
    amax_b = np.abs(ref_vals).reshape(rows, cols // 32, 32).max(-1)
    flip = gs != rsi
    if flip.any():
        edge = 2.0 ** (np.maximum(gs, rsi)[flip] - 127 + 8)   # amax where the exponent steps
        tol = 2.0 ** -12 * edge
        if da is not None:
            tol = np.maximum(tol, da.reshape(rows, cols // 32, 32).max(-1)[flip] * 1.01)
        near = np.abs(amax_b[flip] - edge) <= tol
        assert np.all((np.abs(gs - rsi)[flip] == 1) & near), f"{what}: block scales differ"
    scale = np.repeat(mx.e8m0_decode(gpu_scales), 32, -1)
    gv = mx.mxfp8_dequant(gpu_codes, gpu_scales)
    if da is not None:
        a = np.abs(ref_vals)
        bound = (da + np.maximum(2.0 ** -4 * (a + da), 2.0 ** -10 * scale)
                 + np.maximum(0.0, a + da - 448.0 * scale)) * (1 + 1e-12)
        assert np.all(np.abs(gv - ref_vals) <= bound), f"{what}: codes outside the derived bound"
        return
    rq = mx.e4m3_encode_rne(ref_vals / scale)
    rv = mx.e4m3_decode(rq) * scale
    same = gv == rv
    assert same.mean() > 0.995, f"{what}: only {same.mean():.4f} of codes equal"
    d = np.abs(gv - rv)
    amax = np.repeat(amax_b, 32, -1)
    step = np.abs(rv) * 0.126 + scale * 2.0 ** -9 * 1.01
    assert np.all(d <= np.maximum(step, amax * 2.0 ** -14)), what


def _mfma_step_bound(a, w):
    """Error bound of the GPU's sums a . w over K with the block-scaled FP8 x
    FP4 MFMA.  Measured on this GPU (a probe through the library's GEMM2 with
    hand-set codes): inside one 32-element block the products are summed
    keeping about 13 bits below the block's largest product (a product 2^-13
    of it survives, one of 2^-14 is dropped), while block sums are combined
    and accumulated at fp32 precision.  So each of a block's 32 products
    loses less than 2^-13 of the block maximum (2^-8 per block in all), and
    the fp32 steps add at most 2^-16 of the sum of |products| (<= 32 times the
    block maximum per block).  The block maximum is bounded by the product of
    the block maxima of |a| and |w|, so the bound is a matrix product.
    a [R, K], w [N, K] -> [R, N]."""
    K = a.shape[1]
    am = np.abs(a).reshape(a.shape[0], K // 32, 32).max(-1)
    wm = np.abs(w).reshape(w.shape[0], K // 32, 32).max(-1)
    return (2.0 ** -8 + 32 * 2.0 ** -16) * (am @ wm.T)


def _np_pack(codes, scales):
    """The packed W4A8 layout as include/moe.h defines it, by reshapes."""
    G, R, K2 = codes.shape
    K = 2 * K2
    ns, q16 = K // 128, R // 16
    nq = (ns + 3) // 4
    pc = codes.reshape(G, q16, 16, ns, 4, 16).transpose(0, 1, 3, 4, 2, 5)   # g q s b i byte
    sc = np.zeros((G, q16, 16, nq * 4, 4), np.uint8)                       # g q i step b
    sc[:, :, :, :ns] = scales.reshape(G, q16, 16, ns, 4)
    ps = sc.reshape(G, q16, 16, nq, 4, 4).transpose(0, 1, 3, 5, 2, 4)       # g q c b i u
    return pc.reshape(G, R, K2), ps.reshape(G, -1)


@pytest.mark.parametrize("G,R,K", [(3, 48, 384), (2, 32, 1024), (1, 16, 128)])
def test_mx_pack_weight_layout(G, R, K):
    g = torch.Generator().manual_seed(G * 1000 + R + K)
    codes = torch.randint(0, 256, (G, R, K // 2), generator=g, dtype=torch.uint8)
    scales = torch.randint(100, 140, (G, R, K // 32), generator=g, dtype=torch.uint8)
    pc, ps = B.mx_pack_weight(codes.cuda(), scales.cuda())
    torch.cuda.synchronize()
    rc, rs = _np_pack(codes.numpy(), scales.numpy())
    assert np.array_equal(np_(pc), rc)
    assert np.array_equal(np_(ps), rs)


@pytest.mark.parametrize("name", list(SMALL) + list(WIDE))
def test_mx_grouped_ffn(name):
    L = get_layer({**SMALL, **WIDE}[name])
    cfg = L.cfg
    x = L.dev["x"]
    xq, xs = B.mx_quantize(x)
    logits = B.router_logits(x, L.dev["wr"])
    ids, w = B.gate_topk(logits, cfg.k, L.mode, L.dev["bias"], cfg.routed_scale, cfg.eps)
    counts, offsets, sp, pp = B.route(ids, cfg.E)
    act, act_s = B.grouped_ffn_up(L.weights, xq, xs, cfg.k, sp, offsets)
    y = B.grouped_ffn_down(L.weights, act, act_s, cfg.T, cfg.k, offsets)
    torch.cuda.synchronize()
    xv = mx.mxfp8_dequant(np_(xq), np_(xs))
    sp_np, off = np_(sp), np_(offsets)
    act_c, act_sc = np_(act), np_(act_s)
    act_v = mx.mxfp8_dequant(act_c, act_sc)
    yg = np_(y.float()).astype(np.float64)
    for e in range(cfg.E):
        r0, r1 = off[e], off[e + 1]
        if r1 == r0:
            continue
        w13, w2 = L.expert(e)
        xr = xv[sp_np[r0:r1] // cfg.k]
        I = w13.shape[0] // 2
        g, u = xr @ w13[:I].T, xr @ w13[I:].T
        a = moe.silu(g) * u
        da = None
        if cfg.mx_scales == "wide":
            # values up to ~1e16 whose sums cancel far below their terms: the
            # error of g and u is the MFMA's (_mfma_step_bound), carried
            # through SiLU (slope at most 1.1; |SiLU(g)| <= |g| + 0.3)
            dg, du = _mfma_step_bound(xr, w13[:I]), _mfma_step_bound(xr, w13[I:])
            da = 1.1 * dg * (np.abs(u) + du) + (np.abs(g) + dg + 0.3) * du
        _quant_codes_close(act_c[r0:r1], act_sc[r0:r1], a, f"{name} act expert {e}", da)
        # the down projection on the GPU's own activation codes
        ref = act_v[r0:r1] @ w2.T
        if cfg.mx_scales == "wide":
            # the bf16 rounding of the output (2^-9 |y|, taken as 2^-8) plus
            # the MFMA's accumulation bound; the fixed 1e-2 floor of the unit
            # scale configs means nothing at these magnitudes
            err = np.abs(yg[r0:r1] - ref)
            bad = err > 2.0 ** -8 * np.abs(ref) + _mfma_step_bound(act_v[r0:r1], w2)
            assert not bad.any(), f"{name} y expert {e}: {int(bad.sum())} outside the derived bound"
        else:
            assert_close_bf16(yg[r0:r1], ref, 1e-2, 1e-2, f"{name} y expert {e}")


def _check_act_exponents(gpu_scales, amax, what):
    """The block exponents the GPU took for its SwiGLU outputs against the
    rule on the exact values: equal, or one apart only where the exact
    block maximum lies within 2^-12 (relative) of the power of two between
    the two exponents (the exponent is an integer decided in the kernel's
    fp32).  Rows the oracle did not evaluate (NaN) are skipped."""
    rows = ~np.isnan(amax).any(axis=1)
    ge = gpu_scales[rows].astype(np.int64) - 127
    own = mx.mx_block_exponent(amax[rows], 8)
    flip = ge != own
    if flip.any():
        edge = 2.0 ** (np.maximum(ge, own)[flip] + 8)
        near = np.abs(amax[rows][flip] / edge - 1.0) <= 2.0 ** -12
        assert np.all((np.abs(ge - own)[flip] == 1) & near), f"{what}: act block exponents"
    log(f"[{what}] act block exponents: {int(flip.sum())} of {flip.size} one off at a power of two")


def _layer_check(cfg, tokens=None):
    L = get_layer(cfg)
    layer = L.layer()
    out = layer.forward(L.dev["x"])
    torch.cuda.synchronize()
    b = layer.buf
    gl = np_(b["logits"])
    # the SwiGLU outputs' MXFP8 block exponents are integers the GPU decides
    # from its fp32 values; the oracle quantises its exact values at those
    # exponents (as it gates on the GPU's logits), after they are checked
    act_s = np_(b["act_scales"])
    sh_s = np_(b["shared_act_scales"]) if cfg.shared_I else None
    res = L.oracle(logits=gl, tokens=tokens, act_exponents=act_s.astype(np.int64) - 127,
                   shared_act_exponents=None if sh_s is None else sh_s.astype(np.int64) - 127)
    _check_act_exponents(act_s, res["act_amax"], cfg.name)
    if sh_s is not None:
        toks = np.arange(cfg.T) if tokens is None else np.asarray(tokens)
        _check_act_exponents(sh_s[toks], res["shared_act_amax"], cfg.name + " shared")
    np.testing.assert_allclose(gl, res["logits"], atol=1e-4, rtol=0)
    assert np.array_equal(np_(b["topk_ids"]), res["ids"])
    check_ids_on_oracle_logits(cfg, res["logits"], L.bias(), np_(b["topk_ids"]))
    for key in ("counts", "offsets", "sorted_pair", "pair_pos"):
        assert np.array_equal(np_(b[key]), res[key]), key
    rc, rs = mx.mxfp8_quantize(L.x64())
    assert np.array_equal(np_(b["xq"]), rc) and np.array_equal(np_(b["xq_scales"]), rs)
    og = out.double().cpu().numpy()
    if tokens is not None:
        og = og[np.asarray(tokens)]
    assert_close_bf16(og, res["out"], ATOL, RTOL, f"{cfg.name} out")


@pytest.mark.parametrize("name", list(SMALL))
def test_mx_layer_small(name):
    _layer_check(SMALL[name])


def test_mx_layer_full_decode():
    _layer_check(CFG["qwen3_decode_w4a8"])


def test_mx_layer_full_prefill():
    # 4096 tokens (tiled GEMMs): values on a sample of tokens
    _layer_check(CFG["qwen3_prefill_w4a8"], tokens=[0, 1, 2, 777, 2048, 4094, 4095])


# full-size W4A8 decode weights on both sides of the switch from the
# streaming GEMMs (at most 8 rows per expert on average: T <= 128 at E = 128,
# k = 8) to the tiled ones; values on a sample of tokens
MID = {"qwen3_w4a8_T128": CFG["qwen3_w4a8_T128"],
       "qwen3_w4a8_T136": CFG["qwen3_w4a8_T128"].with_(name="qwen3_w4a8_T136", T=136, x_seed=336)}


@pytest.mark.parametrize("name", list(MID))
def test_mx_layer_mid_size(name):
    T = MID[name].T
    _layer_check(MID[name], tokens=[0, 1, 2, 3, 40, 63, 64, 100, T - 3, T - 2, T - 1])


def test_mx_full_size_expert_rows():
    """The full W4A8 prefill layer: whole experts' GEMM1 act codes (against
    the oracle's SwiGLU of the dequantised x, quantised) and GEMM2 rows (on
    the GPU's own act codes) for the expert with the most rows, the fewest,
    the most ragged last m-tile, the first and last touched ids and a random
    one."""
    cfg = CFG["qwen3_prefill_w4a8"]
    L = get_layer(cfg)
    layer = L.layer()
    layer.forward(L.dev["x"])
    torch.cuda.synchronize()
    b = layer.buf
    off, sp = np_(b["offsets"]), np_(b["sorted_pair"])
    xv = mx.mxfp8_dequant(np_(b["xq"]), np_(b["xq_scales"]))
    experts = expert_rows_to_check(off, seed=5)
    assert len(experts) >= 4
    for e in experts:
        r0, r1 = int(off[e]), int(off[e + 1])
        w13, w2 = L.expert(e)
        xr = xv[sp[r0:r1] // cfg.k]
        a = moe.silu(xr @ w13[:cfg.I].T) * (xr @ w13[cfg.I:].T)
        ac, asc = np_(b["act"][r0:r1]), np_(b["act_scales"][r0:r1])
        _quant_codes_close(ac, asc, a, f"full W4A8 act expert {e} ({r1 - r0} rows)")
        yg = np_(b["y"][r0:r1].float()).astype(np.float64)
        assert_close_bf16(yg, mx.mxfp8_dequant(ac, asc) @ w2.T, 1e-2, 1e-2, f"full W4A8 y expert {e}")
    log("[qwen3_prefill_w4a8] expert rows checked: " + ", ".join(f"{e} ({int(off[e + 1] - off[e])} rows)"
                                                               for e in experts))


@pytest.mark.parametrize("name", ["mx_tiled", "mx_tiled_deep", "mx_tiled_stream"])
def test_mx_tiled_equals_streaming_bit_for_bit(name):
    """A row's GEMM outputs depend only on that row, and both GEMM kernels
    run the same scaled MFMAs over the same K-steps in the same order.  With
    the routing of all T tokens, the first 8*E/k tokens alone (8 rows per
    expert on average: streaming kernels) and all T tokens (tiled kernels)
    give the same bits in every row of those tokens, in both GEMMs."""
    L = get_layer(SMALL[name])
    cfg = L.cfg
    x = L.dev["x"]
    xq, xs = B.mx_quantize(x)
    logits = B.router_logits(x, L.dev["wr"])
    ids, _ = B.gate_topk(logits, cfg.k, L.mode, L.dev["bias"], cfg.routed_scale, cfg.eps)
    nfew = 8 * cfg.E // cfg.k
    outs = []
    for T in (nfew, cfg.T):
        _, offsets, sp, pp = B.route(ids[:T].contiguous(), cfg.E)
        act, act_s = B.grouped_ffn_up(L.weights, xq[:T], xs[:T], cfg.k, sp, offsets)
        y = B.grouped_ffn_down(L.weights, act, act_s, T, cfg.k, offsets)
        rows = pp[: nfew * cfg.k].long()          # rows of the first nfew tokens' pairs
        outs.append((act[rows], act_s[rows], y[rows]))
    torch.cuda.synchronize()
    for few, many, what in zip(outs[0], outs[1], ("act codes", "act scales", "y")):
        assert torch.equal(few, many), what


@pytest.mark.parametrize("name", ["mx_shared", "mx_tiled_deep"])
def test_mx_non_finite_token_stays_in_its_row(name):
    """NaN in one token's hidden state (its MXFP8 blocks, logits, activations
    and shared-expert row): the token still routes to k distinct experts in
    range, and every other token's output equals the clean run's bit for bit
    (each 32-block and each GEMM row is its own)."""
    L = get_layer(SMALL[name])
    cfg = L.cfg
    layer = L.layer()
    clean = layer.forward(L.dev["x"]).clone()
    x = L.dev["x"].clone()
    x[3, ::5] = float("nan")
    out = layer.forward(x).clone()
    torch.cuda.synchronize()
    ids = np_(layer.buf["topk_ids"])
    assert ids.min() >= 0 and ids.max() < cfg.E
    assert all(len(set(row)) == cfg.k for row in ids)
    assert int(np_(layer.buf["counts"]).sum()) == cfg.T * cfg.k
    keep = torch.ones(cfg.T, dtype=torch.bool)
    keep[3] = False
    assert torch.equal(out[keep.cuda()], clean[keep.cuda()])


def test_mx_layer_deterministic_and_graph_capture():
    L = get_layer(SMALL["mx_mid"])
    layer = L.layer()
    x = L.dev["x"]
    eager = layer.forward(x).clone()
    assert torch.equal(layer.forward(x), eager)
    out = torch.empty_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward(x, out)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.forward(x, out)
    for i in range(3):
        out.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        layer.forward(x)
        torch.cuda.synchronize()


def test_mx_quantize_zero_rows():
    codes, scales = B.mx_quantize(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"))
    assert codes.shape == (0, 64) and scales.shape == (0, 2)

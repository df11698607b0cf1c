"""Pins of the CPU oracle to things other than itself: hand-worked cases,
library routines, brute force, closed forms and invariants.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import moe, mx

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


# ------------------------------------------------------------ formats ------

def test_bf16_round_matches_torch_cast():
    # fp32 values (exact in fp64) incl. exact ties between bf16 neighbours
    v = (RNG.standard_normal(200000) * np.exp2(RNG.integers(-30, 30, 200000))).astype(np.float32)
    base = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    ulp = np.abs(base) * 2.0 ** -7
    ties = (base.astype(np.float64) + 0.5 * np.exp2(np.floor(np.log2(np.abs(base))) - 7)).astype(np.float32)
    allv = np.concatenate([v, ties, -ties, np.float32([0.0, 1.0, -3.0, 65504.0])])
    ref = torch.from_numpy(allv).to(torch.bfloat16).to(torch.float64).numpy()
    got = mx.bf16_round(allv.astype(np.float64))
    assert np.array_equal(got, ref)
    assert ulp.size  # silence unused


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = mx.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_e2m1_decode_all_codes():
    # the E2M1 grid of the OCP microscaling format
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = mx.e2m1_decode(np.arange(16))
    assert list(got[:8]) == grid
    assert list(got[8:]) == [-g for g in grid]


def test_e8m0_decode():
    assert mx.e8m0_decode([127])[0] == 1.0
    assert mx.e8m0_decode([0])[0] == 2.0 ** -127
    assert mx.e8m0_decode([254])[0] == 2.0 ** 127
    assert np.isnan(mx.e8m0_decode([255])[0])


def test_fp4_unpack_low_nibble_even():
    packed = np.array([[0x21, 0xF0]], dtype=np.uint8)
    assert mx.unpack_fp4(packed, 4).tolist() == [[1, 2, 0, 15]]


def test_e4m3_encode_matches_torch_in_range():
    # in-range values: torch's fp32 -> float8_e4m3fn cast rounds to nearest-even
    mags = np.exp2(RNG.uniform(-12, np.log2(448.0), 300000))
    v = (mags * RNG.choice([-1.0, 1.0], mags.size)).astype(np.float32)
    # exact midpoints between neighbouring E4M3 values (ties)
    allc = np.arange(0, 0x7E, dtype=np.uint8)
    lo = mx.e4m3_decode(allc)
    hi = mx.e4m3_decode(allc + 1)
    mids = ((lo + hi) / 2).astype(np.float32)
    vals = np.concatenate([v, mids, -mids])
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = mx.e4m3_encode_rne(vals.astype(np.float64))
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates():
    got = mx.e4m3_encode_rne(np.array([448.0, 449.0, 480.0, 500.0, 1e6, -600.0]))
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]


def test_mxfp8_handworked_blocks():
    # all ones: floor(log2 1) - 8 = -8 -> scale code 119, elements 256 = 2^8 -> 0x78
    c, s = mx.mxfp8_quantize(np.ones((1, 32)))
    assert s.tolist() == [[119]] and set(c.ravel().tolist()) == {0x78}
    # amax 448 -> shared exp 0 -> scale code 127; 448 -> 0x7E
    b = np.zeros((1, 32)); b[0, 5] = 448.0; b[0, 6] = -1.0
    c, s = mx.mxfp8_quantize(b)
    assert s.tolist() == [[127]] and c[0, 5] == 0x7E and c[0, 6] == 0xB8 and c[0, 0] == 0
    # amax 500 -> floor(log2 500) = 8 -> scale 1 -> 500 clips to 448
    b[0, 5] = 500.0
    c, s = mx.mxfp8_quantize(b)
    assert s.tolist() == [[127]] and c[0, 5] == 0x7E
    # all-zero block -> scale code 0 (2^-127), zero codes
    c, s = mx.mxfp8_quantize(np.zeros((2, 64)))
    assert s.tolist() == [[0, 0], [0, 0]] and not c.any()


def test_mxfp8_roundtrip_error_bound():
    # RNE to 3 mantissa bits: relative error <= 2^-4 in the normal range,
    # absolute error <= 2^-10 * scale in the subnormal range, and the block
    # maximum saturates by at most (512 - 448) / 512.
    x = RNG.standard_normal((64, 256)) * np.exp2(RNG.integers(-20, 20, (64, 1)))
    c, s = mx.mxfp8_quantize(x)
    dq = mx.mxfp8_dequant(c, s)
    scale = np.repeat(mx.e8m0_decode(s), 32, axis=-1)
    q = np.abs(x) / scale
    err = np.abs(dq - x)
    normal = (q >= 2.0 ** -6) & (q <= 448.0)
    assert np.all(err[normal] <= np.abs(x[normal]) * 2.0 ** -4 + 1e-300)
    sub = q < 2.0 ** -6
    assert np.all(err[sub] <= scale[sub] * 2.0 ** -10)
    sat = q > 448.0
    assert np.all(np.abs(dq[sat]) == 448.0 * scale[sat])
    # scale rule: every block's max lands in [256, 512)
    amax = np.abs(x.reshape(64, -1, 32)).max(-1) / mx.e8m0_decode(s)
    assert np.all((amax >= 256) & (amax < 512))


def test_mxfp4_dequant():
    packed = np.array([[0x21] * 16 + [0x7F] * 16], dtype=np.uint8)  # 64 cols
    scales = np.array([[127, 126]], dtype=np.uint8)
    got = mx.mxfp4_dequant(packed, scales, 64)
    assert got[0, 0] == 0.5 and got[0, 1] == 1.0          # codes 1, 2 at scale 1
    assert got[0, 32] == -6.0 * 0.5 and got[0, 33] == 6.0 * 0.5


# ---------------------------------------------------------------- gate -----

def _brute_topk(key_row, k):
    return [e for _, e in sorted((-float(v), e) for e, v in enumerate(key_row))[:k]]


def test_golden_softmax_case():
    g = json.load(open(os.path.join(GOLDEN, "gate_routing_handworked.json")))["softmax"]
    L = np.array(g["logits"], dtype=np.float32)
    ids, w = moe.gate_topk_softmax(L, g["k"])
    assert ids.tolist() == g["ids"]
    a = 1.0 / (1.0 + math.exp(-1.0))
    exp_w = np.array([[a, 1.0 - a], [0.5, 0.5], [0.5, 0.5]], dtype=np.float32)
    np.testing.assert_allclose(w, exp_w, rtol=1e-7)
    counts, offsets, sp, pp = moe.route(ids, 4)
    assert counts.tolist() == g["counts"] and offsets.tolist() == g["offsets"]
    assert sp.tolist() == g["sorted_pair"] and pp.tolist() == g["pair_pos"]


def test_golden_sigmoid_case():
    g = json.load(open(os.path.join(GOLDEN, "gate_routing_handworked.json")))["sigmoid"]
    ids, w = moe.gate_topk_sigmoid(np.array(g["logits"], np.float32), g["k"],
                                   np.array(g["bias"], np.float32), g["routed_scale"])
    assert ids.tolist() == g["ids"]
    s3 = 1.0 / (1.0 + math.exp(-2.0))
    s2 = 1.0 / (1.0 + math.exp(1.0))
    sc = float(np.float32(2.826))
    np.testing.assert_allclose(w[0], [s3 / (s3 + s2) * sc, s2 / (s3 + s2) * sc], rtol=1e-7)


@pytest.mark.parametrize("E,k", [(8, 2), (128, 8), (192, 8), (37, 5), (6, 6)])
def test_topk_softmax_vs_bruteforce(E, k):
    T = 64
    L = RNG.standard_normal((T, E)).astype(np.float32)
    L[:, E // 2] = L[:, 0]           # planted exact ties: lower id must win
    L[5, :] = 0.25                   # a fully tied row: ids 0..k-1
    ids, w = moe.gate_topk_softmax(L, k)
    for t in range(T):
        assert ids[t].tolist() == _brute_topk(L[t], k)
    assert ids[5].tolist() == list(range(k))
    np.testing.assert_allclose(w.astype(np.float64).sum(1), 1.0, atol=1e-6)
    assert np.all(w > 0)


def test_softmax_k_equals_E_is_dense_softmax():
    L = RNG.standard_normal((32, 16)).astype(np.float32)
    ids, w = moe.gate_topk_softmax(L, 16)
    dense = scipy.special.softmax(L.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(dense, ids.astype(np.int64), 1), rtol=1e-6)


def test_softmax_bias_is_added_to_logits():
    L = RNG.standard_normal((16, 8)).astype(np.float32)
    b = RNG.standard_normal(8).astype(np.float32)
    ids, w = moe.gate_topk_softmax(L, 3, b)
    ids2, w2 = moe.gate_topk_softmax(L + b, 3)
    assert np.array_equal(ids, ids2) and np.array_equal(w, w2)


def test_topk_sigmoid_invariants():
    T, E, k = 128, 192, 8
    L = RNG.standard_normal((T, E)).astype(np.float32)
    b = (RNG.standard_normal(E) * 0.1).astype(np.float32)
    ids, w = moe.gate_topk_sigmoid(L, k, b, 2.826)
    s = scipy.special.expit(L.astype(np.float64))
    for t in range(T):
        assert ids[t].tolist() == _brute_topk(s[t] + b.astype(np.float64), k)
    np.testing.assert_allclose(w.astype(np.float64).sum(1), float(np.float32(2.826)), rtol=1e-6)
    assert np.all(w > 0)
    # zero bias: selection is the plain top-k of the logits (sigmoid is monotone)
    ids0, _ = moe.gate_topk_sigmoid(L, k, None, 2.826)
    for t in range(T):
        assert ids0[t].tolist() == _brute_topk(L[t], k)
    # the bias changes selection but never the weight formula
    sel = np.take_along_axis(s, ids.astype(np.int64), 1)
    np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True) * float(np.float32(2.826)), rtol=1e-6)


# ------------------------------------------------------------- routing -----

@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (257, 128, 8), (1000, 192, 8), (3, 4, 4)])
def test_route_vs_stable_argsort(T, E, k):
    # each token's k ids distinct, as top-k produces
    ids = np.stack([RNG.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, sp, pp = moe.route(ids, E)
    flat = ids.reshape(-1)
    assert np.array_equal(sp, np.argsort(flat, kind="stable"))
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(np.sort(sp), np.arange(T * k))          # bijection
    assert np.array_equal(pp[sp], np.arange(T * k))
    for e in range(E):
        seg = sp[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg // k) > 0)                        # ascending tokens


# ---------------------------------------------------------- expert FFN -----

def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def test_ffn_identity_closed_form():
    # gate = up = identity, down = identity: y = bf16(SiLU(x) * x)
    H = 64
    x = _bf16(RNG.standard_normal((7, H)))
    eye = np.eye(H)
    y = moe.expert_ffn(x, np.concatenate([eye, eye]), eye)
    ref = torch.nn.functional.silu(torch.from_numpy(x)) * torch.from_numpy(x)
    np.testing.assert_array_equal(y, mx.bf16_round(ref.numpy()))


def test_ffn_vs_torch_swiglu_mlp():
    # gate rows first, then up (w13 = [gate; up]); torch fp64 on CPU
    H, I, m = 96, 64, 5
    x = _bf16(RNG.standard_normal((m, H)))
    w13 = _bf16(RNG.standard_normal((2 * I, H)) * 0.1)
    w2 = _bf16(RNG.standard_normal((H, I)) * 0.1)
    tx, t13, t2 = (torch.from_numpy(a) for a in (x, w13, w2))
    a = torch.nn.functional.silu(torch.nn.functional.linear(tx, t13[:I])) * \
        torch.nn.functional.linear(tx, t13[I:])
    a = torch.from_numpy(mx.bf16_round(a.numpy()))
    ref = torch.nn.functional.linear(a, t2).numpy()
    np.testing.assert_allclose(moe.expert_ffn(x, w13, w2), ref, rtol=1e-12, atol=1e-12)
    # swapping gate and up must change the result (the split order matters)
    swapped = np.concatenate([w13[I:], w13[:I]])
    assert np.abs(moe.expert_ffn(x, swapped, w2) - ref).max() > 1e-3


# -------------------------------------------------------------- layer ------

def _tiny_layer(T, H, E, k, I, scale_w=0.1, shared=False):
    x = _bf16(RNG.standard_normal((T, H)))
    wr = (RNG.standard_normal((E, H)) * 0.1).astype(np.float32)
    W = [(_bf16(RNG.standard_normal((2 * I, H)) * scale_w), _bf16(RNG.standard_normal((H, I)) * scale_w))
         for _ in range(E)]
    sh = (_bf16(RNG.standard_normal((2 * I, H)) * scale_w), _bf16(RNG.standard_normal((H, I)) * scale_w)) if shared else None
    return x, wr, W, sh


def _dense_masked(x, wr, W, k, mode, bias=None, scale=1.0, sh=None):
    """Brute force: every expert on every token, multiplied by a dense
    [T, E] weight matrix that is zero off the selected experts."""
    T = x.shape[0]
    E = len(W)
    L = (x @ wr.astype(np.float64).T).astype(np.float32)
    Lk = L.astype(np.float64)
    if mode == "softmax":
        key = (L + (0 if bias is None else bias)).astype(np.float32).astype(np.float64)
    else:
        s = scipy.special.expit(Lk)
        key = s + (0 if bias is None else bias.astype(np.float64))
    M = np.zeros((T, E))
    for t in range(T):
        sel = _brute_topk(key[t], k)
        if mode == "softmax":
            z = np.exp(key[t, sel] - key[t, sel].max())
            M[t, sel] = (z / z.sum()).astype(np.float32)
        else:
            M[t, sel] = (s[t, sel] / s[t, sel].sum() * float(np.float32(scale))).astype(np.float32)
    out = np.zeros((T, x.shape[1]))
    for e in range(E):
        w13, w2 = W[e]
        I = w13.shape[0] // 2
        for t in range(T):
            g = w13[:I] @ x[t]
            u = w13[I:] @ x[t]
            a = mx.bf16_round(g / (1 + np.exp(-g)) * u)
            out[t] += M[t, e] * (w2 @ a)
    if sh is not None:
        w13, w2 = sh
        I = w13.shape[0] // 2
        for t in range(T):
            g = w13[:I] @ x[t]
            u = w13[I:] @ x[t]
            out[t] += w2 @ mx.bf16_round(g / (1 + np.exp(-g)) * u)
    return mx.bf16_round(out)


@pytest.mark.parametrize("mode", ["softmax", "sigmoid"])
def test_layer_vs_dense_masked_bruteforce(mode):
    T, H, E, k, I = 12, 32, 6, 2, 16
    x, wr, W, sh = _tiny_layer(T, H, E, k, I, shared=(mode == "sigmoid"))
    bias = (RNG.standard_normal(E) * 0.1).astype(np.float32) if mode == "sigmoid" else None
    res = moe.layer_forward(x, wr, k, mode, lambda e: W[e], E, bias=bias,
                            routed_scale=2.826 if mode == "sigmoid" else 1.0, shared_weights=sh)
    ref = _dense_masked(x, wr, W, k, mode, bias, 2.826, sh)
    # identical up to fp64 summation order -> equal after bf16 rounding except
    # at rare rounding boundaries
    d = np.abs(res["out"] - ref)
    assert np.mean(d == 0) > 0.98
    assert d.max() <= 2.0 ** -7 * np.abs(ref).max()


@pytest.mark.parametrize("mode,scale", [("softmax", 1.0), ("sigmoid", 2.826)])
def test_identical_experts_independent_of_routing(mode, scale):
    T, H, E, k, I = 10, 32, 5, 3, 16
    x, wr, W, _ = _tiny_layer(T, H, E, k, I)
    W = [W[0]] * E
    res = moe.layer_forward(x, wr, k, mode, lambda e: W[e], E, routed_scale=scale)
    single = moe.expert_ffn(x, *W[0]) * float(np.float32(scale))
    d = np.abs(res["out"] - mx.bf16_round(single))
    assert d.max() <= 2.0 ** -7 * np.abs(single).max()


def test_layer_token_subset_matches_full():
    T, H, E, k, I = 20, 32, 6, 2, 16
    x, wr, W, sh = _tiny_layer(T, H, E, k, I, shared=True)
    full = moe.layer_forward(x, wr, k, "softmax", lambda e: W[e], E, shared_weights=sh)
    sub = moe.layer_forward(x, wr, k, "softmax", lambda e: W[e], E, shared_weights=sh, tokens=[3, 0, 19])
    assert np.array_equal(sub["out"], full["out"][[3, 0, 19]])


def test_router_logits_exact_small_integers():
    # small-integer inputs: every fp64 partial sum is exact
    x = RNG.integers(-4, 5, (9, 40)).astype(np.float64)
    wr = RNG.integers(-3, 4, (7, 40)).astype(np.float32)
    exact = np.einsum("th,eh->te", x.astype(np.int64), wr.astype(np.int64))
    assert np.array_equal(moe.router_logits(x, wr), exact.astype(np.float32))


def test_w4a8_layer_path_quantises_x_and_activation():
    # with x already on the MXFP8 grid and w13, w2 decoded exactly, the only
    # difference from the bf16 layer is the activation quantisation: bounded
    T, H, E, k, I = 8, 64, 4, 2, 32
    x, wr, W, _ = _tiny_layer(T, H, E, k, I)
    res8 = moe.layer_forward(x, wr, k, "softmax", lambda e: W[e], E, fmt="w4a8")
    xq = mx.mxfp8_dequant(*mx.mxfp8_quantize(x))
    assert np.array_equal(res8["x_used"], xq)
    res16 = moe.layer_forward(xq, wr, k, "softmax", lambda e: W[e], E, logits=res8["logits"])
    d = np.abs(res8["out"] - res16["out"])
    assert d.max() <= 0.15 * np.abs(res16["out"]).max()
    assert d.max() > 0   # the activation really was requantised


# ------------------------------------------- W4A8 quantisation points ------

def _quant_points():
    with open(os.path.join(GOLDEN, "w4a8_quant_points_handworked.json")) as f:
        return json.load(f)


def test_w4a8_swiglu_output_quantised_as_one_value():
    """Hand-worked: the SwiGLU output a = SiLU(g) * u is quantised to MXFP8
    along I as one value (not g and u apart, not after a bf16 rounding)."""
    case = _quant_points()["swiglu_output"]
    I, H = 32, 33
    w13 = np.zeros((2 * I, H))
    w13[:I, 32] = 48.0                 # gate: g_j = 48 * x_32 = 48
    w13[I:, :I] = np.eye(I)            # up:   u_j = p_j
    w2 = np.zeros((H, I))
    w2[:I] = np.eye(I)
    assert float(moe.silu(48.0)) == 48.0
    for row in case["rows"]:
        x = np.zeros((1, H))
        x[0, :len(row["p"])] = row["p"]
        x[0, 32] = 1.0
        y = moe.expert_ffn(x, w13, w2, act="mxfp8")
        want = np.zeros(H)
        want[:len(row["y"])] = row["y"]
        np.testing.assert_array_equal(y[0], want)


def test_w4a8_shared_expert_runs_on_quantised_x():
    """Hand-worked: in the W4A8 layer the shared expert takes the MXFP8 x,
    as the routed experts do; zero routed experts leave only its row."""
    case = _quant_points()["shared_on_quantised_x"]
    H, I, E = 64, 32, 2
    zero = (np.zeros((2 * I, H)), np.zeros((H, I)))
    s13 = np.zeros((2 * I, H))
    s13[:I, 32] = 48.0
    s13[I:, :I] = np.eye(I)
    s2 = np.zeros((H, I))
    s2[:I] = np.eye(I)
    rows = case["rows"]
    x = np.zeros((len(rows), H))
    for t, row in enumerate(rows):
        x[t, :len(row["p"])] = row["p"]
        x[t, 32] = 1.0
    wr = np.zeros((E, H), dtype=np.float32)
    res = moe.layer_forward(x, wr, 1, "softmax", lambda e: zero, E, shared_weights=(s13, s2), fmt="w4a8")
    assert res["ids"].ravel().tolist() == [0] * len(rows)   # tied logits -> lower id
    for t, row in enumerate(rows):
        want = np.zeros(H)
        want[:len(row["out"])] = row["out"]
        np.testing.assert_array_equal(res["out"][t], want)


def test_bf16_round_subnormals():
    """The bf16 subnormal range (|a| < 2^-126, grid q = 2^-133): hand-worked
    ties to even, the carry into the smallest normal, and fp32-exact random
    values against torch's bf16 cast."""
    q = 2.0 ** -133
    cases = {1.0: 1.0, 1.5: 2.0, 2.5: 2.0, 0.5: 0.0, 0.75: 1.0, 0.25: 0.0, 126.5: 126.0,
             127.5: 128.0, -3.5: -4.0, 3.25: 3.0}
    got = mx.bf16_round(np.array(list(cases)) * q)
    np.testing.assert_array_equal(got, np.array(list(cases.values())) * q)
    assert mx.bf16_round(np.array([127.5 * q]))[0] == 2.0 ** -126
    # random magnitudes in [2^-149, 2^-126): fp32 subnormals and small
    # normals, exact in fp32 and fp64, so torch's cast rounds them once
    mags = np.exp2(RNG.uniform(-149, -126, 100000)).astype(np.float32)
    v = mags * RNG.choice([-1.0, 1.0], mags.size).astype(np.float32)
    v = v[np.abs(v) < np.float32(2.0 ** -126)]
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(mx.bf16_round(v.astype(np.float64)), ref)
    assert np.any(ref != 0) and np.any(np.abs(ref) < 2.0 ** -126)


def test_mxfp8_quantize_at_given_exponents():
    """Quantising at exponents decided elsewhere: the rule's own exponents
    reproduce the default; a block whose exact maximum 3.99999557 sits just
    below 4 takes exponent floor(log2) - 8 = -7, so that element scales to
    511.9994 and saturates to 448 (3.5), while at exponent -6 it rounds to
    256 (4.0) (hand-worked)."""
    x = RNG.standard_normal((3, 64))
    c0, s0 = mx.mxfp8_quantize(x)
    c1, s1 = mx.mxfp8_quantize(x, s0.astype(np.int64) - 127)
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1)
    b = np.zeros((1, 32))
    b[0, 0] = 3.99999557
    b[0, 1] = 1.0
    c, s = mx.mxfp8_quantize(b)
    assert s.tolist() == [[120]]
    assert mx.mxfp8_dequant(c, s)[0, :2].tolist() == [3.5, 1.0]
    c, s = mx.mxfp8_quantize(b, np.array([[-6]]))
    assert s.tolist() == [[121]]
    assert mx.mxfp8_dequant(c, s)[0, :2].tolist() == [4.0, 1.0]

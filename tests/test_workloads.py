"""The seeded input generators: deterministic, per-tensor seeds, shapes."""
import torch

from expert_routing_grouped_gate_amd import workloads as W


def test_deterministic_and_independent():
    c = W.CONFIGS["tiny"]
    assert torch.equal(W.draw_x(c), W.draw_x(c))
    a13, a2 = W.draw_expert_bf16(c, 3)
    b13, b2 = W.draw_expert_bf16(c, 3)
    assert torch.equal(a13, b13) and torch.equal(a2, b2)
    o13, _ = W.draw_expert_bf16(c, 4)
    assert not torch.equal(a13, o13)
    assert a13.shape == (2 * c.I, c.H) and a2.shape == (c.H, c.I)
    assert a13.dtype == torch.bfloat16


def test_distributions():
    c = W.CONFIGS["tiny"].with_(T=256)
    x = W.draw_x(c).float()
    assert abs(x.std().item() - 1.0) < 0.02
    w13, _ = W.draw_expert_bf16(c, 0)
    assert abs(w13.float().std().item() - 0.02) < 0.001
    assert W.draw_bias(c) is None
    hy = W.CONFIGS["hy3"].with_(T=4, H=64, I=32, shared_I=32)
    b = W.draw_bias(hy)
    assert b.shape == (hy.E,) and abs(b.std().item() - 0.1) < 0.03
    z = W.draw_bias(W.CONFIGS["qwen3_decode_w4a8"])
    assert torch.all(z[1:] < z[:-1])     # Zipf: expert 0 most popular


def test_mx_weights_shapes_and_codes():
    c = W.CONFIGS["qwen3_decode_w4a8"].with_(H=256, I=128)
    c13, s13, c2, s2 = W.draw_expert_mx(c, 0)
    assert c13.shape == (256, 128) and s13.shape == (256, 8)
    assert c2.shape == (256, 64) and s2.shape == (256, 4)
    assert set(torch.unique(s13).tolist()) <= {119, 120, 121}
    assert c13.dtype == torch.uint8


def test_mx_shared_expert_drawn_with_layer():
    c = W.CONFIGS["qwen3_decode_w4a8"].with_(T=2, H=256, E=4, I=128, shared_I=128)
    t = W.draw_layer(c)
    assert t["shared_w13"].shape == (256, 128) and t["shared_w13_scales"].shape == (256, 8)
    assert t["shared_w2"].shape == (256, 64) and t["shared_w2_scales"].shape == (256, 4)
    c13, _, _, _ = W.draw_expert_mx(c, 0)
    assert not torch.equal(t["shared_w13"], c13)   # its own stream, not expert 0's


def test_mx_wide_scales_span_the_range():
    narrow = W.CONFIGS["qwen3_decode_w4a8"].with_(H=256, I=128)
    wide = narrow.with_(mx_scales="wide")
    c13n, s13n, _, _ = W.draw_expert_mx(narrow, 0)
    c13w, s13w, _, s2w = W.draw_expert_mx(wide, 0)
    assert torch.equal(c13n, c13w)                 # same element codes, other scales
    u = set(torch.unique(torch.cat([s13w.ravel(), s2w.ravel()])).tolist())
    assert min(u) == 100 and max(u) == 140 and len(u) == 41


def test_mid_size_configs_share_the_decode_weights():
    for T in (64, 128, 256, 320, 512, 1024):
        c = W.CONFIGS[f"qwen3_T{T}"]
        assert c.T == T and c.family_seed == W.CONFIGS["qwen3_decode"].family_seed
        assert (c.H, c.E, c.k, c.I) == (4096, 128, 8, 1536)
    for T in (64, 128, 256, 512, 1024):
        c = W.CONFIGS[f"qwen3_w4a8_T{T}"]
        d = W.CONFIGS["qwen3_decode_w4a8"]
        assert c.T == T and (c.family_seed, c.fmt, c.bias) == (d.family_seed, d.fmt, d.bias)
        assert (c.H, c.E, c.k, c.I) == (4096, 128, 8, 1536)


def test_hy3_decode_shares_the_hy3_weights():
    c, h = W.CONFIGS["hy3_decode"], W.CONFIGS["hy3"]
    assert c.T == 16 and c.x_seed != h.x_seed
    assert (c.H, c.E, c.k, c.I, c.shared_I, c.gate, c.bias, c.family_seed) == \
        (h.H, h.E, h.k, h.I, h.shared_I, h.gate, h.bias, h.family_seed)

"""The no-allocation layer entry point (moe_layer_forward_noalloc): the same
layer as moe_layer_forward with the library's static scratch in place of the
caller's workspace.  Through the C ABI, every output of two calls in a row
(the second with fewer tokens, so the scratch holds the first call's data
when the second starts) must equal moe_layer_forward's bit for bit: the same
kernels run over the same inputs.  The shapes use the scratch for the
router's K-split partial tiles and the routing histograms (700 tokens) and
for the few-token router partials (9 tokens)."""
import pytest
import torch

from expert_routing_grouped_gate_amd import binding as B
from expert_routing_grouped_gate_amd import workloads as W
from tests.layer_fixtures import get_layer

pytestmark = pytest.mark.gpu

KEYS = ("logits", "topk_ids", "topk_w", "counts", "offsets", "sorted_pair", "pair_pos", "act", "y")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    B.load()


def _pair(cfg, T):
    L = get_layer(cfg)
    x = L.dev["x"][:T].contiguous()
    ref_layer, na_layer = L.layer(), L.layer()
    ref_out = ref_layer.forward(x)
    assert ref_layer.buf["workspace"].numel() > 16, "shape must use the workspace"
    na_out = na_layer.forward_noalloc(x)
    torch.cuda.synchronize()
    return ref_layer, ref_out, na_layer, na_out


@pytest.mark.parametrize("name,cfg,Ts", [
    ("softmax", W.CONFIGS["tiny"].with_(name="na_softmax", T=700, E=8, k=2, x_seed=51), (700, 300, 9)),
    ("sigmoid_shared", W.CONFIGS["hy3"].with_(name="na_hy3", T=600, H=512, E=16, k=4, I=384, shared_I=384,
                                              x_seed=52, family_seed=1052), (600, 130, 16)),
])
def test_noalloc_equals_layer_forward(name, cfg, Ts):
    for T in Ts:                       # two or more calls in a row, each smaller
        ref_layer, ref_out, na_layer, na_out = _pair(cfg, T)
        assert torch.equal(na_out, ref_out), f"{name} T={T} out"
        for key in KEYS + (("shared_y",) if cfg.shared_I else ()):
            assert torch.equal(na_layer.buf[key], ref_layer.buf[key]), f"{name} T={T} {key}"
        assert int(na_layer.buf["dev_status"][0]) == 0

"""Host-side logic of bench.py: the algorithmic bytes and flops that the
roofline fractions divide by, pinned to figures derived by hand from the
layer shapes (expert weight sizes, router weight, x in and out, 2 flops per
multiply-add of the three expert projections), and the refusal of more than
one GPU.  No GPU needed."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from expert_routing_grouped_gate_amd import workloads as W  # noqa: E402


def counts_touching(E, n):
    c = np.zeros(E, dtype=np.int32)
    c[:n] = 1
    return c


def test_bf16_decode_bytes():
    # per expert: w13 2 x 1536 x 4096 bf16 + w2 4096 x 1536 bf16 = 37,748,736 B;
    # plus the fp32 router weight (2 MiB) and x in + out (2 x 16 x 4096 x 2 B)
    w = bench.workload_bytes_flops(W.CONFIGS["qwen3_decode"], counts_touching(128, 80))
    assert w["n_touched"] == 80
    assert w["layer_bytes"] == 80 * 37_748_736 + 128 * 4096 * 4 + 2 * 16 * 4096 * 2
    assert w["flops"] == 2 * 16 * 8 * 3 * 1536 * 4096          # 4.83 GFLOP
    # GEMM1: the touched w13 slices, x, and the bf16 activations it writes
    assert w["g1_bytes"] == 80 * 25_165_824 + 16 * 4096 * 2 + 16 * 8 * 1536 * 2
    assert w["g1_flops"] == 2 * 16 * 8 * 2 * 1536 * 4096


def test_prefill_flops():
    w = bench.workload_bytes_flops(W.CONFIGS["qwen3_prefill"], counts_touching(128, 128))
    assert w["flops"] == 1_236_950_581_248                         # 1.2370 TFLOP
    assert w["g1_flops"] == 824_633_720_832                         # 824.6 GFLOP
    assert w["layer_bytes"] == 128 * 37_748_736 + 128 * 4096 * 4 + 2 * 4096 * 4096 * 2


def test_hy3_adds_the_shared_expert_and_bias():
    w = bench.workload_bytes_flops(W.CONFIGS["hy3"], counts_touching(192, 155))
    shared = 3 * 1536 * 4096 * 2
    assert w["layer_bytes"] == (155 * 37_748_736 + shared + 192 * 4096 * 4 + 192 * 4
                                + 2 * 4096 * 4096 * 2)
    assert w["flops"] == 1_236_950_581_248 + 2 * 4096 * 3 * 1536 * 4096   # 1.3916 TFLOP
    # the shared expert runs inside the GEMM1 launch: its w13 (2 x 1536 x 4096
    # bf16) is read, its 4096 x 1536 bf16 activations written, its flops done
    assert w["g1_shared"]
    assert w["g1_bytes"] == (155 * 25_165_824 + 4096 * 4096 * 2 + 4096 * 8 * 1536 * 2
                             + 25_165_824 + 4096 * 1536 * 2)
    assert w["g1_flops"] == 824_633_720_832 + 2 * 4096 * 2 * 1536 * 4096
    # not folded: at most 16 tokens (streaming GEMMs), or no shared expert
    assert not bench.workload_bytes_flops(W.CONFIGS["hy3"].with_(T=16), counts_touching(192, 80))["g1_shared"]
    assert not bench.workload_bytes_flops(W.CONFIGS["qwen3_prefill"], counts_touching(128, 128))["g1_shared"]


def test_w4a8_bytes():
    # per expert: E2M1 codes (half a byte each) + one E8M0 scale per 32 values:
    # w13 6,291,456 + 393,216 B, w2 3,145,728 + 196,608 B = 10,027,008 B
    cfg = W.CONFIGS["qwen3_decode_w4a8"]
    w = bench.workload_bytes_flops(cfg, counts_touching(128, 42))
    assert w["layer_bytes"] == 42 * 10_027_008 + 128 * 4096 * 4 + 128 * 4 + 2 * 16 * 4096 * 2
    # GEMM1 writes MXFP8 activations: one byte per value + one scale per 32
    assert w["g1_bytes"] == 42 * (6_291_456 + 393_216) + 16 * 4096 * 2 + 16 * 8 * (1536 + 48)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_gemm1_traffic_is_keyed_to_the_config_and_its_sources(tmp_path, monkeypatch):
    assert bench.gemm1_family(W.CONFIGS["hy3"]) == "bf16_tiled"
    assert bench.gemm1_family(W.CONFIGS["qwen3_decode"]) == "bf16_stream"
    assert bench.gemm1_family(W.CONFIGS["qwen3_decode_w4a8"]) == "w4a8_stream"
    assert bench.gemm1_family(W.CONFIGS["qwen3_prefill_w4a8"]) == "w4a8_tiled"
    # the library's switch: bf16 above 3 rows per expert (T > 48 at E = 128,
    # top-8), W4A8 above 8 (T > 128), bf16 with a foldable shared expert above
    # 16 tokens
    assert bench.gemm1_family(W.CONFIGS["qwen3_decode"].with_(T=48)) == "bf16_stream"
    assert bench.gemm1_family(W.CONFIGS["qwen3_decode"].with_(T=56)) == "bf16_tiled"
    assert bench.gemm1_family(W.CONFIGS["qwen3_decode_w4a8"].with_(T=128)) == "w4a8_stream"
    assert bench.gemm1_family(W.CONFIGS["qwen3_decode_w4a8"].with_(T=136)) == "w4a8_tiled"
    assert bench.gemm1_family(W.CONFIGS["hy3"].with_(T=16)) == "bf16_stream"
    assert bench.gemm1_family(W.CONFIGS["hy3"].with_(T=17)) == "bf16_tiled"
    cfg = W.CONFIGS["hy3"]
    md = tmp_path / "hbm_counters_hy3.md"
    monkeypatch.setattr(bench, "counters_md", lambda name: str(tmp_path / f"hbm_counters_{name}.md"))
    assert bench.measured_gemm1_traffic(cfg) is None                     # no summary
    h = bench.gemm1_source_hash("bf16_tiled")
    md.write_text(f"kernel_source_sha256_16: {h}\nkernel_read_bytes: 1000\nkernel_write_bytes: 24\n")
    assert bench.measured_gemm1_traffic(cfg) == 1024
    md.write_text("kernel_source_sha256_16: 0000000000000000\nkernel_read_bytes: 1000\nkernel_write_bytes: 24\n")
    assert bench.measured_gemm1_traffic(cfg) is None                     # taken on other sources
    assert h != bench.gemm1_source_hash("bf16_stream")
    # the norm configs grade their one kernel, keyed to the norm sources
    assert bench.graded_kernel("combine_add_rmsnorm")[1] == "combine_add_rmsnorm_kernel"
    hn = bench.source_hash(bench.graded_kernel("add_rmsnorm")[0])
    (tmp_path / "hbm_counters_add_rmsnorm.md").write_text(
        f"kernel_source_sha256_16: {hn}\nkernel_read_bytes: 7\nkernel_write_bytes: 3\n")
    assert bench.measured_traffic("add_rmsnorm") == 10


def test_host_cpu_model_is_named():
    assert isinstance(bench.host_cpu_model(), str) and bench.host_cpu_model()

"""bench.py host logic on the CPU: the algorithmic byte and FLOP counts behind the roofline
fraction (hand-computed values), the counter-table lookup behind `traffic`, and the one-GPU
guard."""
import importlib.util
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


# T = 4 tokens, d = 256, E = 8, k = 2, H = 512: rows = 8; experts 1, 3 and 6 touched
SHAPE = dict(T=4, d=256, E=8, k=2, H=512)
COUNTS = np.array([0, 3, 0, 4, 0, 0, 1, 0])


def _inp(dtype):
    return SimpleNamespace(dtype=dtype, **SHAPE)


def test_algorithmic_bf16(bench):
    a = bench.algorithmic(_inp("bf16"), COUNTS)
    assert a["touched"] == 3
    # gate/up kernel: 3 experts x (gate + up) x 512 x 256 bf16 = 1572864 B, 8 gathered x rows of
    # 256 bf16 = 4096 B, 8 h rows of 512 bf16 = 8192 B
    assert a["gu_bytes"] == 1572864 + 4096 + 8192
    assert a["gu_flops"] == 4 * 256 * 512 * 8 == 4194304
    # whole step: 3 x 3 matrices = 2359296 B, x 2048 B, router 4096 B, fp32 y 4096 B,
    # ids + weights 64 B
    assert a["step_bytes"] == 2359296 + 2048 + 4096 + 4096 + 64
    assert a["step_flops"] == 6 * 256 * 512 * 8 + 2 * 4 * 256 * 8


def test_algorithmic_int8(bench):
    a = bench.algorithmic(_inp("bf16"), COUNTS, "int8")
    # one byte per weight (786432 B) + one fp32 scale per gate and up row (3 x 1024 x 4 B)
    assert a["gu_bytes"] == 786432 + 12288 + 4096 + 8192
    # three matrices (1179648 B) + scales of the gate, up and down rows (3 x 1280 x 4 B)
    assert a["step_bytes"] == 1179648 + 15360 + 2048 + 4096 + 4096 + 64


def test_algorithmic_q4(bench):
    a = bench.algorithmic(_inp("bf16"), COUNTS, "q4")
    # 786432 weights: half a byte each (393216 B) + a 4-byte (scale, bias) pair per 64 weights
    # (12288 pairs, 49152 B)
    assert a["gu_bytes"] == 393216 + 49152 + 4096 + 8192


def test_algorithmic_fragment_major_equals_row_major(bench):
    # the fragment-major orders move exactly the bytes of the storage they reorder
    for frag, base in (("frag", "native"), ("int8-frag", "int8"), ("q4-frag", "q4")):
        assert bench.algorithmic(_inp("bf16"), COUNTS, frag) == \
            bench.algorithmic(_inp("bf16"), COUNTS, base)


def test_algorithmic_fp32(bench):
    a = bench.algorithmic(_inp("f32"), COUNTS)
    assert a["gu_bytes"] == 2 * 1572864 + 2 * 4096 + 2 * 8192


def test_measured_traffic_lookup(bench, tmp_path, monkeypatch):
    h = bench.kernel_source_hash()
    table = tmp_path / "traffic.md"
    table.write_text(
        "| kernel | workload | src | FETCH_SIZE KiB | WRITE_SIZE KiB | fetch scale | write scale |\n"
        "|---|---|---|---|---|---|---|\n"
        f"| k_a | w1 | {h} | 100.0 | 10.0 | 2.0 | 1.0 |\n"
        "| k_b | w1 | 0000000000000000 | 100.0 | 10.0 | 2.0 | 1.0 |\n")
    monkeypatch.setattr(bench, "TRAFFIC_TABLE", str(table))
    assert bench.measured_traffic("k_a", "w1") == (100.0 * 2.0 + 10.0) * 1024.0
    assert bench.measured_traffic("k_b", "w1") is None   # counters of another kernel source
    assert bench.measured_traffic("k_a", "w2") is None   # no row


def test_committed_traffic_table_parses(bench):
    """Every data row of the committed table has the seven cells the lookup reads."""
    with open(bench.TRAFFIC_TABLE) as f:
        rows = [l for l in f if l.startswith("| ") and not l.startswith("| kernel")]
    assert rows
    for line in rows:
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        assert len(cells) == 7, line
        assert len(cells[2]) == 16
        [float(c) for c in cells[3:7]]


def test_traffic_table_names_the_kernels_the_bench_reports(bench):
    """Each bf16 workload's dominant kernel, as bench.py names it, has a row in the committed
    table for that workload (a renamed kernel would otherwise leave `traffic` null)."""
    from expert_routing_grouped_moe_amd import inputs as gen
    with open(bench.TRAFFIC_TABLE) as f:
        keys = {tuple(c.strip() for c in l.strip().strip("|").split("|")[:2])
                for l in f if l.startswith("| ") and not l.startswith("| kernel")}
    for name in ("zonos2-skewed-prefill", "zonos3mini-prefill", "zonos2-decode",
                 "zonos3mini-decode-cfg"):
        wl = gen.WORKLOADS[name]
        inp = SimpleNamespace(dtype="bf16", T=wl.T, d=wl.d, E=wl.E, k=wl.k, H=wl.H)
        assert (bench.dominant_kernel(inp), name) in keys, name
    wl = gen.WORKLOADS["zonos3mini-prefill"]
    inp = SimpleNamespace(dtype="bf16", T=wl.T, d=wl.d, E=wl.E, k=wl.k, H=wl.H)
    assert (bench.dominant_kernel(inp, "frag"), "zonos3mini-prefill/frag") in keys


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"] and msg["n_gpus"] == 2


def test_spread(bench):
    s = bench._spread([0.5, 0.1, 0.4, 0.2, 0.3])      # ms, unordered
    assert s["median"] == pytest.approx(300.0) and s["n"] == 5
    assert s["p10"] == pytest.approx(100.0) and s["p90"] == pytest.approx(500.0)


def test_kernel_hash_ignores_comments_only(bench):
    a = "int f(int x) { // doubles\n  return 2 * x; /* fast */ }\n"
    b = "int f(int x) {\n  /* twice x */\n  return 2 * x;\n}\n"
    c = "int f(int x) { return 3 * x; }\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)


def test_dominant_kernel_names(bench):
    mk = lambda T, d, E, k, H, dt="bf16": SimpleNamespace(T=T, d=d, E=E, k=k, H=H, dtype=dt)
    # decode shapes: the weight-streaming gate/up kernel, two-group passes while (H/16)*E <= 2048
    # (2816 / 16) * 16 = 2816 blocks: one-group passes; (512 / 16) * 64 = 2048: two-group passes
    assert bench.dominant_kernel(mk(64, 2048, 16, 1, 2816)) == "ffn_stream_kernel<true, 1, 0>"
    assert bench.dominant_kernel(mk(64, 1024, 64, 2, 512)) == "ffn_stream_kernel<true, 2, 0>"
    assert bench.dominant_kernel(mk(64, 1024, 64, 2, 512), "q4") == "ffn_stream_kernel<true, 2, 2>"
    # fragment-major: the weight-format template argument carries the order flag (4)
    assert bench.dominant_kernel(mk(64, 2048, 16, 1, 2816), "frag") == "ffn_stream_kernel<true, 1, 4>"
    assert bench.dominant_kernel(mk(64, 2048, 16, 1, 2816), "int8-frag") == "ffn_stream_kernel<true, 1, 5>"
    assert bench.dominant_kernel(mk(64, 1024, 64, 2, 512), "q4-frag") == "ffn_stream_kernel<true, 2, 6>"
    # prefill shapes: the grouped GEMM, wide tiles once experts average 256 rows
    assert bench.dominant_kernel(mk(8192, 2048, 16, 1, 2816)) == \
        "gemm_dma_kernel<true, 256, 256, 2, 64, 64, false>"
    assert bench.dominant_kernel(mk(8192, 2048, 16, 1, 2816), "frag") == \
        "gemm_dma_kernel<true, 256, 256, 2, 64, 64, true>"
    assert bench.dominant_kernel(mk(4096, 1024, 64, 2, 512)).startswith("gemm_dma_kernel<true, 128, 256")
    assert bench.dominant_kernel(mk(64, 128, 8, 1, 256, "f32")) == "ffn_f32_kernel<true>"


def test_bench_defaults_headline_the_skewed_prefill(bench):
    assert bench.HEADLINE == "zonos2-skewed-prefill"
    assert bench.FIVE[-1] == bench.HEADLINE and len(bench.FIVE) == 5

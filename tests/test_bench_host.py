"""Host logic of the benchmark, on the CPU: its refusal of more than one GPU, the
algorithmic work that the roofline fraction divides by (per-unit figures times
units, written out here from the workload shapes), and the rule that the counter
record is used only for the kernel sources it was taken on."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_several_gpus_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2, r
    assert "one GPU" in r.stderr
    assert r.stdout == ""


# (workload, algorithmic bytes per unit, units per launch, flop per unit,
#  bytes per unit as launched (o in the launch's dtype), final-state bytes)
CHUNK_WORK = [
    # normalized d64: q, k, v, o bf16; launched with o in fp32
    ("normalized_bf16_b8h16_l2048_d64", (3 * 64 + 64) * 2, 8 * 16 * 2048, 2 * 64 * (64 + 64) + 4 * 64 * 64,
     3 * 64 * 2 + 64 * 4, 8 * 16 * 64 * 64 * 4),
    # decay d128: + one fp32 log-gate per token; launched with o in bf16
    ("decay_bf16_b4h32_l8192_d128", 4 * 128 * 2 + 4, 4 * 32 * 8192, 2 * 64 * 256 + 4 * 128 * 128,
     4 * 128 * 2 + 4, 4 * 32 * 128 * 128 * 4),
    # vector decay d128: + one fp32 log-gate per token and key channel
    ("vector_decay_bf16_b4h32_l8192_d128", 4 * 128 * 2 + 128 * 4, 4 * 32 * 8192, 2 * 64 * 256 + 4 * 128 * 128,
     3 * 128 * 2 + 128 * 4 + 128 * 4, 4 * 32 * 128 * 128 * 4),
    # gated delta d128: + log-gate and beta per token
    ("gated_delta_bf16_b2h16_l8192_d128", 4 * 128 * 2 + 4 + 4, 2 * 16 * 8192,
     (2 * 64 * 64 * (3 * 128 + 2 * 128) + 6 * 64 * 128 * 128 + 64 ** 3 / 3) / 64,
     3 * 128 * 2 + 128 * 4 + 4 + 4, 2 * 16 * 128 * 128 * 4),
]


@pytest.mark.parametrize("name,per_unit,units,flop_unit,launched_unit,state", CHUNK_WORK)
def test_chunk_work(name, per_unit, units, flop_unit, launched_unit, state):
    flop, nbytes, launched = bench.chunk_work(W.CONFIGS[name])
    assert nbytes == per_unit * units
    assert launched == launched_unit * units + state
    assert flop == pytest.approx(flop_unit * units, rel=1e-12)


def test_headline_is_the_largest_single_gpu_workload_with_algorithmic_bytes():
    # decay B4 H32 L8192 d128: q, k, v, o bf16 (1,073,741,824 B) + fp32 log-gates (4 MiB)
    assert bench.HEADLINE == "decay_bf16_b4h32_l8192_d128"
    assert bench.chunk_work(W.CONFIGS[bench.HEADLINE])[1] == 1_077_936_128
    # the normalized workload: q, k, v, o bf16 = 134.2 MB
    assert bench.chunk_work(W.CONFIGS["normalized_bf16_b8h16_l2048_d64"])[1] == 134_217_728


def test_decode_work():
    # per sequence-head: the fp32 128 x 128 state read and written, q, k, v in
    # bf16, the gate, and o in bf16
    flop, nbytes = bench.decode_work(W.CONFIGS["decode_decay_bf16_n512h32_d128"])
    assert nbytes == 512 * 32 * (2 * 128 * 128 * 4 + 3 * 128 * 2 + 4 + 128 * 2) == 2_164_326_400
    assert flop == 5 * 128 * 128 * 512 * 32


def test_conv_work():
    c = W.CONFIGS["short_conv_qkv_bf16_b2h16_l8192_d128_k4"]
    flop, nbytes = bench.conv_work(c)
    elems = 2 * 16 * 8192 * 3 * 128
    assert nbytes == 2 * elems * 2 + 16 * 3 * 128 * 4 * 4
    assert flop == 2 * 4 * elems


def test_counter_record_follows_code_not_comments(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("// a kernel\nint f(int x) {\n    return x + 1;  // one more\n}\n")
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    h0 = bench.kernel_source_hash()
    src.write_text("/* another comment */\nint f(int x) {\n\n    return x + 1;\n}\n")
    assert bench.kernel_source_hash() == h0
    src.write_text("int f(int x) {\n    return x + 2;\n}\n")
    assert bench.kernel_source_hash() != h0


def test_traffic_null_for_other_sources(monkeypatch):
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "not-the-profiled-sources")
    assert bench.traffic_for(bench.HEADLINE) is None

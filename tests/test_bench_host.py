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


# (workload, bytes per unit, units per launch, final-state bytes, flop per unit)
CHUNK_WORK = [
    # normalized d64: q, k, v bf16 in, o fp32 out
    ("normalized_bf16_b8h16_l2048_d64", (2 * 64 + 64) * 2 + 64 * 4, 8 * 16 * 2048, 8 * 16 * 64 * 64 * 4,
     2 * 64 * (64 + 64) + 4 * 64 * 64),
    # decay d128: + one fp32 log-gate per token
    ("decay_bf16_b4h32_l8192_d128", 384 * 2 + 512 + 4, 4 * 32 * 8192, 4 * 32 * 128 * 128 * 4,
     2 * 64 * 256 + 4 * 128 * 128),
    # vector decay d128: + one fp32 log-gate per token and key channel
    ("vector_decay_bf16_b4h32_l8192_d128", 384 * 2 + 128 * 4 + 512, 4 * 32 * 8192, 4 * 32 * 128 * 128 * 4,
     2 * 64 * 256 + 4 * 128 * 128),
    # gated delta d128: + log-gate and beta per token
    ("gated_delta_bf16_b2h16_l8192_d128", 384 * 2 + 512 + 4 + 4, 2 * 16 * 8192, 2 * 16 * 128 * 128 * 4,
     (2 * 64 * 64 * (3 * 128 + 2 * 128) + 6 * 64 * 128 * 128 + 64 ** 3 / 3) / 64),
]


@pytest.mark.parametrize("name,per_unit,units,state,flop_unit", CHUNK_WORK)
def test_chunk_work(name, per_unit, units, state, flop_unit):
    flop, nbytes = bench.chunk_work(W.CONFIGS[name])
    assert nbytes == per_unit * units + state
    assert flop == pytest.approx(flop_unit * units, rel=1e-12)


def test_headline_bytes():
    # 640 bytes per token-head over 262,144 token-heads plus a 2 MiB final state
    assert bench.chunk_work(W.CONFIGS[bench.HEADLINE])[1] == 169_869_312


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

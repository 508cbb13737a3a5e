"""bench.py's host-side contract, CPU only: more than one GPU is refused with a
message, the algorithmic FLOP count of a prompt chunk is the closed form, and
the CPU baseline of the prefill oracle reports the documented fields."""
import os
import subprocess
import sys

import numpy as np

import mla_synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_prefill_flops_closed_form():
    case = mla_synth.prefill_chunk(5, 12, 16)
    pos = np.arange(7, 12)
    attn = 16 * 640 * int(np.sum(pos + 1))               # 2 (192 + 128) per visible (query, key, head)
    expand = 16 * 2 * 512 * 256 * 12
    assert bench.prefill_flops(case) == attn + expand


def test_prefill_cpu_baseline_fields():
    case = mla_synth.prefill_chunk(128, 128, 16)
    b = bench.cpu_baseline_prefill(case, budget_s=0.01)
    assert b["kind"] == "oracle" and b["unit"] == "TFLOP/s" and b["value"] > 0 and b["cores"] >= 1
    assert "64" in b["sample"]


def test_decode_cpu_baseline_fields():
    """The decode CPU baseline: float32 oracle, median of three runs, with the
    host's CPU model and BLAS recorded (bf16 and a quantised cache)."""
    for dt in (0, 1):
        case = mla_synth.small_decode(case_id=33, H=16, seq_lens=[300, 200, 100, 50], normalise=dt == 0)
        b = bench.cpu_baseline(case, dt, budget_s=0.01)
        assert b["kind"] == "oracle" and b["unit"] == "GB/s" and b["value"] > 0 and b["cores"] >= 1
        assert "median of 3" in b["sample"] and "float32" in b["sample"]
        assert b["cpu_model"] and b["blas"]

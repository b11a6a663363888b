"""Host-side logic of bench.py, no GPU: the timing rounds, the algorithmic byte counts the roofline
divides by, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_timed_rounds_reports_the_median_round():
    vals = iter([12.0, 10.0, 11.0])
    ms, r = bench.timed_rounds(3, 4, lambda: next(vals))
    assert ms == 11.0
    assert r["n"] == 3 and r["ms_per_step"] == [3.0, 2.5, 2.75]
    assert r["min"] == 2.5 and r["max"] == 3.0 and r["value_from"] == "median round"


def test_kv_bytes_per_position_closed_form():
    # K and V of every layer: 49 layers x 2 x 4 kv heads x 128 dims x 2 bytes (bf16)
    assert bench.kv_bytes_per_position(synth.CONFIGS["int4_49"]) == 49 * 2 * 4 * 128 * 2 == 100352


def test_weight_bytes_of_the_int4_49_step():
    # counted from the model's shapes: an int4 group-64 matrix of r x c weights is r c / 2 bytes of codes
    # plus r c / 64 bf16 scales; norms fp32; one bf16 embedding row and the whole bf16 lm_head
    H, V, QKV, QD = 2048, 65536, (16 + 2 * 4) * 128, 16 * 128

    def m(r, c):
        return r * c // 2 + r * (c // 64) * 2

    attn = m(QKV, H) + m(H, QD) + 2 * H * 4
    dense = 2 * m(6144, H) + m(H, 6144)
    moe = m(64, H) + 6 * (2 * m(768, H) + m(H, 768))
    total = 2 * (attn + dense) + 47 * (attn + moe) + H * 2 + V * H * 2 + H * 4
    assert bench.weight_bytes_per_step(synth.CONFIGS["int4_49"]) == total == 1292492800
    # the mean over the 256 timed positions from 8,022: the bytes the default line divides by
    mean = sum(bench.step_bytes(synth.CONFIGS["int4_49"], 8022 + i) for i in range(256)) / 256
    assert mean == 2110411776


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr

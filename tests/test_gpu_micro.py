"""The measurement helpers through the C ABI: each returns a plausible figure on the GPU."""
import pytest

import synth
from stream_moe_decode_amd import micro

from gpu_common import build

pytestmark = pytest.mark.gpu


def test_micro_helpers():
    model = build(synth.CONFIGS["tiny"])
    m = micro(model.ctx)
    print("micro", m)
    assert 500.0 < m["stream_read_gbs"] < 8000.0  # below the 8 TB/s peak
    for g, us in list(m["exchange_us_per_round"].items()) + list(m["exchange_xcd_us_per_round"].items()):
        assert 0.0 < us < 100.0, (g, us)
    assert 0.0 < m["empty_launch_us"] < 100.0
    model.free()

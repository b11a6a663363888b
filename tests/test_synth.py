"""The seeded generators are pure functions of (seed, tensor id, index)."""
import numpy as np

import synth


def test_streams_are_sliceable_and_deterministic():
    tid = synth.tensor_id(synth.QKV, 4, 0)
    full = synth.normal_f32(tid, 5000, 0.02)
    np.testing.assert_array_equal(full[1234:2345], synth.normal_f32(tid, 1111, 0.02, off=1234))
    np.testing.assert_array_equal(full, synth.normal_f32(tid, 5000, 0.02))
    assert not np.array_equal(full, synth.normal_f32(tid + 1, 5000, 0.02))
    c1, s1 = synth.int4g64(tid, 10, 256, 0.02)
    c2, s2 = synth.int4g64(tid, 4, 256, 0.02, row0=6)
    np.testing.assert_array_equal(c1[6:], c2)
    np.testing.assert_array_equal(s1[6:], s2)


def test_normal_moments_and_bf16_rounding():
    x = synth.normal_f32(99, 400000, 1.0)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    b = synth.normal_bf16(99, 1000, 1.0)
    f = synth.normal_f32(99, 1000, 1.0)
    fb = (b.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.abs(fb - f) <= np.abs(f) * 2 ** -8)


def test_uniform_ints_in_range():
    t = synth.uniform_int(5, 10000, 512, 8192)
    assert t.min() >= 512 and t.max() <= 8192 and len(np.unique(t)) > 5000

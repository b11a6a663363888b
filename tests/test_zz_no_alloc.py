"""flint_decode_step_noalloc (the entry point for callers that cannot allocate device memory) against
flint_decode_step, through the C ABI: two calls in a row on a model and cache, then a second context with a
smaller model and cache, each compared bit for bit with the existing entry point on an identical cache (ids,
lengths and the K/V the step appended in every layer); the shared fixed array keeps the previous call's
contents, so the later calls also show that nothing stale leaks between calls.  A model whose exchange
scratch exceeds the fixed array is refused with FLINT_EINVAL."""
import numpy as np
import pytest
import torch

import synth
from stream_moe_decode_amd import (FLINT_EINVAL, FlintError, decode_step, decode_step_noalloc, kv_get_lengths,
                                   sync)

from gpu_common import build, gpu_kv_positions

pytestmark = pytest.mark.gpu


def _twin_caches(cfg, model, res, cap):
    kvs = []
    for _ in range(2):
        kv = model.kv(1, cap)
        for l in range(cfg.n_layers):
            if res:
                k, v = synth.resident_kv(cfg, l, 0, res)
                kv.load_resident(l, 0, k, v)
        kv.set_lengths([res])
        kvs.append(kv)
    return kvs


def _compare(cfg, model, kv_a, kv_b, tokens, what):
    dev = model.device
    ta = torch.tensor([tokens[0]], dtype=torch.int32, device=dev)
    tb = ta.clone()
    for i in range(len(tokens)):
        p = kv_get_lengths(kv_a.handle, 1)[0]
        decode_step(model.ctx, ta.data_ptr(), kv_a.handle, ta.data_ptr())
        decode_step_noalloc(model.ctx, tb.data_ptr(), kv_b.handle, tb.data_ptr())
        sync(model.ctx)
        ia, ib = int(ta.item()), int(tb.item())
        ka, va = gpu_kv_positions(kv_a, 0, p, 1)
        kb, vb = gpu_kv_positions(kv_b, 0, p, 1)
        print(f"{what} call {i} at position {p}: ids {ia} / {ib}", flush=True)
        assert ia == ib
        assert np.array_equal(ka, kb) and np.array_equal(va, vb)
        assert kv_get_lengths(kv_a.handle, 1) == kv_get_lengths(kv_b.handle, 1) == [p + 1]
    return int(tb.item())


def test_noalloc_matches_decode_step_then_a_smaller_model():
    # two calls in a row on the narrowed int4 model over 300 cached positions
    cfg = synth.CONFIGS["int4_b16_small"].replace(name="int4_small_noalloc", batch=1)
    model = build(cfg)
    kv_a, kv_b = _twin_caches(cfg, model, 300, 310)
    tok = int(synth.tokens(cfg, 1, stream=83)[0])
    _compare(cfg, model, kv_a, kv_b, [tok, tok], "int4 small")
    model.free()
    # a second context with a smaller model and cache: the fp32 two-layer model at 5 positions
    small = synth.CONFIGS["tiny"]
    model2 = build(small)
    kv_a, kv_b = _twin_caches(small, model2, 5, 12)
    _compare(small, model2, kv_a, kv_b, [int(synth.tokens(small, 1, stream=89)[0])], "tiny")
    model2.free()


def test_noalloc_refuses_a_model_beyond_the_fixed_array():
    # one kv head for 8 query heads on 256 workgroups: 256 attention splits, about 4.3 MB of partials
    cfg = synth.CONFIGS["moe_layer"].replace(name="one_kv_head", n_q_heads=8, n_kv_heads=1, vocab=1024)
    model = build(cfg)
    kv = model.kv(1, 8)
    t = torch.zeros(1, dtype=torch.int32, device=model.device)
    with pytest.raises(FlintError) as e:
        decode_step_noalloc(model.ctx, t.data_ptr(), kv.handle, t.data_ptr())
    assert e.value.status == FLINT_EINVAL
    assert kv_get_lengths(kv.handle, 1) == [0]
    model.free()

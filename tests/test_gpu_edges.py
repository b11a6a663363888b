"""GPU edge cases through the C ABI: the renormalised router (weights of the picked experts summing to
one) on both decode paths, sequences decoding from an empty cache, the capacity limit, an out-of-range
token (the kernel's own check latches it, the next call reports it), and prefill chunk sizes at the
boundary between a batched pass and the long-chunk kernels."""
import numpy as np
import pytest
import torch

import synth
from stream_moe_decode_amd import (FLINT_ECAPACITY, FLINT_EDEVICE, FlintError, decode_step, decode_step_debug,
                                   kv_get_lengths, prefill_chunk, sync)
from stream_moe_decode_amd.loader import make_debug

from gpu_common import TIE_EPS, Stepper, build, check_step, make_oracle

pytestmark = pytest.mark.gpu

# the narrowed int4 model of the batched-path tests (3 layers, 1 dense, hidden 512, 16 experts top-4)
SMALL = synth.CONFIGS["int4_b16"].replace(name="int4_b16_small", n_layers=3, n_dense_layers=1, hidden=512,
                                          n_q_heads=8, n_kv_heads=2, vocab=4096, dense_inter=1024, n_experts=16,
                                          top_k=4, expert_inter=256, ragged=(1, 300))


def _cache(cfg, lens, cap):
    model = build(cfg)
    kv = model.kv(len(lens), cap)
    orc = make_oracle(cfg, cap, batch=len(lens))
    for b, n in enumerate(lens):
        if n == 0:
            continue
        for l in range(cfg.n_layers):
            k, v = synth.resident_kv(cfg, l, b, n)
            kv.load_resident(l, b, k, v)
            orc.set_resident(b, l, k, v)
    kv.set_lengths(list(lens))
    orc.len = list(lens)
    return model, kv, orc


def _batched_steps(cfg, lens, steps, cap=None):
    model, kv, orc = _cache(cfg, lens, cap or max(lens) + steps + 4)
    dev, B = model.device, len(lens)
    tok = torch.from_numpy(synth.tokens(cfg, B, stream=37)).to(dev)
    out = torch.zeros(B, dtype=torch.int32, device=dev)
    for s in range(steps):
        dbg, t = make_debug(cfg, B, dev)
        toks = tok.cpu().numpy()
        decode_step_debug(model.ctx, tok.data_ptr(), kv.handle, out.data_ptr(), dbg)
        sync(model.ctx)
        for b in range(B):
            check_step(cfg, orc, b, int(toks[b]), t["logits"][b].cpu().numpy(), t["routes"][b].cpu().numpy(),
                       int(out[b].item()), what=f"step {s} sequence {b}: ", g_z=t["router_logits"][b].cpu().numpy())
        tok.copy_(out)
    assert kv_get_lengths(kv.handle, B) == [n + steps for n in lens]
    model.free()


def test_router_renorm_both_paths():
    cfg = SMALL.replace(name="int4_small_renorm", router_renorm=1)
    _batched_steps(cfg, [37, 180, 5, 260], 2)   # batched path
    model, kv, orc = _cache(cfg, [90], 96)        # persistent kernel
    st = Stepper(cfg, model, kv, orc)
    tok = int(synth.tokens(cfg, 1, stream=41)[0])
    for _ in range(2):
        tok = st.step(tok)
    model.free()


def test_batch_from_empty_cache():
    # two of four sequences start at length 0: their first step attends to its own position only
    _batched_steps(SMALL, [0, 7, 0, 200], 2)


def test_capacity_limit_both_paths():
    for lens, cap in (([19], 20), ([9, 3, 3], 10)):
        model, kv, orc = _cache(SMALL, lens, cap)
        dev, B = model.device, len(lens)
        tok = torch.from_numpy(synth.tokens(SMALL, B, stream=43)).to(dev)
        decode_step(model.ctx, tok.data_ptr(), kv.handle, tok.data_ptr())   # the last position fits
        sync(model.ctx)
        with pytest.raises(FlintError) as e:
            decode_step(model.ctx, tok.data_ptr(), kv.handle, tok.data_ptr())
        assert e.value.status == FLINT_ECAPACITY
        assert kv_get_lengths(kv.handle, B) == [n + 1 for n in lens]
        model.free()


def test_bad_token_is_reported_once():
    for lens in ([12], [12, 30, 4]):
        model, kv, orc = _cache(SMALL, lens, 64)
        dev, B = model.device, len(lens)
        tok = torch.from_numpy(synth.tokens(SMALL, B, stream=47)).to(dev)
        tok[B - 1] = SMALL.vocab   # outside [0, vocab)
        decode_step(model.ctx, tok.data_ptr(), kv.handle, tok.data_ptr())
        with pytest.raises(FlintError) as e:
            sync(model.ctx)
        assert e.value.status == FLINT_EDEVICE
        tok.copy_(torch.from_numpy(synth.tokens(SMALL, B, stream=53)).to(dev))
        decode_step(model.ctx, tok.data_ptr(), kv.handle, tok.data_ptr())   # reported once, then cleared
        sync(model.ctx)
        model.free()


def test_prefill_chunk_sizes_at_the_path_boundary():
    # 1 token (one batched pass), 17 (the smallest long chunk: one ragged block), 16 (one full pass)
    cfg = SMALL
    model = build(cfg)
    cap = 64
    kv = model.kv(1, cap)
    orc = make_oracle(cfg, cap)
    dev = model.device
    prompt = synth.tokens(cfg, 34, stream=59)
    toks = torch.from_numpy(prompt).to(dev)
    out = torch.zeros(1, dtype=torch.int32, device=dev)
    i0 = 0
    for n in (1, 17, 16):
        prefill_chunk(model.ctx, kv.handle, 0, toks.data_ptr() + 4 * i0, n, out.data_ptr())
        sync(model.ctx)
        r = orc.forward(0, prompt[i0:i0 + n])
        gpu_id, o_id, gap = int(out.item()), int(r["ids"][-1]), float(r["gap"][-1])
        print(f"chunk of {n}: gpu id {gpu_id} oracle id {o_id} gap {gap:.3g}", flush=True)
        assert gpu_id == o_id or gap < TIE_EPS
        i0 += n
    assert kv_get_lengths(kv.handle, 1) == [34]
    st = Stepper(cfg, model, kv, orc)
    st.step(int(out.item()))
    model.free()

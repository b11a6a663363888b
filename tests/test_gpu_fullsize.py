"""GPU parity at the full model sizes, through the C ABI: the oracle is
teacher-forced on the GPU's tokens (and, at near ties, its routes) and every
step's logits, routes and id are compared (rules in gpu_common).  These build
the 49-layer models, so each test takes tens of seconds."""
import numpy as np
import pytest
import torch

import synth
from stream_moe_decode_amd import decode_step_debug, prefill_chunk, sync
from stream_moe_decode_amd.loader import make_debug

from gpu_common import Stepper, build, check_step, make_oracle

pytestmark = pytest.mark.gpu


def _cached(cfg):
    cache = {}

    def fn(l):
        if l not in cache:
            cache[l] = synth.layer(cfg, l)
        return cache[l]
    return fn, cache


def test_int4_49_decode_at_8022_positions():
    # the int4 49-layer model over the 8,022-position synthetic cache, 3 greedy steps
    cfg = synth.CONFIGS["int4_49"]
    fn, cache = _cached(cfg)
    print(f"{cfg.name}: generating the weights", flush=True)
    layers = {l: fn(l) for l in range(cfg.n_layers)}
    print(f"{cfg.name}: building the device model", flush=True)
    model = build(cfg, layers=layers)
    cap = cfg.resident + 8
    kv = model.kv(1, cap)
    orc = make_oracle(cfg, cap, layers=layers)
    for l in range(cfg.n_layers):
        k, v = synth.resident_kv(cfg, l, 0, cfg.resident)
        kv.load_resident(l, 0, k, v)
        orc.set_resident(0, l, k, v)
    kv.set_lengths([cfg.resident])
    orc.len[0] = cfg.resident
    st = Stepper(cfg, model, kv, orc)
    tok = int(synth.tokens(cfg, 1, stream=11)[0])
    for i in range(3):
        print(f"int4_49 step {i} at position {cfg.resident + i}", flush=True)
        tok = st.step(tok)
    model.free()
    print("int4_49 report", st.report)


def test_bf16_49_prefill_then_decode():
    # the bf16 49-layer model: a 32-token prompt through flint_prefill_chunk, then 2 greedy steps
    cfg = synth.CONFIGS["bf16_49"].replace(prompt=32, decode=2)
    fn, cache = _cached(cfg)
    print(f"{cfg.name}: generating the weights", flush=True)
    layers = {l: fn(l) for l in range(cfg.n_layers)}
    print(f"{cfg.name}: building the device model", flush=True)
    model = build(cfg, layers=layers)
    cap = cfg.prompt + cfg.decode + 4
    kv = model.kv(1, cap)
    orc = make_oracle(cfg, cap, layers=layers)
    prompt = synth.tokens(cfg, cfg.prompt)
    dev = model.device
    toks = torch.from_numpy(prompt).to(dev)
    out = torch.zeros(1, dtype=torch.int32, device=dev)
    print("bf16_49 prefill", flush=True)
    prefill_chunk(model.ctx, kv.handle, 0, toks.data_ptr(), len(prompt) - 1, out.data_ptr())
    sync(model.ctx)
    orc.forward(0, prompt[:-1], want_logits=False)
    st = Stepper(cfg, model, kv, orc)
    tok = int(prompt[-1])
    for i in range(cfg.decode + 1):
        print(f"bf16_49 step {i}", flush=True)
        tok = st.step(tok)
    model.free()
    print("bf16_49 report", st.report)


def test_int4_batch16_fullsize_all_sequences():
    # the batched path on the full int4 model, 16 sequences with lengths in [512, 8192]: every sequence's
    # first step against the oracle, one sequence at a time (a single-slot oracle per sequence keeps the
    # host copy of the K/V to one sequence's)
    cfg = synth.CONFIGS["int4_b16"]
    fn, cache = _cached(cfg)
    print(f"{cfg.name}: generating the weights", flush=True)
    layers = {l: fn(l) for l in range(cfg.n_layers)}
    print(f"{cfg.name}: building the device model", flush=True)
    lens = [int(x) for x in synth.lengths(cfg)]
    B = cfg.batch
    model = build(cfg, layers=layers)
    cap = max(lens) + 4
    kv = model.kv(B, cap)
    for b in range(B):
        for l in range(cfg.n_layers):
            k, v = synth.resident_kv(cfg, l, b, lens[b])
            kv.load_resident(l, b, k, v)
    kv.set_lengths(lens)
    dev = model.device
    tok = torch.from_numpy(synth.tokens(cfg, B, stream=11)).to(dev)
    out = torch.zeros(B, dtype=torch.int32, device=dev)
    dbg, t = make_debug(cfg, B, dev)
    decode_step_debug(model.ctx, tok.data_ptr(), kv.handle, out.data_ptr(), dbg)
    sync(model.ctx)
    g_logits, g_routes, g_ids, toks = (t["logits"].cpu().numpy(), t["routes"].cpu().numpy(), out.cpu().numpy(),
                                       tok.cpu().numpy())
    g_z = t["router_logits"].cpu().numpy()
    model.free()
    for b in range(B):
        orc = make_oracle(cfg, lens[b] + 4, layers=layers)
        for l in range(cfg.n_layers):
            k, v = synth.resident_kv(cfg, l, b, lens[b])
            orc.set_resident(0, l, k, v)
        orc.len[0] = lens[b]
        check_step(cfg, orc, 0, int(toks[b]), g_logits[b], g_routes[b], int(g_ids[b]),
                   what=f"sequence {b} ({lens[b]} positions): ", g_z=g_z[b])
        del orc

"""GPU parity at the full model sizes, through the C ABI (rules in gpu_common).
These build the 49-layer models, so each test takes tens of seconds.

  * int4, 8,022 resident positions: 16 greedy steps, each end to end against
    the oracle, every 4th (and the last) layer by layer; likewise 10 steps from
    8,188 positions (the contexts cross 64 x 128 positions: two attention chunks
    per split, the second a short tail).
  * bf16, a 2,048-token prompt through the long-chunk prefill: the prefill is
    run twice and must write bit-identical K/V and id; at sampled prompt
    positions the oracle runs one step from the GPU's cache of the earlier
    positions and its K/V must match the GPU's in every layer (the last
    position also gives the greedy id); then 8 greedy steps checked end to end
    and layer by layer.
  * int4, 16 sequences with ragged lengths in [512, 8192] on the batched path:
    the step is run twice (bit-identical logits and ids) and every sequence is
    checked end to end and layer by layer.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from stream_moe_decode_amd import decode_step_debug, kv_get_lengths, kv_set_lengths, prefill_chunk, sync
from stream_moe_decode_amd.loader import make_debug

from gpu_common import (Stepper, build, check_layers, check_step, gpu_kv_positions, make_oracle, margins, rel_err,
                        token_margin)

pytestmark = pytest.mark.gpu


def _layers(cfg):
    print(f"{cfg.name}: generating the weights", flush=True)
    return {l: synth.layer(cfg, l) for l in range(cfg.n_layers)}


@pytest.mark.parametrize("resident,steps", [(8022, 16), (8188, 10)])
def test_int4_49_decode_steps(resident, steps):
    # 8,022 positions: the metric's context, one attention chunk per split.  From 8,188: the contexts
    # cross 64 x 128 positions, where a split's second chunk is a short tail (its rows requested early)
    cfg = synth.CONFIGS["int4_49"].replace(resident=resident)
    layers = _layers(cfg)
    print(f"{cfg.name}: building the device model", flush=True)
    model = build(cfg, layers=layers)
    cap = cfg.resident + steps + 4
    kv = model.kv(1, cap)
    orc = make_oracle(cfg, cap, layers=layers)
    tf = make_oracle(cfg, cap, layers=layers)
    for l in range(cfg.n_layers):
        k, v = synth.resident_kv(cfg, l, 0, cfg.resident)
        kv.load_resident(l, 0, k, v)
        orc.set_resident(0, l, k, v)
        tf.set_resident(0, l, k, v)
    kv.set_lengths([cfg.resident])
    orc.len[0] = tf.len[0] = cfg.resident
    st = Stepper(cfg, model, kv, orc, tf=tf)
    tok = int(synth.tokens(cfg, 1, stream=11)[0])
    for i in range(steps):
        print(f"int4_49 step {i} at position {cfg.resident + i}", flush=True)
        tok = st.step(tok, layers=(i % 4 == 0 or i == steps - 1))
    model.free()
    print("int4_49 report", st.report)


def _oracle_with_gpu_cache(cfg, layers, cap, gk, gv, n):
    o = make_oracle(cfg, cap, layers=layers)
    for l in range(cfg.n_layers):
        o.K[l][0][:, :n] = gk[l]
        o.V[l][0][:, :n] = gv[l]
    o.len[0] = n
    return o


def test_bf16_49_prompt_2048_then_decode():
    cfg = synth.CONFIGS["bf16_49"]
    n = cfg.prompt - 1           # the prompt's last token is the first decode step's input
    steps = 8
    layers = _layers(cfg)
    print(f"{cfg.name}: building the device model", flush=True)
    model = build(cfg, layers=layers)
    cap = cfg.prompt + steps + 4
    kv = model.kv(1, cap)
    prompt = synth.tokens(cfg, cfg.prompt)
    dev = model.device
    toks = torch.from_numpy(prompt).to(dev)
    out = torch.zeros(1, dtype=torch.int32, device=dev)
    ids, caches = [], []
    for rep in range(2):
        print(f"bf16_49: prefill of {n} tokens (run {rep})", flush=True)
        kv_set_lengths(kv.handle, [0])
        prefill_chunk(model.ctx, kv.handle, 0, toks.data_ptr(), n, out.data_ptr())
        sync(model.ctx)
        ids.append(int(out.item()))
        caches.append(gpu_kv_positions(kv, 0, 0, n))
    assert kv_get_lengths(kv.handle, 1) == [n]
    assert ids[0] == ids[1]
    for a, b in zip(caches[0], caches[1]):
        assert np.array_equal(a, b), "two prefills of the same prompt wrote different K/V"
    gk, gv = caches[0]
    del caches
    M = margins(cfg)
    # sampled positions: the oracle's step at p from the GPU's cache of positions < p
    for p in (0, 1, 17, 64, 500, 1023, 1500, n - 1):
        o = _oracle_with_gpu_cache(cfg, layers, p + 2, gk[:, :, :p], gv[:, :, :p], p)
        r = o.forward(0, prompt[p:p + 1])
        worst = 0.0
        for l in range(cfg.n_layers):
            for j in range(cfg.n_kv_heads):
                worst = max(worst, rel_err(gk[l, j, p], o.K[l][0][j, p]), rel_err(gv[l, j, p], o.V[l][0][j, p]))
        print(f"bf16_49 prompt position {p}: appended K/V rel err {worst:.3g}", flush=True)
        assert worst <= M["free_kv_bound"], f"position {p}: K/V rel err {worst:.3g} > {M['free_kv_bound']:.3g}"
        if p == n - 1:
            o_id, gap = int(r["ids"][0]), float(r["gap"][0])
            print(f"bf16_49 after the prompt: gpu id {ids[0]} oracle id {o_id} gap {gap:.3g}", flush=True)
            assert ids[0] == o_id or gap < token_margin(cfg)
        del o
    orc = _oracle_with_gpu_cache(cfg, layers, cap, gk, gv, n)
    tf = _oracle_with_gpu_cache(cfg, layers, cap, gk, gv, n)
    del gk, gv
    st = Stepper(cfg, model, kv, orc, tf=tf)
    tok = int(prompt[-1])
    for i in range(steps):
        print(f"bf16_49 step {i} at position {n + i}", flush=True)
        tok = st.step(tok)
    model.free()
    print("bf16_49 report", st.report)


def test_int4_batch16_fullsize_all_sequences():
    cfg = synth.CONFIGS["int4_b16"]
    layers = _layers(cfg)
    lens = [int(x) for x in synth.lengths(cfg)]
    B = cfg.batch
    print(f"{cfg.name}: building the device model", flush=True)
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
    runs = []
    for rep in range(2):
        kv.set_lengths(lens)
        dbg, t = make_debug(cfg, B, dev, resid=True)
        decode_step_debug(model.ctx, tok.data_ptr(), kv.handle, out.data_ptr(), dbg)
        sync(model.ctx)
        runs.append({k: v.cpu().numpy() for k, v in t.items()} | {"ids": out.cpu().numpy()})
    for key in ("logits", "ids", "routes", "resid"):
        assert np.array_equal(runs[0][key], runs[1][key]), f"two batched steps gave different {key}"
    g = runs[0]
    toks = tok.cpu().numpy()
    new_k, new_v = [], []
    for b in range(B):
        k, v = gpu_kv_positions(kv, b, lens[b], 1)
        new_k.append(k[:, :, 0])
        new_v.append(v[:, :, 0])
    model.free()
    for b in range(B):
        what = f"sequence {b} ({lens[b]} positions): "
        orc = make_oracle(cfg, lens[b] + 4, layers=layers)
        tf = make_oracle(cfg, lens[b] + 4, layers=layers)
        for l in range(cfg.n_layers):
            k, v = synth.resident_kv(cfg, l, b, lens[b])
            orc.set_resident(0, l, k, v)
            tf.set_resident(0, l, k, v)
        orc.len[0] = tf.len[0] = lens[b]
        check_layers(cfg, tf, 0, int(toks[b]), g["resid"][b], g["router_logits"][b], g["routes"][b],
                     g["logits"][b], int(g["ids"][b]), new_k[b], new_v[b], what=what)
        check_step(cfg, orc, 0, int(toks[b]), g["logits"][b], g["routes"][b], int(g["ids"][b]), what=what,
                   g_z=g["router_logits"][b])
        del orc, tf

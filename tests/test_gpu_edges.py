"""GPU edge cases through the C ABI: the renormalised router (weights of the picked experts summing to
one) on both decode paths, sequences decoding from an empty cache, the capacity limit, an out-of-range
token (the kernel's own check latches it, the next call reports it), prefill chunk sizes at the
boundary between a batched pass and the long-chunk kernels, exact ties (an all-zero router: the lowest
experts; equal top logits: the lowest id) on both decode paths, and one sequence on the batched pass."""
import numpy as np
import pytest
import torch

import oracle as oracle_mod
import synth
from stream_moe_decode_amd import (FLINT_ECAPACITY, FLINT_EDEVICE, FlintError, decode_step, decode_step_debug,
                                   kv_get_lengths, prefill_chunk, sync)
from stream_moe_decode_amd.loader import DeviceModel, make_debug

from gpu_common import Stepper, build, check_step, make_oracle, token_margin

pytestmark = pytest.mark.gpu

# the narrowed int4 model of the batched-path tests (3 layers, 1 dense, hidden 512, 16 experts top-4)
SMALL = synth.CONFIGS["int4_b16_small"]


def gpu_build(cfg, layers, head):
    return DeviceModel(cfg, lambda l: layers[l], head)


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
        assert gpu_id == o_id or gap < token_margin(cfg)
        i0 += n
    assert kv_get_lengths(kv.handle, 1) == [34]
    st = Stepper(cfg, model, kv, orc)
    st.step(int(out.item()))
    model.free()


def _zero_router(cfg, layers):
    for l in range(cfg.n_dense_layers, cfg.n_layers):
        r = layers[l]["router"]
        if "s" in r:   # int4: code 8 (q = 0) with scale 0
            layers[l]["router"] = {"w": np.full_like(r["w"], 0x88), "s": np.zeros_like(r["s"])}
        else:
            layers[l]["router"] = {"w": np.zeros_like(r["w"])}


@pytest.mark.parametrize("lens", [[40], [40, 7, 120, 300]])
def test_zero_router_ties_pick_the_lowest_experts(lens):
    # every router logit is exactly 0: the top-k is experts 0 .. k-1 in index order and each weight is
    # 1 / n_experts (1 / k renormalised), on the persistent kernel (one sequence) and the batched pass (four)
    for renorm in (0, 1):
        cfg = SMALL.replace(name="int4_small_zero_router", router_renorm=renorm)
        layers = {l: synth.layer(cfg, l) for l in range(cfg.n_layers)}
        _zero_router(cfg, layers)
        model = build(cfg, layers=layers)
        B = len(lens)
        kv = model.kv(B, max(lens) + 4)
        orc = make_oracle(cfg, max(lens) + 4, layers=layers, batch=B)
        for b, n in enumerate(lens):
            for l in range(cfg.n_layers):
                k, v = synth.resident_kv(cfg, l, b, n)
                kv.load_resident(l, b, k, v)
                orc.set_resident(b, l, k, v)
        kv.set_lengths(lens)
        orc.len = list(lens)
        dev = model.device
        tok = torch.from_numpy(synth.tokens(cfg, B, stream=61)).to(dev)
        out = torch.zeros(B, dtype=torch.int32, device=dev)
        dbg, t = make_debug(cfg, B, dev)
        decode_step_debug(model.ctx, tok.data_ptr(), kv.handle, out.data_ptr(), dbg)
        sync(model.ctx)
        routes, rw, z = t["routes"].cpu().numpy(), t["route_w"].cpu().numpy(), t["router_logits"].cpu().numpy()
        moe = list(range(cfg.n_dense_layers, cfg.n_layers))
        want_w = np.float32(1.0 / cfg.top_k) if renorm else np.float32(1.0 / cfg.n_experts)
        for b in range(B):
            assert (z[b, moe] == 0).all()
            assert (routes[b, moe] == np.arange(cfg.top_k)).all(), routes[b, moe]
            np.testing.assert_allclose(rw[b, moe], want_w, rtol=1e-6)
            check_step(cfg, orc, b, int(tok[b].item()), t["logits"][b].cpu().numpy(), routes[b], int(out[b].item()),
                       what=f"renorm {renorm} sequence {b}: ", g_z=z[b])
        model.free()


@pytest.mark.parametrize("lens", [[40], [40, 7, 120, 300]])
def test_equal_top_logits_pick_the_lowest_id(lens):
    # the lm_head row that wins for sequence 0 (per the oracle) is copied to a lower row owned by another
    # workgroup and to a higher one: three exactly equal top logits, the lowest id must win on both paths
    cfg = SMALL.replace(name="int4_small_argmax_tie")
    layers = {l: synth.layer(cfg, l) for l in range(cfg.n_layers)}
    head = synth.head(cfg)
    B = len(lens)
    kvs = {(b, l): synth.resident_kv(cfg, l, b, n) for b, n in enumerate(lens) for l in range(cfg.n_layers)}

    def oracle_for(hw):
        o = oracle_mod.Oracle(cfg, lambda l: layers[l], hw, cap=max(lens) + 4, batch=B)
        for (b, l), (k, v) in kvs.items():
            o.set_resident(b, l, k, v)
        o.len = list(lens)
        return o

    # pick the first candidate token whose winning row leads the next distinct row by a clear margin
    for cand in synth.tokens(cfg, 8, stream=67):
        r = oracle_for(head).forward(0, np.array([cand], np.int32))
        lg = r["logits"][0]
        win = int(np.argmax(lg))
        if r["gap"][0] > 2 * token_margin(cfg) and win >= 64 and win + 1 < cfg.vocab:
            break
    else:
        pytest.skip("no candidate token with a clear winner")
    lo, hi = win - 48, win + 1    # 48 rows below: another workgroup's share on every path
    head = dict(head)
    head["lm_head"] = head["lm_head"].copy()
    head["lm_head"][lo] = head["lm_head"][win]
    head["lm_head"][hi] = head["lm_head"][win]
    r = oracle_for(head).forward(0, np.array([cand], np.int32))
    assert int(r["ids"][0]) == lo
    model = gpu_build(cfg, layers, head)
    kv = model.kv(B, max(lens) + 4)
    for (b, l), (k, v) in kvs.items():
        kv.load_resident(l, b, k, v)
    kv.set_lengths(lens)
    dev = model.device
    toks = synth.tokens(cfg, B, stream=71)
    toks[0] = cand
    tok = torch.from_numpy(toks).to(dev)
    out = torch.zeros(B, dtype=torch.int32, device=dev)
    dbg, t = make_debug(cfg, B, dev)
    decode_step_debug(model.ctx, tok.data_ptr(), kv.handle, out.data_ptr(), dbg)
    sync(model.ctx)
    g = t["logits"][0].cpu().numpy()
    print(f"winning row {win}, copies at {lo} and {hi}: gpu id {int(out[0].item())}, "
          f"logits {g[lo]!r} {g[win]!r} {g[hi]!r}", flush=True)
    assert g[lo] == g[win] == g[hi] == g.max()
    assert int(out[0].item()) == lo
    model.free()


def test_one_column_batched_pass_matches_oracle(monkeypatch):
    # the fusion experiment's configuration: one sequence routed to the batched pass of ordinary kernels
    # (FLINT_BATCH_MIN=1, read at context creation), checked end to end and layer by layer
    from gpu_common import check_layers, gpu_kv_positions
    monkeypatch.setenv("FLINT_BATCH_MIN", "1")
    cfg = SMALL
    model, kv, orc = _cache(cfg, [150], 160)
    monkeypatch.delenv("FLINT_BATCH_MIN")
    tf = make_oracle(cfg, 160)
    for l in range(cfg.n_layers):
        k, v = synth.resident_kv(cfg, l, 0, 150)
        tf.set_resident(0, l, k, v)
    tf.len[0] = 150
    st = Stepper(cfg, model, kv, orc, tf=tf)
    tok = int(synth.tokens(cfg, 1, stream=73)[0])
    for _ in range(3):
        tok = st.step(tok)
    model.free()


def test_wait_limit_timeout_is_reported_once_and_recovers():
    # the persistent kernel's bounded waits, forced from the host: with every wait bounded by 1 us some wait of
    # the step gives up, every workgroup winds down and exits, the step writes -1 in place of its id and leaves
    # the length as it was; the next call reports FLINT_ETIMEOUT once; with the default bound restored the
    # same position decodes and matches the oracle
    from stream_moe_decode_amd import FLINT_ETIMEOUT, set_wait_limit
    cfg = SMALL
    model, kv, orc = _cache(cfg, [50], 64)
    dev = model.device
    tok = int(synth.tokens(cfg, 1, stream=79)[0])
    t = torch.tensor([tok], dtype=torch.int32, device=dev)
    out = torch.full((1,), 7, dtype=torch.int32, device=dev)
    set_wait_limit(model.ctx, 1)
    timed_out = False
    for attempt in range(3):
        decode_step(model.ctx, t.data_ptr(), kv.handle, out.data_ptr())
        try:
            sync(model.ctx)
        except FlintError as e:
            assert e.status == FLINT_ETIMEOUT
            timed_out = True
            break
        print(f"attempt {attempt}: every wait ended within 1 us; rolling back", flush=True)
        kv.set_lengths([50])
    assert timed_out
    assert int(out.item()) == -1
    assert kv_get_lengths(kv.handle, 1) == [50]
    sync(model.ctx)   # reported once
    set_wait_limit(model.ctx, 0)
    st = Stepper(cfg, model, kv, orc)
    tok = st.step(tok)
    tok = st.step(tok)
    assert kv_get_lengths(kv.handle, 1) == [52]
    model.free()

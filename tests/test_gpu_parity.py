"""GPU parity of the persistent decode kernel against the CPU oracle, called
through the C ABI (include/flint.h) via the Python binding.  Every step is
checked end to end and layer by layer (rules in gpu_common)."""
import numpy as np
import pytest
import torch

import synth
from stream_moe_decode_amd import prefill_chunk, sync

from gpu_common import Stepper, build, check_layers, check_step, logits_tol, make_oracle, rel_err

pytestmark = pytest.mark.gpu


def _greedy(cfg, grid=0):
    model = build(cfg, grid=grid)
    cap = cfg.prompt + cfg.decode + 4
    kv = model.kv(1, cap)
    orc = make_oracle(cfg, cap)
    tf = make_oracle(cfg, cap)
    prompt = synth.tokens(cfg, cfg.prompt)
    dev = model.device
    toks = torch.from_numpy(prompt).to(dev)
    out = torch.zeros(1, dtype=torch.int32, device=dev)
    prefill_chunk(model.ctx, kv.handle, 0, toks.data_ptr(), len(prompt) - 1, out.data_ptr())
    sync(model.ctx)
    orc.forward(0, prompt[:-1])
    st = Stepper(cfg, model, kv, orc, tf=tf)
    tok = int(prompt[-1])
    ids = []
    for _ in range(cfg.decode + 1):
        tok = st.step(tok)
        ids.append(tok)
    model.free()
    return ids, st.report


def test_tiny_fp32_greedy_matches_oracle():
    cfg = synth.CONFIGS["tiny"]
    ids, rep = _greedy(cfg)
    print("tiny ids", ids, "max err", max(r["err"] for r in rep))
    assert len(ids) == cfg.decode + 1


def test_tiny_fp32_distinct_norm_weights():
    # RMSNorm weights 1 + N(0, 0.1), different in every layer and norm: the kernel must take each layer's own
    cfg = synth.CONFIGS["tiny"].replace(name="tiny_norms", norm_sigma=0.1, decode=6)
    _greedy(cfg)


def test_tiny_fp32_small_grid():
    # a grid that is not one workgroup per CU exercises the uneven work splits
    cfg = synth.CONFIGS["tiny"].replace(decode=4)
    _greedy(cfg, grid=60)


def test_tiny_bf16_and_int4_variants():
    for wt in (synth.BF16, synth.INT4G64):
        cfg = synth.CONFIGS["tiny"].replace(weight_type=wt, decode=6, norm_sigma=0.1)
        _greedy(cfg)


@pytest.mark.parametrize("resident", [1024, 9000, 16383])
def test_moe_layer_bf16_one_step(resident):
    # one MoE layer at full width over the resident positions: the layer's output residual against the
    # oracle's at 2e-2 (end to end) and at the per-layer bound, routes, logits.  The attention splits of
    # 64 per kv head take 1,025 positions as one chunk each, 9,001 as two chunks of which the second is
    # ragged, and 16,384 as two whole chunks of 128 (the online softmax carried across chunks)
    cfg = synth.CONFIGS["moe_layer"].replace(resident=resident)
    model = build(cfg)
    cap = cfg.resident + 8
    kv = model.kv(1, cap)
    orc = make_oracle(cfg, cap)
    tf = make_oracle(cfg, cap)
    k, v = synth.resident_kv(cfg, 0, 0, cfg.resident)
    kv.load_resident(0, 0, k, v)
    for o in (orc, tf):
        o.set_resident(0, 0, k, v)
        o.len[0] = cfg.resident
    kv.set_lengths([cfg.resident])
    st = Stepper(cfg, model, kv, orc, tf=tf)
    tok = int(synth.tokens(cfg, 1, stream=7)[0])
    st.step(tok)
    g_res = st.t["resid"][0, 0].cpu().numpy()
    model.free()
    ref = make_oracle(cfg, cap)
    ref.set_resident(0, 0, k, v)
    ref.len[0] = cfg.resident
    r = ref.forward(0, np.array([tok], np.int32), resid_all=True)
    err = rel_err(g_res, r["resid"][0, 0])
    print("moe_layer residual rel err", err, "report", st.report)
    assert err <= logits_tol(cfg)


def test_deterministic_bitwise():
    cfg = synth.CONFIGS["tiny"].replace(decode=3)
    a, _ = _greedy(cfg)
    b, _ = _greedy(cfg)
    assert a == b

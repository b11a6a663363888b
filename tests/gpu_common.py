"""Shared helpers of the GPU parity tests (device model from the seeded
generator, and the comparison rules).

Comparison rules (the tolerances stated for this library):
  * logits: max |gpu - oracle| / max |oracle| <= 1e-4 (fp32 model) or 2e-2 (bf16 / int4);
  * routes: the GPU's top-k set equals the oracle's, or, where the oracle's
    k-th / (k+1)-th router logits are within 1e-3 * max|z|, is a valid top-k
    within that margin (the oracle then follows the GPU's set);
  * token ids: identical unless the oracle's top-2 logit gap is below 1e-3 of
    max |logit| or below twice the step's measured logit error (then the
    oracle follows the GPU's token).
"""
import numpy as np
import torch

import oracle
import synth
from stream_moe_decode_amd import decode_step_debug, prefill_chunk, sync
from stream_moe_decode_amd.loader import DeviceModel, make_debug

TIE_EPS = 1e-3


def logits_tol(cfg):
    return 1e-4 if cfg.weight_type == synth.F32 else 2e-2


def rel_err(g, o):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    return float(np.max(np.abs(g - o)) / max(np.max(np.abs(o)), 1e-30))


def build(cfg, grid=0, layers=None):
    if layers is None:
        def layer_fn(l):
            return synth.layer(cfg, l)
    else:
        def layer_fn(l):
            return layers[l]
    return DeviceModel(cfg, layer_fn, synth.head(cfg), grid=grid)


def make_oracle(cfg, cap, layers=None, batch=1):
    fn = (lambda l: synth.layer(cfg, l)) if layers is None else (lambda l: layers[l])
    return oracle.Oracle(cfg, fn, synth.head(cfg), cap=cap, batch=batch)


class Stepper:
    """Runs GPU decode steps with debug outputs and checks each against the oracle."""

    def __init__(self, cfg, model, kv, orc, seq=0):
        self.cfg, self.model, self.kv, self.orc, self.seq = cfg, model, kv, orc, seq
        self.dev = model.device
        self.tok = torch.zeros(kv.batch, dtype=torch.int32, device=self.dev)
        self.out = torch.zeros(kv.batch, dtype=torch.int32, device=self.dev)
        self.dbg, self.t = make_debug(cfg, kv.batch, self.dev, resid_layer=0)
        self.report = []

    def step(self, token: int):
        """One GPU step on `token` and the oracle's step on the same token; returns the checked GPU id."""
        cfg = self.cfg
        self.tok[self.seq] = token
        decode_step_debug(self.model.ctx, self.tok.data_ptr(), self.kv.handle, self.out.data_ptr(), self.dbg)
        sync(self.model.ctx)
        g_logits = self.t["logits"][self.seq].cpu().numpy()
        g_routes = self.t["routes"][self.seq].cpu().numpy()
        g_id = int(self.out[self.seq].item())
        g_z = self.t["router_logits"][self.seq].cpu().numpy() if "router_logits" in self.t else None
        self.report.append(check_step(cfg, self.orc, self.seq, token, g_logits, g_routes, g_id, g_z=g_z))
        return g_id


def check_step(cfg, orc, seq, token, g_logits, g_routes, g_id, what="", g_z=None):
    """The oracle's step of sequence `seq` on `token` (following the GPU's routes and token where the
    oracle's own margin is below the tolerance) against the GPU's logits, routes and id; returns a report.
    g_z: the GPU's router logits [n_layers][n_experts], which widen the route tolerance of a layer to
    twice their measured deviation from the oracle's."""
    r = orc.forward(seq, np.array([token], np.int32), ref_routes=g_routes[None], tie_eps=TIE_EPS,
                    ref_z=None if g_z is None else g_z[None])
    err = rel_err(g_logits, r["logits"][0])
    moe = [l for l in range(cfg.n_layers) if l >= cfg.n_dense_layers]
    flags = r["route_flags"][0, moe] if moe else np.zeros(0)
    assert not (flags == 2).any(), f"{what}routes differ beyond a near tie at layers {np.nonzero(flags == 2)[0]}"
    assert err <= logits_tol(cfg), f"{what}logits max rel err {err:.3g} > {logits_tol(cfg)}"
    o_id = int(r["ids"][0])
    # the token may differ where the oracle's top-2 gap is below 1e-3 of max |logit|, or below twice this
    # step's measured logit error: one bf16 rounding flip of the final norm's output moves the logits by
    # about 1e-3 of their maximum at these sizes, so a smaller gap is not resolved by the tolerance itself
    near = r["gap"][0] < max(TIE_EPS, 2.0 * err)
    print(f"{what}logits rel err {err:.3g}, gpu id {g_id}, oracle id {o_id}, oracle gap {r['gap'][0]:.3g}, "
          f"oracle logit of gpu id {(r['logits'][0][o_id] - r['logits'][0][g_id]) / np.max(np.abs(r['logits'][0])):.3g} "
          f"below its max")
    assert g_id == o_id or near, f"{what}token {g_id} != oracle {o_id} (gap {r['gap'][0]:.3g})"
    assert g_id == int(np.argmax(g_logits)) or np.max(g_logits) == g_logits[g_id]
    return {"err": err, "near_route": int((flags == 1).sum()), "near_token": bool(near and g_id != o_id)}

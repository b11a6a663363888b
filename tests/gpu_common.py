"""Shared helpers of the GPU parity tests (device model from the seeded
generator, and the comparison rules).

Two comparisons per checked step, both against the CPU oracle:

  * Per layer (``check_layers``): layer l of the oracle is fed the GPU's own
    residual after layer l - 1 (the embedding for layer 0) and a cache that
    holds the GPU's K/V for every earlier position; its router logits, expert
    set, output residual and appended K/V are compared with the GPU's, and the
    head with the GPU's final residual.  This isolates each layer's
    arithmetic: the router logits must agree within ``layer_z_bound``, the
    expert set must be the oracle's exactly unless the oracle's k-th/(k+1)-th
    gap is below ``layer_route_margin`` (then a different set must be a valid
    top-k within it; such adoptions are counted and capped), and the greedy id
    must be the oracle's unless its top-2 gap is below ``head_token_margin``.
  * End to end (``check_step``): the oracle runs the whole step from the
    token.  Logits within max rel err 2e-2 (bf16 / int4) or 1e-4 (fp32); the
    router logits within ``free_z_bound``; where the GPU's expert set differs it
    must be a valid top-k within ``free_route_margin`` and the oracle follows
    it; the greedy id must be the oracle's unless the top-2 gap is below
    ``free_token_margin`` (then the oracle follows the GPU's token).

The bf16 / int4 margins are fixed numbers in ``golden/margins.json``, written
by ``golden/derive_margins.py`` from the oracle alone (its drift under fp32-size
rounding noise, per group of models); nothing in them comes from the GPU.  The
fp32 model has no bf16 rounding: its margins are the stated 1e-4 logit
tolerance and a 1e-3 relative gap.
"""
import json
import os

import numpy as np
import torch

import oracle
import synth
from stream_moe_decode_amd import decode_step_debug, sync
from stream_moe_decode_amd.loader import DeviceModel, make_debug

_MARGINS = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "margins.json")))
FP32_MARGINS = {"layer_z_bound": 1e-4, "layer_route_margin": 1e-3, "layer_resid_bound": 1e-4,
                "layer_kv_bound": 1e-4, "head_logit_bound": 1e-4, "head_token_margin": 1e-3,
                "free_z_bound": 1e-4, "free_route_margin": 1e-3, "free_logit_bound": 1e-4,
                "free_token_margin": 1e-3}
# per-layer expert-set adoptions allowed per checked step: a tenth of the MoE layers, at least one
ADOPT_FRACTION = 0.1


def margin_group(cfg) -> str:
    if cfg.n_layers >= 10:
        return "deep"
    if cfg.n_layers == 1:
        return "one_layer"
    if cfg.hidden <= 256:
        return "tiny"
    return "small"


def margins(cfg) -> dict:
    """The fixed margins for cfg's group of models (fp32: the stated tolerances)."""
    if cfg.weight_type == synth.F32:
        return FP32_MARGINS
    return _MARGINS["groups"][margin_group(cfg)]


def logits_tol(cfg):
    return 1e-4 if cfg.weight_type == synth.F32 else 2e-2


def token_margin(cfg):
    """Relative top-2 gap below which an end-to-end greedy id may differ."""
    return margins(cfg)["free_token_margin"]


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


def gpu_kv_positions(kv, seq: int, p0: int, n: int):
    """The device cache's K, V at positions p0 .. p0 + n - 1 of every layer as fp32 [L][n_kv][n][hd]."""
    cfg = kv.model.cfg
    ks, vs = [], []
    for l in range(cfg.n_layers):
        k, v = kv.read_positions(l, seq, p0, n)
        if k.dtype == np.uint16:
            k, v = oracle.bf16_bits_to_f32(k), oracle.bf16_bits_to_f32(v)
        ks.append(k)
        vs.append(v)
    return np.stack(ks), np.stack(vs)


def sync_tf_cache(tf, kv, seq: int, tf_seq: int, upto: int):
    """Copy the GPU's K/V of positions tf.len[tf_seq] .. upto - 1 into the teacher-forced oracle."""
    p0 = tf.len[tf_seq]
    if upto > p0:
        k, v = gpu_kv_positions(kv, seq, p0, upto - p0)
        for l in range(tf.cfg.n_layers):
            tf.K[l][tf_seq][:, p0:upto] = k[l]
            tf.V[l][tf_seq][:, p0:upto] = v[l]
        tf.len[tf_seq] = upto


def check_layers(cfg, tf, tf_seq, token, g_resid, g_z, g_routes, g_logits, g_id, g_k, g_v, what=""):
    """Per-layer comparison of one GPU step (see the module docstring).

    tf: an oracle whose sequence tf_seq holds the GPU's cache for every earlier position (tf.len[tf_seq] is
    the step's position).  g_resid [L][H], g_z [L][E], g_routes [L][K], g_logits [V], g_id: the GPU's
    debug outputs; g_k, g_v [L][n_kv][hd]: the K/V the GPU appended at the position.  Afterwards the oracle's
    cache holds the GPU's K/V at the position and tf.len[tf_seq] has advanced."""
    M = margins(cfg)
    p = tf.len[tf_seq]
    L = cfg.n_layers
    moe = [l for l in range(L) if l >= cfg.n_dense_layers]
    worst = {"z": 0.0, "resid": 0.0, "kv": 0.0}
    adopted = 0
    for l in range(L):
        x = tf.embed(np.array([token], np.int32)) if l == 0 else np.asarray(g_resid[l - 1], np.float64)[None].copy()
        ref = np.asarray(g_routes[l], np.int32)[None] if l in moe else None
        routes, _, flags, gap, z = tf.layer(l, tf_seq, x, p, ref_routes=ref, route_margin=M["layer_route_margin"])
        if l in moe:
            ez = rel_err(g_z[l], z[0])
            worst["z"] = max(worst["z"], ez)
            assert ez <= M["layer_z_bound"], f"{what}layer {l}: router logits rel err {ez:.3g} > {M['layer_z_bound']:.3g}"
            assert flags[0] != 2, (f"{what}layer {l}: experts {sorted(g_routes[l])} != oracle {sorted(routes[0])} "
                                   f"(oracle gap {gap[0]:.3g})")
            adopted += int(flags[0] == 1)
        er = rel_err(g_resid[l], x[0])
        worst["resid"] = max(worst["resid"], er)
        assert er <= M["layer_resid_bound"], f"{what}layer {l}: residual rel err {er:.3g} > {M['layer_resid_bound']:.3g}"
        for j in range(cfg.n_kv_heads):
            ek = max(rel_err(g_k[l][j], tf.K[l][tf_seq][j, p]), rel_err(g_v[l][j], tf.V[l][tf_seq][j, p]))
            worst["kv"] = max(worst["kv"], ek)
            assert ek <= M["layer_kv_bound"], f"{what}layer {l} kv head {j}: appended K/V rel err {ek:.3g}"
        # the cache continues with the GPU's K/V (teacher forcing)
        tf.K[l][tf_seq][:, p] = g_k[l]
        tf.V[l][tf_seq][:, p] = g_v[l]
    cap = max(1, int(ADOPT_FRACTION * len(moe)))
    assert adopted <= cap, f"{what}{adopted} near-tie expert sets adopted (cap {cap})"
    logits, ids, gap = tf.head(np.asarray(g_resid[L - 1], np.float64)[None].copy())
    eh = rel_err(g_logits, logits[0])
    assert eh <= M["head_logit_bound"], f"{what}head: logits rel err {eh:.3g} > {M['head_logit_bound']:.3g}"
    assert g_id == int(ids[0]) or gap[0] < M["head_token_margin"], \
        f"{what}head: token {g_id} != oracle {int(ids[0])} (gap {gap[0]:.3g})"
    tf.len[tf_seq] = p + 1
    print(f"{what}per layer: router {worst['z']:.3g}, residual {worst['resid']:.3g}, kv {worst['kv']:.3g}, "
          f"head {eh:.3g}, adopted {adopted}", flush=True)
    return {"layer_z": worst["z"], "layer_resid": worst["resid"], "layer_kv": worst["kv"], "head": eh,
            "adopted_layer": adopted}


def check_step(cfg, orc, seq, token, g_logits, g_routes, g_id, what="", g_z=None):
    """End-to-end comparison: the oracle's step of sequence `seq` on `token` (following the GPU's expert sets
    where they are a valid top-k within the free margin) against the GPU's logits, routes, router logits and
    id; returns a report."""
    M = margins(cfg)
    r = orc.forward(seq, np.array([token], np.int32), ref_routes=g_routes[None],
                    route_margin=M["free_route_margin"])
    err = rel_err(g_logits, r["logits"][0])
    moe = [l for l in range(cfg.n_layers) if l >= cfg.n_dense_layers]
    flags = r["route_flags"][0, moe] if moe else np.zeros(0)
    assert not (flags == 2).any(), f"{what}routes differ beyond the free margin at layers {np.array(moe)[flags == 2]}"
    ez = 0.0
    if g_z is not None:
        for l in moe:
            ez = max(ez, rel_err(g_z[l], r["router_z"][0, l]))
        assert ez <= M["free_z_bound"], f"{what}router logits rel err {ez:.3g} > {M['free_z_bound']:.3g}"
    assert err <= logits_tol(cfg), f"{what}logits max rel err {err:.3g} > {logits_tol(cfg)}"
    o_id = int(r["ids"][0])
    near = r["gap"][0] < M["free_token_margin"]
    print(f"{what}logits rel err {err:.3g}, router {ez:.3g}, gpu id {g_id}, oracle id {o_id}, "
          f"oracle gap {r['gap'][0]:.3g}, followed expert sets {int((flags == 1).sum())}", flush=True)
    assert g_id == o_id or near, f"{what}token {g_id} != oracle {o_id} (gap {r['gap'][0]:.3g})"
    assert g_id == int(np.argmax(g_logits)) or np.max(g_logits) == g_logits[g_id]
    return {"err": err, "z": ez, "near_route": int((flags == 1).sum()), "near_token": bool(near and g_id != o_id)}


class Stepper:
    """Runs GPU decode steps with debug outputs and checks each against the oracle, end to end (`orc`) and,
    on steps with ``layers=True``, layer by layer against a teacher-forced oracle (`tf`, built lazily with
    the same resident cache as `orc` had at construction: the caller passes it)."""

    def __init__(self, cfg, model, kv, orc, seq=0, tf=None):
        self.cfg, self.model, self.kv, self.orc, self.seq, self.tf = cfg, model, kv, orc, seq, tf
        self.dev = model.device
        self.tok = torch.zeros(kv.batch, dtype=torch.int32, device=self.dev)
        self.out = torch.zeros(kv.batch, dtype=torch.int32, device=self.dev)
        self.dbg, self.t = make_debug(cfg, kv.batch, self.dev, resid=tf is not None)
        self.report = []

    def step(self, token: int, layers: bool = True):
        """One GPU step on `token` and the oracle's step(s) on the same token; returns the checked GPU id."""
        cfg = self.cfg
        self.tok[self.seq] = token
        decode_step_debug(self.model.ctx, self.tok.data_ptr(), self.kv.handle, self.out.data_ptr(), self.dbg)
        sync(self.model.ctx)
        g_logits = self.t["logits"][self.seq].cpu().numpy()
        g_routes = self.t["routes"][self.seq].cpu().numpy()
        g_id = int(self.out[self.seq].item())
        g_z = self.t["router_logits"][self.seq].cpu().numpy()
        rep = {}
        if self.tf is not None and layers:
            p = self.orc.len[self.seq]
            sync_tf_cache(self.tf, self.kv, self.seq, 0, p)
            k, v = gpu_kv_positions(self.kv, self.seq, p, 1)
            rep = check_layers(cfg, self.tf, 0, token, self.t["resid"][self.seq].cpu().numpy(), g_z, g_routes,
                               g_logits, g_id, k[:, :, 0], v[:, :, 0], what=f"position {p}: ")
        rep.update(check_step(cfg, self.orc, self.seq, token, g_logits, g_routes, g_id, g_z=g_z))
        self.report.append(rep)
        return g_id

"""Derive the fixed comparison margins of the GPU parity tests on the CPU alone.

The GPU sums in fp32 in its own order; the oracle sums in double.  Where a
value is rounded to bf16 (the norm outputs, the attention output, the SwiGLU
product, the final norm output, K/V on append) two such sums a few fp32 ulps
apart can land on different sides of a bf16 rounding boundary, and such a
one-ulp flip moves everything downstream.  How far these flips carry is a
property of the oracle's own arithmetic on the seeded inputs, so it is
measured here with the oracle alone: the same steps run once plainly and then
with every pre-rounding value multiplied by (1 + rel * u), u uniform in
[-1, 1) (the oracle's rounding noise), following the plain run's expert
choices so that only rounding differences are measured.

rel = 2^-18 (3.8e-6) is the size of an fp32 reordering difference of a
2048-term dot product (about sqrt(2048) fp32 ulps of the result, 2^-24 * 45).

Two comparisons are derived, each with a factor 3 above the largest drift seen
over every noisy run, step and layer:

Per layer (the test feeds layer l the GPU's own residual after layer l - 1 and
checks that one layer; the head gets the GPU's final residual):
  layer_z_bound      router logits   max|z' - z| / max|z|
  layer_route_margin = max(1e-3, 2 * layer_z_bound): two logits each within the bound can swap order
                       only if their gap is below twice it; a different expert set is accepted only
                       there and only if it is a valid top-k within the margin
  layer_resid_bound  residual after the layer, max|x' - x| / max|x|
  layer_kv_bound     K and V appended at the new position, max|k' - k| / max|k| per kv head
  head_logit_bound   logits from the final residual
  head_token_margin  = max(1e-3, 2 * head_logit_bound): the greedy id may differ only where the
                       oracle's top-2 gap is below it

End to end (the oracle runs the whole step from the token, following the GPU's
tokens and, within the free margins, its expert sets):
  free_z_bound, free_route_margin = 2 * free_z_bound, free_logit_bound,
  free_token_margin = max(1e-3, 2 * free_logit_bound),
  free_kv_bound (the K/V a whole step appends, per layer and kv head)

Margins are derived per group of models (``GROUPS``): the drift grows with depth, so the 49-layer
models get their own, and so do the one-layer, narrowed and two-layer models of the faster tests.

Run:  python3 tests/golden/derive_margins.py  (writes tests/golden/margins.json; a few minutes on
8 cores; the 49-layer bf16 model needs about 35 GB of host memory).
"""
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

REL = 2.0 ** -18
SEEDS = (1, 2, 3)
FACTOR = 3.0
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "margins.json")


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


def drift(cfg, resident, prompt, steps, tok_stream):
    """Plain vs noisy oracle runs: a block of `prompt` tokens after `resident` synthetic positions (the
    prefill's last position compared), then `steps` greedy steps."""
    t0 = time.time()
    layers = {l: synth.layer(cfg, l) for l in range(cfg.n_layers)}
    head = synth.head(cfg)
    kvs = [synth.resident_kv(cfg, l, 0, resident) for l in range(cfg.n_layers)] if resident else []
    cap = resident + prompt + steps + 2
    L = cfg.n_layers
    moe = list(range(cfg.n_dense_layers, L))
    print(f"{cfg.name}: model ready in {time.time() - t0:.0f} s", flush=True)

    def fresh(seed):
        o = oracle.Oracle(cfg, lambda l: layers[l], head, cap=cap)
        for l, (k, v) in enumerate(kvs):
            o.set_resident(0, l, k, v)
        o.len[0] = resident
        if seed:
            o.set_noise(REL, seed)
        return o

    # plain run; after each step, every layer rerun alone with rounding noise from the plain residual
    plain = fresh(0)
    ptoks = synth.tokens(cfg, prompt, stream=tok_stream + 100) if prompt else None
    pr = plain.forward(0, ptoks) if prompt else None
    tok = int(synth.tokens(cfg, 1, stream=tok_stream)[0])
    toks, runs = [], []
    lz, lx, lkv, hl = [], [], [], []
    for s in range(steps):
        p = plain.len[0]
        r = plain.forward(0, np.array([tok], np.int32), resid_all=True)
        runs.append(r)
        toks.append(tok)
        for seed in SEEDS:
            plain.set_noise(REL, 1000 * seed + s)
            for l in range(L):
                xin = plain.embed(np.array([tok], np.int32)) if l == 0 else r["resid"][:, l - 1].copy()
                K0 = plain.K[l][0][:, p].copy()
                V0 = plain.V[l][0][:, p].copy()
                _, _, _, _, z = plain.layer(l, 0, xin, p, ref_routes=r["routes"][:, l], route_margin=np.inf)
                if l in moe:
                    lz.append(rel_err(z[0], r["router_z"][0, l]))
                lx.append(rel_err(xin[0], r["resid"][0, l]))
                for j in range(cfg.n_kv_heads):
                    lkv.append(rel_err(plain.K[l][0][j, p], K0[j]))
                    lkv.append(rel_err(plain.V[l][0][j, p], V0[j]))
                plain.K[l][0][:, p] = K0
                plain.V[l][0][:, p] = V0
            lg, _, _ = plain.head(r["resid"][:, L - 1].copy())
            hl.append(rel_err(lg[0], r["logits"][0]))
            plain.noise = None
        tok = int(r["ids"][0])
        print(f"{cfg.name}: plain step {s}, per-layer drift: z {max(lz) if lz else 0:.3g}, resid {max(lx):.3g}, "
              f"kv {max(lkv):.3g}, head {max(hl):.3g} ({time.time() - t0:.0f} s)", flush=True)
    # whole steps with noise, following the plain run's expert sets
    zd, ld, kd = [], [], []
    zd_layer = np.zeros(L)
    for seed in SEEDS:
        o = fresh(seed)
        if prompt:  # the prompt block's last position
            r = o.forward(0, ptoks, ref_routes=pr["routes"], route_margin=np.inf)
            for l in moe:
                zd.append(rel_err(r["router_z"][-1, l], pr["router_z"][-1, l]))
            ld.append(rel_err(r["logits"][-1], pr["logits"][-1]))
            print(f"{cfg.name}: seed {seed} prompt of {prompt}: logits drift {ld[-1]:.3g}", flush=True)
        for s, tk in enumerate(toks):
            ref = runs[s]
            p = o.len[0]
            r = o.forward(0, np.array([tk], np.int32), ref_routes=ref["routes"], route_margin=np.inf)
            for l in range(L):  # the K/V the whole step appended, against the plain run's
                for j in range(cfg.n_kv_heads):
                    kd.append(rel_err(o.K[l][0][j, p], plain.K[l][0][j, p]))
                    kd.append(rel_err(o.V[l][0][j, p], plain.V[l][0][j, p]))
            for l in moe:
                d = rel_err(r["router_z"][0, l], ref["router_z"][0, l])
                zd.append(d)
                zd_layer[l] = max(zd_layer[l], d)
            ld.append(rel_err(r["logits"][0], ref["logits"][0]))
            print(f"{cfg.name}: seed {seed} step {s}: router drift {max(zd[-len(moe):]):.3g}, "
                  f"logits drift {ld[-1]:.3g} ({time.time() - t0:.0f} s)", flush=True)
    del layers, kvs
    return {"steps": steps, "resident": resident, "prompt": prompt, "seeds": list(SEEDS),
            "layer_z_drift_max": max(lz), "layer_resid_drift_max": max(lx), "layer_kv_drift_max": max(lkv),
            "head_logits_drift_max": max(hl),
            "free_z_drift_max": max(zd), "free_z_drift_median": float(np.median(zd)),
            "free_z_drift_by_layer": [round(float(v), 7) for v in zd_layer],
            "free_logits_drift_max": max(ld), "free_logits_drift_median": float(np.median(ld)),
            "free_kv_drift_max": max(kd)}


# workloads measured, grouped by the tests' model families (the margins of a group hold for its models)
GROUPS = {
    # name: (config, resident positions, prompt tokens, greedy steps, token stream)
    "deep": {  # the 49-layer models
        "int4_49": (synth.CONFIGS["int4_49"], 8022, 0, 3, 11),
        "bf16_49": (synth.CONFIGS["bf16_49"], 2048, 32, 2, 12),
    },
    "one_layer": {"moe_layer": (synth.CONFIGS["moe_layer"], 1024, 0, 2, 7)},
    "small": {  # the narrowed batch-16 model and its bf16 variant
        "int4_b16_small": (synth.CONFIGS["int4_b16_small"], 300, 300, 4, 5),
        "bf16_b16_small": (synth.CONFIGS["int4_b16_small"].replace(name="bf16_b16_small", weight_type=synth.BF16),
                           300, 300, 4, 5),
    },
    "tiny": {  # the two-layer model in bf16 and int4
        "tiny_bf16": (synth.CONFIGS["tiny"].replace(name="tiny_bf16", weight_type=synth.BF16), 0, 8, 6, 3),
        "tiny_int4": (synth.CONFIGS["tiny"].replace(name="tiny_int4", weight_type=synth.INT4G64), 0, 8, 6, 3),
    },
}


def margins(res):
    def worst(key):
        return max(r[key] for r in res.values())

    out = {}
    out["layer_z_bound"] = FACTOR * worst("layer_z_drift_max")
    out["layer_route_margin"] = max(1e-3, 2.0 * out["layer_z_bound"])
    out["layer_resid_bound"] = FACTOR * worst("layer_resid_drift_max")
    out["layer_kv_bound"] = FACTOR * worst("layer_kv_drift_max")
    out["head_logit_bound"] = FACTOR * worst("head_logits_drift_max")
    out["head_token_margin"] = max(1e-3, 2.0 * out["head_logit_bound"])
    out["free_z_bound"] = FACTOR * worst("free_z_drift_max")
    out["free_route_margin"] = 2.0 * out["free_z_bound"]
    out["free_logit_bound"] = FACTOR * worst("free_logits_drift_max")
    out["free_token_margin"] = max(1e-3, 2.0 * out["free_logit_bound"])
    out["free_kv_bound"] = FACTOR * worst("free_kv_drift_max")
    return out


def main():
    out = {"noise_rel": REL, "factor": FACTOR, "groups": {}, "workloads": {}}
    for group in ("tiny", "small", "one_layer", "deep"):
        res = {}
        for name, (cfg, resident, prompt, steps, stream) in GROUPS[group].items():
            res[name] = drift(cfg, resident, prompt, steps, stream)
        out["workloads"].update(res)
        out["groups"][group] = margins(res)
        print(group, json.dumps(out["groups"][group], indent=1), flush=True)
    with open(OUT, "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()

"""Seeded synthetic inputs shared by the oracle and the GPU path.

Nothing here computes any step of the decode method: the module only draws
numbers (``synth.c``) and names the shapes of the workloads.  Every tensor is a
pure function of ``(seed, tensor id, element index)``, so a layer can be
regenerated on its own, which keeps the 49-layer models out of host memory.

RMSNorm weights are 1 in the tiny model (as that configuration states) and
1 + N(0, 0.1), distinct per layer and per norm, everywhere else.

Workloads (shapes from the page "Flint Inference on Apple Silicon: rec
Megakernel and Tempo9 Compared", section 2: 49 layers, 2048-wide residual,
top-6 routing, layers 0 and 1 dense; the remaining sizes are the stated
synthetic configurations of this library):

* ``tiny``      fp32, 2 layers (dense + MoE 8 experts top-2), hidden 256.
* ``moe_layer`` bf16, one MoE layer at full width, 1,024 resident positions.
* ``bf16_49``   bf16, 49 layers, 2,048-token prompt then 256 greedy tokens.
* ``int4_49``   int4 group-64 weights (bf16 embeddings and lm_head),
                8,022 resident positions, 256 greedy tokens.
* ``int4_b16``  ``int4_49`` at batch 16 with ragged lengths in [512, 8192].
* ``int4_b16_small``  a 3-layer, 512-wide narrowing of ``int4_b16`` for fast checks.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None

F32, BF16, INT4G64 = 0, 1, 2
WEIGHT_SIGMA = 0.02
KV_SIGMA = 1.0

# tensor kinds of the stream ids
EMBED, LMHEAD, QKV, OPROJ, DGATE, DUP, DDOWN, ROUTER, EGATE, EUP, EDOWN, KCACHE, VCACHE, TOKENS, LENGTHS = range(1, 16)
ANORM, PNORM, FNORM = range(16, 19)


def build(force: bool = False) -> str:
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", src, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.synth_splitmix64.argtypes = [u64]
        L.synth_splitmix64.restype = u64
        L.synth_normal_f32.argtypes = [u64, u64, dbl, i64, i64, vp]
        L.synth_normal_bf16.argtypes = [u64, u64, dbl, i64, i64, vp]
        L.synth_int4g64.argtypes = [u64, u64, dbl, i64, i64, i64, vp, vp]
        L.synth_uniform_int.argtypes = [u64, u64, i64, i64, i64, i64, vp]
        for f in (L.synth_normal_f32, L.synth_normal_bf16, L.synth_int4g64, L.synth_uniform_int):
            f.restype = None
        _lib = L
    return _lib


def tensor_id(kind: int, layer: int = 0, expert: int = 0) -> int:
    return (kind << 40) | (layer << 20) | expert


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    n_layers: int
    n_dense_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    vocab: int
    dense_inter: int
    n_experts: int
    top_k: int
    expert_inter: int
    weight_type: int
    rope_theta: float = 1e4
    rms_eps: float = 1e-6
    router_renorm: int = 0
    batch: int = 1
    resident: int = 0          # synthetic resident KV positions (values ~N(0, 1))
    prompt: int = 0            # random prompt tokens processed before decoding
    decode: int = 1            # greedy tokens generated
    ragged: tuple = ()         # (lo, hi) of uniform per-sequence lengths, batch > 1
    seed: int = 0
    norm_sigma: float = 0.1    # RMSNorm weights 1 + N(0, norm_sigma), distinct per layer and per norm (0: all 1)

    @property
    def qkv_rows(self):
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def q_dim(self):
        return self.n_q_heads * self.head_dim

    @property
    def n_moe_layers(self):
        return self.n_layers - self.n_dense_layers

    @property
    def act_is_f32(self):
        return self.weight_type == F32

    def replace(self, **kw):
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "tiny": Config("tiny", n_layers=2, n_dense_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                   vocab=1024, dense_inter=512, n_experts=8, top_k=2, expert_inter=128, weight_type=F32,
                   prompt=8, decode=16, norm_sigma=0.0),
    "moe_layer": Config("moe_layer", n_layers=1, n_dense_layers=0, hidden=2048, n_q_heads=16, n_kv_heads=4,
                        head_dim=128, vocab=65536, dense_inter=6144, n_experts=64, top_k=6, expert_inter=768,
                        weight_type=BF16, resident=1024, decode=1),
    "bf16_49": Config("bf16_49", n_layers=49, n_dense_layers=2, hidden=2048, n_q_heads=16, n_kv_heads=4,
                      head_dim=128, vocab=65536, dense_inter=6144, n_experts=64, top_k=6, expert_inter=768,
                      weight_type=BF16, prompt=2048, decode=256),
    "int4_49": Config("int4_49", n_layers=49, n_dense_layers=2, hidden=2048, n_q_heads=16, n_kv_heads=4,
                      head_dim=128, vocab=65536, dense_inter=6144, n_experts=64, top_k=6, expert_inter=768,
                      weight_type=INT4G64, resident=8022, decode=256),
    "int4_b16": Config("int4_b16", n_layers=49, n_dense_layers=2, hidden=2048, n_q_heads=16, n_kv_heads=4,
                       head_dim=128, vocab=65536, dense_inter=6144, n_experts=64, top_k=6, expert_inter=768,
                       weight_type=INT4G64, batch=16, ragged=(512, 8192), decode=1),
    # int4_b16 narrowed so that the oracle runs in seconds (the batched-path parity tests): 3 layers (1 dense),
    # hidden 512, 8 query / 2 kv heads of 128, 16 experts top-4 of 256, lengths uniform in [1, 300]
    "int4_b16_small": Config("int4_b16_small", n_layers=3, n_dense_layers=1, hidden=512, n_q_heads=8,
                             n_kv_heads=2, head_dim=128, vocab=4096, dense_inter=1024, n_experts=16, top_k=4,
                             expert_inter=256, weight_type=INT4G64, batch=16, ragged=(1, 300), decode=1),
}


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def normal_f32(tid: int, n: int, sigma: float, seed: int = 0, off: int = 0) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().synth_normal_f32(seed, tid, sigma, off, n, _ptr(out))
    return out


def normal_bf16(tid: int, n: int, sigma: float, seed: int = 0, off: int = 0) -> np.ndarray:
    out = np.empty(n, np.uint16)
    lib().synth_normal_bf16(seed, tid, sigma, off, n, _ptr(out))
    return out


def int4g64(tid: int, rows: int, cols: int, sigma: float, seed: int = 0, row0: int = 0):
    assert cols % 64 == 0
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 64), np.uint16)
    lib().synth_int4g64(seed, tid, sigma, cols, row0, rows, _ptr(codes), _ptr(scales))
    return codes, scales


def uniform_int(tid: int, n: int, lo: int, hi: int, seed: int = 0, off: int = 0) -> np.ndarray:
    out = np.empty(n, np.int32)
    lib().synth_uniform_int(seed, tid, lo, hi, off, n, _ptr(out))
    return out


def matrix(cfg: Config, kind: int, layer: int, expert: int, rows: int, cols: int, wtype: int | None = None):
    """One weight matrix [rows][cols] ~ N(0, 0.02) in the configuration's format.

    Returns ``{"w": array}`` for fp32 / bf16 (bf16 as raw uint16 bits) or
    ``{"w": codes, "s": scales}`` for int4 group-64.
    """
    wt = cfg.weight_type if wtype is None else wtype
    tid = tensor_id(kind, layer, expert)
    if wt == F32:
        return {"w": normal_f32(tid, rows * cols, WEIGHT_SIGMA, cfg.seed).reshape(rows, cols)}
    if wt == BF16:
        return {"w": normal_bf16(tid, rows * cols, WEIGHT_SIGMA, cfg.seed).reshape(rows, cols)}
    c, s = int4g64(tid, rows, cols, WEIGHT_SIGMA, cfg.seed)
    return {"w": c, "s": s}


def _stack(mats):
    out = {"w": np.stack([m["w"] for m in mats])}
    if "s" in mats[0]:
        out["s"] = np.stack([m["s"] for m in mats])
    return out


def embed_like(cfg: Config, kind: int):
    """Embedding / lm_head [vocab][hidden]: fp32 for the fp32 model, else bf16."""
    wt = F32 if cfg.weight_type == F32 else BF16
    return matrix(cfg, kind, 0, 0, cfg.vocab, cfg.hidden, wtype=wt)["w"]


def norm_weights(cfg: Config, kind: int, layer: int = 0) -> np.ndarray:
    """RMSNorm weights [hidden]: 1 + N(0, norm_sigma) (all 1 when norm_sigma is 0)."""
    if cfg.norm_sigma == 0:
        return np.ones(cfg.hidden, np.float32)
    return (1.0 + normal_f32(tensor_id(kind, layer), cfg.hidden, cfg.norm_sigma, cfg.seed)).astype(np.float32)


def layer(cfg: Config, l: int) -> dict:
    """All weights of layer ``l`` in the canonical layout."""
    H = cfg.hidden
    d = {
        "attn_norm": norm_weights(cfg, ANORM, l),
        "post_norm": norm_weights(cfg, PNORM, l),
        "qkv": matrix(cfg, QKV, l, 0, cfg.qkv_rows, H),
        "o": matrix(cfg, OPROJ, l, 0, H, cfg.q_dim),
    }
    if l < cfg.n_dense_layers:
        d["dense_gate"] = matrix(cfg, DGATE, l, 0, cfg.dense_inter, H)
        d["dense_up"] = matrix(cfg, DUP, l, 0, cfg.dense_inter, H)
        d["dense_down"] = matrix(cfg, DDOWN, l, 0, H, cfg.dense_inter)
    else:
        E = cfg.n_experts
        d["router"] = matrix(cfg, ROUTER, l, 0, E, H)
        d["exp_gate"] = _stack([matrix(cfg, EGATE, l, e, cfg.expert_inter, H) for e in range(E)])
        d["exp_up"] = _stack([matrix(cfg, EUP, l, e, cfg.expert_inter, H) for e in range(E)])
        d["exp_down"] = _stack([matrix(cfg, EDOWN, l, e, H, cfg.expert_inter) for e in range(E)])
    return d


def head(cfg: Config) -> dict:
    return {"embed": embed_like(cfg, EMBED), "lm_head": embed_like(cfg, LMHEAD),
            "final_norm": norm_weights(cfg, FNORM)}


def resident_kv(cfg: Config, l: int, seq: int, n_pos: int):
    """Synthetic resident K and V of one layer and sequence: [n_kv][n_pos][head_dim] ~ N(0, 1).

    bf16 bits for the bf16 / int4 models, fp32 for the fp32 model.
    """
    shape = (cfg.n_kv_heads, n_pos, cfg.head_dim)
    n = int(np.prod(shape))
    f = normal_f32 if cfg.weight_type == F32 else normal_bf16
    k = f(tensor_id(KCACHE, l, seq), n, KV_SIGMA, cfg.seed).reshape(shape)
    v = f(tensor_id(VCACHE, l, seq), n, KV_SIGMA, cfg.seed).reshape(shape)
    return k, v


def tokens(cfg: Config, n: int, stream: int = 0) -> np.ndarray:
    return uniform_int(tensor_id(TOKENS, 0, stream), n, 0, cfg.vocab - 1, cfg.seed)


def lengths(cfg: Config) -> np.ndarray:
    lo, hi = cfg.ragged
    return uniform_int(tensor_id(LENGTHS), cfg.batch, lo, hi, cfg.seed)

"""CPU oracle for the decode step (ctypes wrapper around ``oracle.cpp``).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline of ``bench.py`` may import this package.  The GPU library never does,
and this package imports nothing from it.

The composition below (embedding, then every layer in order, then the head)
follows the operator list of one decode step on the page "Flint Inference on
Apple Silicon: rec Megakernel and Tempo9 Compared", section 2; the per-step
arithmetic lives in ``oracle.cpp``.  A block of known tokens is run
layer-major (all positions through layer l, then layer l + 1), which is the
same function as running the positions one decode step at a time.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16, INT4G64 = 0, 1, 2


def build(force: bool = False) -> str:
    src = os.path.join(_HERE, "oracle.cpp")
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["g++", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c++17", src, "-o", tmp])
        os.replace(tmp, _SO)
    return _SO


class OMat(ctypes.Structure):
    _fields_ = [("wtype", ctypes.c_int32), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("pad", ctypes.c_int32), ("w", ctypes.c_void_p), ("s", ctypes.c_void_p)]


class OCfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("router_renorm", ctypes.c_int32), ("act_bf16", ctypes.c_int32),
                ("pad", ctypes.c_int32), ("rope_theta", ctypes.c_double), ("rms_eps", ctypes.c_double)]


class ONoise(ctypes.Structure):
    _fields_ = [("rel", ctypes.c_double), ("state", ctypes.c_uint64)]


class OLayer(ctypes.Structure):
    _fields_ = [("attn_norm", ctypes.c_void_p), ("post_norm", ctypes.c_void_p), ("qkv", OMat), ("o", OMat),
                ("dense", ctypes.c_int32), ("pad", ctypes.c_int32), ("gate", OMat), ("up", OMat), ("down", OMat),
                ("router", OMat), ("exp_gate", ctypes.c_void_p), ("exp_up", ctypes.c_void_p),
                ("exp_down", ctypes.c_void_p)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.oracle_round_bf16.argtypes = [dbl]
        L.oracle_round_bf16.restype = dbl
        L.oracle_weight.argtypes = [vp, i64, i64]
        L.oracle_weight.restype = dbl
        L.oracle_linear.argtypes = [vp, vp, vp]
        L.oracle_rmsnorm.argtypes = [vp, vp, i32, dbl, i32, vp]
        L.oracle_rope.argtypes = [vp, i32, i32, dbl]
        L.oracle_softmax.argtypes = [vp, i32, vp]
        L.oracle_topk.argtypes = [vp, i32, i32, vp]
        L.oracle_argmax.argtypes = [vp, i64]
        L.oracle_argmax.restype = i32
        L.oracle_attention_head.argtypes = [vp, vp, vp, i32, i32, i64, vp]
        L.oracle_layer.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, vp, dbl, vp, vp, vp, vp, vp, vp]
        L.oracle_layer.restype = i32
        L.oracle_embed.argtypes = [vp, vp, i32, vp]
        L.oracle_head.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, vp]
        for f in (L.oracle_linear, L.oracle_rmsnorm, L.oracle_rope, L.oracle_softmax, L.oracle_topk,
                  L.oracle_attention_head, L.oracle_embed, L.oracle_head):
            f.restype = None
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "contiguous numpy array expected"
    return a.ctypes.data


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def mat(m: dict, wtype: int, keep: list) -> OMat:
    """OMat view of a weight dict {"w": ..., ["s": ...]} (arrays kept alive in ``keep``)."""
    w = np.ascontiguousarray(m["w"])
    keep.append(w)
    s = None
    if wtype == INT4G64:
        s = np.ascontiguousarray(m["s"])
        keep.append(s)
        rows, cols = w.shape[-2], w.shape[-1] * 2
    else:
        rows, cols = w.shape[-2], w.shape[-1]
    return OMat(wtype, rows, cols, 0, _p(w), _p(s))


# ----------------------------------------------------------------- primitives

def round_bf16(v: float) -> float:
    return lib().oracle_round_bf16(float(v))


def weight(m: dict, wtype: int, r: int, c: int) -> float:
    keep = []
    om = mat(m, wtype, keep)
    return lib().oracle_weight(ctypes.byref(om), r, c)


def linear(m: dict, wtype: int, x) -> np.ndarray:
    keep = []
    om = mat(m, wtype, keep)
    x = _f64(x)
    out = np.empty(om.rows, np.float64)
    lib().oracle_linear(ctypes.byref(om), _p(x), _p(out))
    return out


def rmsnorm(x, g, eps: float, round_bf16_out: bool = False) -> np.ndarray:
    x = _f64(x)
    g = np.ascontiguousarray(g, np.float32)
    y = np.empty_like(x)
    lib().oracle_rmsnorm(_p(x), _p(g), x.size, eps, int(round_bf16_out), _p(y))
    return y


def rope(v, pos: int, theta: float) -> np.ndarray:
    v = _f64(v).copy()
    lib().oracle_rope(_p(v), v.size, pos, theta)
    return v


def softmax(z) -> np.ndarray:
    z = _f64(z)
    p = np.empty_like(z)
    lib().oracle_softmax(_p(z), z.size, _p(p))
    return p


def topk(z, k: int) -> np.ndarray:
    z = _f64(z)
    idx = np.empty(k, np.int32)
    lib().oracle_topk(_p(z), z.size, k, _p(idx))
    return idx


def argmax(z) -> int:
    z = _f64(z)
    return lib().oracle_argmax(_p(z), z.size)


def attention_head(q, K, V) -> np.ndarray:
    """q [d], K/V [T][d] (fp32 values)."""
    q = _f64(q)
    K = np.ascontiguousarray(K, np.float32)
    V = np.ascontiguousarray(V, np.float32)
    T, d = K.shape
    out = np.empty(d, np.float64)
    lib().oracle_attention_head(_p(q), _p(K), _p(V), T, d, d, _p(out))
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- the model

class Oracle:
    """Plain CPU model: per-sequence KV store, block (layer-major) forward pass.

    ``cfg``: a ``synth.Config``-like object; ``layer_weights(l)`` returns the
    canonical weight dict of layer l; ``head_weights`` holds embed, lm_head
    and final_norm.  KV capacity ``cap`` positions per sequence.
    """

    def __init__(self, cfg, layer_weights, head_weights, cap: int, batch: int = 1, cache_layers: bool = True):
        self.cfg = cfg
        self._layer_weights = layer_weights
        self._cache = {} if cache_layers else None
        self.head_w = head_weights
        self.cap = cap
        self.batch = batch
        self.wt = cfg.weight_type
        self.bf = 0 if cfg.weight_type == F32 else 1
        self.len = [0] * batch
        shape = (cfg.n_kv_heads, cap, cfg.head_dim)
        self.K = [[np.zeros(shape, np.float32) for _ in range(batch)] for _ in range(cfg.n_layers)]
        self.V = [[np.zeros(shape, np.float32) for _ in range(batch)] for _ in range(cfg.n_layers)]
        self.noise = None
        self.ocfg = OCfg(cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_experts, cfg.top_k,
                         cfg.expert_inter, cfg.router_renorm, self.bf, 0, cfg.rope_theta, cfg.rms_eps)

    def weights(self, l: int) -> dict:
        if self._cache is None:
            return self._layer_weights(l)
        if l not in self._cache:
            self._cache[l] = self._layer_weights(l)
        return self._cache[l]

    def set_resident(self, seq: int, l: int, k: np.ndarray, v: np.ndarray):
        """Resident cache of layer l: k, v [n_kv][n][d], fp32 values or bf16 bits."""
        n = k.shape[1]
        if k.dtype == np.uint16:
            k, v = bf16_bits_to_f32(k), bf16_bits_to_f32(v)
        self.K[l][seq][:, :n] = k
        self.V[l][seq][:, :n] = v

    def _olayer(self, l: int, keep: list) -> OLayer:
        w = self.weights(l)
        cfg, wt = self.cfg, self.wt
        an = np.ascontiguousarray(w["attn_norm"], np.float32)
        pn = np.ascontiguousarray(w["post_norm"], np.float32)
        keep += [an, pn]
        L = OLayer()
        L.attn_norm, L.post_norm = _p(an), _p(pn)
        L.qkv = mat(w["qkv"], wt, keep)
        L.o = mat(w["o"], wt, keep)
        if l < cfg.n_dense_layers:
            L.dense = 1
            L.gate = mat(w["dense_gate"], wt, keep)
            L.up = mat(w["dense_up"], wt, keep)
            L.down = mat(w["dense_down"], wt, keep)
        else:
            L.dense = 0
            L.router = mat(w["router"], wt, keep)
            E = cfg.n_experts
            arrs = []
            for name in ("exp_gate", "exp_up", "exp_down"):
                t = w[name]
                a = (OMat * E)()
                for e in range(E):
                    sub = {"w": t["w"][e]}
                    if "s" in t:
                        sub["s"] = t["s"][e]
                    a[e] = mat(sub, wt, keep)
                keep.append(a)
                arrs.append(ctypes.cast(a, ctypes.c_void_p))
            L.exp_gate, L.exp_up, L.exp_down = arrs
        return L

    def embed(self, toks) -> np.ndarray:
        keep = []
        E = mat({"w": self.head_w["embed"]}, F32 if self.wt == F32 else BF16, keep)
        toks = np.ascontiguousarray(toks, np.int32)
        x = np.empty((toks.size, self.cfg.hidden), np.float64)
        lib().oracle_embed(ctypes.byref(E), _p(toks), toks.size, _p(x))
        return x

    def _noise(self):
        return None if self.noise is None else ctypes.byref(self.noise)

    def set_noise(self, rel: float, seed: int):
        """Rounding noise of relative size `rel` before every bf16 rounding (0: none); see ``oracle.cpp``."""
        self.noise = None if rel == 0 else ONoise(rel, (seed * 0x9E3779B97F4A7C15 + 1) & 0xFFFFFFFFFFFFFFFF or 1)

    def layer(self, l: int, seq: int, x: np.ndarray, p0: int, ref_routes=None, route_margin: float = 0.0):
        """Run layer l over the block x ([n][hidden], modified) at positions p0.. of sequence seq.

        ref_routes [n][top_k]: another implementation's routes; a different set is adopted when it is a
        valid top-k within the fixed relative margin ``route_margin`` (see ``oracle_layer``)."""
        n = x.shape[0]
        keep = []
        L = self._olayer(l, keep)
        K, E = self.cfg.top_k, max(self.cfg.n_experts, 1)
        routes = np.full((n, K), -1, np.int32)
        rw = np.zeros((n, K), np.float32)
        flags = np.zeros(n, np.int32)
        gap = np.full(n, np.inf, np.float32)
        z = np.zeros((n, E), np.float64)
        ref = None if ref_routes is None else np.ascontiguousarray(ref_routes, np.int32).reshape(n, K)
        rc = lib().oracle_layer(ctypes.byref(self.ocfg), ctypes.byref(L), _p(self.K[l][seq]), _p(self.V[l][seq]),
                                self.cap, p0, n, _p(x), _p(ref), route_margin, self._noise(), _p(routes), _p(rw),
                                _p(flags), _p(gap), _p(z))
        if rc != 0:
            raise ValueError("oracle_layer: capacity exceeded")
        return routes, rw, flags, gap, z

    def head(self, x: np.ndarray, want_logits: bool = True):
        keep = []
        lm = mat({"w": self.head_w["lm_head"]}, F32 if self.wt == F32 else BF16, keep)
        gf = np.ascontiguousarray(self.head_w["final_norm"], np.float32)
        n = x.shape[0]
        logits = np.empty((n, self.cfg.vocab), np.float32) if want_logits else None
        ids = np.empty(n, np.int32)
        gap = np.empty(n, np.float64)
        lib().oracle_head(ctypes.byref(self.ocfg), ctypes.byref(lm), _p(gf), _p(x), n, _p(logits), _p(ids), _p(gap),
                          self._noise())
        return logits, ids, gap

    def forward(self, seq: int, toks, ref_routes=None, route_margin: float = 0.0, want_logits: bool = True,
                resid_all: bool = False):
        """Block pass over known tokens at positions len..len+n-1; advances len.

        ref_routes: [n][n_layers][top_k] candidate routes, adopted where they are a valid top-k within
        ``route_margin`` (see ``oracle_layer``).
        Returns a dict with logits [n][vocab], ids [n], gap [n], routes, route_w, route_flags, route_gap
        ([n][n_layers][...], -1 / 0 on dense layers), router_z [n][n_layers][n_experts] (0 on dense layers)
        and, with resid_all, the residual after every layer, resid [n][n_layers][hidden].
        """
        cfg = self.cfg
        toks = np.ascontiguousarray(toks, np.int32)
        n = toks.size
        p0 = self.len[seq]
        x = self.embed(toks)
        Ln, K, E = cfg.n_layers, cfg.top_k, max(cfg.n_experts, 1)
        routes = np.full((n, Ln, K), -1, np.int32)
        rw = np.zeros((n, Ln, K), np.float32)
        flags = np.zeros((n, Ln), np.int32)
        rgap = np.full((n, Ln), np.inf, np.float32)
        rz = np.zeros((n, Ln, E), np.float64)
        resid = np.zeros((n, Ln, cfg.hidden), np.float64) if resid_all else None
        for l in range(Ln):
            ref = None if ref_routes is None else np.ascontiguousarray(np.asarray(ref_routes)[:, l, :])
            r, w, f, g, z = self.layer(l, seq, x, p0, ref, route_margin)
            routes[:, l], rw[:, l], flags[:, l], rgap[:, l] = r, w, f, g
            if l >= cfg.n_dense_layers:
                rz[:, l] = z
            if resid_all:
                resid[:, l] = x
        logits, ids, gap = self.head(x, want_logits)
        self.len[seq] = p0 + n
        return {"logits": logits, "ids": ids, "gap": gap, "routes": routes, "route_w": rw,
                "route_flags": flags, "route_gap": rgap, "router_z": rz, "resid": resid, "x": x}

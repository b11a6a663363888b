"""Device-side plumbing for callers of the library: upload canonical weights,
create a context, and fill a resident KV cache.

Weights arrive as numpy arrays in the canonical layout of ``include/flint.h``
(fp32, bf16 bits as uint16, or int4 codes + bf16 scales), one layer at a
time, so a 49-layer model never has to sit in host memory whole.  PyTorch
provides the device memory and the stream; the library copies the weights
into memory it owns, after which the staging tensors are released.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import (W_F32, W_INT4G64, Config, Debug, Mat, Weights, decode_free, decode_init, kv_alloc, kv_free,
               kv_layer_ptrs, kv_set_lengths)

_hip = None


def hip_memcpy(dst: int, src: int, nbytes: int, kind: int):
    """hipMemcpy through the HIP runtime already loaded by torch (kind: 1 H2D, 2 D2H, 3 D2D)."""
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so.7")  # the process's runtime (torch loaded it first)
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        _hip.hipMemcpy.restype = ctypes.c_int
    rc = _hip.hipMemcpy(dst, src, nbytes, kind)
    if rc != 0:
        raise RuntimeError(f"hipMemcpy failed with {rc}")


def _t(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a)


class DeviceModel:
    """A flint context built from a layer provider.

    ``cfg`` needs the attributes of ``synth.Config`` (dimensions, weight_type,
    rope_theta, rms_eps, router_renorm); ``layer_fn(l)`` returns the weight
    dict of layer l and ``head`` holds embed, lm_head and final_norm.
    """

    def __init__(self, cfg, layer_fn, head: dict, device: str = "cuda", grid: int = 0):
        self.cfg = cfg
        self.device = torch.device(device)
        self.stream = torch.cuda.current_stream(self.device)
        wt = cfg.weight_type
        L, ND = cfg.n_layers, cfg.n_dense_layers
        NM = L - ND
        H, E = cfg.hidden, cfg.n_experts
        staging = {}

        def alloc(name, count, rows, cols):
            if count == 0:
                return
            if wt == W_INT4G64:
                staging[name] = (torch.empty((count, rows, cols // 2), dtype=torch.uint8, device=self.device),
                                 torch.empty((count, rows, cols // 64), dtype=torch.int16, device=self.device))
            else:
                dt = torch.float32 if wt == W_F32 else torch.int16
                staging[name] = (torch.empty((count, rows, cols), dtype=dt, device=self.device), None)

        alloc("qkv", L, cfg.qkv_rows, H)
        alloc("o", L, H, cfg.q_dim)
        alloc("dense_gate", ND, cfg.dense_inter, H)
        alloc("dense_up", ND, cfg.dense_inter, H)
        alloc("dense_down", ND, H, cfg.dense_inter)
        alloc("router", NM, E, H)
        alloc("exp_gate", NM * E, cfg.expert_inter, H)
        alloc("exp_up", NM * E, cfg.expert_inter, H)
        alloc("exp_down", NM * E, H, cfg.expert_inter)
        attn_norm = torch.empty((L, H), dtype=torch.float32, device=self.device)
        post_norm = torch.empty((L, H), dtype=torch.float32, device=self.device)

        def put(name, idx, m):
            w, s = staging[name]
            w[idx].copy_(_t(m["w"]).reshape(w[idx].shape))
            if s is not None:
                s[idx].copy_(_t(m["s"]).reshape(s[idx].shape))

        for l in range(L):
            d = layer_fn(l)
            attn_norm[l].copy_(torch.from_numpy(np.ascontiguousarray(d["attn_norm"], np.float32)))
            post_norm[l].copy_(torch.from_numpy(np.ascontiguousarray(d["post_norm"], np.float32)))
            put("qkv", l, d["qkv"])
            put("o", l, d["o"])
            if l < ND:
                for n in ("dense_gate", "dense_up", "dense_down"):
                    put(n, l, d[n])
            else:
                m = l - ND
                put("router", m, d["router"])
                for n in ("exp_gate", "exp_up", "exp_down"):
                    put(n, slice(m * E, (m + 1) * E), d[n])
            del d
        embed = _t(head["embed"]).to(self.device)
        lm_head = _t(head["lm_head"]).to(self.device)
        final_norm = torch.from_numpy(np.ascontiguousarray(head["final_norm"], np.float32)).to(self.device)

        w = Weights()
        w.embed, w.lm_head, w.final_norm = embed.data_ptr(), lm_head.data_ptr(), final_norm.data_ptr()
        w.attn_norm, w.post_norm = attn_norm.data_ptr(), post_norm.data_ptr()
        for name, (tw, ts) in staging.items():
            setattr(w, name, Mat(tw.data_ptr(), ts.data_ptr() if ts is not None else None))
        c = Config(n_layers=L, n_dense_layers=ND, hidden=H, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                   head_dim=cfg.head_dim, vocab=cfg.vocab, dense_inter=cfg.dense_inter, n_experts=E,
                   top_k=cfg.top_k, expert_inter=cfg.expert_inter, weight_type=wt,
                   router_renorm=cfg.router_renorm, grid=grid, rope_theta=cfg.rope_theta, rms_eps=cfg.rms_eps)
        self.ctx = decode_init(c, w, self.stream.cuda_stream)
        del staging, embed, lm_head, final_norm, attn_norm, post_norm
        self.kvs = []

    def kv(self, batch: int, max_tokens: int) -> "DeviceKV":
        k = DeviceKV(self, batch, max_tokens)
        self.kvs.append(k)
        return k

    def free(self):
        for k in self.kvs:
            k.free()
        self.kvs = []
        if self.ctx:
            decode_free(self.ctx)
            self.ctx = None


class DeviceKV:
    def __init__(self, model: DeviceModel, batch: int, max_tokens: int):
        self.model = model
        self.batch = batch
        self.max_tokens = max_tokens
        self.handle = kv_alloc(model.ctx, batch, max_tokens)

    def load_resident(self, layer: int, seq: int, k: np.ndarray, v: np.ndarray):
        """Write K, V ([n_kv][n][head_dim], fp32 or bf16 bits) at positions 0..n-1 of (layer, seq)."""
        cfg = self.model.cfg
        kp, vp = kv_layer_ptrs(self.handle, layer)
        k = np.ascontiguousarray(k)
        v = np.ascontiguousarray(v)
        eb = k.dtype.itemsize
        n = k.shape[1]
        for j in range(cfg.n_kv_heads):
            off = ((seq * cfg.n_kv_heads + j) * self.max_tokens) * cfg.head_dim * eb
            hip_memcpy(kp + off, k[j].ctypes.data, n * cfg.head_dim * eb, 1)
            hip_memcpy(vp + off, v[j].ctypes.data, n * cfg.head_dim * eb, 1)

    def read_layer(self, layer: int, seq: int, n: int):
        """K, V of (layer, seq) at positions 0..n-1 as numpy [n_kv][n][head_dim] (fp32 or bf16 bits)."""
        return self.read_positions(layer, seq, 0, n)

    def read_positions(self, layer: int, seq: int, p0: int, n: int):
        """K, V of (layer, seq) at positions p0..p0+n-1 as numpy [n_kv][n][head_dim] (fp32 or bf16 bits)."""
        cfg = self.model.cfg
        assert 0 <= p0 and p0 + n <= self.max_tokens
        dt = np.float32 if cfg.weight_type == W_F32 else np.uint16
        kp, vp = kv_layer_ptrs(self.handle, layer)
        eb = np.dtype(dt).itemsize
        k = np.empty((cfg.n_kv_heads, n, cfg.head_dim), dt)
        v = np.empty_like(k)
        for j in range(cfg.n_kv_heads):
            off = ((seq * cfg.n_kv_heads + j) * self.max_tokens + p0) * cfg.head_dim * eb
            hip_memcpy(k[j].ctypes.data, kp + off, n * cfg.head_dim * eb, 2)
            hip_memcpy(v[j].ctypes.data, vp + off, n * cfg.head_dim * eb, 2)
        return k, v

    def set_lengths(self, lengths):
        kv_set_lengths(self.handle, list(lengths))

    def free(self):
        if self.handle:
            kv_free(self.handle)
            self.handle = None


def make_debug(cfg, batch: int, device, logits=True, routes=True, resid=False, phase_ts=False,
               router_logits=None) -> tuple:
    """Allocate the optional outputs of decode_step_debug; returns (Debug, dict of tensors)."""
    t = {}
    dbg = Debug()
    if logits:
        t["logits"] = torch.empty((batch, cfg.vocab), dtype=torch.float32, device=device)
        dbg.logits = t["logits"].data_ptr()
    if routes:
        t["routes"] = torch.empty((batch, cfg.n_layers, cfg.top_k), dtype=torch.int32, device=device)
        t["route_w"] = torch.empty((batch, cfg.n_layers, cfg.top_k), dtype=torch.float32, device=device)
        dbg.routes, dbg.route_w = t["routes"].data_ptr(), t["route_w"].data_ptr()
    if resid:  # residual after every layer
        t["resid"] = torch.empty((batch, cfg.n_layers, cfg.hidden), dtype=torch.float32, device=device)
        dbg.resid = t["resid"].data_ptr()
    if phase_ts:
        t["phase_ts"] = torch.zeros((cfg.n_layers + 1, 16), dtype=torch.int64, device=device)
        dbg.phase_ts = t["phase_ts"].data_ptr()
    if router_logits if router_logits is not None else routes:  # with the routes unless asked otherwise
        t["router_logits"] = torch.zeros((batch, cfg.n_layers, cfg.n_experts), dtype=torch.float32, device=device)
        dbg.router_logits = t["router_logits"].data_ptr()
    return dbg, t

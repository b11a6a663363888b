"""Python binding of the MI355X decode library (``libflint.so``, C ABI in ``include/flint.h``).

Argument marshalling only: every step of the decode path runs in the library's
HIP kernels.  PyTorch is used by callers for device memory and streams; this
module passes raw device pointers (``tensor.data_ptr()``) and the HIP stream
handle through.  Importing the module does not load the library; the first
call does, and raises if ``libflint.so`` has not been built (there is no
fallback path).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libflint.so")

OK, EINVAL, ENOMEM, EHIP, ECAPACITY, ETIMEOUT, ENORESIDENT, EDEVICE = range(8)
W_F32, W_BF16, W_INT4G64 = 0, 1, 2
(FLINT_OK, FLINT_EINVAL, FLINT_ENOMEM, FLINT_EHIP, FLINT_ECAPACITY, FLINT_ETIMEOUT, FLINT_ENORESIDENT,
 FLINT_EDEVICE) = range(8)
STATUS_NAMES = {0: "FLINT_OK", 1: "FLINT_EINVAL", 2: "FLINT_ENOMEM", 3: "FLINT_EHIP", 4: "FLINT_ECAPACITY",
                5: "FLINT_ETIMEOUT", 6: "FLINT_ENORESIDENT", 7: "FLINT_EDEVICE"}

# every symbol include/flint.h declares
EXPORTS = ("flint_decode_init", "flint_decode_free", "flint_kv_alloc", "flint_kv_free", "flint_kv_set_lengths",
           "flint_kv_get_lengths", "flint_kv_tokens", "flint_kv_prefix_match", "flint_kv_layer_ptrs",
           "flint_decode_step", "flint_decode_step_seqs", "flint_decode_step_noalloc",
           "flint_decode_step_debug", "flint_prefill_chunk", "flint_micro_stream_read", "flint_micro_exchange", "flint_micro_exchange_xcd",
           "flint_micro_launch", "flint_sync", "flint_set_wait_limit", "flint_device_info", "flint_last_error")


class FlintError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "n_dense_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "vocab", "dense_inter",
        "n_experts", "top_k", "expert_inter", "weight_type", "router_renorm", "grid")] + [
        ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float)]


class Mat(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class Weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("lm_head", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("attn_norm", ctypes.c_void_p), ("post_norm", ctypes.c_void_p)] + [
        (n, Mat) for n in ("qkv", "o", "dense_gate", "dense_up", "dense_down", "router", "exp_gate", "exp_up",
                           "exp_down")]


class Debug(ctypes.Structure):
    _fields_ = [("logits", ctypes.c_void_p), ("routes", ctypes.c_void_p), ("route_w", ctypes.c_void_p),
                ("resid", ctypes.c_void_p), ("phase_ts", ctypes.c_void_p), ("router_logits", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libflint.so (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is None:
        try:  # bind to the HIP runtime torch ships, so the process has exactly one
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, P = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER
        sig = {
            "flint_decode_init": [P(Config), P(Weights), vp, P(vp)],
            "flint_decode_free": [vp],
            "flint_kv_alloc": [vp, i32, i32, P(vp)],
            "flint_kv_free": [vp],
            "flint_kv_set_lengths": [vp, vp],
            "flint_kv_get_lengths": [vp, vp],
            "flint_kv_tokens": [vp, i32, P(i32), i32],
            "flint_kv_prefix_match": [vp, i32, P(i32), i32, P(i32)],
            "flint_kv_layer_ptrs": [vp, i32, P(vp), P(vp)],
            "flint_decode_step": [vp, vp, vp, vp],
            "flint_decode_step_seqs": [vp, vp, P(i32), i32, vp, vp],
            "flint_decode_step_noalloc": [vp, vp, vp, vp],
            "flint_decode_step_debug": [vp, vp, vp, vp, P(Debug)],
            "flint_prefill_chunk": [vp, vp, i32, vp, i32, vp],
            "flint_micro_stream_read": [vp, ctypes.c_size_t, i32, P(ctypes.c_float)],
            "flint_micro_exchange": [vp, i32, i32, P(ctypes.c_float)],
            "flint_micro_exchange_xcd": [vp, i32, i32, P(ctypes.c_float)],
            "flint_micro_launch": [vp, i32, P(ctypes.c_float)],
            "flint_sync": [vp],
            "flint_set_wait_limit": [vp, ctypes.c_uint32],
            "flint_device_info": [vp, P(i32), P(i32), P(i32)],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.flint_last_error.argtypes = []
        L.flint_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(rc: int):
    if rc != OK:
        raise FlintError(rc, lib().flint_last_error().decode())


def last_error() -> str:
    return lib().flint_last_error().decode()


def decode_init(cfg: Config, weights: Weights, stream: int = 0) -> int:
    ctx = ctypes.c_void_p()
    _check(lib().flint_decode_init(ctypes.byref(cfg), ctypes.byref(weights), ctypes.c_void_p(stream),
                                   ctypes.byref(ctx)))
    return ctx.value


def decode_free(ctx: int):
    _check(lib().flint_decode_free(ctx))


def kv_alloc(ctx: int, batch: int, max_tokens: int) -> int:
    kv = ctypes.c_void_p()
    _check(lib().flint_kv_alloc(ctx, batch, max_tokens, ctypes.byref(kv)))
    return kv.value


def kv_free(kv: int):
    _check(lib().flint_kv_free(kv))


def kv_set_lengths(kv: int, lengths):
    arr = (ctypes.c_int32 * len(lengths))(*lengths)
    _check(lib().flint_kv_set_lengths(kv, ctypes.cast(arr, ctypes.c_void_p)))


def kv_get_lengths(kv: int, batch: int):
    arr = (ctypes.c_int32 * batch)()
    _check(lib().flint_kv_get_lengths(kv, ctypes.cast(arr, ctypes.c_void_p)))
    return list(arr)


def kv_layer_ptrs(kv: int, layer: int):
    k, v = ctypes.c_void_p(), ctypes.c_void_p()
    _check(lib().flint_kv_layer_ptrs(kv, layer, ctypes.byref(k), ctypes.byref(v)))
    return k.value, v.value


def decode_step(ctx: int, tokens_ptr: int, kv: int, out_ptr: int):
    _check(lib().flint_decode_step(ctx, tokens_ptr, kv, out_ptr))


def decode_step_noalloc(ctx: int, tokens_ptr: int, kv: int, out_ptr: int):
    """flint_decode_step with the exchange scratch in the library's fixed device array (allocates nothing)."""
    _check(lib().flint_decode_step_noalloc(ctx, tokens_ptr, kv, out_ptr))


def kv_tokens(kv: int, seq: int, n: int):
    """The first n token ids the sequence's cache holds (-1 where unknown)."""
    arr = (ctypes.c_int32 * max(n, 1))()
    _check(lib().flint_kv_tokens(kv, seq, arr, n))
    return list(arr)[:n]


def kv_prefix_match(kv: int, seq: int, tokens) -> int:
    """Leading tokens of `tokens` that the sequence's cache already holds."""
    arr = (ctypes.c_int32 * max(len(tokens), 1))(*[int(x) for x in tokens])
    out = ctypes.c_int32()
    _check(lib().flint_kv_prefix_match(kv, seq, arr, len(tokens), ctypes.byref(out)))
    return out.value


def micro(ctx: int) -> dict:
    """The measurement helpers: stream-read GB/s (1 GiB, 10 reads), exchange us per round at 64 / 128 / 256
    workgroups (1,000 rounds), the same round confined to each XCD at 256 workgroups, empty-launch us (1,000
    launches)."""
    L, f = lib(), ctypes.c_float()
    _check(L.flint_micro_stream_read(ctx, 1 << 30, 10, ctypes.byref(f)))
    out = {"stream_read_gbs": round(f.value, 1), "exchange_us_per_round": {}}
    for g in (64, 128, 256):
        _check(L.flint_micro_exchange(ctx, g, 1000, ctypes.byref(f)))
        out["exchange_us_per_round"][str(g)] = round(f.value, 3)
    _check(L.flint_micro_exchange_xcd(ctx, 256, 1000, ctypes.byref(f)))
    out["exchange_xcd_us_per_round"] = {"256": round(f.value, 3)}
    _check(L.flint_micro_launch(ctx, 1000, ctypes.byref(f)))
    out["empty_launch_us"] = round(f.value, 3)
    return out


def decode_step_seqs(ctx: int, kv: int, seqs, tokens_ptr: int, out_ptr: int):
    """One greedy step for the listed sequences only (tokens / out_ids indexed by list position)."""
    arr = (ctypes.c_int32 * len(seqs))(*[int(x) for x in seqs])
    _check(lib().flint_decode_step_seqs(ctx, kv, arr, len(seqs), tokens_ptr, out_ptr))


def decode_step_debug(ctx: int, tokens_ptr: int, kv: int, out_ptr: int, dbg: Debug | None):
    _check(lib().flint_decode_step_debug(ctx, tokens_ptr, kv, out_ptr, ctypes.byref(dbg) if dbg is not None else None))


def set_wait_limit(ctx: int, microseconds: int):
    """Bound of every cross-workgroup wait of the persistent kernel (0: the default, 1 s)."""
    _check(lib().flint_set_wait_limit(ctx, microseconds))


def prefill_chunk(ctx: int, kv: int, seq: int, tokens_ptr: int, n: int, out_ptr: int):
    _check(lib().flint_prefill_chunk(ctx, kv, seq, tokens_ptr, n, out_ptr))


def sync(ctx: int):
    _check(lib().flint_sync(ctx))


def device_info(ctx: int):
    g, b, l = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().flint_device_info(ctx, ctypes.byref(g), ctypes.byref(b), ctypes.byref(l)))
    return g.value, b.value, l.value

"""The C ABI without a GPU: the library loads and exports exactly the entry
points include/flint.h declares, the Python structures match the C layout,
and configuration / argument validation fails cleanly before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

import stream_moe_decode_amd as fl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flint.h")
SO = os.path.join(ROOT, "stream_moe_decode_amd", "libflint.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:int|const char\*)\s+(flint_\w+)\s*\(", text, flags=re.M))


def test_header_declarations_match_the_binding():
    decl = declared_functions()
    assert decl == set(fl.EXPORTS), (decl ^ set(fl.EXPORTS))


@pytest.mark.skipif(not os.path.exists(SO), reason="libflint.so not built")
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(SO)
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", SO], capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l and l.split()[-1].startswith("flint_")}
    assert exported == declared_functions(), exported ^ declared_functions()


C_LAYOUT = r"""
#include <stddef.h>
#include <stdio.h>
#include "flint.h"
#define F(S, M) printf(#S "." #M " %zu\n", offsetof(S, M));
int main(void) {
  printf("flint_config %zu\nflint_mat %zu\nflint_weights %zu\nflint_debug %zu\n", sizeof(flint_config),
         sizeof(flint_mat), sizeof(flint_weights), sizeof(flint_debug));
  F(flint_config, grid) F(flint_config, rope_theta) F(flint_config, rms_eps)
  F(flint_weights, attn_norm) F(flint_weights, qkv) F(flint_weights, exp_down)
  F(flint_debug, resid) F(flint_debug, phase_ts)
  return 0;
}
"""


def test_python_structures_match_the_c_layout(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(C_LAYOUT)
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    c = dict(l.rsplit(" ", 1) for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                      check=True).stdout.splitlines())
    assert int(c["flint_config"]) == ctypes.sizeof(fl.Config)
    assert int(c["flint_mat"]) == ctypes.sizeof(fl.Mat)
    assert int(c["flint_weights"]) == ctypes.sizeof(fl.Weights)
    assert int(c["flint_debug"]) == ctypes.sizeof(fl.Debug)
    for key, cls in (("flint_config", fl.Config), ("flint_weights", fl.Weights), ("flint_debug", fl.Debug)):
        for k, v in c.items():
            if k.startswith(key + "."):
                assert getattr(cls, k.split(".")[1]).offset == int(v), k


def _cfg(**kw):
    base = dict(n_layers=2, n_dense_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, vocab=1024,
                dense_inter=512, n_experts=8, top_k=2, expert_inter=128, weight_type=fl.W_F32, router_renorm=0,
                grid=0, rope_theta=1e4, rms_eps=1e-6)
    base.update(kw)
    return fl.Config(**base)


BAD_CONFIGS = [
    (dict(weight_type=7), "weight_type"),
    (dict(n_layers=0), "n_layers"),
    (dict(n_dense_layers=3), "n_dense_layers"),
    (dict(hidden=100), "hidden"),
    (dict(hidden=4096), "hidden"),
    (dict(head_dim=96), "head_dim"),
    (dict(n_q_heads=6, n_kv_heads=4), "n_q_heads"),
    (dict(n_q_heads=32, n_kv_heads=2), "n_q_heads"),
    (dict(n_q_heads=64, head_dim=64), "n_q_heads"),
    (dict(vocab=0), "vocab"),
    (dict(dense_inter=100), "dense_inter"),
    (dict(n_experts=65), "n_experts"),
    (dict(top_k=9), "top_k"),
    (dict(top_k=3, n_experts=2), "top_k"),
    (dict(expert_inter=96), "expert_inter"),
    (dict(weight_type=fl.W_INT4G64, hidden=320), "int4"),
    (dict(rms_eps=-1.0), "rms_eps"),
    (dict(router_renorm=2), "router_renorm"),
    (dict(grid=-1), "grid"),
]


@pytest.mark.skipif(not os.path.exists(SO), reason="libflint.so not built")
@pytest.mark.parametrize("kw,word", BAD_CONFIGS)
def test_bad_configuration_is_rejected_before_any_device_call(kw, word):
    lib = fl.lib()
    out = ctypes.c_void_p(1)
    w = fl.Weights()
    rc = lib.flint_decode_init(ctypes.byref(_cfg(**kw)), ctypes.byref(w), None, ctypes.byref(out))
    assert rc == fl.FLINT_EINVAL
    assert out.value is None  # *out cleared on failure
    assert word in lib.flint_last_error().decode()


@pytest.mark.skipif(not os.path.exists(SO), reason="libflint.so not built")
def test_null_arguments_are_rejected():
    lib = fl.lib()
    w = fl.Weights()
    assert lib.flint_decode_init(ctypes.byref(_cfg()), ctypes.byref(w), None, None) == fl.FLINT_EINVAL
    out = ctypes.c_void_p()
    assert lib.flint_decode_init(None, ctypes.byref(w), None, ctypes.byref(out)) == fl.FLINT_EINVAL
    assert lib.flint_decode_init(ctypes.byref(_cfg()), None, None, ctypes.byref(out)) == fl.FLINT_EINVAL
    assert lib.flint_decode_free(None) == fl.FLINT_OK
    assert lib.flint_kv_free(None) == fl.FLINT_OK
    assert lib.flint_kv_alloc(None, 1, 16, ctypes.byref(out)) == fl.FLINT_EINVAL
    assert lib.flint_decode_step(None, None, None, None) == fl.FLINT_EINVAL
    assert lib.flint_decode_step_seqs(None, None, None, 0, None, None) == fl.FLINT_EINVAL
    assert lib.flint_kv_tokens(None, 0, None, 0) == fl.FLINT_EINVAL
    assert lib.flint_micro_stream_read(None, 1 << 20, 1, None) == fl.FLINT_EINVAL
    assert lib.flint_micro_exchange(None, 2, 1, None) == fl.FLINT_EINVAL
    assert lib.flint_micro_launch(None, 1, None) == fl.FLINT_EINVAL
    assert lib.flint_kv_prefix_match(None, 0, None, 0, None) == fl.FLINT_EINVAL
    assert lib.flint_prefill_chunk(None, None, 0, None, 1, None) == fl.FLINT_EINVAL
    assert lib.flint_sync(None) == fl.FLINT_EINVAL
    assert lib.flint_kv_set_lengths(None, None) == fl.FLINT_EINVAL
    assert lib.flint_kv_get_lengths(None, None) == fl.FLINT_EINVAL
    assert lib.flint_last_error() != b""

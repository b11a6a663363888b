"""The oracle pins must catch plausible mistakes: each case below plants one
mistake in a copy of ``oracle/oracle.cpp`` (on the CPU, in a temporary
directory), rebuilds that copy and runs ``test_oracle_pins.py`` against it;
at least one pin has to fail.  The mistakes are the ones a reader could make
when writing the operators of the decode step listed in section 2 of the page
"Flint Inference on Apple Silicon: rec Megakernel and Tempo9 Compared": the
sign in SiLU, SiLU on the wrong branch of SwiGLU, the expert outputs averaged
instead of weighted by the router, attention that leaves out the new token,
the wrong norm weights, the RoPE rotation turned the other way, ties in the
top-k broken towards the higher index, and the scale of the scores."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# name: (text of oracle.cpp, its replacement[, extra replacement])
MUTATIONS = {
    "silu_sign": ("return u / (1.0 + exp(-u));", "return u / (1.0 + exp(u));"),
    "silu_on_up_dense": ("hh[e] = RN(silu(g[e]) * u[e], bf, noise);", "hh[e] = RN(silu(u[e]) * g[e], bf, noise);"),
    "silu_on_up_experts": ("hh[r] = RN(silu(g[r]) * u[r], bf, noise);", "hh[r] = RN(silu(u[r]) * g[r], bf, noise);"),
    "combine_mean": ("acc[r] += w[j] * y[r];", "acc[r] += y[r] / K;"),
    "attention_excludes_self": ("Vc + (size_t)j * cap * d, p + 1, d, d,", "Vc + (size_t)j * cap * d, p > 0 ? p : 1, d, d,"),
    "post_norm_is_attn_norm": ("rmsnorm_n(xi, L->post_norm, H,", "rmsnorm_n(xi, L->attn_norm, H,"),
    "final_norm_ignored": ("rmsnorm_n(x + (size_t)i * H, gf, H,", "rmsnorm_n(x + (size_t)i * H, ones.data(), H,",
                           ("  std::vector<double> f(H), l(V);",
                            "  std::vector<double> f(H), l(V);\n  std::vector<float> ones(H, 1.0f);")),
    "rope_turned_back": ("v[i] = a * c - b * s;", "v[i] = a * c + b * s;"),
    "topk_ties_higher_index": ("if (!used[i] && (best < 0 || z[i] > z[best])) best = i;",
                               "if (!used[i] && (best < 0 || z[i] >= z[best])) best = i;"),
    "score_scale_1_over_d": ("double scale = 1.0 / sqrt((double)d);", "double scale = 1.0 / (double)d;"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_a_planted_mistake(name, tmp_path):
    spec = MUTATIONS[name]
    src = open(os.path.join(ROOT, "oracle", "oracle.cpp")).read()
    assert spec[0] in src, f"mutation {name} no longer applies"
    src = src.replace(spec[0], spec[1])
    if len(spec) > 2:
        assert spec[2][0] in src
        src = src.replace(spec[2][0], spec[2][1])
    d = tmp_path / "repo"
    (d / "tests").mkdir(parents=True)
    shutil.copytree(os.path.join(ROOT, "oracle"), d / "oracle", ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "synth"), d / "synth", ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copy(os.path.join(ROOT, "tests", "test_oracle_pins.py"), d / "tests")
    (d / "tests" / "conftest.py").write_text(
        "import os, sys\nsys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))\n")
    (d / "oracle" / "oracle.cpp").write_text(src)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_oracle_pins.py"],
                       cwd=d, capture_output=True, text=True, timeout=600)
    failed = [l for l in r.stdout.splitlines() if l.startswith("FAILED")]
    print(name, "caught by", failed)
    assert failed, f"no pin fails with the mistake {name!r} planted in the oracle"

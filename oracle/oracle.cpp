/*
 * CPU oracle for one greedy decode step (and a block of steps) of the top-k
 * mixture-of-experts transformer described on the page "Flint Inference on
 * Apple Silicon: rec Megakernel and Tempo9 Compared" (section 2, the list of
 * operators inside one decode step: input RMSNorm, QKV projection, RoPE, KV
 * writes, attention over the resident cache, o_proj, post-attention RMSNorm,
 * router, top-6, expert gate/up and down, dense MLP on layers 0 and 1, final
 * norm, lm_head, argmax).
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU baseline may load this file.  It shares nothing with the GPU library:
 * plain scalar loops, double accumulation, every step written out in the
 * order of the definition.  The page states that the persistent kernel's
 * gain comes from fusion and fewer memory round trips (section 3), i.e. the
 * fused kernel computes the same function up to floating-point order, so the
 * oracle is the plain definition of the step.
 *
 * Readings where the page is silent (all listed in the design notes):
 *  - RMSNorm y_i = x_i / sqrt(mean(x^2) + eps) * g_i.
 *  - RoPE rotates pairs (i, i + d/2) of every q and k head by p * base^(-2i/d),
 *    p = 0-based absolute position of the token.
 *  - attention: scale 1/sqrt(d), causal including the new token, head h reads
 *    kv head h / (n_q / n_kv).
 *  - MLP: down(silu(gate . b) * (up . b)), silu(u) = u / (1 + e^-u).
 *  - router: softmax over all experts, the k largest logits selected (equal
 *    logits: lower index first), weight of a selected expert = its softmax
 *    probability (optionally renormalised over the selection).
 *  - bf16 models round to bf16 (nearest even, from fp32) exactly these
 *    tensors: the RMSNorm outputs, the attention output o, the SwiGLU product
 *    h and K/V when appended.  The residual, q, scores, router logits and
 *    logits stay wide.
 *  - int4 group-64 weights dequantise as scale * (nibble - 8).
 *
 * Rounding noise (off unless a caller passes an ONoise): every value about to
 * be rounded to bf16 is first multiplied by (1 + rel * u), u uniform in
 * [-1, 1) from a xorshift64* stream (Vigna, "An experimental exploration of
 * Marsaglia's xorshift generators, scrambled", 2016).  It models an
 * implementation whose fp32 sums land a few ulps away from the double sums,
 * and only serves to measure on the CPU how far such rounding differences
 * carry through the layers (the tolerances of the GPU comparison are derived
 * from it).  With no ONoise the functions below are the plain definition.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

extern "C" {

enum { O_F32 = 0, O_BF16 = 1, O_INT4G64 = 2 };

struct OMat {
  int32_t wtype, rows, cols, pad;
  const void* w;       /* F32: float[rows][cols]; BF16: uint16[rows][cols]; INT4G64: uint8[rows][cols/2] */
  const uint16_t* s;   /* INT4G64 only: bf16 scales [rows][cols/64] */
};

struct OCfg {
  int32_t hidden, n_q_heads, n_kv_heads, head_dim;
  int32_t n_experts, top_k, inter, router_renorm;
  int32_t act_bf16, pad;
  double rope_theta, rms_eps;
};

struct ONoise {
  double rel;          /* relative size of the perturbation before each bf16 rounding */
  uint64_t state;      /* xorshift64* state (non-zero), advanced by every use */
};

struct OLayer {
  const float* attn_norm;
  const float* post_norm;
  OMat qkv, o;
  int32_t dense, pad;
  OMat gate, up, down;          /* dense MLP (dense != 0) */
  OMat router;                  /* MoE (dense == 0) */
  const OMat* exp_gate;         /* [n_experts] */
  const OMat* exp_up;
  const OMat* exp_down;
};

static double bf16_bits_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* R(v): round to bf16, nearest even, from the fp32 value of v. */
double oracle_round_bf16(double v) {
  float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  u &= 0xFFFF0000u;
  memcpy(&f, &u, 4);
  return (double)f;
}

static inline double R(double v, int bf16) { return bf16 ? oracle_round_bf16(v) : v; }

/* Uniform deviate in [-1, 1) from the noise stream. */
static double noise_u(ONoise* nz) {
  uint64_t x = nz->state;
  x ^= x >> 12;
  x ^= x << 25;
  x ^= x >> 27;
  nz->state = x;
  return (double)((x * 0x2545F4914F6CDD1Dull) >> 11) * (1.0 / 9007199254740992.0) * 2.0 - 1.0;
}

/* R with the optional rounding noise (only where a value is rounded to bf16). */
static inline double RN(double v, int bf16, ONoise* nz) {
  if (nz && bf16 && nz->rel != 0.0) v *= 1.0 + nz->rel * noise_u(nz);
  return R(v, bf16);
}

/* Dequantised weight W[r][c]. */
double oracle_weight(const OMat* m, int64_t r, int64_t c) {
  switch (m->wtype) {
    case O_F32: return (double)((const float*)m->w)[r * m->cols + c];
    case O_BF16: return bf16_bits_to_double(((const uint16_t*)m->w)[r * m->cols + c]);
    default: {
      uint8_t byte = ((const uint8_t*)m->w)[r * (m->cols / 2) + c / 2];
      int u = (c & 1) ? (byte >> 4) : (byte & 15);
      double s = bf16_bits_to_double(m->s[r * (m->cols / 64) + c / 64]);
      return s * (double)(u - 8);
    }
  }
}

/* out = W in, out[r] = sum_c W[r][c] in[c]. */
void oracle_linear(const OMat* m, const double* in, double* out) {
#pragma omp parallel for schedule(static)
  for (int32_t r = 0; r < m->rows; ++r) {
    double acc = 0.0;
    for (int32_t c = 0; c < m->cols; ++c) acc += oracle_weight(m, r, c) * in[c];
    out[r] = acc;
  }
}

/* y_i = R(x_i / sqrt(mean_j x_j^2 + eps) * g_i). */
static void rmsnorm_n(const double* x, const float* g, int32_t n, double eps, int32_t round_bf16, ONoise* nz,
                      double* y) {
  double ss = 0.0;
  for (int32_t i = 0; i < n; ++i) ss += x[i] * x[i];
  double inv = 1.0 / sqrt(ss / n + eps);
  for (int32_t i = 0; i < n; ++i) y[i] = RN(x[i] * inv * (double)g[i], round_bf16, nz);
}
void oracle_rmsnorm(const double* x, const float* g, int32_t n, double eps, int32_t round_bf16, double* y) {
  rmsnorm_n(x, g, n, eps, round_bf16, nullptr, y);
}

/* Rotate pairs (i, i + d/2) of one head by pos * theta^(-2i/d). */
void oracle_rope(double* v, int32_t d, int32_t pos, double theta) {
  for (int32_t i = 0; i < d / 2; ++i) {
    double ang = (double)pos * pow(theta, -2.0 * (double)i / (double)d);
    double c = cos(ang), s = sin(ang);
    double a = v[i], b = v[i + d / 2];
    v[i] = a * c - b * s;
    v[i + d / 2] = b * c + a * s;
  }
}

/* p = softmax(z), max-subtracted. */
void oracle_softmax(const double* z, int32_t n, double* p) {
  double m = z[0];
  for (int32_t i = 1; i < n; ++i) m = z[i] > m ? z[i] : m;
  double sum = 0.0;
  for (int32_t i = 0; i < n; ++i) {
    p[i] = exp(z[i] - m);
    sum += p[i];
  }
  for (int32_t i = 0; i < n; ++i) p[i] /= sum;
}

/* idx = the k largest z, in descending order; equal values: lower index first. */
void oracle_topk(const double* z, int32_t n, int32_t k, int32_t* idx) {
  std::vector<char> used(n, 0);
  for (int32_t j = 0; j < k; ++j) {
    int32_t best = -1;
    for (int32_t i = 0; i < n; ++i)
      if (!used[i] && (best < 0 || z[i] > z[best])) best = i;
    used[best] = 1;
    idx[j] = best;
  }
}

/* argmax, equal values: lowest index. */
int32_t oracle_argmax(const double* z, int64_t n) {
  int64_t best = 0;
  for (int64_t i = 1; i < n; ++i)
    if (z[i] > z[best]) best = i;
  return (int32_t)best;
}

/* One head over T positions: out = sum_t softmax_t(q.K_t / sqrt(d)) V_t.
 * Row t of K (V) starts at K + t * stride. */
void oracle_attention_head(const double* q, const float* K, const float* V, int32_t T, int32_t d, int64_t stride,
                           double* out) {
  std::vector<double> s(T), p(T);
  double scale = 1.0 / sqrt((double)d);
  for (int32_t t = 0; t < T; ++t) {
    double acc = 0.0;
    for (int32_t i = 0; i < d; ++i) acc += q[i] * (double)K[t * stride + i];
    s[t] = acc * scale;
  }
  oracle_softmax(s.data(), T, p.data());
  for (int32_t i = 0; i < d; ++i) out[i] = 0.0;
  for (int32_t t = 0; t < T; ++t)
    for (int32_t i = 0; i < d; ++i) out[i] += p[t] * (double)V[t * stride + i];
}

static double silu(double u) { return u / (1.0 + exp(-u)); }

/*
 * One layer for positions p0 .. p0 + n - 1 of one sequence, in position order.
 * x: [n][hidden] residual in/out.  Kc, Vc: this layer's cache of this
 * sequence, [n_kv][cap][head_dim]; positions < p0 must already be there, the
 * new positions are appended.
 *
 * Routing (MoE layers): the oracle selects its own top-k.  If ref_routes
 * ([n][top_k]) is given and names a different set, that set is accepted only
 * when it is a valid top-k within the fixed relative margin route_margin:
 * min over the set >= max outside the set - route_margin * max|z|, which
 * can only hold where the oracle's own k-th / (k+1)-th gap is below the
 * margin.  Then it is adopted (flag 1); otherwise the oracle keeps its own set
 * (flag 2).  Equal sets: flag 0.
 * routes_out [n][top_k], rw_out [n][top_k], flags_out [n], gap_out [n]
 * ((z_(k) - z_(k+1)) / max|z|) and z_out [n][n_experts] (router logits) may
 * each be NULL.  noise: optional rounding noise (NULL = none).
 */
int32_t oracle_layer(const OCfg* cfg, const OLayer* L, float* Kc, float* Vc, int32_t cap, int32_t p0, int32_t n,
                     double* x, const int32_t* ref_routes, double route_margin, ONoise* noise, int32_t* routes_out,
                     float* rw_out, int32_t* flags_out, float* gap_out, double* z_out) {
  const int32_t H = cfg->hidden, d = cfg->head_dim, nq = cfg->n_q_heads, nkv = cfg->n_kv_heads;
  const int32_t group = nq / nkv, bf = cfg->act_bf16;
  if (p0 + n > cap) return 1;
  std::vector<double> a(H), qkv((size_t)(nq + 2 * nkv) * d), o((size_t)nq * d), y(H), b(H);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t p = p0 + i;
    double* xi = x + (size_t)i * H;
    /* attention half */
    rmsnorm_n(xi, L->attn_norm, H, cfg->rms_eps, bf, noise, a.data());
    oracle_linear(&L->qkv, a.data(), qkv.data());
    double* q = qkv.data();
    double* k = q + (size_t)nq * d;
    double* v = k + (size_t)nkv * d;
    for (int32_t h = 0; h < nq; ++h) oracle_rope(q + (size_t)h * d, d, p, cfg->rope_theta);
    for (int32_t j = 0; j < nkv; ++j) oracle_rope(k + (size_t)j * d, d, p, cfg->rope_theta);
    for (int32_t j = 0; j < nkv; ++j)
      for (int32_t e = 0; e < d; ++e) {
        Kc[((size_t)j * cap + p) * d + e] = (float)RN(k[(size_t)j * d + e], bf, noise);
        Vc[((size_t)j * cap + p) * d + e] = (float)RN(v[(size_t)j * d + e], bf, noise);
      }
    for (int32_t h = 0; h < nq; ++h) {
      int32_t j = h / group;
      oracle_attention_head(q + (size_t)h * d, Kc + (size_t)j * cap * d, Vc + (size_t)j * cap * d, p + 1, d, d,
                            o.data() + (size_t)h * d);
    }
    for (size_t e = 0; e < o.size(); ++e) o[e] = RN(o[e], bf, noise);
    oracle_linear(&L->o, o.data(), y.data());
    for (int32_t e = 0; e < H; ++e) xi[e] += y[e];
    /* MLP half */
    rmsnorm_n(xi, L->post_norm, H, cfg->rms_eps, bf, noise, b.data());
    if (L->dense) {
      const int32_t I = L->gate.rows;
      std::vector<double> g(I), u(I), hh(I);
      oracle_linear(&L->gate, b.data(), g.data());
      oracle_linear(&L->up, b.data(), u.data());
      for (int32_t e = 0; e < I; ++e) hh[e] = RN(silu(g[e]) * u[e], bf, noise);
      oracle_linear(&L->down, hh.data(), y.data());
      for (int32_t e = 0; e < H; ++e) xi[e] += y[e];
    } else {
      const int32_t E = cfg->n_experts, K = cfg->top_k;
      std::vector<double> z(E), pr(E);
      std::vector<int32_t> sel(K);
      oracle_linear(&L->router, b.data(), z.data());
      if (z_out)
        for (int32_t e = 0; e < E; ++e) z_out[(size_t)i * E + e] = z[e];
      oracle_topk(z.data(), E, K, sel.data());
      double zmax = 0.0;
      for (int32_t e = 0; e < E; ++e) zmax = fabs(z[e]) > zmax ? fabs(z[e]) : zmax;
      if (gap_out) {
        std::vector<int32_t> s1(K + 1 <= E ? K + 1 : K);
        oracle_topk(z.data(), E, (int32_t)s1.size(), s1.data());
        double gap = (int32_t)s1.size() > K ? z[s1[K - 1]] - z[s1[K]] : INFINITY;
        gap_out[i] = (float)(zmax > 0 ? gap / zmax : gap);
      }
      int32_t flag = 0;
      if (ref_routes) {
        const int32_t* ref = ref_routes + (size_t)i * K;
        std::vector<char> in_ref(E, 0), in_own(E, 0);
        int32_t valid = 1;
        for (int32_t j = 0; j < K; ++j) {
          if (ref[j] < 0 || ref[j] >= E || in_ref[ref[j]]) valid = 0;
          else in_ref[ref[j]] = 1;
          in_own[sel[j]] = 1;
        }
        int32_t same = valid;
        for (int32_t e = 0; e < E && same; ++e) same = in_ref[e] == in_own[e];
        if (!same) {
          if (valid) {
            double min_in = INFINITY, max_out = -INFINITY;
            for (int32_t e = 0; e < E; ++e) {
              if (in_ref[e]) min_in = std::min(min_in, z[e]);
              else max_out = std::max(max_out, z[e]);
            }
            valid = min_in >= max_out - route_margin * zmax;
          }
          if (valid) {
            flag = 1;
            for (int32_t j = 0; j < K; ++j) sel[j] = ref[j];
          } else {
            flag = 2;
          }
        }
      }
      oracle_softmax(z.data(), E, pr.data());
      std::vector<double> w(K);
      double wsum = 0.0;
      for (int32_t j = 0; j < K; ++j) {
        w[j] = pr[sel[j]];
        wsum += w[j];
      }
      if (cfg->router_renorm)
        for (int32_t j = 0; j < K; ++j) w[j] /= wsum;
      const int32_t I = cfg->inter;
      std::vector<double> g(I), u(I), hh(I), acc(H, 0.0);
      for (int32_t j = 0; j < K; ++j) {
        const int32_t e = sel[j];
        oracle_linear(&L->exp_gate[e], b.data(), g.data());
        oracle_linear(&L->exp_up[e], b.data(), u.data());
        for (int32_t r = 0; r < I; ++r) hh[r] = RN(silu(g[r]) * u[r], bf, noise);
        oracle_linear(&L->exp_down[e], hh.data(), y.data());
        for (int32_t r = 0; r < H; ++r) acc[r] += w[j] * y[r];
      }
      for (int32_t r = 0; r < H; ++r) xi[r] += acc[r];
      if (routes_out)
        for (int32_t j = 0; j < K; ++j) routes_out[(size_t)i * K + j] = sel[j];
      if (rw_out)
        for (int32_t j = 0; j < K; ++j) rw_out[(size_t)i * K + j] = (float)w[j];
      if (flags_out) flags_out[i] = flag;
    }
  }
  return 0;
}

/* x_i = E[tokens_i] (embedding row, fp32 or bf16). */
void oracle_embed(const OMat* E, const int32_t* tok, int32_t n, double* x) {
  for (int32_t i = 0; i < n; ++i)
    for (int32_t c = 0; c < E->cols; ++c) x[(size_t)i * E->cols + c] = oracle_weight(E, tok[i], c);
}

/*
 * Final norm, lm_head and argmax for n positions.  logits [n][vocab] (fp32,
 * may be NULL), ids [n], gap [n] = (l_(1) - l_(2)) / max|l| (may be NULL),
 * noise: optional rounding noise (NULL = none).
 */
void oracle_head(const OCfg* cfg, const OMat* lm, const float* gf, const double* x, int32_t n, float* logits,
                 int32_t* ids, double* gap, ONoise* noise) {
  const int32_t H = cfg->hidden, V = lm->rows;
  std::vector<double> f(H), l(V);
  for (int32_t i = 0; i < n; ++i) {
    rmsnorm_n(x + (size_t)i * H, gf, H, cfg->rms_eps, cfg->act_bf16, noise, f.data());
    oracle_linear(lm, f.data(), l.data());
    ids[i] = oracle_argmax(l.data(), V);
    if (logits)
      for (int32_t r = 0; r < V; ++r) logits[(size_t)i * V + r] = (float)l[r];
    if (gap) {
      double top = l[ids[i]], second = -INFINITY, amax = 0.0;
      for (int32_t r = 0; r < V; ++r) {
        if (r != ids[i] && l[r] > second) second = l[r];
        amax = fabs(l[r]) > amax ? fabs(l[r]) : amax;
      }
      gap[i] = amax > 0 ? (top - second) / amax : INFINITY;
    }
  }
}

} /* extern "C" */

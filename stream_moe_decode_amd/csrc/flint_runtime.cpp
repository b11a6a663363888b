// Host runtime behind the C ABI of include/flint.h: argument checks, the
// library-owned copies of the weights, the KV cache, the RoPE table (computed
// in double), the kernel's scratch, and one persistent-kernel launch per
// sequence and step.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <new>
#include <string>
#include <vector>

#include "../../include/flint.h"
#include "flint_internal.h"

using namespace flint;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

#define HIPCHECK(x)                                                                              \
  do {                                                                                           \
    hipError_t e_ = (x);                                                                         \
    if (e_ != hipSuccess) return fail(FLINT_EHIP, "%s failed: %s", #x, hipGetErrorString(e_)); \
  } while (0)

size_t elem_bytes_act(int wt) { return wt == FLINT_W_F32 ? 4 : 2; }

// Bytes of a [rows][in] matrix in the layer weight format (codes only for int4).
size_t mat_bytes(int wt, size_t rows, size_t in) {
  return wt == FLINT_W_F32 ? rows * in * 4 : (wt == FLINT_W_BF16 ? rows * in * 2 : rows * in / 2);
}
size_t scale_bytes(int wt, size_t rows, size_t in) { return wt == FLINT_W_INT4G64 ? rows * (in / 64) * 2 : 0; }

}  // namespace

struct flint_ctx {
  flint_config cfg;
  hipStream_t stream;
  int device;
  int grid;
  int S;
  std::vector<void*> allocs;  // library-owned device memory
  KStatic base;               // weights, dimensions and scratch (host copy)
  KStatic* kdev;              // the same, in device memory, read by the kernel
  bool stat;                  // the compile-time 2048-wide kernel applies
  bool batch_ok;              // batches of several sequences take the batched MFMA path
  int batch_min;              // fewest sequences of a step that take it (FLINT_BATCH_MIN overrides)
  bool tiled;                 // the batched path's tiled weight copies exist
  const uint8_t* lmt;         // lm_head in the tiled layout (with `tiled`)
  uint32_t* herr_host;        // host-mapped error word
  uint64_t* xbuf;
  size_t xbuf_words;          // exchange slots; the argmax hand-off counters follow (16 words)
  uint64_t* na_ptr;           // this device's fixed scratch array (flint_decode_step_noalloc), or null
  hipError_t na_status;       // result of finding it
  uint64_t launches;
  int live_kv;
  uint32_t resync_gen;        // bumped when a reported error may have left device lengths behind the host's
};

struct flint_kv {
  flint_ctx* ctx;
  int batch, max_tokens;
  void* k;
  void* v;
  int32_t* len;
  int32_t* hist;              // [batch][max_tokens] token consumed at each position, -1 where unknown
  float* rope;
  std::vector<int32_t> hlen;
  void* bscratch;             // scratch of the batched path (batch > 1), null otherwise
  BArgs bargs;                // its buffers and the pass-invariant arguments
  void* pscratch;             // scratch of the long-chunk prefill (made by its first use), null otherwise
  BArgs pargs;                // bargs with the buffers pointed at pscratch
  uint32_t resync_gen;        // ctx->resync_gen when hlen was last known to match the device lengths
};

namespace {

int dalloc(flint_ctx* c, void** p, size_t bytes) {
  *p = nullptr;
  if (bytes == 0) return FLINT_OK;
  hipError_t e = hipMalloc(p, bytes);
  if (e != hipSuccess) return fail(FLINT_ENOMEM, "hipMalloc(%zu bytes): %s", bytes, hipGetErrorString(e));
  c->allocs.push_back(*p);
  return FLINT_OK;
}

void release(flint_ctx* c) {
  for (void* p : c->allocs) (void)hipFree(p);
  c->allocs.clear();
  if (c->herr_host) (void)hipHostFree(c->herr_host);
  c->herr_host = nullptr;
}

int check_config(const flint_config* c) {
  if (!c) return fail(FLINT_EINVAL, "cfg is NULL");
  if (c->weight_type < FLINT_W_F32 || c->weight_type > FLINT_W_INT4G64)
    return fail(FLINT_EINVAL, "weight_type %d unknown", c->weight_type);
  if (c->n_layers < 1 || c->n_layers > 120) return fail(FLINT_EINVAL, "n_layers %d not in [1, 120]", c->n_layers);
  if (c->n_dense_layers < 0 || c->n_dense_layers > c->n_layers)
    return fail(FLINT_EINVAL, "n_dense_layers %d not in [0, n_layers]", c->n_dense_layers);
  if (c->hidden < 64 || c->hidden > MAX_H || c->hidden % 64)
    return fail(FLINT_EINVAL, "hidden %d must be a multiple of 64 in [64, %d]", c->hidden, MAX_H);
  if (c->head_dim != 64 && c->head_dim != 128) return fail(FLINT_EINVAL, "head_dim %d must be 64 or 128", c->head_dim);
  if (c->n_kv_heads < 1 || c->n_q_heads < c->n_kv_heads || c->n_q_heads % c->n_kv_heads ||
      c->n_q_heads / c->n_kv_heads > MAX_GQ)
    return fail(FLINT_EINVAL, "n_q_heads %d / n_kv_heads %d: need a divisor ratio <= %d", c->n_q_heads, c->n_kv_heads,
                MAX_GQ);
  if (c->n_q_heads * c->head_dim > MAX_QD)
    return fail(FLINT_EINVAL, "n_q_heads * head_dim = %d exceeds %d", c->n_q_heads * c->head_dim, MAX_QD);
  if (c->vocab < 1) return fail(FLINT_EINVAL, "vocab %d", c->vocab);
  if (c->n_dense_layers > 0 && (c->dense_inter < 64 || c->dense_inter % 64 || c->dense_inter > (c->weight_type == FLINT_W_F32 ? MAX_HBUF / 2 : MAX_HBUF)))
    return fail(FLINT_EINVAL, "dense_inter %d must be a multiple of 64 in [64, %d]", c->dense_inter, MAX_HBUF);
  if (c->n_dense_layers < c->n_layers) {
    if (c->n_experts < 1 || c->n_experts > MAX_E) return fail(FLINT_EINVAL, "n_experts %d not in [1, %d]", c->n_experts, MAX_E);
    if (c->top_k < 1 || c->top_k > MAX_K || c->top_k > c->n_experts)
      return fail(FLINT_EINVAL, "top_k %d not in [1, min(%d, n_experts)]", c->top_k, MAX_K);
    if (c->expert_inter < 64 || c->expert_inter % 64 || c->top_k * c->expert_inter > (c->weight_type == FLINT_W_F32 ? MAX_HBUF / 2 : MAX_HBUF))
      return fail(FLINT_EINVAL, "expert_inter %d must be a multiple of 64 with top_k * expert_inter <= %d",
                  c->expert_inter, MAX_HBUF);
  }
  if (c->weight_type == FLINT_W_INT4G64 &&
      (c->hidden % 128 || (c->n_q_heads * c->head_dim) % 128 ||
       (c->n_dense_layers > 0 && c->dense_inter % 128) || (c->n_dense_layers < c->n_layers && c->expert_inter % 128)))
    return fail(FLINT_EINVAL, "int4 weights need every input width to be a multiple of 128");
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f)) return fail(FLINT_EINVAL, "rms_eps / rope_theta invalid");
  if (c->router_renorm != 0 && c->router_renorm != 1) return fail(FLINT_EINVAL, "router_renorm must be 0 or 1");
  if (c->grid < 0) return fail(FLINT_EINVAL, "grid %d < 0", c->grid);
  return FLINT_OK;
}

// Per-phase sizes a workgroup keeps in LDS for grid G.
int check_grid(const flint_config* c, int G) {
  auto ceil_div = [](long a, long b) { return (a + b - 1) / b; };
  const int hd = c->head_dim, QD = c->n_q_heads * hd;
  if (G < c->n_kv_heads) return fail(FLINT_EINVAL, "grid %d smaller than n_kv_heads", G);
  const int S = G / c->n_kv_heads;
  long need = 2 * ceil_div((c->n_q_heads + 2 * c->n_kv_heads) * hd / 2, G);
  if (c->n_dense_layers > 0) need = std::max(need, 4 * ceil_div(c->dense_inter / 2, G));
  if (c->n_dense_layers < c->n_layers) {
    need = std::max(need, 4 * ceil_div(c->top_k * c->expert_inter / 2, G));
    need = std::max(need, (long)c->top_k * ceil_div(c->hidden, G));
  }
  need = std::max(need, ceil_div(c->hidden, G));
  need = std::max(need, 2 * ceil_div(QD / 2, G));  // merged attention dims
  if (need > MAX_YROWS) return fail(FLINT_EINVAL, "grid %d too small: %ld rows per workgroup > %d", G, need, MAX_YROWS);
  const long pairs = ceil_div((c->n_q_heads + 2 * c->n_kv_heads) * hd / 2, G);
  if (pairs > MAX_QPAIRS) return fail(FLINT_EINVAL, "grid %d too small: %ld RoPE pairs per workgroup > %d", G, pairs, MAX_QPAIRS);
  long ne = std::min<long>(hd, 2 * ceil_div(QD / 2, G));
  if ((2 + ne) * S > MAX_GATHER)
    return fail(FLINT_EINVAL, "grid %d: attention merge needs %ld words > %d", G, (2 + ne) * S, MAX_GATHER);
  return FLINT_OK;
}

int copy_in(flint_ctx* c, const void* src, size_t bytes, const uint8_t** dst, const char* what) {
  if (bytes == 0) {
    *dst = nullptr;
    return FLINT_OK;
  }
  if (!src) return fail(FLINT_EINVAL, "weights.%s is NULL", what);
  void* p;
  int rc = dalloc(c, &p, bytes);
  if (rc) return rc;
  HIPCHECK(hipMemcpyAsync(p, src, bytes, hipMemcpyDeviceToDevice, c->stream));
  *dst = (const uint8_t*)p;
  return FLINT_OK;
}

int copy_mat(flint_ctx* c, const flint_mat& m, size_t count, size_t rows, size_t in, Mat* out, const char* what) {
  const int wt = c->cfg.weight_type;
  int rc = copy_in(c, m.w, count * mat_bytes(wt, rows, in), &out->w, what);
  if (rc) return rc;
  out->s = nullptr;
  if (wt == FLINT_W_INT4G64 && count) {
    const uint8_t* s;
    if (!m.scales) return fail(FLINT_EINVAL, "weights.%s.scales is NULL", what);
    rc = copy_in(c, m.scales, count * scale_bytes(wt, rows, in), &s, what);
    if (rc) return rc;
    out->s = (const uint16_t*)s;
  }
  return FLINT_OK;
}

int latched_error(flint_ctx* c) {
  uint32_t e = __atomic_load_n(c->herr_host, __ATOMIC_ACQUIRE);
  if (!e) return FLINT_OK;
  // clear the device and host words so the error is reported once.  A step whose wait gave up (and every
  // step queued behind it before this report) left its sequence's length unchanged while the host mirror
  // advanced: every cache of this ctx re-reads its lengths at its next use.
  (void)hipStreamSynchronize(c->stream);
  e |= __atomic_load_n(c->herr_host, __ATOMIC_ACQUIRE);
  __atomic_store_n(c->herr_host, 0u, __ATOMIC_RELEASE);
  (void)hipMemsetAsync(c->base.err, 0, sizeof(uint32_t), c->stream);
  (void)hipStreamSynchronize(c->stream);
  if (e & ERR_TIMEOUT) {
    c->resync_gen++;
    return fail(FLINT_ETIMEOUT, "a cross-workgroup wait timed out in an earlier step (its length was not advanced)");
  }
  if (e & ERR_TOKEN) return fail(FLINT_EDEVICE, "an earlier step read a token id outside [0, vocab)");
  return fail(FLINT_EDEVICE, "an earlier step found a device length outside [0, max_tokens)");
}

// Host mirror of the lengths brought back in line with the device after a reported timeout.
int resync(flint_kv* kv) {
  flint_ctx* c = kv->ctx;
  if (kv->resync_gen == c->resync_gen) return FLINT_OK;
  HIPCHECK(hipStreamSynchronize(c->stream));
  HIPCHECK(hipMemcpy(kv->hlen.data(), kv->len, sizeof(int32_t) * kv->batch, hipMemcpyDeviceToHost));
  kv->resync_gen = c->resync_gen;
  return FLINT_OK;
}

// Entry of every call that uses a cache: report a latched error once, then make the host lengths current.
int enter(flint_ctx* c, flint_kv* kv) {
  const int rc = latched_error(c);
  const int rs = resync(kv);
  return rc ? rc : rs;
}

int launch(flint_ctx* c, flint_kv* kv, const int32_t* tokens, int tok_idx, int seq, int32_t* out, int out_idx,
           const flint_debug* dbg, bool noalloc = false) {
  KDyn a;
  memset(&a, 0, sizeof a);
  uint64_t n;
  if (noalloc) {
    // the fixed scratch is shared by every context on this device: tags come from the device's own count
    n = noalloc_next_launch(c->device);
    if (n > 0 && n % (1ull << 22) == 0) HIPCHECK(launch_fill(c->na_ptr, NOALLOC_SCRATCH_WORDS, c->stream));
    a.xbase = c->na_ptr;
  } else {
    n = c->launches;
    if (n > 0 && n % (1ull << 22) == 0) {
      // tags restart: clear every exchange slot so no stale tag can match
      HIPCHECK(launch_fill(c->xbuf, c->xbuf_words, c->stream));
    }
  }
  a.kc = (uint8_t*)kv->k;
  a.vc = (uint8_t*)kv->v;
  a.B = kv->batch;
  a.cap = kv->max_tokens;
  a.rope = (const float2*)kv->rope;
  a.len = kv->len;
  a.hist = kv->hist;
  a.tokens = tokens;
  a.tok_idx = tok_idx;
  a.seq = seq;
  a.out_ids = out;
  a.out_idx = out_idx;
  a.epoch = 1u + (uint32_t)(n % (1ull << 22)) * (uint32_t)TAGS_PER_LAUNCH;
  if (dbg) {
    const int H = c->cfg.hidden, V = c->cfg.vocab, L = c->cfg.n_layers, K = c->cfg.top_k;
    a.dbg_logits = dbg->logits ? dbg->logits + (size_t)seq * V : nullptr;
    a.dbg_routes = dbg->routes ? dbg->routes + (size_t)seq * L * K : nullptr;
    a.dbg_rw = dbg->route_w ? dbg->route_w + (size_t)seq * L * K : nullptr;
    a.dbg_resid = dbg->resid ? dbg->resid + (size_t)seq * L * H : nullptr;
    a.dbg_ts = seq == 0 ? dbg->phase_ts : nullptr;
    a.dbg_z = dbg->router_logits ? dbg->router_logits + (size_t)seq * L * c->cfg.n_experts : nullptr;
  }
  HIPCHECK(launch_decode(c->cfg.weight_type, c->stat, c->kdev, a, c->grid, c->stream));
  if (!noalloc) c->launches++;
  return FLINT_OK;
}

// The batched path's weight copies in 16-row tiles of MFMA operand chunks (made once per context, on
// the first cache of several sequences).
int tile_weights(flint_ctx* c) {
  if (c->tiled) return FLINT_OK;
  const flint_config& cfg = c->cfg;
  KStatic& k = c->base;
  const int wt = cfg.weight_type;
  const size_t L = cfg.n_layers, ND = cfg.n_dense_layers, NM = L - ND, H = cfg.hidden, hd = cfg.head_dim;
  const size_t QR = (cfg.n_q_heads + 2 * cfg.n_kv_heads) * hd, QD = cfg.n_q_heads * hd;
  const size_t DI = cfg.dense_inter, E = cfg.n_experts, EI = cfg.expert_inter;
  struct T {
    Mat* m;
    size_t rows, in;
    int rope;
  } mats[] = {{&k.qkv, L * QR, H, (int)hd}, {&k.o, L * H, QD, 0},        {&k.dg, ND * DI, H, 0},
              {&k.du, ND * DI, H, 0},       {&k.dd, ND * H, DI, 0},       {&k.eg, NM * E * EI, H, 0},
              {&k.eu, NM * E * EI, H, 0},   {&k.ed, NM * E * H, EI, 0}};
  int rc;
  for (const T& t : mats) {
    if (!t.rows) continue;
    void* p;
    if ((rc = dalloc(c, &p, mat_bytes(wt, t.rows, t.in)))) return rc;
    if (launch_tile_weights(wt == FLINT_W_INT4G64 ? W_I4 : W_BF16, t.m->w, (uint8_t*)p, t.rows, (int)t.in, t.rope,
                            c->stream) != hipSuccess)
      return fail(FLINT_EHIP, "weight tiling failed");
    t.m->wt = (const uint8_t*)p;
  }
  void* p;
  if ((rc = dalloc(c, &p, (size_t)cfg.vocab * H * 2))) return rc;
  if (launch_tile_weights(W_BF16, k.lmhead, (uint8_t*)p, cfg.vocab, (int)H, 0, c->stream) != hipSuccess)
    return fail(FLINT_EHIP, "lm_head tiling failed");
  c->lmt = (const uint8_t*)p;
  if (hipStreamSynchronize(c->stream) != hipSuccess) return fail(FLINT_EHIP, "weight tiling failed");
  c->tiled = true;
  return FLINT_OK;
}

// Scratch of the batched path, one allocation carved into the buffers of BArgs, plus the arguments
// that stay the same for every pass.
int batch_scratch(flint_ctx* c, flint_kv* kv) {
  const flint_config& cfg = c->cfg;
  int trc = tile_weights(c);
  if (trc) return trc;
  const KStatic& k = c->base;
  BArgs& a = kv->bargs;
  memset(&a, 0, sizeof a);
  a.H = cfg.hidden;
  a.nq = cfg.n_q_heads;
  a.nkv = cfg.n_kv_heads;
  a.hd = cfg.head_dim;
  a.V = cfg.vocab;
  a.L = cfg.n_layers;
  a.n_dense = cfg.n_dense_layers;
  a.DI = cfg.dense_inter;
  a.E = cfg.n_experts;
  a.K = cfg.top_k;
  a.EI = cfg.expert_inter;
  a.renorm = cfg.router_renorm;
  a.eps = cfg.rms_eps;
  a.embed = k.embed;
  a.lmhead = k.lmhead;
  a.lmt = c->lmt;
  a.fnorm = k.fnorm;
  a.anorm = k.anorm;
  a.pnorm = k.pnorm;
  a.qkv = k.qkv;
  a.o = k.o;
  a.dg = k.dg;
  a.du = k.du;
  a.dd = k.dd;
  a.router = k.router;
  a.eg = k.eg;
  a.eu = k.eu;
  a.ed = k.ed;
  a.Bc = kv->batch;
  a.cap = kv->max_tokens;
  a.kc = (uint8_t*)kv->k;
  a.vc = (uint8_t*)kv->v;
  a.rope = (const float2*)kv->rope;
  a.len = kv->len;
  a.hist = kv->hist;
  a.err = k.err;
  a.herr = k.herr;
  const size_t H = cfg.hidden, QD = (size_t)cfg.n_q_heads * cfg.head_dim;
  a.astride = (int)std::max(H, QD);
  a.nsmax = (kv->max_tokens + ATT_P - 1) / ATT_P;
  const size_t ND = cfg.n_dense_layers, NM = cfg.n_layers - ND;
  a.hstride = (int)std::max(ND ? (size_t)cfg.dense_inter : 0, NM ? (size_t)cfg.top_k * cfg.expert_inter : 0);
  // byte sizes, each rounded up to 256
  auto r256 = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const size_t sx = r256(BT * H * 4), sact = r256(BT * (size_t)a.astride * 2), sq = r256(BT * QD * 4);
  const size_t spart = r256((size_t)BT * cfg.n_q_heads * a.nsmax * (cfg.head_dim + 2) * 4);
  const size_t sop = r256(OKC * BT * H * 4), sdp = r256(DKC * BT * H * 4), sh = r256(BT * (size_t)a.hstride * 2);
  const size_t ssel = r256(BT * MAX_K * 4), sam = r256(BT * 8 + 64), scnt = r256((H / 16 + H / 64) * 4);
  const size_t total = sx + sact + sq + spart + sop + sdp + sh + 2 * ssel + sam + scnt;
  if (hipMalloc(&kv->bscratch, total) != hipSuccess) {
    kv->bscratch = nullptr;
    return fail(FLINT_ENOMEM, "batched-path scratch of %zu bytes", total);
  }
  char* p = (char*)kv->bscratch;
  auto take = [&](size_t b) {
    char* q = p;
    p += b;
    return q;
  };
  a.x = (float*)take(sx);
  a.act = (uint16_t*)take(sact);
  a.q = (float*)take(sq);
  a.part = (float*)take(spart);
  a.opart = (float*)take(sop);
  a.dpart = (float*)take(sdp);
  a.h = (uint16_t*)take(sh);
  a.sel = (int32_t*)take(ssel);
  a.wsel = (float*)take(ssel);
  a.amax = (unsigned long long*)take(sam);
  a.done = (uint32_t*)(a.amax + BT);
  a.cnt = (uint32_t*)take(scnt);
  if (hipMemsetAsync(kv->bscratch, 0, total, c->stream) != hipSuccess || hipStreamSynchronize(c->stream) != hipSuccess)
    return fail(FLINT_EHIP, "batched-path scratch initialisation failed");
  return FLINT_OK;
}

// Scratch of the long-chunk prefill (chunks of up to PF_MAXN tokens), carved like batch_scratch.
constexpr int PF_MAXN = 4096;
int prefill_scratch(flint_ctx* c, flint_kv* kv) {
  const flint_config& cfg = c->cfg;
  BArgs a = kv->bargs;
  const size_t N = PF_MAXN, H = cfg.hidden, QD = (size_t)cfg.n_q_heads * cfg.head_dim, K = cfg.top_k;
  const size_t ND = cfg.n_dense_layers, NM = cfg.n_layers - ND;
  const size_t hw = std::max(ND ? (size_t)cfg.dense_inter : 0, NM ? K * cfg.expert_inter : 0);
  auto r256 = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const size_t sx = r256(N * H * 4), sact = r256(N * a.astride * 2), sq = r256(N * QD * 4);
  const size_t spart = r256(prefill_part_floats(cfg.n_q_heads, a.nsmax, cfg.head_dim) * 4);
  const size_t sh = r256(N * hw * 2), ssel = r256(N * K * 4), sy = r256(N * K * H * 4);
  const size_t secnt = r256(((size_t)cfg.n_experts + 1) * 4), sblk = r256(((N * K + 63) / 64 + cfg.n_experts) * 3 * 4);
  const size_t total = sx + sact + sq + spart + sh + 3 * ssel + sy + secnt + sblk;
  if (hipMalloc(&kv->pscratch, total) != hipSuccess) {
    kv->pscratch = nullptr;
    return fail(FLINT_ENOMEM, "prefill scratch of %zu bytes", total);
  }
  char* p = (char*)kv->pscratch;
  auto take = [&](size_t b) {
    char* q = p;
    p += b;
    return q;
  };
  a.x = (float*)take(sx);
  a.act = (uint16_t*)take(sact);
  a.q = (float*)take(sq);
  a.part = (float*)take(spart);
  a.h = (uint16_t*)take(sh);
  a.sel = (int32_t*)take(ssel);
  a.wsel = (float*)take(ssel);
  a.lst = (int32_t*)take(ssel);
  a.y = (float*)take(sy);
  a.ecnt = (int32_t*)take(secnt);
  a.nblk = a.ecnt + cfg.n_experts;
  a.blk = (int32_t*)take(sblk);
  kv->pargs = a;
  if (hipMemsetAsync(kv->pscratch, 0, total, c->stream) != hipSuccess || hipStreamSynchronize(c->stream) != hipSuccess)
    return fail(FLINT_EHIP, "prefill scratch initialisation failed");
  return FLINT_OK;
}

// Fewest sequences of a step that take the batched pass: below it, one persistent launch per sequence is
// faster (int4 49-layer model, ragged lengths up to 8,192: 2 sequences 2.5 ms as two launches, 3.4 ms
// as one pass; 4 sequences 3.7 ms as one pass).
constexpr int BATCH_MIN = 3;

// Positions of a pass's columns from the host's mirror of the lengths, and the attention splits per column.
void set_positions(BArgs& a, const std::vector<int32_t>& hlen) {
  if (a.prefill) a.p0 = hlen[a.seq0];
  a.asp[0] = 0;
  for (int n = 0; n < BT; ++n) {
    a.pos[n] = n < a.B ? (a.prefill ? hlen[a.seq0] + n : hlen[a.cseq[n]]) : 0;
    a.asp[n + 1] = a.asp[n] + (n < a.B ? (a.pos[n] + 1 + ATT_P - 1) / ATT_P : 0);
  }
}

}  // namespace

extern "C" {

const char* flint_last_error(void) { return g_last_error.c_str(); }

int flint_decode_init(const flint_config* cfg, const flint_weights* w, void* hip_stream, flint_ctx** out) {
  if (!out) return fail(FLINT_EINVAL, "out is NULL");
  *out = nullptr;
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!w) return fail(FLINT_EINVAL, "weights is NULL");
  flint_ctx* c = new (std::nothrow) flint_ctx();
  if (!c) return fail(FLINT_ENOMEM, "host allocation failed");
  c->cfg = *cfg;
  c->stream = (hipStream_t)hip_stream;
  c->herr_host = nullptr;
  auto bail = [&](int code) {
    release(c);
    delete c;
    return code;
  };
  if (hipGetDevice(&c->device) != hipSuccess) return bail(fail(FLINT_EHIP, "hipGetDevice failed"));
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, c->device) != hipSuccess) return bail(fail(FLINT_EHIP, "hipGetDeviceProperties failed"));
  int per_cu = 0;
  if (kernel_occupancy(cfg->weight_type, &per_cu) != hipSuccess) return bail(fail(FLINT_EHIP, "occupancy query failed"));
  const int resident = per_cu * prop.multiProcessorCount;
  c->grid = cfg->grid ? cfg->grid : prop.multiProcessorCount;
  if (c->grid > resident)
    return bail(fail(FLINT_ENORESIDENT, "grid %d exceeds the %d workgroups that can be co-resident", c->grid, resident));
  if ((rc = check_grid(cfg, c->grid))) return bail(rc);
  c->S = c->grid / cfg->n_kv_heads;

  const int wt = cfg->weight_type;
  const size_t L = cfg->n_layers, ND = cfg->n_dense_layers, NM = L - ND, H = cfg->hidden, V = cfg->vocab;
  const size_t hd = cfg->head_dim, QR = (cfg->n_q_heads + 2 * cfg->n_kv_heads) * hd, QD = cfg->n_q_heads * hd;
  const size_t DI = cfg->dense_inter, E = cfg->n_experts, EI = cfg->expert_inter;
  KStatic& a = c->base;
  memset(&a, 0, sizeof a);
  a.H = (int)H;
  a.nq = cfg->n_q_heads;
  a.nkv = cfg->n_kv_heads;
  a.hd = (int)hd;
  a.V = (int)V;
  a.L = (int)L;
  a.n_dense = (int)ND;
  a.DI = (int)DI;
  a.E = NM ? (int)E : 0;
  a.K = cfg->top_k;
  a.EI = (int)EI;
  a.renorm = cfg->router_renorm;
  a.eps = cfg->rms_eps;
  a.S = c->S;
  // exchange polling: tuning knobs for experiments (defaults are the measured best)
  a.poll_sleep = getenv("FLINT_POLL_SLEEP") ? atoi(getenv("FLINT_POLL_SLEEP")) : 0;
  a.sentinels = getenv("FLINT_SENTINELS") ? atoi(getenv("FLINT_SENTINELS")) : 0;
  a.spin_limit = SPIN_TIMEOUT;
  if (a.sentinels < 0) a.sentinels = 0;
  if (a.sentinels > 64) a.sentinels = 64;
  if (a.poll_sleep < 0) a.poll_sleep = 0;

  const size_t eb = elem_bytes_act(wt);
  if ((rc = copy_in(c, w->embed, V * H * eb, &a.embed, "embed"))) return bail(rc);
  if ((rc = copy_in(c, w->lm_head, V * H * eb, &a.lmhead, "lm_head"))) return bail(rc);
  const uint8_t* p;
  if ((rc = copy_in(c, w->final_norm, H * 4, &p, "final_norm"))) return bail(rc);
  a.fnorm = (const float*)p;
  if ((rc = copy_in(c, w->attn_norm, L * H * 4, &p, "attn_norm"))) return bail(rc);
  a.anorm = (const float*)p;
  if ((rc = copy_in(c, w->post_norm, L * H * 4, &p, "post_norm"))) return bail(rc);
  a.pnorm = (const float*)p;
  if ((rc = copy_mat(c, w->qkv, L, QR, H, &a.qkv, "qkv"))) return bail(rc);
  if ((rc = copy_mat(c, w->o, L, H, QD, &a.o, "o"))) return bail(rc);
  if ((rc = copy_mat(c, w->dense_gate, ND, DI, H, &a.dg, "dense_gate"))) return bail(rc);
  if ((rc = copy_mat(c, w->dense_up, ND, DI, H, &a.du, "dense_up"))) return bail(rc);
  if ((rc = copy_mat(c, w->dense_down, ND, H, DI, &a.dd, "dense_down"))) return bail(rc);
  if ((rc = copy_mat(c, w->router, NM, E, H, &a.router, "router"))) return bail(rc);
  if ((rc = copy_mat(c, w->exp_gate, NM * E, EI, H, &a.eg, "exp_gate"))) return bail(rc);
  if ((rc = copy_mat(c, w->exp_up, NM * E, EI, H, &a.eu, "exp_up"))) return bail(rc);
  if ((rc = copy_mat(c, w->exp_down, NM * E, H, EI, &a.ed, "exp_down"))) return bail(rc);

  // scratch: tagged exchange slots
  const bool act32 = wt == FLINT_W_F32;
  a.qkv_rows = (int)QR;
  a.o_slots = (int)(act32 ? QD : QD / 2);
  size_t hmax = std::max(ND ? DI : 0, NM ? (size_t)cfg->top_k * EI : 0);
  a.h_slots = (int)std::max<size_t>(1, act32 ? hmax : hmax / 2);
  const size_t n_qkv = NCOPY * 2 * QR, n_part = 2 * (size_t)cfg->n_q_heads * (hd + 2) * c->S;
  const size_t n_o = NCOPY * 2 * (size_t)a.o_slots, n_res = NCOPY * 2 * H, n_h = NCOPY * 2 * (size_t)a.h_slots;
  const size_t n_z = NCOPY * 2 * (size_t)std::max(1, cfg->n_experts);
  c->xbuf_words = n_qkv + n_part + n_o + 2 * n_res + n_h + n_z;
  // the argmax hand-off counters follow the slots in the same buffer (16 words, two 64-byte lines)
  void* xb;
  if ((rc = dalloc(c, &xb, (c->xbuf_words + 16) * 8 + 256))) return bail(rc);
  c->xbuf = (uint64_t*)xb;
  a.x_qkv = c->xbuf;
  a.x_part = a.x_qkv + n_qkv;
  a.x_o = a.x_part + n_part;
  a.x_res1 = a.x_o + n_o;
  a.x_h = a.x_res1 + n_res;
  a.x_res2 = a.x_h + n_h;
  a.x_z = a.x_res2 + n_res;
  void* misc;
  if ((rc = dalloc(c, &misc, 256))) return bail(rc);
  a.err = (uint32_t*)misc;
  a.amax = (unsigned long long*)(c->xbuf + c->xbuf_words);
  a.done = (uint32_t*)(c->xbuf + c->xbuf_words + 8);
  if (hipHostMalloc((void**)&c->herr_host, 64, hipHostMallocMapped) != hipSuccess)
    return bail(fail(FLINT_ENOMEM, "hipHostMalloc of the error word failed"));
  *c->herr_host = 0;
  void* herr_dev = nullptr;
  if (hipHostGetDevicePointer(&herr_dev, c->herr_host, 0) != hipSuccess)
    return bail(fail(FLINT_EHIP, "hipHostGetDevicePointer failed"));
  a.herr = (uint32_t*)herr_dev;
  c->stat = cfg->weight_type != FLINT_W_F32 && shape_is_static(a, c->grid) && !getenv("FLINT_GENERIC_KERNEL");
  // the batched path: bf16 activations, 128-dim heads with at most 4 query heads per kv head (attention
  // scores on MFMA), row counts in whole 16-row tiles and 64-row gate/up blocks
  c->batch_ok = cfg->weight_type != FLINT_W_F32 && hd == 128 && cfg->n_q_heads / cfg->n_kv_heads <= 4 &&
                H % 128 == 0 && QD % 128 == 0 && (ND == 0 || DI % 256 == 0) && (NM == 0 || EI % 256 == 0) &&
                V % 16 == 0 &&
                !getenv("FLINT_NO_BATCH_PATH");
  c->batch_min = BATCH_MIN;
  if (const char* bm = getenv("FLINT_BATCH_MIN")) c->batch_min = std::max(1, atoi(bm));
  if (c->batch_ok && wt == FLINT_W_INT4G64) {  // int4 scales regrouped by 4 rows for the batched contractions
    struct R {
      Mat* m;
      size_t rows, in;
    } regs[] = {{&a.qkv, L * QR, H}, {&a.o, L * H, QD}, {&a.dg, ND * DI, H}, {&a.du, ND * DI, H},
                {&a.dd, ND * H, DI}, {&a.eg, NM * E * EI, H}, {&a.eu, NM * E * EI, H}, {&a.ed, NM * E * H, EI}};
    for (const R& r : regs) {
      if (!r.rows || !r.m->s) continue;
      void* p4;
      if ((rc = dalloc(c, &p4, r.rows * (r.in / 64) * 2))) return bail(rc);
      if (launch_regroup_scales(r.m->s, (uint16_t*)p4, r.rows, (int)(r.in / 64), c->stream) != hipSuccess)
        return bail(fail(FLINT_EHIP, "scale regrouping failed"));
      r.m->s4 = (const uint16_t*)p4;
    }
  }
  void* kd;
  if ((rc = dalloc(c, &kd, sizeof(KStatic)))) return bail(rc);
  c->kdev = (KStatic*)kd;
  if (hipMemcpyAsync(kd, &a, sizeof(KStatic), hipMemcpyHostToDevice, c->stream) != hipSuccess)
    return bail(fail(FLINT_EHIP, "copy of the kernel constants failed"));
  if (launch_fill(c->xbuf, c->xbuf_words + 16, c->stream) != hipSuccess) return bail(fail(FLINT_EHIP, "fill kernel failed"));
  // the fixed exchange scratch of flint_decode_step_noalloc on this device (found once per device)
  c->na_ptr = nullptr;
  c->na_status = noalloc_scratch(c->device, c->stream, &c->na_ptr);
  if (hipMemsetAsync(misc, 0, 256, c->stream) != hipSuccess) return bail(fail(FLINT_EHIP, "hipMemsetAsync failed"));
  if (hipStreamSynchronize(c->stream) != hipSuccess) return bail(fail(FLINT_EHIP, "hipStreamSynchronize failed"));
  c->launches = 0;
  c->live_kv = 0;
  c->resync_gen = 0;
  *out = c;
  return FLINT_OK;
}

int flint_decode_free(flint_ctx* c) {
  if (!c) return FLINT_OK;
  if (c->live_kv) return fail(FLINT_EINVAL, "free the %d flint_kv of this ctx first", c->live_kv);
  (void)hipStreamSynchronize(c->stream);
  release(c);
  delete c;
  return FLINT_OK;
}

int flint_kv_alloc(flint_ctx* c, int32_t batch, int32_t max_tokens, flint_kv** out) {
  if (!out) return fail(FLINT_EINVAL, "out is NULL");
  *out = nullptr;
  if (!c) return fail(FLINT_EINVAL, "ctx is NULL");
  if (batch < 1 || batch > 4096) return fail(FLINT_EINVAL, "batch %d not in [1, 4096]", batch);
  if (max_tokens < 1 || max_tokens > (1 << 22)) return fail(FLINT_EINVAL, "max_tokens %d not in [1, 2^22]", max_tokens);
  const flint_config& cfg = c->cfg;
  const size_t per = (size_t)cfg.n_layers * batch * cfg.n_kv_heads * max_tokens * cfg.head_dim *
                     elem_bytes_act(cfg.weight_type);
  flint_kv* kv = new (std::nothrow) flint_kv();
  if (!kv) return fail(FLINT_ENOMEM, "host allocation failed");
  kv->ctx = c;
  kv->batch = batch;
  kv->max_tokens = max_tokens;
  kv->k = kv->v = nullptr;
  kv->len = nullptr;
  kv->hist = nullptr;
  kv->rope = nullptr;
  kv->bscratch = nullptr;
  kv->pscratch = nullptr;
  auto bail = [&](int code) {
    if (kv->k) (void)hipFree(kv->k);
    if (kv->v) (void)hipFree(kv->v);
    if (kv->len) (void)hipFree(kv->len);
    if (kv->hist) (void)hipFree(kv->hist);
    if (kv->rope) (void)hipFree(kv->rope);
    if (kv->bscratch) (void)hipFree(kv->bscratch);
    delete kv;
    return code;
  };
  if (hipMalloc(&kv->k, per) != hipSuccess || hipMalloc(&kv->v, per) != hipSuccess)
    return bail(fail(FLINT_ENOMEM, "KV cache of 2 x %zu bytes", per));
  if (hipMalloc((void**)&kv->len, sizeof(int32_t) * batch) != hipSuccess) return bail(fail(FLINT_ENOMEM, "lengths"));
  const size_t hist_bytes = sizeof(int32_t) * (size_t)batch * max_tokens;
  if (hipMalloc((void**)&kv->hist, hist_bytes) != hipSuccess) return bail(fail(FLINT_ENOMEM, "token record"));
  // RoPE table: cos, sin of p * theta^(-2i/d) in double, stored fp32 [max_tokens][d/2][2]
  const int half = cfg.head_dim / 2;
  std::vector<float> tab((size_t)max_tokens * half * 2);
  for (int pos = 0; pos < max_tokens; ++pos)
    for (int i = 0; i < half; ++i) {
      const double ang = (double)pos * pow((double)cfg.rope_theta, -2.0 * i / (double)cfg.head_dim);
      tab[((size_t)pos * half + i) * 2] = (float)cos(ang);
      tab[((size_t)pos * half + i) * 2 + 1] = (float)sin(ang);
    }
  if (hipMalloc((void**)&kv->rope, tab.size() * 4) != hipSuccess) return bail(fail(FLINT_ENOMEM, "RoPE table"));
  if (hipMemsetAsync(kv->k, 0, per, c->stream) != hipSuccess || hipMemsetAsync(kv->v, 0, per, c->stream) != hipSuccess ||
      hipMemsetAsync(kv->len, 0, sizeof(int32_t) * batch, c->stream) != hipSuccess ||
      hipMemsetAsync(kv->hist, 0xFF, hist_bytes, c->stream) != hipSuccess ||
      hipMemcpyAsync(kv->rope, tab.data(), tab.size() * 4, hipMemcpyHostToDevice, c->stream) != hipSuccess ||
      hipStreamSynchronize(c->stream) != hipSuccess)
    return bail(fail(FLINT_EHIP, "KV cache initialisation failed"));
  kv->hlen.assign(batch, 0);
  kv->resync_gen = c->resync_gen;
  kv->bscratch = nullptr;
  if (batch > 1 && c->batch_ok && max_tokens <= ATT_P * MAX_SPLITS) {
    int rc2 = batch_scratch(c, kv);
    if (rc2) return bail(rc2);
  }
  c->live_kv++;
  *out = kv;
  return FLINT_OK;
}

int flint_kv_free(flint_kv* kv) {
  if (!kv) return FLINT_OK;
  (void)hipStreamSynchronize(kv->ctx->stream);
  if (kv->bscratch) (void)hipFree(kv->bscratch);
  if (kv->pscratch) (void)hipFree(kv->pscratch);
  (void)hipFree(kv->k);
  (void)hipFree(kv->v);
  (void)hipFree(kv->len);
  (void)hipFree(kv->hist);
  (void)hipFree(kv->rope);
  kv->ctx->live_kv--;
  delete kv;
  return FLINT_OK;
}

int flint_kv_set_lengths(flint_kv* kv, const int32_t* lengths) {
  if (!kv || !lengths) return fail(FLINT_EINVAL, "kv or lengths is NULL");
  for (int b = 0; b < kv->batch; ++b)
    if (lengths[b] < 0 || lengths[b] > kv->max_tokens)
      return fail(FLINT_EINVAL, "length[%d] = %d not in [0, %d]", b, lengths[b], kv->max_tokens);
  HIPCHECK(hipMemcpyAsync(kv->len, lengths, sizeof(int32_t) * kv->batch, hipMemcpyHostToDevice, kv->ctx->stream));
  HIPCHECK(hipStreamSynchronize(kv->ctx->stream));
  kv->hlen.assign(lengths, lengths + kv->batch);
  kv->resync_gen = kv->ctx->resync_gen;
  return FLINT_OK;
}

int flint_kv_get_lengths(flint_kv* kv, int32_t* lengths) {
  if (!kv || !lengths) return fail(FLINT_EINVAL, "kv or lengths is NULL");
  HIPCHECK(hipMemcpyAsync(lengths, kv->len, sizeof(int32_t) * kv->batch, hipMemcpyDeviceToHost, kv->ctx->stream));
  HIPCHECK(hipStreamSynchronize(kv->ctx->stream));
  return FLINT_OK;
}

int flint_kv_tokens(flint_kv* kv, int32_t seq, int32_t* tokens, int32_t n) {
  if (!kv || !tokens) return fail(FLINT_EINVAL, "NULL argument");
  if (seq < 0 || seq >= kv->batch) return fail(FLINT_EINVAL, "seq %d not in [0, %d)", seq, kv->batch);
  int rc = resync(kv);
  if (rc) return rc;
  if (n < 0 || n > kv->hlen[seq]) return fail(FLINT_EINVAL, "n %d not in [0, %d]", n, kv->hlen[seq]);
  if (n == 0) return FLINT_OK;
  HIPCHECK(hipStreamSynchronize(kv->ctx->stream));
  HIPCHECK(hipMemcpy(tokens, kv->hist + (size_t)seq * kv->max_tokens, sizeof(int32_t) * n, hipMemcpyDeviceToHost));
  return FLINT_OK;
}

int flint_kv_prefix_match(flint_kv* kv, int32_t seq, const int32_t* tokens, int32_t n, int32_t* matched) {
  if (!kv || !matched || (n > 0 && !tokens)) return fail(FLINT_EINVAL, "NULL argument");
  if (seq < 0 || seq >= kv->batch) return fail(FLINT_EINVAL, "seq %d not in [0, %d)", seq, kv->batch);
  if (n < 0) return fail(FLINT_EINVAL, "n %d < 0", n);
  int rc0 = resync(kv);
  if (rc0) return rc0;
  const int m = std::min<int>(n, kv->hlen[seq]);
  std::vector<int32_t> rec(m);
  int rc = flint_kv_tokens(kv, seq, rec.data(), m);
  if (rc) return rc;
  int k = 0;
  while (k < m && rec[k] == tokens[k]) ++k;
  *matched = k;
  return FLINT_OK;
}

int flint_kv_layer_ptrs(flint_kv* kv, int32_t layer, void** k, void** v) {
  if (!kv || !k || !v) return fail(FLINT_EINVAL, "NULL argument");
  const flint_config& cfg = kv->ctx->cfg;
  if (layer < 0 || layer >= cfg.n_layers) return fail(FLINT_EINVAL, "layer %d not in [0, %d)", layer, cfg.n_layers);
  const size_t per_layer = (size_t)kv->batch * cfg.n_kv_heads * kv->max_tokens * cfg.head_dim *
                           elem_bytes_act(cfg.weight_type);
  *k = (char*)kv->k + per_layer * layer;
  *v = (char*)kv->v + per_layer * layer;
  return FLINT_OK;
}

int flint_decode_step_debug(flint_ctx* c, const int32_t* tokens, flint_kv* kv, int32_t* out_ids,
                            const flint_debug* dbg) {
  if (!c || !kv || !tokens || !out_ids) return fail(FLINT_EINVAL, "NULL argument");
  if (kv->ctx != c) return fail(FLINT_EINVAL, "kv belongs to another ctx");
  int rc = enter(c, kv);
  if (rc) return rc;
  for (int b = 0; b < kv->batch; ++b)
    if (kv->hlen[b] + 1 > kv->max_tokens)
      return fail(FLINT_ECAPACITY, "sequence %d: length %d + 1 exceeds max_tokens %d", b, kv->hlen[b], kv->max_tokens);
  if (kv->bscratch && kv->batch >= c->batch_min) {  // batched path: passes of up to BT sequences
    BArgs a = kv->bargs;
    a.tokens = tokens;
    a.out_ids = out_ids;
    a.dbg_logits = dbg ? dbg->logits : nullptr;
    a.dbg_routes = dbg ? dbg->routes : nullptr;
    a.dbg_rw = dbg ? dbg->route_w : nullptr;
    a.dbg_resid = dbg ? dbg->resid : nullptr;
    a.dbg_z = dbg ? dbg->router_logits : nullptr;
    for (int s0 = 0; s0 < kv->batch; s0 += BT) {
      a.B = std::min(BT, kv->batch - s0);
      for (int q = 0; q < BT; ++q) a.cseq[q] = q < a.B ? s0 + q : 0;
      a.tokens = tokens + s0;
      a.out_ids = out_ids + s0;
      set_positions(a, kv->hlen);
      HIPCHECK(launch_batch_pass(c->cfg.weight_type, a, c->stream));
    }
    for (int b = 0; b < kv->batch; ++b) kv->hlen[b]++;
    return FLINT_OK;
  }
  for (int b = 0; b < kv->batch; ++b) {
    rc = launch(c, kv, tokens, b, b, out_ids, b, dbg);
    if (rc) return rc;
    kv->hlen[b]++;
  }
  return FLINT_OK;
}

int flint_decode_step(flint_ctx* c, const int32_t* tokens, flint_kv* kv, int32_t* out_ids) {
  return flint_decode_step_debug(c, tokens, kv, out_ids, nullptr);
}

int flint_decode_step_noalloc(flint_ctx* c, const int32_t* tokens, flint_kv* kv, int32_t* out_ids) {
  if (!c || !kv || !tokens || !out_ids) return fail(FLINT_EINVAL, "NULL argument");
  if (kv->ctx != c) return fail(FLINT_EINVAL, "kv belongs to another ctx");
  const size_t need = c->xbuf_words + 16;
  if (need > NOALLOC_SCRATCH_WORDS)
    return fail(FLINT_EINVAL, "this model needs %zu bytes of exchange scratch; the fixed array holds %zu", need * 8,
                NOALLOC_SCRATCH_WORDS * 8);
  if (c->na_status != hipSuccess || !c->na_ptr)
    return fail(FLINT_EHIP, "the fixed scratch array was not found at init: %s", hipGetErrorString(c->na_status));
  int rc = enter(c, kv);
  if (rc) return rc;
  for (int b = 0; b < kv->batch; ++b)
    if (kv->hlen[b] + 1 > kv->max_tokens)
      return fail(FLINT_ECAPACITY, "sequence %d: length %d + 1 exceeds max_tokens %d", b, kv->hlen[b], kv->max_tokens);
  for (int b = 0; b < kv->batch; ++b) {  // every sequence on the persistent kernel
    rc = launch(c, kv, tokens, b, b, out_ids, b, nullptr, true);
    if (rc) return rc;
    kv->hlen[b]++;
  }
  return FLINT_OK;
}

int flint_decode_step_seqs(flint_ctx* c, flint_kv* kv, const int32_t* seqs, int32_t n, const int32_t* tokens,
                           int32_t* out_ids) {
  if (!c || !kv || !seqs || !tokens || !out_ids) return fail(FLINT_EINVAL, "NULL argument");
  if (kv->ctx != c) return fail(FLINT_EINVAL, "kv belongs to another ctx");
  if (n < 1 || n > kv->batch) return fail(FLINT_EINVAL, "n %d not in [1, %d]", n, kv->batch);
  int rc = enter(c, kv);
  if (rc) return rc;
  std::vector<char> seen(kv->batch, 0);
  for (int i = 0; i < n; ++i) {
    const int b = seqs[i];
    if (b < 0 || b >= kv->batch) return fail(FLINT_EINVAL, "seqs[%d] = %d not in [0, %d)", i, b, kv->batch);
    if (seen[b]) return fail(FLINT_EINVAL, "sequence %d listed twice", b);
    seen[b] = 1;
    if (kv->hlen[b] + 1 > kv->max_tokens)
      return fail(FLINT_ECAPACITY, "sequence %d: length %d + 1 exceeds max_tokens %d", b, kv->hlen[b], kv->max_tokens);
  }
  if (kv->bscratch && n >= c->batch_min) {  // batched passes over the listed sequences
    BArgs a = kv->bargs;
    for (int i0 = 0; i0 < n; i0 += BT) {
      a.B = std::min(BT, n - i0);
      for (int q = 0; q < BT; ++q) a.cseq[q] = q < a.B ? seqs[i0 + q] : 0;
      a.tokens = tokens + i0;
      a.out_ids = out_ids + i0;
      set_positions(a, kv->hlen);
      HIPCHECK(launch_batch_pass(c->cfg.weight_type, a, c->stream));
    }
    for (int i = 0; i < n; ++i) kv->hlen[seqs[i]]++;
    return FLINT_OK;
  }
  for (int i = 0; i < n; ++i) {
    rc = launch(c, kv, tokens, i, seqs[i], out_ids, i, nullptr);
    if (rc) return rc;
    kv->hlen[seqs[i]]++;
  }
  return FLINT_OK;
}

int flint_prefill_chunk(flint_ctx* c, flint_kv* kv, int32_t seq, const int32_t* tokens, int32_t n, int32_t* out_id) {
  if (!c || !kv || !tokens || !out_id) return fail(FLINT_EINVAL, "NULL argument");
  if (kv->ctx != c) return fail(FLINT_EINVAL, "kv belongs to another ctx");
  if (seq < 0 || seq >= kv->batch) return fail(FLINT_EINVAL, "seq %d not in [0, %d)", seq, kv->batch);
  if (n < 1 || n > 4096) return fail(FLINT_EINVAL, "n %d not in [1, 4096]", n);
  int rc = enter(c, kv);
  if (rc) return rc;
  if (kv->hlen[seq] + n > kv->max_tokens)
    return fail(FLINT_ECAPACITY, "sequence %d: length %d + %d exceeds max_tokens %d", seq, kv->hlen[seq], n,
                kv->max_tokens);
  if (c->batch_ok && !kv->bscratch && kv->max_tokens <= ATT_P * MAX_SPLITS) {
    rc = batch_scratch(c, kv);
    if (rc) return rc;
  }
  if (kv->bscratch && n > BT) {  // long chunk: contractions over 64 tokens per workgroup
    if (!kv->pscratch) {
      rc = prefill_scratch(c, kv);
      if (rc) return rc;
    }
    BArgs a = kv->pargs;
    a.seq0 = seq;
    a.tokens = tokens;
    a.out_ids = out_id;
    a.p0 = kv->hlen[seq];
    HIPCHECK(launch_prefill(c->cfg.weight_type, a, n, c->stream));
    kv->hlen[seq] += n;
    return FLINT_OK;
  }
  if (kv->bscratch) {  // batched path: up to BT prompt tokens per pass, causal over the shared cache
    BArgs a = kv->bargs;
    a.prefill = 1;
    a.seq0 = seq;
    a.tokens = tokens;
    a.out_ids = out_id;
    for (int i0 = 0; i0 < n; i0 += BT) {
      a.tok0 = i0;
      a.B = std::min(BT, n - i0);
      a.lenadd = a.B;
      set_positions(a, kv->hlen);
      HIPCHECK(launch_batch_pass(c->cfg.weight_type, a, c->stream));
      kv->hlen[seq] += a.B;
    }
    return FLINT_OK;
  }
  // positions in order; each launch writes its greedy id to out_id[0], the
  // last one is the id after the chunk
  for (int i = 0; i < n; ++i) {
    rc = launch(c, kv, tokens, i, seq, out_id, 0, nullptr);
    if (rc) return rc;
    kv->hlen[seq]++;
  }
  return FLINT_OK;
}

int flint_micro_stream_read(flint_ctx* c, size_t bytes, int32_t reps, float* gbps) {
  if (!c || !gbps) return fail(FLINT_EINVAL, "NULL argument");
  if (bytes < (1u << 20) || reps < 1) return fail(FLINT_EINVAL, "bytes %zu < 1 MiB or reps %d < 1", bytes, reps);
  bytes &= ~(size_t)15;
  hipDeviceProp_t prop;
  HIPCHECK(hipGetDeviceProperties(&prop, c->device));
  void* buf = nullptr;
  uint32_t* sink = nullptr;
  if (hipMalloc(&buf, bytes) != hipSuccess) return fail(FLINT_ENOMEM, "stream-read buffer of %zu bytes", bytes);
  if (hipMalloc((void**)&sink, 64) != hipSuccess) {
    (void)hipFree(buf);
    return fail(FLINT_ENOMEM, "stream-read sink");
  }
  hipEvent_t e0 = nullptr, e1 = nullptr;
  float ms = 0.f;
  hipError_t e = hipMemsetAsync(buf, 0, bytes, c->stream);
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) e = launch_micro_read(buf, bytes, sink, 2 * prop.multiProcessorCount, c->stream);  // warm-up
  if (e == hipSuccess) e = hipEventRecord(e0, c->stream);
  for (int r = 0; r < reps && e == hipSuccess; ++r) e = launch_micro_read(buf, bytes, sink, 2 * prop.multiProcessorCount, c->stream);
  if (e == hipSuccess) e = hipEventRecord(e1, c->stream);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipFree(buf);
  (void)hipFree(sink);
  if (e != hipSuccess) return fail(FLINT_EHIP, "stream read: %s", hipGetErrorString(e));
  const size_t read = bytes / (2 * prop.multiProcessorCount) / 1024 * 1024 * (2 * prop.multiProcessorCount);
  *gbps = (float)((double)read * reps / (ms * 1e-3) / 1e9);
  return FLINT_OK;
}

namespace {
int micro_exchange(flint_ctx* c, int32_t workgroups, int32_t rounds, float* us_per_round, bool xcd) {
  if (!c || !us_per_round) return fail(FLINT_EINVAL, "NULL argument");
  hipDeviceProp_t prop;
  HIPCHECK(hipGetDeviceProperties(&prop, c->device));
  if (workgroups < 2 || workgroups > prop.multiProcessorCount || rounds < 1)
    return fail(FLINT_EINVAL, "workgroups %d not in [2, %d] or rounds %d < 1", workgroups, prop.multiProcessorCount, rounds);
  if (xcd && (workgroups % NCOPY != 0 || workgroups < 2 * NCOPY))
    return fail(FLINT_EINVAL, "workgroups %d: a multiple of %d, at least %d", workgroups, NCOPY, 2 * NCOPY);
  void* mem = nullptr;
  const size_t bytes = 8 * (size_t)NCOPY * workgroups + 64;  // NCOPY replicas of the slots, then the error word
  if (hipMalloc(&mem, bytes) != hipSuccess) return fail(FLINT_ENOMEM, "exchange slots");
  unsigned long long* slots = (unsigned long long*)mem;
  uint32_t* err = (uint32_t*)(slots + (size_t)NCOPY * workgroups);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  float ms = 0.f;
  uint32_t herr = 0;
  hipError_t e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) e = hipMemsetAsync(mem, 0, bytes, c->stream);
  if (e == hipSuccess) e = hipEventRecord(e0, c->stream);
  if (e == hipSuccess) e = launch_micro_exchange(slots, workgroups, rounds, err, c->stream, xcd);
  if (e == hipSuccess) e = hipEventRecord(e1, c->stream);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  if (e == hipSuccess) e = hipMemcpy(&herr, err, 4, hipMemcpyDeviceToHost);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipFree(mem);
  if (e != hipSuccess) return fail(FLINT_EHIP, "exchange: %s", hipGetErrorString(e));
  if (herr) return fail(FLINT_ETIMEOUT, "exchange: a wait exceeded its bound");
  *us_per_round = ms * 1e3f / rounds;
  return FLINT_OK;
}
}  // namespace

int flint_micro_exchange(flint_ctx* c, int32_t workgroups, int32_t rounds, float* us_per_round) {
  return micro_exchange(c, workgroups, rounds, us_per_round, false);
}

int flint_micro_exchange_xcd(flint_ctx* c, int32_t workgroups, int32_t rounds, float* us_per_round) {
  return micro_exchange(c, workgroups, rounds, us_per_round, true);
}

int flint_micro_launch(flint_ctx* c, int32_t launches, float* us_per_launch) {
  if (!c || !us_per_launch) return fail(FLINT_EINVAL, "NULL argument");
  if (launches < 1) return fail(FLINT_EINVAL, "launches %d < 1", launches);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  float ms = 0.f;
  hipError_t e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) e = launch_micro_empty(c->stream);
  if (e == hipSuccess) e = hipEventRecord(e0, c->stream);
  for (int i = 0; i < launches && e == hipSuccess; ++i) e = launch_micro_empty(c->stream);
  if (e == hipSuccess) e = hipEventRecord(e1, c->stream);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (e != hipSuccess) return fail(FLINT_EHIP, "empty launches: %s", hipGetErrorString(e));
  *us_per_launch = ms * 1e3f / launches;
  return FLINT_OK;
}

int flint_sync(flint_ctx* c) {
  if (!c) return fail(FLINT_EINVAL, "ctx is NULL");
  HIPCHECK(hipStreamSynchronize(c->stream));
  return latched_error(c);
}

int flint_set_wait_limit(flint_ctx* c, uint32_t microseconds) {
  if (!c) return fail(FLINT_EINVAL, "ctx is NULL");
  // 100 MHz clock; bounds beyond 2^32 ticks (42.9 s) are clamped
  const uint64_t t64 = microseconds ? (uint64_t)microseconds * 100u : SPIN_TIMEOUT;
  const uint32_t ticks = t64 > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)t64;
  HIPCHECK(hipStreamSynchronize(c->stream));
  c->base.spin_limit = ticks;
  HIPCHECK(hipMemcpy(&c->kdev->spin_limit, &ticks, sizeof ticks, hipMemcpyHostToDevice));
  return FLINT_OK;
}

int flint_device_info(flint_ctx* c, int32_t* grid, int32_t* block, int32_t* lds_bytes) {
  if (!c) return fail(FLINT_EINVAL, "ctx is NULL");
  if (grid) *grid = c->grid;
  if (block) *block = NT;
  if (lds_bytes) *lds_bytes = kernel_lds_bytes(c->cfg.weight_type);
  return FLINT_OK;
}

}  // extern "C"

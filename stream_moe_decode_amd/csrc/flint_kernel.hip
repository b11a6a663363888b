// Persistent decode kernel for gfx950 (MI355X).
//
// One launch runs one greedy decode step of one sequence through every layer
// and the head, the arrangement described in section 2 of the page "Flint
// Inference on Apple Silicon: rec Megakernel and Tempo9 Compared": all
// operators inside a single dispatch, every workgroup recomputing the two
// RMSNorms and the top-k itself, and cross-workgroup synchronisation only
// where data really crosses workgroups.
//
// Exchanges between workgroups use 8-byte "tagged" slots: 32 bits of payload
// and a 32-bit tag that names the producing phase of this launch.  A producer
// writes the slot with one system-scope 64-bit store (written through the
// XCD's L2 to memory); a consumer polls with system-scope 64-bit loads until
// every slot it needs carries the expected tag.  On MI355X each of the eight
// XCDs has its own L2 and agent-scope stores stay in the writer's L2, so
// system scope is what makes a slot visible on the other XCDs.  Slots read by
// every workgroup are replicated once per XCD so that each replica is polled
// by the 32 workgroups of one XCD only.  Tags are unique per launch, layer
// and phase, so no flag ever needs resetting; buffers alternate by layer
// parity so a slot is rewritten only after every reader has consumed it.
//
// Per layer the exchanges are: q/k/v -> attention partials -> merged
// attention output -> residual after o_proj -> SwiGLU output -> residual
// after the MLP.  Every wait is bounded (1 s); a timeout latches an error
// word that every other wait also checks, so a failed step always ends.

#include "flint_internal.h"

namespace flint {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// ---------------------------------------------------------------- scalars

__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ uint32_t f2bf(float f) {  // round to nearest even (finite inputs)
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float round_bf16(float f) { return __uint_as_float(f2bf(f) << 16); }
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}
__device__ __forceinline__ uint64_t now() { return __builtin_amdgcn_s_memrealtime(); }
__device__ __forceinline__ uint32_t xcc_id() { return __builtin_amdgcn_s_getreg((31 << 11) | 20); }
__device__ __forceinline__ uint64_t xload(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void xstore(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ uint64_t slot(uint32_t tag, uint32_t payload) { return ((uint64_t)tag << 32) | payload; }
__device__ __forceinline__ int part(int total, int G, int w) { return (int)(((long long)total * w) / G); }

template <int WT> constexpr bool kAct32 = (WT == W_F32);
template <int WT> constexpr int kChunkElems = WT == W_F32 ? 4 : (WT == W_BF16 ? 8 : 32);
template <int WT> __device__ __forceinline__ long long row_bytes(int in) {
  return WT == W_F32 ? 4ll * in : (WT == W_BF16 ? 2ll * in : in / 2);
}
// Activation value as the GEMV input: bf16-rounded unless the model is fp32.
template <int WT> __device__ __forceinline__ float act_round(float v) { return kAct32<WT> ? v : round_bf16(v); }

// ---------------------------------------------------------------- shared memory

struct Smem {
  float xres[MAX_H];                 // residual (every workgroup keeps all of it)
  uint32_t actA[MAX_QD];             // GEMV input: fp32 words or bf16 pairs
  float asumA[MAX_QD / 32];          // int4: sum of each 32-element chunk of actA
  uint32_t hbuf[MAX_HBUF];           // SwiGLU output as GEMV input
  float asumH[MAX_HBUF / 32];
  float ytmp[MAX_YROWS];             // this workgroup's GEMV results of a phase
  uint32_t gbuf[MAX_GATHER];         // gathered attention partials
  float qs[MAX_GQ * MAX_HD];         // scaled queries of one kv-head group
  float kn[MAX_HD], vn[MAX_HD];      // the new token's k, v
  float sc[MAX_GQ * MAX_P];          // scores / probabilities of a chunk
  float red[MAX_GQ * 512];           // P.V partial sums of thread subsets
  float ocur[MAX_GQ * MAX_HD];       // running attention output
  float mrun[MAX_GQ], lrun[MAX_GQ], alpha[MAX_GQ], lsum[MAX_GQ];
  float z[MAX_E];                    // router logits
  int sel[MAX_K];
  float wsel[MAX_K];
  float wred[NW * 2];
  unsigned long long best[NW];
  int flag;
};

// ---------------------------------------------------------------- reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
// Sum over the workgroup; every thread gets the same value.
__device__ float block_sum(Smem& sm, float v) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sm.wred[wave] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) t += sm.wred[w];
  return t;
}

// ---------------------------------------------------------------- activations in LDS

// int4 GEMV reads each 8-element group of the activation as the bf16 pairs
// (0,4) (1,5) (2,6) (3,7), the order in which one 32-bit word of nibbles is
// unpacked; fp32 / bf16 GEMVs read natural order.
template <int WT> __device__ __forceinline__ void act_put(uint32_t* act, int e, float v) {
  if constexpr (kAct32<WT>) {
    act[e] = __float_as_uint(v);
  } else {
    int p = WT == W_I4 ? ((e & ~7) | ((e & 3) << 1) | ((e >> 2) & 1)) : e;
    reinterpret_cast<uint16_t*>(act)[p] = (uint16_t)f2bf(v);
  }
}
// After act_put of n elements (and a barrier): chunk sums for the int4 bias.
template <int WT> __device__ void act_sums(const uint32_t* act, float* asum, int n) {
  if constexpr (WT == W_I4) {
    for (int c = threadIdx.x; c < n / 32; c += NT) {
      float s = 0.f;
      for (int k = 0; k < 16; ++k) {
        uint32_t w = act[c * 16 + k];
        s += bf2f(w & 0xFFFFu) + bf2f(w >> 16);
      }
      asum[c] = s;
    }
  }
}

// ---------------------------------------------------------------- GEMV

struct RowSrc {
  const uint8_t* w;
  const uint16_t* s;
  const uint32_t* act;
  const float* asum;
};

template <int WT>
__device__ __forceinline__ RowSrc mrow(const Mat& m, long long row, int in, const uint32_t* act, const float* asum) {
  RowSrc r;
  r.w = m.w + row * row_bytes<WT>(in);
  r.s = WT == W_I4 ? m.s + row * (in / 64) : nullptr;
  r.act = act;
  r.asum = asum;
  return r;
}

// Dot product of one 16-byte weight chunk with the matching activation chunk.
template <int WT>
__device__ __forceinline__ float chunk_dot(uint4 w, const RowSrc& r, int c, float scale) {
  if constexpr (WT == W_F32) {
    float4 x = *reinterpret_cast<const float4*>(r.act + 4 * c);
    float acc = __uint_as_float(w.x) * x.x;
    acc = fmaf(__uint_as_float(w.y), x.y, acc);
    acc = fmaf(__uint_as_float(w.z), x.z, acc);
    return fmaf(__uint_as_float(w.w), x.w, acc);
  } else if constexpr (WT == W_BF16) {
    uint4 x = *reinterpret_cast<const uint4*>(r.act + 4 * c);
    float acc = dot2(w.x, x.x, 0.f);
    acc = dot2(w.y, x.y, acc);
    acc = dot2(w.z, x.z, acc);
    return dot2(w.w, x.w, acc);
  } else {
    // nibble n of a word becomes bf16 (128 + n) via 0x4300 | n; the chunk sum
    // of the activation removes the 128 + 8 offset: sum (u - 8) a = sum (128 + u) a - 136 sum a
    const uint4* xp = reinterpret_cast<const uint4*>(r.act + 16 * c);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint4 x = xp[k];
      uint32_t q = ww[k];
      acc = dot2((q & 0x000F000Fu) | 0x43004300u, x.x, acc);
      acc = dot2(((q >> 4) & 0x000F000Fu) | 0x43004300u, x.y, acc);
      acc = dot2(((q >> 8) & 0x000F000Fu) | 0x43004300u, x.z, acc);
      acc = dot2(((q >> 12) & 0x000F000Fu) | 0x43004300u, x.w, acc);
    }
    return scale * (acc - 136.0f * r.asum[c]);
  }
}

// Dot products of `nrows` rows (length `in`) with their activations.  Each row
// is read in 16-byte chunks by a group of lanes (64, or fewer for short rows,
// several rows per wave); PU rows per wave are in flight at once.  outfn(row,
// value) runs on one lane of the row's group.
template <int WT, int PU, class RowFn, class OutFn>
__device__ void gemv(int nrows, int in, RowFn rowfn, OutFn outfn) {
  constexpr int CE = kChunkElems<WT>;
  const int C = in / CE;
  int LPR = 64;
  while (LPR > 1 && LPR / 2 >= C) LPR >>= 1;
  const int RPW = 64 / LPR, CPL = (C + LPR - 1) / LPR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / LPR, li = lane % LPR;
  const int step = NW * RPW;
  for (int rb = wave * RPW; rb < nrows; rb += step * PU) {
    float acc[PU];
    RowSrc src[PU];
    bool rv[PU];
#pragma unroll
    for (int p = 0; p < PU; ++p) {
      const int r = rb + p * step + sub;
      rv[p] = r < nrows;
      src[p] = rowfn(rv[p] ? r : 0);
      acc[p] = 0.f;
    }
    for (int j = 0; j < CPL; ++j) {
      const int c = li + j * LPR;
      const bool cv = c < C;
      uint4 wv[PU];
      float scl[PU];
#pragma unroll
      for (int p = 0; p < PU; ++p) {
        if (rv[p] && cv) {
          wv[p] = *reinterpret_cast<const uint4*>(src[p].w + 16ll * c);
          scl[p] = WT == W_I4 ? bf2f(src[p].s[c >> 1]) : 1.f;
        }
      }
#pragma unroll
      for (int p = 0; p < PU; ++p)
        if (rv[p] && cv) acc[p] += chunk_dot<WT>(wv[p], src[p], c, scl[p]);
    }
#pragma unroll
    for (int p = 0; p < PU; ++p) {
      float v = acc[p];
      for (int off = LPR / 2; off > 0; off >>= 1) v += __shfl_xor(v, off);
      if (li == 0 && rv[p]) outfn(rb + p * step + sub, v);
    }
  }
}

// ---------------------------------------------------------------- exchanges

struct Waiter {
  uint32_t* err;
  uint32_t* herr;
  bool abort;
};

// Latch an error: atomically in device memory, by a plain system-scope store
// in the host-mapped word (the host only tests it for non-zero).
__device__ __forceinline__ void raise_error(const Waiter& wt, uint32_t bits) {
  __hip_atomic_fetch_or(wt.err, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  __hip_atomic_store(wt.herr, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Wait until the n slots src[index(i)] carry `tag` and hand each payload to
// put(i, payload).  Each thread keeps up to 8 loads in flight.
template <class IndexFn, class PutFn>
__device__ void gather(const uint64_t* src, int n, uint32_t tag, IndexFn index, PutFn put, Waiter& wt) {
  for (int b0 = 0; b0 < n; b0 += 8 * NT) {
    uint64_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = b0 + (int)threadIdx.x + k * NT;
      v[k] = (i < n && !wt.abort) ? xload(src + index(i)) : slot(tag, 0);
    }
    uint32_t pending = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if ((uint32_t)(v[k] >> 32) != tag) pending |= 1u << k;
    if (pending) {
      const uint64_t t0 = now();
      uint32_t it = 0;
      while (pending) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (pending & (1u << k)) v[k] = xload(src + index(b0 + (int)threadIdx.x + k * NT));
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if ((pending & (1u << k)) && (uint32_t)(v[k] >> 32) == tag) pending &= ~(1u << k);
        if (pending && (++it & 15) == 0) {
          if (__hip_atomic_load(wt.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) & ERR_TIMEOUT) {
            wt.abort = true;
            break;
          }
          if (now() - t0 > SPIN_TIMEOUT) {
            raise_error(wt, ERR_TIMEOUT);
            wt.abort = true;
            break;
          }
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = b0 + (int)threadIdx.x + k * NT;
      if (i < n) put(i, (uint32_t)v[k]);
    }
  }
}

// Make a thread's abort decision the workgroup's (uniform) decision.
__device__ __forceinline__ bool sync_abort(Smem& sm, Waiter& wt) {
  __syncthreads();
  if (threadIdx.x == 0) sm.flag = 0;
  __syncthreads();
  if (wt.abort) sm.flag = 1;
  __syncthreads();
  wt.abort = sm.flag != 0;
  return wt.abort;
}

// Replicated exchange buffer: [NCOPY][2 parities][n] slots.
__device__ __forceinline__ void put_all(uint64_t* base, int n, int par, int idx, uint64_t v) {
#pragma unroll
  for (int c = 0; c < NCOPY; ++c) xstore(base + (size_t)(c * 2 + par) * n + idx, v);
}
__device__ __forceinline__ const uint64_t* copy_of(const uint64_t* base, int n, int par) {
  return base + (size_t)((xcc_id() & (NCOPY - 1)) * 2 + par) * n;
}

// ---------------------------------------------------------------- the kernel

template <int WT>
__global__ void __launch_bounds__(NT, 1) decode_kernel(const KArgs a) {
  __shared__ Smem sm;
  const int G = gridDim.x, W = blockIdx.x, tid = threadIdx.x;
  const int H = a.H, hd = a.hd, nq = a.nq, nkv = a.nkv, QD = nq * hd, Gq = nq / nkv;
  Waiter wt{a.err, a.herr, false};

  // token and position of this step (every workgroup makes the same choice)
  int tok = a.tokens[a.tok_idx];
  const int pos = a.len[a.seq];
  if (pos < 0 || pos >= a.cap) {
    if (W == 0 && tid == 0) raise_error(wt, ERR_POS);
    return;
  }
  if (tok < 0 || tok >= a.V) {
    if (W == 0 && tid == 0) raise_error(wt, ERR_TOKEN);
    tok = 0;
  }
  const bool ts = a.dbg_ts != nullptr && W == 0 && tid == 0;
  if (ts) a.dbg_ts[0] = now();

  // embedding row -> residual
  for (int e = tid; e < H; e += NT) {
    if constexpr (kAct32<WT>)
      sm.xres[e] = reinterpret_cast<const float*>(a.embed)[(long long)tok * H + e];
    else
      sm.xres[e] = bf2f(reinterpret_cast<const uint16_t*>(a.embed)[(long long)tok * H + e]);
  }
  __syncthreads();

  const int T = pos + 1;
  const int S = a.S;
  const int aj = W / S, as = W % S;  // attention work: kv head aj, split as
  const bool attn = aj < nkv;
  const int t0 = attn ? part(T, S, as) : 0, t1 = attn ? part(T, S, as + 1) : 0;
  const float qscale = 1.0f / sqrtf((float)hd);
  bool ok = true;  // false once a wait failed: skip to the argmax hand-off so the launch still ends cleanly
  const size_t kvstride = (size_t)a.cap * hd;  // elements per (layer, seq, kv head)

  for (int l = 0; l < a.L; ++l) {
    const uint32_t tag = a.epoch + (uint32_t)l * 8u;
    const int par = l & 1;
    uint64_t* stamp = ts ? a.dbg_ts + (size_t)(l + 1) * 8 : nullptr;

    // ---------------- input RMSNorm (recomputed by every workgroup)
    {
      float ss = 0.f;
      for (int e = tid; e < H; e += NT) ss += sm.xres[e] * sm.xres[e];
      ss = block_sum(sm, ss);
      const float inv = 1.0f / sqrtf(ss / (float)H + a.eps);
      const float* g = a.anorm + (size_t)l * H;
      for (int e = tid; e < H; e += NT) act_put<WT>(sm.actA, e, act_round<WT>(sm.xres[e] * inv * g[e]));
      __syncthreads();
      act_sums<WT>(sm.actA, sm.asumA, H);
      __syncthreads();
    }

    // ---------------- QKV rows (RoPE pairs i, i + hd/2 stay in one workgroup), RoPE, KV append
    {
      const int half = hd / 2, NPAIR = a.qkv_rows / 2;
      const int pb = part(NPAIR, G, W), pe = part(NPAIR, G, W + 1);
      const int nrows = 2 * (pe - pb);
      const long long lbase = (long long)l * a.qkv_rows;
      auto rowfn = [&](int q) {
        const int u = pb + q / 2, head = u / half, i = u % half;
        return mrow<WT>(a.qkv, lbase + head * hd + i + (q & 1) * half, H, sm.actA, sm.asumA);
      };
      gemv<WT, 4>(nrows, H, rowfn, [&](int q, float v) { sm.ytmp[q] = v; });
      __syncthreads();
      for (int q2 = tid; q2 < pe - pb; q2 += NT) {
        const int u = pb + q2, head = u / half, i = u % half;
        float y0 = sm.ytmp[2 * q2], y1 = sm.ytmp[2 * q2 + 1];
        if (head < nq + nkv) {  // q and k heads are rotated
          const float2 cs = a.rope[(size_t)pos * half + i];
          const float r0 = y0 * cs.x - y1 * cs.y, r1 = y1 * cs.x + y0 * cs.y;
          y0 = r0;
          y1 = r1;
        }
        const int row0 = head * hd + i, row1 = row0 + half;
        put_all(a.x_qkv, a.qkv_rows, par, row0, slot(tag + 0, __float_as_uint(y0)));
        put_all(a.x_qkv, a.qkv_rows, par, row1, slot(tag + 0, __float_as_uint(y1)));
        if (head >= nq) {  // append K or V of kv head j at position pos
          const bool isk = head < nq + nkv;
          const int j = isk ? head - nq : head - nq - nkv;
          const size_t off = (((size_t)l * a.B + a.seq) * nkv + j) * kvstride + (size_t)pos * hd;
          uint8_t* base = isk ? a.kc : a.vc;
          if constexpr (kAct32<WT>) {
            reinterpret_cast<float*>(base)[off + i] = y0;
            reinterpret_cast<float*>(base)[off + i + half] = y1;
          } else {
            reinterpret_cast<uint16_t*>(base)[off + i] = (uint16_t)f2bf(y0);
            reinterpret_cast<uint16_t*>(base)[off + i + half] = (uint16_t)f2bf(y1);
          }
        }
      }
    }
    if (stamp) stamp[0] = now();

    // ---------------- attention partial over positions [t0, t1) of kv head aj
    if (attn) {
      const int h0 = aj * Gq;
      if (t0 < t1) {
        const uint64_t* src = copy_of(a.x_qkv, a.qkv_rows, par);
        gather(src, Gq * hd, tag + 0, [&](int i) { return h0 * hd + i; },
               [&](int i, uint32_t p) { sm.qs[i] = __uint_as_float(p) * qscale; }, wt);
        if (t1 == T) {  // this split holds the new token: its k, v come from the exchange
          gather(src, 2 * hd, tag + 0,
                 [&](int i) { return i < hd ? (nq + aj) * hd + i : (nq + nkv + aj) * hd + (i - hd); },
                 [&](int i, uint32_t p) {
                   const float v = act_round<WT>(__uint_as_float(p));
                   if (i < hd) sm.kn[i] = v; else sm.vn[i - hd] = v;
                 },
                 wt);
        }
      }
      if (sync_abort(sm, wt)) {
        ok = false;
        break;
      }
      if (tid < Gq) {
        sm.mrun[tid] = -INFINITY;
        sm.lrun[tid] = 0.f;
      }
      for (int i = tid; i < Gq * hd; i += NT) sm.ocur[i] = 0.f;
      __syncthreads();
      const size_t cbase = (((size_t)l * a.B + a.seq) * nkv + aj) * kvstride;
      for (int c0 = t0; c0 < t1; c0 += MAX_P) {
        const int np = min(MAX_P, t1 - c0);
        // scores: one thread per position
        for (int i = tid; i < np; i += NT) {
          const int tau = c0 + i;
          float s[MAX_GQ];
#pragma unroll
          for (int h = 0; h < MAX_GQ; ++h) s[h] = 0.f;
          if (tau == pos) {
            for (int e = 0; e < hd; ++e) {
              const float kv = sm.kn[e];
#pragma unroll
              for (int h = 0; h < MAX_GQ; ++h)
                if (h < Gq) s[h] = fmaf(sm.qs[h * hd + e], kv, s[h]);
            }
          } else if constexpr (kAct32<WT>) {
            const float4* kr = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.kc) + cbase + (size_t)tau * hd);
            for (int e4 = 0; e4 < hd / 4; ++e4) {
              const float4 k4 = kr[e4];
#pragma unroll
              for (int h = 0; h < MAX_GQ; ++h)
                if (h < Gq) {
                  const float* q = sm.qs + h * hd + e4 * 4;
                  s[h] = fmaf(q[0], k4.x, fmaf(q[1], k4.y, fmaf(q[2], k4.z, fmaf(q[3], k4.w, s[h]))));
                }
            }
          } else {
            const uint4* kr = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.kc) + cbase + (size_t)tau * hd);
            for (int e8 = 0; e8 < hd / 8; ++e8) {
              const uint4 k8 = kr[e8];
              const float kf[8] = {bf2f(k8.x & 0xFFFF), bf2f(k8.x >> 16), bf2f(k8.y & 0xFFFF), bf2f(k8.y >> 16),
                                   bf2f(k8.z & 0xFFFF), bf2f(k8.z >> 16), bf2f(k8.w & 0xFFFF), bf2f(k8.w >> 16)};
#pragma unroll
              for (int h = 0; h < MAX_GQ; ++h)
                if (h < Gq) {
                  const float* q = sm.qs + h * hd + e8 * 8;
                  float t = s[h];
#pragma unroll
                  for (int k = 0; k < 8; ++k) t = fmaf(q[k], kf[k], t);
                  s[h] = t;
                }
            }
          }
#pragma unroll
          for (int h = 0; h < MAX_GQ; ++h)
            if (h < Gq) sm.sc[h * MAX_P + i] = s[h];
        }
        __syncthreads();
        // chunk max per head (wave w handles heads w, w + NW, ...)
        {
          const int lane = tid & 63, wave = tid >> 6;
          for (int h = wave; h < Gq; h += NW) {
            float m = -INFINITY;
            for (int i = lane; i < np; i += 64) m = fmaxf(m, sm.sc[h * MAX_P + i]);
            m = wave_max(m);
            if (lane == 0) {
              const float mn = fmaxf(sm.mrun[h], m);
              sm.alpha[h] = sm.mrun[h] == -INFINITY ? 0.f : __expf(sm.mrun[h] - mn);
              sm.mrun[h] = mn;
            }
          }
        }
        __syncthreads();
        for (int i = tid; i < Gq * np; i += NT) {
          const int h = i / np, k = i % np;
          sm.sc[h * MAX_P + k] = __expf(sm.sc[h * MAX_P + k] - sm.mrun[h]);
        }
        __syncthreads();
        {
          const int lane = tid & 63, wave = tid >> 6;
          for (int h = wave; h < Gq; h += NW) {
            float t = 0.f;
            for (int i = lane; i < np; i += 64) t += sm.sc[h * MAX_P + i];
            t = wave_sum(t);
            if (lane == 0) sm.lsum[h] = t;
          }
        }
        // P.V: thread = (dim pair dp, subset sb); subsets stride over positions
        {
          const int DP = hd / 2, NS = NT / DP;
          const int dp = tid % DP, sb = tid / DP;
          float acc0[MAX_GQ], acc1[MAX_GQ];
#pragma unroll
          for (int h = 0; h < MAX_GQ; ++h) acc0[h] = acc1[h] = 0.f;
          for (int i = sb; i < np; i += NS) {
            const int tau = c0 + i;
            float v0, v1;
            if (tau == pos) {
              v0 = sm.vn[2 * dp];
              v1 = sm.vn[2 * dp + 1];
            } else if constexpr (kAct32<WT>) {
              const float2 v2 = reinterpret_cast<const float2*>(reinterpret_cast<const float*>(a.vc) + cbase + (size_t)tau * hd)[dp];
              v0 = v2.x;
              v1 = v2.y;
            } else {
              const uint32_t v2 = reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(a.vc) + cbase + (size_t)tau * hd)[dp];
              v0 = bf2f(v2 & 0xFFFF);
              v1 = bf2f(v2 >> 16);
            }
#pragma unroll
            for (int h = 0; h < MAX_GQ; ++h)
              if (h < Gq) {
                const float p = sm.sc[h * MAX_P + i];
                acc0[h] = fmaf(p, v0, acc0[h]);
                acc1[h] = fmaf(p, v1, acc1[h]);
              }
          }
#pragma unroll
          for (int h = 0; h < MAX_GQ; ++h)
            if (h < Gq) {
              sm.red[(sb * MAX_GQ + h) * hd + 2 * dp] = acc0[h];
              sm.red[(sb * MAX_GQ + h) * hd + 2 * dp + 1] = acc1[h];
            }
          __syncthreads();
          for (int i = tid; i < Gq * hd; i += NT) {
            const int h = i / hd, e = i % hd;
            float t = 0.f;
            for (int k = 0; k < NS; ++k) t += sm.red[(k * MAX_GQ + h) * hd + e];
            sm.ocur[i] = sm.ocur[i] * sm.alpha[h] + t;
          }
          __syncthreads();
          if (tid < Gq) sm.lrun[tid] = sm.lrun[tid] * sm.alpha[tid] + sm.lsum[tid];
          __syncthreads();
        }
      }
      // publish (m, l, o) of each head: slot ((h * (hd + 2) + field) * S + split)
      uint64_t* dst = a.x_part + (size_t)par * nq * (hd + 2) * S;
      for (int i = tid; i < Gq * (hd + 2); i += NT) {
        const int h = i / (hd + 2), f = i % (hd + 2);
        const float v = f == 0 ? sm.mrun[h] : (f == 1 ? sm.lrun[h] : sm.ocur[h * hd + f - 2]);
        xstore(dst + ((size_t)(h0 + h) * (hd + 2) + f) * S + as, slot(tag + 1, __float_as_uint(v)));
      }
    }
    if (stamp) stamp[1] = now();

    // ---------------- merge the splits: this workgroup's pairs of output dims
    {
      const int NPO = QD / 2;
      const int pb = part(NPO, G, W), pe = part(NPO, G, W + 1);
      const uint64_t* srcp = a.x_part + (size_t)par * nq * (hd + 2) * S;
      int e0 = 2 * pb;
      while (e0 < 2 * pe) {  // one head at a time (uniform loop)
        const int h = e0 / hd, eh0 = e0 % hd;
        const int ne = min(2 * pe, (h + 1) * hd) - e0;  // elements of head h in range (even)
        const int n = (2 + ne) * S;
        gather(srcp, n, tag + 1,
               [&](int i) {
                 const int f = i / S, s = i % S;
                 const int field = f < 2 ? f : 2 + eh0 + (f - 2);
                 return ((size_t)h * (hd + 2) + field) * S + s;
               },
               [&](int i, uint32_t p) { sm.gbuf[i] = p; }, wt);
        if (sync_abort(sm, wt)) {
          ok = false;
          break;
        }
        for (int k = tid; k < ne / 2; k += NT) {
          float M = -INFINITY;
          for (int s = 0; s < S; ++s) M = fmaxf(M, __uint_as_float(sm.gbuf[s]));
          float Lsum = 0.f, O0 = 0.f, O1 = 0.f;
          for (int s = 0; s < S; ++s) {
            const float m = __uint_as_float(sm.gbuf[s]);
            const float w = m == -INFINITY ? 0.f : __expf(m - M);
            Lsum = fmaf(w, __uint_as_float(sm.gbuf[S + s]), Lsum);
            O0 = fmaf(w, __uint_as_float(sm.gbuf[(2 + 2 * k) * S + s]), O0);
            O1 = fmaf(w, __uint_as_float(sm.gbuf[(3 + 2 * k) * S + s]), O1);
          }
          const float o0 = act_round<WT>(O0 / Lsum), o1 = act_round<WT>(O1 / Lsum);
          const int e = e0 + 2 * k;
          if constexpr (kAct32<WT>) {
            put_all(a.x_o, a.o_slots, par, e, slot(tag + 2, __float_as_uint(o0)));
            put_all(a.x_o, a.o_slots, par, e + 1, slot(tag + 2, __float_as_uint(o1)));
          } else {
            put_all(a.x_o, a.o_slots, par, e / 2, slot(tag + 2, f2bf(o0) | (f2bf(o1) << 16)));
          }
        }
        __syncthreads();
        e0 += ne;
      }
    }
    if (!ok) break;
    if (stamp) stamp[2] = now();

    // ---------------- o_proj rows + residual
    {
      const uint64_t* src = copy_of(a.x_o, a.o_slots, par);
      gather(src, a.o_slots, tag + 2, [](int i) { return i; },
             [&](int i, uint32_t p) {
               if constexpr (kAct32<WT>) {
                 act_put<WT>(sm.actA, i, __uint_as_float(p));
               } else {
                 act_put<WT>(sm.actA, 2 * i, bf2f(p & 0xFFFF));
                 act_put<WT>(sm.actA, 2 * i + 1, bf2f(p >> 16));
               }
             },
             wt);
      if (sync_abort(sm, wt)) {
        ok = false;
        break;
      }
      act_sums<WT>(sm.actA, sm.asumA, QD);
      __syncthreads();
      const int rb = part(H, G, W), re = part(H, G, W + 1);
      const long long lbase = (long long)l * H;
      gemv<WT, 4>(re - rb, QD, [&](int q) { return mrow<WT>(a.o, lbase + rb + q, QD, sm.actA, sm.asumA); },
                  [&](int q, float v) {
                    const int r = rb + q;
                    put_all(a.x_res1, H, par, r, slot(tag + 3, __float_as_uint(sm.xres[r] + v)));
                  });
      __syncthreads();
      gather(copy_of(a.x_res1, H, par), H, tag + 3, [](int i) { return i; },
             [&](int i, uint32_t p) { sm.xres[i] = __uint_as_float(p); }, wt);
      if (sync_abort(sm, wt)) {
        ok = false;
        break;
      }
    }
    if (stamp) stamp[3] = now();

    // ---------------- post-attention RMSNorm (recomputed by every workgroup)
    {
      float ss = 0.f;
      for (int e = tid; e < H; e += NT) ss += sm.xres[e] * sm.xres[e];
      ss = block_sum(sm, ss);
      const float inv = 1.0f / sqrtf(ss / (float)H + a.eps);
      const float* g = a.pnorm + (size_t)l * H;
      for (int e = tid; e < H; e += NT) act_put<WT>(sm.actA, e, act_round<WT>(sm.xres[e] * inv * g[e]));
      __syncthreads();
      act_sums<WT>(sm.actA, sm.asumA, H);
      __syncthreads();
    }

    const bool dense = l < a.n_dense;
    int nunit, inner;  // SwiGLU elements this layer produces, and the down projection's input width
    if (dense) {
      nunit = a.DI;
      inner = a.DI;
    } else {
      // ------------ router (every workgroup computes all logits) and top-k
      const int lm = l - a.n_dense;
      gemv<WT, 4>(a.E, H, [&](int q) { return mrow<WT>(a.router, (long long)lm * a.E + q, H, sm.actA, sm.asumA); },
                  [&](int q, float v) { sm.z[q] = v; });
      __syncthreads();
      if (tid < 64) {
        const int lane = tid;
        const float zl = lane < a.E ? sm.z[lane] : -INFINITY;
        float zsel = zl;
        const float zmax = wave_max(zl);
        const float den = wave_sum(lane < a.E ? __expf(zl - zmax) : 0.f);
        float wsum = 0.f;
        for (int r = 0; r < a.K; ++r) {
          float bv = zsel;
          int bi = lane;
#pragma unroll
          for (int off = 32; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off);
            const int oi = __shfl_xor(bi, off);
            if (ov > bv || (ov == bv && oi < bi)) {
              bv = ov;
              bi = oi;
            }
          }
          if (lane == bi) zsel = -INFINITY;
          const float w = __expf(bv - zmax) / den;
          wsum += w;
          if (lane == 0) {
            sm.sel[r] = bi;
            sm.wsel[r] = w;
          }
        }
        if (a.renorm && lane < a.K) sm.wsel[lane] = sm.wsel[lane] / wsum;
      }
      __syncthreads();
      if (W == 0 && tid < a.K) {
        if (a.dbg_routes) a.dbg_routes[(size_t)l * a.K + tid] = sm.sel[tid];
        if (a.dbg_rw) a.dbg_rw[(size_t)l * a.K + tid] = sm.wsel[tid];
      }
      nunit = a.K * a.EI;
      inner = a.EI;
    }
    if (dense && W == 0 && tid < a.K) {
      if (a.dbg_routes) a.dbg_routes[(size_t)l * a.K + tid] = -1;
      if (a.dbg_rw) a.dbg_rw[(size_t)l * a.K + tid] = 0.f;
    }
    if (stamp) stamp[4] = now();

    // ---------------- gate/up rows of this workgroup's SwiGLU elements
    {
      const int NPU = nunit / 2;
      const int pb = part(NPU, G, W), pe = part(NPU, G, W + 1);
      const int e0 = 2 * pb, ne = 2 * (pe - pb);
      const int lm = l - a.n_dense;
      auto rowfn = [&](int q) {
        const int u = e0 + q / 2;
        const Mat& m = (q & 1) ? (dense ? a.du : a.eu) : (dense ? a.dg : a.eg);
        long long row;
        if (dense) row = (long long)l * a.DI + u;
        else row = ((long long)lm * a.E + sm.sel[u / a.EI]) * a.EI + u % a.EI;
        return mrow<WT>(m, row, H, sm.actA, sm.asumA);
      };
      gemv<WT, 4>(2 * ne, H, rowfn, [&](int q, float v) { sm.ytmp[q] = v; });
      __syncthreads();
      for (int k = tid; k < ne / 2; k += NT) {
        float hv[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const float g = sm.ytmp[4 * k + 2 * t], u = sm.ytmp[4 * k + 2 * t + 1];
          hv[t] = act_round<WT>(g / (1.0f + __expf(-g)) * u);
        }
        const int e = e0 + 2 * k;
        if constexpr (kAct32<WT>) {
          put_all(a.x_h, a.h_slots, par, e, slot(tag + 4, __float_as_uint(hv[0])));
          put_all(a.x_h, a.h_slots, par, e + 1, slot(tag + 4, __float_as_uint(hv[1])));
        } else {
          put_all(a.x_h, a.h_slots, par, e / 2, slot(tag + 4, f2bf(hv[0]) | (f2bf(hv[1]) << 16)));
        }
      }
    }
    // ---------------- gather the SwiGLU output, down projection + residual
    {
      const int nslots = kAct32<WT> ? nunit : nunit / 2;
      gather(copy_of(a.x_h, a.h_slots, par), nslots, tag + 4, [](int i) { return i; },
             [&](int i, uint32_t p) {
               // element e of rank r lives at hbuf element r * inner + e: the same flat index
               if constexpr (kAct32<WT>) {
                 act_put<WT>(sm.hbuf, i, __uint_as_float(p));
               } else {
                 act_put<WT>(sm.hbuf, 2 * i, bf2f(p & 0xFFFF));
                 act_put<WT>(sm.hbuf, 2 * i + 1, bf2f(p >> 16));
               }
             },
             wt);
      if (sync_abort(sm, wt)) {
        ok = false;
        break;
      }
      act_sums<WT>(sm.hbuf, sm.asumH, nunit);
      __syncthreads();
      const int rb = part(H, G, W), re = part(H, G, W + 1);
      if (stamp) stamp[5] = now();
      if (dense) {
        gemv<WT, 4>(re - rb, inner,
                    [&](int q) { return mrow<WT>(a.dd, (long long)l * H + rb + q, inner, sm.hbuf, sm.asumH); },
                    [&](int q, float v) {
                      const int r = rb + q;
                      put_all(a.x_res2, H, par, r, slot(tag + 5, __float_as_uint(sm.xres[r] + v)));
                    });
      } else {
        const int K = a.K, lm = l - a.n_dense;
        const int wstride = kAct32<WT> ? inner : inner / 2;  // words of one rank's h
        gemv<WT, 4>((re - rb) * K, inner,
                    [&](int q) {
                      const int r = rb + q / K, k = q % K;
                      return mrow<WT>(a.ed, ((long long)lm * a.E + sm.sel[k]) * H + r, inner, sm.hbuf + k * wstride,
                                      sm.asumH + k * (inner / 32));
                    },
                    [&](int q, float v) { sm.ytmp[q] = v; });
        __syncthreads();
        for (int q = tid; q < re - rb; q += NT) {
          float y = 0.f;
          for (int k = 0; k < K; ++k) y = fmaf(sm.wsel[k], sm.ytmp[q * K + k], y);
          const int r = rb + q;
          put_all(a.x_res2, H, par, r, slot(tag + 5, __float_as_uint(sm.xres[r] + y)));
        }
      }
      __syncthreads();
      gather(copy_of(a.x_res2, H, par), H, tag + 5, [](int i) { return i; },
             [&](int i, uint32_t p) { sm.xres[i] = __uint_as_float(p); }, wt);
      if (sync_abort(sm, wt)) {
        ok = false;
        break;
      }
    }
    if (stamp) stamp[6] = now();
    if (a.dbg_resid && W == 0 && l == a.dbg_resid_layer)
      for (int e = tid; e < H; e += NT) a.dbg_resid[e] = sm.xres[e];
  }

  // ---------------- final norm, lm_head, argmax
  {
    float ss = 0.f;
    for (int e = tid; e < H; e += NT) ss += sm.xres[e] * sm.xres[e];
    ss = block_sum(sm, ss);
    const float inv = 1.0f / sqrtf(ss / (float)H + a.eps);
    for (int e = tid; e < H; e += NT) act_put<WT>(sm.actA, e, act_round<WT>(sm.xres[e] * inv * a.fnorm[e]));
    __syncthreads();
    // the head is bf16 (or fp32) even when the layers are int4
    constexpr int HW = WT == W_I4 ? W_BF16 : WT;
    if constexpr (WT == W_I4) {  // lm_head reads natural order: undo the int4 pairing
      for (int e = tid; e < H; e += NT) {
        const float v = act_round<WT>(sm.xres[e] * inv * a.fnorm[e]);
        reinterpret_cast<uint16_t*>(sm.hbuf)[e] = (uint16_t)f2bf(v);
      }
      __syncthreads();
    }
    const uint32_t* fact = WT == W_I4 ? sm.hbuf : sm.actA;
    const int vb = ok ? part(a.V, G, W) : 0, ve = ok ? part(a.V, G, W + 1) : 0;
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    Mat lmh{a.lmhead, nullptr};
    gemv<HW, 4>(ve - vb, H, [&](int q) { return mrow<HW>(lmh, vb + q, H, fact, nullptr); },
                [&](int q, float v) {
                  const int r = vb + q;
                  if (a.dbg_logits) a.dbg_logits[r] = v;
                  if (v > bv || (v == bv && r < bi)) {
                    bv = v;
                    bi = r;
                  }
                });
    // best of the workgroup: max logit, then lowest id
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    const uint32_t u = __float_as_uint(bv);
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    const unsigned long long key = bi == 0x7FFFFFFF ? 0ull : (((unsigned long long)ord << 32) | (0xFFFFFFFFu - (uint32_t)bi));
    if ((tid & 63) == 0) sm.best[tid >> 6] = key;
    __syncthreads();
    if (tid == 0) {
      unsigned long long k = 0;
      for (int w = 0; w < NW; ++w) k = sm.best[w] > k ? sm.best[w] : k;
      __hip_atomic_fetch_max(a.amax, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t prev = __hip_atomic_fetch_add(a.done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      if (prev == (uint32_t)G - 1) {  // last workgroup: publish the token, reset for the next launch
        const unsigned long long fin = __hip_atomic_exchange(a.amax, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        a.out_ids[a.out_idx] = (int32_t)(0xFFFFFFFFu - (uint32_t)(fin & 0xFFFFFFFFull));
        a.len[a.seq] = pos + 1;
        if (a.dbg_ts) a.dbg_ts[2] = now();
      }
    }
  }
  if (ts) a.dbg_ts[1] = now();
}

__global__ void fill_kernel(uint64_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0;
}

hipError_t launch_decode(int wt, const KArgs& a, int grid, hipStream_t stream) {
  switch (wt) {
    case W_F32: hipLaunchKernelGGL(decode_kernel<W_F32>, dim3(grid), dim3(NT), 0, stream, a); break;
    case W_BF16: hipLaunchKernelGGL(decode_kernel<W_BF16>, dim3(grid), dim3(NT), 0, stream, a); break;
    default: hipLaunchKernelGGL(decode_kernel<W_I4>, dim3(grid), dim3(NT), 0, stream, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_fill(uint64_t* p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3(256), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

int kernel_lds_bytes(int) { return (int)sizeof(Smem); }

hipError_t kernel_occupancy(int wt, int* per_cu) {
  switch (wt) {
    case W_F32: return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, decode_kernel<W_F32>, NT, 0);
    case W_BF16: return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, decode_kernel<W_BF16>, NT, 0);
    default: return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, decode_kernel<W_I4>, NT, 0);
  }
}

}  // namespace flint

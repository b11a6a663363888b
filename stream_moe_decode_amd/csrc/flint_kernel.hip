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
// XCD's L2 to memory); a consumer reads it with system-scope 64-bit loads.
// On MI355X each of the eight XCDs has its own L2 and agent-scope stores stay
// in the writer's L2, so system scope is what makes a slot visible on the
// other XCDs.  A consumer first lets one wave poll a sample of 64 slots
// ("sentinels") and only then reads every slot once, re-polling the few that
// are still stale, so the waiting workgroups do not flood the memory system
// with loads.  Slots read by every workgroup are replicated once per XCD so
// that each replica is read by the 32 workgroups of one XCD only.  Tags are
// unique per launch, layer and phase, so no flag ever needs resetting;
// buffers alternate by layer parity so a slot is rewritten only after every
// reader has consumed it.
//
// Weights of a phase are loaded into registers before the exchange that
// precedes the phase is waited for, so the HBM latency of activation-
// independent bytes hides behind the exchange; only the selected experts'
// weights are fetched after the routing decision.
//
// Per layer the exchanges are: q/k/v -> attention partials -> merged
// attention output -> residual after o_proj -> SwiGLU output -> residual
// after the MLP.  Every wait is bounded (1 s); a timeout latches an error
// word that every other wait also checks, so a failed step always ends.

#include "flint_internal.h"

namespace flint {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((address_space(3))) void lds_void;

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
// Start of workgroup w's share of `total` items split over G (total * G < 2^32).
__device__ __forceinline__ int part(int total, int G, int w) { return (int)(((uint32_t)total * (uint32_t)w) / (uint32_t)G); }
// q = n / d for 0 <= n < 2^22 and a small positive d, through a float reciprocal and one correction.
__device__ __forceinline__ int div_small(int n, int d, float inv) {
  int q = (int)((float)n * inv);
  q += (q + 1) * d <= n;
  q -= q * d > n;
  return q;
}
// wait until every vector memory operation of this wave has completed (vmcnt(0))
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int WT> constexpr bool kAct32 = (WT == W_F32);
template <int WT> constexpr int kChunkElems = WT == W_F32 ? 4 : (WT == W_BF16 ? 8 : 32);
template <int WT> __device__ __forceinline__ long long row_bytes(int in) {
  return WT == W_F32 ? 4ll * in : (WT == W_BF16 ? 2ll * in : in / 2);
}
// Activation value as the GEMV input: bf16-rounded unless the model is fp32.
template <int WT> __device__ __forceinline__ float act_round(float v) { return kAct32<WT> ? v : round_bf16(v); }

// ---------------------------------------------------------------- shared memory

struct AttnLds {
  float qs[MAX_GQ * MAX_HD];             // scaled queries of one kv-head group
  float kn[MAX_HD], vn[MAX_HD];          // the new token's k, v
  float sc[MAX_GQ * MAX_CHUNK_POS];      // scores / probabilities of a chunk
  float red[MAX_GQ * 512];               // P.V partial sums of thread subsets
  float ocur[MAX_GQ * MAX_HD];           // running attention output
  uint4 vbuf[KV_CHUNK_BYTES / 16];       // V rows of a chunk (LDS DMA target)
};
// Weight staging in LDS: item i of wave w is 64 lanes x 16 B at w16[(i * NW + w) * 64 + lane]
// and, for int4, the dword holding the item's scale at s32[(i * NW + w) * 64 + lane].
template <int CAP> struct StageLds {
  uint4 w16[CAP * NW * 64];
  uint32_t s32[CAP * NW * 64];
};
struct MlpLds {
  uint32_t hbuf[MAX_HBUF / 2];           // SwiGLU output as GEMV input (also the lm_head input)
  float asumH[MAX_HBUF / 32];
  StageLds<GU_CAP> gu;                   // gate/up weights
  StageLds<DN_CAP> dn;                   // down weights
};

struct Smem {
  float xres[MAX_H];                     // residual (every workgroup keeps all of it)
  uint32_t actA[MAX_QD];                 // GEMV input: fp32 words or bf16 pairs
  float asumA[MAX_QD / 32];              // int4: sum of each 32-element chunk of actA
  float ytmp[MAX_YROWS];                 // this workgroup's GEMV results of a phase
  StageLds<QKV_CAP> sq;                  // QKV weights (staged during the previous layer)
  StageLds<O_CAP> so;                    // o_proj weights (staged during the merge)
  union {
    AttnLds att;
    StageLds<R_CAP> rt;                  // router weights (staged during the o_proj exchange)
    MlpLds mlp;
    uint32_t gbuf[MAX_GATHER];           // gathered attention partials
  } u;
  float mrun[MAX_GQ], lrun[MAX_GQ], alpha[MAX_GQ], lsum[MAX_GQ];
  float z[MAX_E];                        // router logits
  int sel[MAX_K];
  float wsel[MAX_K];
  float wred[NW * 2];
  unsigned long long best[NW];
  int flag;
};

// ---------------------------------------------------------------- reductions

// Cross-lane moves without LDS: DPP within rows of 16 lanes, permlane swaps
// across rows.  Every butterfly step combines a lane with its partner
// (lane ^ 1, ^ 2, mirrored within 8 and 16, ^ 16, ^ 32), so after the steps
// every lane of the group holds the same reduced value.
template <int CTRL> __device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL> __device__ __forceinline__ int dppi(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;
// value of the partner lane across 16 / 32 lanes (lane ^ 16, lane ^ 32)
__device__ __forceinline__ float swap16(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float((threadIdx.x & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float swap32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
__device__ __forceinline__ int swap16i(int v) {
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return (threadIdx.x & 16) ? r[0] : r[1];
}
__device__ __forceinline__ int swap32i(int v) {
  auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (threadIdx.x & 32) ? r[0] : r[1];
}
// Sum over aligned groups of n lanes (n = 1, 2, 4, ..., 64).
__device__ __forceinline__ float group_sum(float v, int n) {
  if (n >= 2) v += dpp<DPP_XOR1>(v);
  if (n >= 4) v += dpp<DPP_XOR2>(v);
  if (n >= 8) v += dpp<DPP_HALF_MIRROR>(v);
  if (n >= 16) v += dpp<DPP_MIRROR>(v);
  if (n >= 32) v += swap16(v);
  if (n >= 64) v += swap32(v);
  return v;
}
__device__ __forceinline__ float wave_sum(float v) { return group_sum(v, 64); }
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<DPP_XOR1>(v));
  v = fmaxf(v, dpp<DPP_XOR2>(v));
  v = fmaxf(v, dpp<DPP_HALF_MIRROR>(v));
  v = fmaxf(v, dpp<DPP_MIRROR>(v));
  v = fmaxf(v, swap16(v));
  return fmaxf(v, swap32(v));
}
// (value, index) maximum over the wave: larger value, then lower index.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#define FLINT_ARGSTEP(MOVV, MOVI)            \
  {                                          \
    const float ov = MOVV;                   \
    const int oi = MOVI;                     \
    if (ov > v || (ov == v && oi < i)) {     \
      v = ov;                                \
      i = oi;                                \
    }                                        \
  }
  FLINT_ARGSTEP(dpp<DPP_XOR1>(v), dppi<DPP_XOR1>(i))
  FLINT_ARGSTEP(dpp<DPP_XOR2>(v), dppi<DPP_XOR2>(i))
  FLINT_ARGSTEP(dpp<DPP_HALF_MIRROR>(v), dppi<DPP_HALF_MIRROR>(i))
  FLINT_ARGSTEP(dpp<DPP_MIRROR>(v), dppi<DPP_MIRROR>(i))
  FLINT_ARGSTEP(swap16(v), swap16i(i))
  FLINT_ARGSTEP(swap32(v), swap32i(i))
#undef FLINT_ARGSTEP
}
// Sum over the workgroup; every thread gets the same value.
__device__ __forceinline__ float block_sum(Smem& sm, float v) {
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
template <int WT> __device__ __forceinline__ void act_sums(const uint32_t* act, float* asum, int n) {
  if constexpr (WT == W_I4) {
    for (int c = threadIdx.x; c < n / 32; c += NT) {
      const uint4* p = reinterpret_cast<const uint4*>(act + c * 16);
      const uint4 x0 = p[0], x1 = p[1], x2 = p[2], x3 = p[3];
      float s0 = 0.f, s1 = 0.f;
      const uint32_t w[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                              x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
#pragma unroll
      for (int k = 0; k < 16; k += 2) {
        s0 += bf2f(w[k] & 0xFFFFu) + bf2f(w[k] >> 16);
        s1 += bf2f(w[k + 1] & 0xFFFFu) + bf2f(w[k + 1] >> 16);
      }
      asum[c] = s0 + s1;
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
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint4 x = xp[k];
      uint32_t q = ww[k];
      a0 = dot2((q & 0x000F000Fu) | 0x43004300u, x.x, a0);
      a1 = dot2(((q >> 4) & 0x000F000Fu) | 0x43004300u, x.y, a1);
      a0 = dot2(((q >> 8) & 0x000F000Fu) | 0x43004300u, x.z, a0);
      a1 = dot2(((q >> 12) & 0x000F000Fu) | 0x43004300u, x.w, a1);
    }
    return scale * ((a0 + a1) - 136.0f * r.asum[c]);
  }
}

// Lane geometry of a GEMV over `nrows` rows of width `in`: each row is read in
// 16-byte chunks by a group of LPR lanes (64, or fewer for short rows, several
// rows per wave).  A lane's work is a list of NI items (row pass p, chunk j),
// processed in register-staged blocks of R items whose loads are all in flight
// together.
struct Geo {
  int nrows, C, LPR, RPW, CPL, NI, sub, li, wave;
};
template <int WT> __device__ __forceinline__ Geo geo(int nrows, int in) {
  Geo g;
  g.nrows = nrows;
  g.C = in / kChunkElems<WT>;
  int LPR = 64;
  while (LPR > 1 && LPR / 2 >= g.C) LPR >>= 1;
  g.LPR = LPR;
  g.RPW = 64 / LPR;
  g.CPL = (g.C + LPR - 1) / LPR;
  const int lane = threadIdx.x & 63;
  g.wave = threadIdx.x >> 6;
  g.sub = lane / LPR;
  g.li = lane % LPR;
  const int npass = (nrows + NW * g.RPW - 1) / (NW * g.RPW);
  g.NI = npass * g.CPL;
  return g;
}

template <int R> struct Stage {
  uint4 w[R];
  float s[R];
};

template <int WT, int R, class RowFn>
__device__ __forceinline__ void stage_load(Stage<R>& st, const Geo& g, int blk, RowFn rowfn) {
  int p = (blk * R) / g.CPL, j = blk * R - p * g.CPL;
#pragma unroll
  for (int i = 0; i < R; ++i, (++j == g.CPL ? (j = 0, ++p) : 0)) {
    const int k = blk * R + i;
    if (k < g.NI) {
      const int r = g.wave * g.RPW + p * NW * g.RPW + g.sub, c = g.li + j * g.LPR;
      if (r < g.nrows && c < g.C) {
        const RowSrc src = rowfn(r);
        st.w[i] = *reinterpret_cast<const uint4*>(src.w + 16ll * c);
        if constexpr (WT == W_I4) st.s[i] = bf2f(src.s[c >> 1]);
      }
    }
  }
}

template <int WT, int R, class RowFn, class OutFn>
__device__ __forceinline__ void stage_compute(const Stage<R>& st, const Geo& g, int blk, float& acc, RowFn rowfn,
                                              OutFn outfn) {
  int p = (blk * R) / g.CPL, j = blk * R - p * g.CPL;
#pragma unroll
  for (int i = 0; i < R; ++i, (++j == g.CPL ? (j = 0, ++p) : 0)) {
    const int k = blk * R + i;
    if (k < g.NI) {  // uniform across the wave
      const int r = g.wave * g.RPW + p * NW * g.RPW + g.sub, c = g.li + j * g.LPR;
      if (r < g.nrows && c < g.C) acc += chunk_dot<WT>(st.w[i], rowfn(r), c, WT == W_I4 ? st.s[i] : 1.f);
      if (j == g.CPL - 1) {
        const float v = group_sum(acc, g.LPR);
        if (g.li == 0 && r < g.nrows) outfn(r, v);
        acc = 0.f;
      }
    }
  }
}

// Run a GEMV whose first block may already be staged (`pre`).  With DB the
// blocks are double-buffered (the next block's loads are in flight during
// compute); without it a phase that fits one block holds a single stage.
template <int WT, int R, bool DB, class RowFn, class OutFn>
__device__ __forceinline__ void gemv_run(const Geo& g, Stage<R>& A, bool pre, RowFn rowfn, OutFn outfn) {
  const int nb = (g.NI + R - 1) / R;
  float acc = 0.f;
  if constexpr (DB) {
    if (!pre) stage_load<WT, R>(A, g, 0, rowfn);
    Stage<R> B;
    for (int b = 0; b < nb; b += 2) {
      if (b + 1 < nb) stage_load<WT, R>(B, g, b + 1, rowfn);
      stage_compute<WT, R>(A, g, b, acc, rowfn, outfn);
      if (b + 1 < nb) {
        if (b + 2 < nb) stage_load<WT, R>(A, g, b + 2, rowfn);
        stage_compute<WT, R>(B, g, b + 1, acc, rowfn, outfn);
      }
    }
  } else {
    for (int b = 0; b < nb; ++b) {
      if (b > 0 || !pre) stage_load<WT, R>(A, g, b, rowfn);
      stage_compute<WT, R>(A, g, b, acc, rowfn, outfn);
    }
  }
}

// LDS-staged GEMV: the items of a phase are brought into LDS by DMA (no
// registers held, so every load of the phase is in flight at once and the
// loads can be issued long before the activation is ready), then each wave
// computes its own items from LDS.  Phases with more items than the staging
// area holds run in rounds.
struct LStage {
  uint4* w16;
  uint32_t* s32;
  int cap;
};
template <int CAP> __device__ __forceinline__ LStage lstage(StageLds<CAP>& s) { return LStage{s.w16, s.s32, CAP}; }

__device__ __forceinline__ void dma16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)l, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, void* l) { __builtin_amdgcn_global_load_lds(g, (lds_void*)l, 4, 0, 0); }
// wait until this wave's LDS reads have completed (lgkmcnt(0))
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

template <int WT, class RowFn>
__device__ __forceinline__ void lstage_issue(const LStage& st, const Geo& g, int round, RowFn rowfn) {
  const int k0 = round * st.cap;
  const int n = min(st.cap, g.NI - k0);
  int p = k0 / g.CPL, j = k0 - p * g.CPL;
  for (int i = 0; i < n; ++i) {
    const int r = g.wave * g.RPW + p * NW * g.RPW + g.sub, c = g.li + j * g.LPR;
    if (r < g.nrows && c < g.C) {
      const RowSrc src = rowfn(r);
      dma16(src.w + 16ll * c, &st.w16[(i * NW + g.wave) * 64]);
      if constexpr (WT == W_I4) dma4(src.s + ((c >> 1) & ~1), &st.s32[(i * NW + g.wave) * 64]);
    }
    if (++j == g.CPL) {
      j = 0;
      ++p;
    }
  }
}

template <int WT, class RowFn, class OutFn>
__device__ __forceinline__ void lstage_compute(const LStage& st, const Geo& g, int round, float& acc, RowFn rowfn,
                                               OutFn outfn) {
  const int k0 = round * st.cap;
  const int n = min(st.cap, g.NI - k0);
  const int lane = threadIdx.x & 63;
  int p = k0 / g.CPL, j = k0 - p * g.CPL;
#pragma unroll 2
  for (int i = 0; i < n; ++i) {
    const int r = g.wave * g.RPW + p * NW * g.RPW + g.sub, c = g.li + j * g.LPR;
    if (r < g.nrows && c < g.C) {
      const uint4 w = st.w16[(i * NW + g.wave) * 64 + lane];
      float scale = 1.f;
      if constexpr (WT == W_I4) {
        const uint32_t sw = st.s32[(i * NW + g.wave) * 64 + lane];
        scale = bf2f(((c >> 1) & 1) ? (sw >> 16) : (sw & 0xFFFFu));
      }
      acc += chunk_dot<WT>(w, rowfn(r), c, scale);
    }
    if (j == g.CPL - 1) {  // uniform across the wave
      const float v = group_sum(acc, g.LPR);
      if (g.li == 0 && r < g.nrows) outfn(r, v);
      acc = 0.f;
    }
    if (++j == g.CPL) {
      j = 0;
      ++p;
    }
  }
}

// Run a staged GEMV; `issued`: round 0 was already issued.  The activation
// (read through rowfn) must be in LDS and visible to this wave.
template <int WT, class RowFn, class OutFn>
__device__ __forceinline__ void gemv_lds(const LStage& st, const Geo& g, bool issued, RowFn rowfn, OutFn outfn) {
  const int nr = (g.NI + st.cap - 1) / st.cap;
  float acc = 0.f;
  for (int b = 0; b < nr; ++b) {
    if (b > 0) wait_lds();
    if (b > 0 || !issued) lstage_issue<WT>(st, g, b, rowfn);
    wait_vmem();
    lstage_compute<WT>(st, g, b, acc, rowfn, outfn);
  }
}

// ---------------------------------------------------------------- exchanges

struct Waiter {
  uint32_t* err;
  uint32_t* herr;
  int sleep;
  int sentinels;
  bool abort;
};
__device__ __forceinline__ void backoff(const Waiter& wt) {
  __builtin_amdgcn_s_sleep(1);
  for (int z = 0; z < wt.sleep; ++z) __builtin_amdgcn_s_sleep(8);
}

// Latch an error: atomically in device memory, by a plain system-scope store
// in the host-mapped word (the host only tests it for non-zero).
__device__ __forceinline__ void raise_error(const Waiter& wt, uint32_t bits) {
  __hip_atomic_fetch_or(wt.err, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  __hip_atomic_store(wt.herr, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// True once this wait should give up: another wait has timed out, or this one
// has run for longer than the timeout (which it then reports).
__device__ __forceinline__ bool poll_timed_out(const Waiter& wt, uint64_t t0, uint32_t it) {
  if ((it & 15) == 0 &&
      (__hip_atomic_load(wt.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) & ERR_TIMEOUT))
    return true;
  if (now() - t0 > SPIN_TIMEOUT) {
    raise_error(wt, ERR_TIMEOUT);
    return true;
  }
  return false;
}

// Make a thread's abort decision the workgroup's (uniform) decision.
__device__ __forceinline__ bool sync_ok(Smem& sm, Waiter& wt) {
  __syncthreads();
  if (threadIdx.x == 0) sm.flag = 0;
  __syncthreads();
  if (wt.abort) sm.flag = 1;
  __syncthreads();
  wt.abort = sm.flag != 0;
  return !wt.abort;
}

// Wait until the n slots src[index(i)] carry `tag` and hand each payload to
// put(i, payload).  Wave 0 first polls up to 64 sentinel items (i = sent(k),
// k < nsent); then every thread reads its items once (8 loads in flight) and
// re-polls only those still stale.  Called by the whole workgroup; returns
// false (uniformly) if a wait failed.
template <class IndexFn, class SentFn, class PutFn>
__device__ __forceinline__ bool gather(Smem& sm, const uint64_t* src, int n, uint32_t tag, IndexFn index, SentFn sent, int nsent,
                       PutFn put, Waiter& wt) {
  const int tid = threadIdx.x;
  if (nsent > wt.sentinels) nsent = wt.sentinels;
  if (tid < 64 && tid < nsent && !wt.abort) {
    const uint64_t* p = src + index(sent(tid, nsent));
    if ((uint32_t)(xload(p) >> 32) != tag) {
      const uint64_t t0 = now();
      uint32_t it = 0;
      while ((uint32_t)(xload(p) >> 32) != tag) {
        backoff(wt);
        if (poll_timed_out(wt, t0, ++it)) {
          wt.abort = true;
          break;
        }
      }
    }
  }
  if (!sync_ok(sm, wt)) return false;
  for (int b0 = 0; b0 < n; b0 += 8 * NT) {
    uint64_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = b0 + tid + k * NT;
      v[k] = i < n ? xload(src + index(i)) : slot(tag, 0);
    }
    uint32_t pending = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if ((uint32_t)(v[k] >> 32) != tag) pending |= 1u << k;
    if (pending) {
      const uint64_t t0 = now();
      uint32_t it = 0;
      while (pending) {
        backoff(wt);
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (pending & (1u << k)) v[k] = xload(src + index(b0 + tid + k * NT));
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if ((pending & (1u << k)) && (uint32_t)(v[k] >> 32) == tag) pending &= ~(1u << k);
        if (pending && poll_timed_out(wt, t0, ++it)) {
          wt.abort = true;
          break;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = b0 + tid + k * NT;
      if (i < n) put(i, (uint32_t)v[k]);
    }
  }
  return sync_ok(sm, wt);
}

// Gather n contiguous slots, sentinels spread evenly.
template <class PutFn>
__device__ __forceinline__ bool gather_flat(Smem& sm, const uint64_t* src, int n, uint32_t tag, PutFn put,
                                            Waiter& wt) {
  const int ns = n < 64 ? n : 64;
  return gather(
      sm, src, n, tag, [](int i) { return i; }, [=](int k, int m) { return (int)(((long long)(k + 1) * n) / m) - 1; },
      ns, put, wt);
}

// Replicated exchange buffer: [NCOPY][2 parities][n] slots.
__device__ __forceinline__ void put_all(uint64_t* base, int n, int par, int idx, uint64_t v) {
#pragma unroll
  for (int c = 0; c < NCOPY; ++c) xstore(base + (size_t)(c * 2 + par) * n + idx, v);
}
__device__ __forceinline__ const uint64_t* copy_of(const uint64_t* base, int n, int par) {
  return base + (size_t)((xcc_id() & (NCOPY - 1)) * 2 + par) * n;
}

// ---------------------------------------------------------------- attention data

// K rows of positions [c0, c0 + np) to registers: TPP threads per row, 64 B each,
// KV_PASSES passes of NT / TPP positions; rows past np re-read the last one.
template <int WT>
__device__ __forceinline__ void load_k(uint4 (&kreg)[KV_PASSES][4], const uint8_t* kbase, int c0, int np, int rowb) {
  const int TPP = rowb / 64, PPP = NT / TPP;
  const int pp = threadIdx.x / TPP, pt = threadIdx.x % TPP;
#pragma unroll
  for (int p = 0; p < KV_PASSES; ++p) {
    const int i = p * PPP + pp;
    const int tau = c0 + (i < np ? i : np - 1);
    const uint4* src = reinterpret_cast<const uint4*>(kbase + (size_t)tau * rowb + pt * 64);
#pragma unroll
    for (int k = 0; k < 4; ++k) kreg[p][k] = src[k];
  }
}
// V rows of positions [c0, c0 + np) into LDS by DMA, 1 KB per wave instruction.
__device__ __forceinline__ void load_v(uint4* vbuf, const uint8_t* vbase, int c0, int np, int rowb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint8_t* vsrc = vbase + (size_t)c0 * rowb;
  const int units = np * rowb / 16;
#pragma unroll
  for (int q = 0; q < KV_CHUNK_BYTES / (NT * 16); ++q) {
    const int gi = q * NW + wave;
    if (gi * 64 < units) {
      const int unit = min(gi * 64 + lane, units - 1);
      __builtin_amdgcn_global_load_lds(vsrc + (size_t)unit * 16, (lds_void*)&vbuf[gi * 64], 16, 0, 0);
    }
  }
}

// ---------------------------------------------------------------- the kernel

// Model shapes known at compile time let every index, partition and row
// address fold to constants; DynShape reads them from the context instead.
struct DynShape {
  static constexpr bool kStatic = false;
  static constexpr int G = 0, H = 0, HD = 0, NQ = 0, NKV = 0, V = 0, DI = 0, E = 0, K = 0, EI = 0;
};
// 2048-wide residual, GQA 16 / 4 x 128, vocab 65536, dense MLP 6144,
// 64 experts top-6 of width 768, on a 256-workgroup grid.
struct Shape2048 {
  static constexpr bool kStatic = true;
  static constexpr int G = 256, H = 2048, HD = 128, NQ = 16, NKV = 4, V = 65536, DI = 6144, E = 64, K = 6, EI = 768;
};

template <int WT, class SH>
__global__ void __launch_bounds__(NT, 1) decode_kernel(const KStatic* __restrict__ ksp, const KDyn d) {
  __shared__ Smem sm;
  const KStatic& ks = *ksp;
  constexpr bool SS = SH::kStatic;
  const int G = SS ? SH::G : (int)gridDim.x, W = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = SS ? SH::H : ks.H, hd = SS ? SH::HD : ks.hd, nq = SS ? SH::NQ : ks.nq, nkv = SS ? SH::NKV : ks.nkv;
  const int QD = nq * hd, Gq = nq / nkv, L = ks.L;
  const int V_ = SS ? SH::V : ks.V, DI_ = SS ? SH::DI : ks.DI, E_ = SS ? SH::E : ks.E, K_ = SS ? SH::K : ks.K;
  const int EI_ = SS ? SH::EI : ks.EI;
  const int QR = (nq + 2 * nkv) * hd;                            // q, k, v rows
  const int OSL = kAct32<WT> ? QD : QD / 2;                      // slots of the merged attention output
  const int HSLOTS = ks.h_slots;                                 // slots of the SwiGLU output exchange
  Waiter wt{ks.err, ks.herr, ks.poll_sleep, ks.sentinels, false};
  uint8_t* const kc = d.kc;
  uint8_t* const vc = d.vc;
  const int seq = d.seq, B = d.B, cap = d.cap;
  const float2* const rope = d.rope;
  uint64_t* const stamps = (d.dbg_ts != nullptr && W == 0 && tid == 0) ? d.dbg_ts : nullptr;

  // token and position of this step (every workgroup makes the same choice)
  int tok = d.tokens[d.tok_idx];
  const int pos = d.len[seq];
  if (pos < 0 || pos >= cap) {
    if (W == 0 && tid == 0) raise_error(wt, ERR_POS);
    return;
  }
  if (tok < 0 || tok >= V_) {
    if (W == 0 && tid == 0) raise_error(wt, ERR_TOKEN);
    tok = 0;
  }
  if (stamps) stamps[0] = now();

  // embedding row -> residual
  for (int e = tid; e < H; e += NT) {
    if constexpr (kAct32<WT>)
      sm.xres[e] = reinterpret_cast<const float*>(ks.embed)[(long long)tok * H + e];
    else
      sm.xres[e] = bf2f(reinterpret_cast<const uint16_t*>(ks.embed)[(long long)tok * H + e]);
  }

  const int T = pos + 1;
  const int S = nkv > 0 ? G / nkv : 0;  // attention splits per kv head
  const int aj = W / S, as = W % S;  // attention work: kv head aj, split as
  const bool attn = aj < nkv;
  const int t0 = attn ? part(T, S, as) : 0, t1 = attn ? part(T, S, as + 1) : 0;
  const float qscale = 1.0f / sqrtf((float)hd);
  const int ebytes = kAct32<WT> ? 4 : 2;
  const int rowb = hd * ebytes;                 // bytes of one cached K or V row
  const int TPP = rowb / 64;                    // threads per K row (64 B each)
  const int PPP = NT / TPP;                     // positions per register pass
  const int CHP = KV_PASSES * PPP;              // positions per attention chunk
  const size_t kvstride = (size_t)cap * hd;     // elements per (layer, seq, kv head)
  bool ok = true;  // false once a wait failed: skip to the argmax hand-off so the launch still ends cleanly

  // QKV rows of this workgroup: RoPE pairs (i, i + hd/2) stay together
  const int half = hd / 2, NPAIR = QR / 2;
  const int qpb = part(NPAIR, G, W), qpe = part(NPAIR, G, W + 1);
  const Geo gq = geo<WT>(2 * (qpe - qpb), H);
  auto qkv_rowfn = [&](int l) {
    return [&, l](int q) {
      const int u = qpb + q / 2, head = u / half, i = u % half;
      return mrow<WT>(ks.qkv, (long long)l * QR + head * hd + i + (q & 1) * half, H, sm.actA, sm.asumA);
    };
  };
  lstage_issue<WT>(lstage(sm.sq), gq, 0, qkv_rowfn(0));
  // this workgroup's shares of every other phase (the same in every layer)
  const int orb = part(H, G, W), ore = part(H, G, W + 1);               // o_proj and down rows
  const int mpb = part(QD / 2, G, W), mpe = part(QD / 2, G, W + 1);     // merged output dim pairs
  const int dpb = part(DI_ / 2, G, W), dpe = part(DI_ / 2, G, W + 1);  // dense SwiGLU pairs
  const int xpb = part(K_ * EI_ / 2, G, W), xpe = part(K_ * EI_ / 2, G, W + 1);  // expert pairs
  const float inv_ei = 1.0f / (float)EI_, inv_k = 1.0f / (float)K_;
  __syncthreads();

  for (int l = 0; l < L; ++l) {
    const uint32_t tag = d.epoch + (uint32_t)l * 8u;
    const int par = l & 1;
    uint64_t* stamp = stamps ? stamps + (size_t)(l + 1) * 16 : nullptr;
    const size_t cbase = (((size_t)l * B + seq) * nkv + (attn ? aj : 0)) * kvstride;
    const uint8_t* const kbase = kc + cbase * ebytes;
    const uint8_t* const vbase = vc + cbase * ebytes;

    // ---------------- attention data of the first chunk: K rows to registers, V rows to LDS
    uint4 kreg[KV_PASSES][4];
    if (attn && t1 > t0) {
      const int np0 = min(CHP, t1 - t0);
      load_k<WT>(kreg, kbase, t0, np0, rowb);
      load_v(sm.u.att.vbuf, vbase, t0, np0, rowb);
    }

    // ---------------- input RMSNorm (recomputed by every workgroup)
    {
      float ss = 0.f;
      for (int e = tid; e < H; e += NT) ss += sm.xres[e] * sm.xres[e];
      ss = block_sum(sm, ss);
      const float inv = 1.0f / sqrtf(ss / (float)H + ks.eps);
      const float* g = ks.anorm + (size_t)l * H;
      for (int e = tid; e < H; e += NT) act_put<WT>(sm.actA, e, act_round<WT>(sm.xres[e] * inv * g[e]));
      __syncthreads();
      act_sums<WT>(sm.actA, sm.asumA, H);
      __syncthreads();
    }

    if (stamp) stamp[7] = now();
    // ---------------- QKV rows (staged earlier), RoPE, KV append, publish
    gemv_lds<WT>(lstage(sm.sq), gq, true, qkv_rowfn(l), [&](int q, float v) { sm.ytmp[q] = v; });
    if (stamp) stamp[8] = now();
    __syncthreads();
    for (int q2 = tid; q2 < qpe - qpb; q2 += NT) {
      const int u = qpb + q2, head = u / half, i = u % half;
      float y0 = sm.ytmp[2 * q2], y1 = sm.ytmp[2 * q2 + 1];
      if (head < nq + nkv) {  // q and k heads are rotated
        const float2 cs = rope[(size_t)pos * half + i];
        const float r0 = y0 * cs.x - y1 * cs.y, r1 = y1 * cs.x + y0 * cs.y;
        y0 = r0;
        y1 = r1;
      }
      const int row0 = head * hd + i, row1 = row0 + half;
      put_all(ks.x_qkv, QR, par, row0, slot(tag + 0, __float_as_uint(y0)));
      put_all(ks.x_qkv, QR, par, row1, slot(tag + 0, __float_as_uint(y1)));
      if (head >= nq) {  // append K or V of kv head j at position pos
        const bool isk = head < nq + nkv;
        const int j = isk ? head - nq : head - nq - nkv;
        const size_t off = (((size_t)l * B + seq) * nkv + j) * kvstride + (size_t)pos * hd;
        uint8_t* base = isk ? kc : vc;
        if constexpr (kAct32<WT>) {
          reinterpret_cast<float*>(base)[off + i] = y0;
          reinterpret_cast<float*>(base)[off + i + half] = y1;
        } else {
          reinterpret_cast<uint16_t*>(base)[off + i] = (uint16_t)f2bf(y0);
          reinterpret_cast<uint16_t*>(base)[off + i + half] = (uint16_t)f2bf(y1);
        }
      }
    }
    if (stamp) stamp[0] = now();

    // ---------------- attention partial over positions [t0, t1) of kv head aj
    if (attn) {
      const int h0 = aj * Gq;
      AttnLds& at = sm.u.att;
      if (t0 < t1) {
        const uint64_t* src = copy_of(ks.x_qkv, QR, par);
        const int nqs = Gq * hd;
        const bool last = t1 == T;  // this split holds the new token: its k, v come from the exchange
        const int n = nqs + (last ? 2 * hd : 0);
        const int ns = n < 64 ? n : 64;
        ok = gather(
            sm, src, n, tag + 0,
            [&](int i) {
              return i < nqs ? h0 * hd + i
                             : (i < nqs + hd ? (nq + aj) * hd + (i - nqs) : (nq + nkv + aj) * hd + (i - nqs - hd));
            },
            [=](int k, int m) { return (int)(((long long)(k + 1) * n) / m) - 1; }, ns,
            [&](int i, uint32_t p) {
              const float v = __uint_as_float(p);
              if (i < nqs) at.qs[i] = v * qscale;
              else if (i < nqs + hd) at.kn[i - nqs] = act_round<WT>(v);
              else at.vn[i - nqs - hd] = act_round<WT>(v);
            },
            wt);
      } else {
        ok = sync_ok(sm, wt);
      }
      if (!ok) break;
      if (stamp) stamp[9] = now();
      if (tid < Gq) {
        sm.mrun[tid] = -INFINITY;
        sm.lrun[tid] = 0.f;
      }
      for (int i = tid; i < Gq * hd; i += NT) at.ocur[i] = 0.f;
      for (int c0 = t0; c0 < t1; c0 += CHP) {
        const int np = min(CHP, t1 - c0);
        if (c0 != t0) {  // later chunks (long contexts): load now
          load_k<WT>(kreg, kbase, c0, np, rowb);
          load_v(at.vbuf, vbase, c0, np, rowb);
        }
        wait_vmem();
        __syncthreads();
        if (stamp && c0 == t0) stamp[10] = now();
        // the new token's V row replaces whatever the DMA read for it
        if (pos >= c0 && pos < c0 + np)
          for (int e = tid; e < hd; e += NT) {
            uint8_t* row = reinterpret_cast<uint8_t*>(at.vbuf) + (size_t)(pos - c0) * rowb;
            if constexpr (kAct32<WT>) reinterpret_cast<float*>(row)[e] = at.vn[e];
            else reinterpret_cast<uint16_t*>(row)[e] = (uint16_t)f2bf(at.vn[e]);
          }
        // scores: TPP threads per position, 64 B of the K row each, from registers
        {
          const int pp = tid / TPP, pt = tid % TPP;
          constexpr int DPT = kAct32<WT> ? 16 : 32;  // dims per thread
#pragma unroll
          for (int p = 0; p < KV_PASSES; ++p) {
            const int i = p * PPP + pp;
            const int tau = c0 + i;
            float kf[DPT];
            if (tau == pos) {
#pragma unroll
              for (int e = 0; e < DPT; ++e) kf[e] = at.kn[pt * DPT + e];
            } else if constexpr (kAct32<WT>) {
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                kf[4 * k] = __uint_as_float(kreg[p][k].x);
                kf[4 * k + 1] = __uint_as_float(kreg[p][k].y);
                kf[4 * k + 2] = __uint_as_float(kreg[p][k].z);
                kf[4 * k + 3] = __uint_as_float(kreg[p][k].w);
              }
            } else {
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                const uint4 x = kreg[p][k];
                kf[8 * k] = bf2f(x.x & 0xFFFF);
                kf[8 * k + 1] = bf2f(x.x >> 16);
                kf[8 * k + 2] = bf2f(x.y & 0xFFFF);
                kf[8 * k + 3] = bf2f(x.y >> 16);
                kf[8 * k + 4] = bf2f(x.z & 0xFFFF);
                kf[8 * k + 5] = bf2f(x.z >> 16);
                kf[8 * k + 6] = bf2f(x.w & 0xFFFF);
                kf[8 * k + 7] = bf2f(x.w >> 16);
              }
            }
#pragma unroll 1
            for (int h = 0; h < Gq; ++h) {
              const float4* q4 = reinterpret_cast<const float4*>(at.qs + h * hd + pt * DPT);
              float t = 0.f;
#pragma unroll
              for (int e = 0; e < DPT / 4; ++e) {
                const float4 q = q4[e];
                t = fmaf(q.x, kf[4 * e], t);
                t = fmaf(q.y, kf[4 * e + 1], t);
                t = fmaf(q.z, kf[4 * e + 2], t);
                t = fmaf(q.w, kf[4 * e + 3], t);
              }
              t = group_sum(t, TPP);
              if (pt == 0 && i < np) at.sc[h * CHP + i] = t;
            }
          }
        }
        __syncthreads();
        // chunk max per head (wave w handles heads w, w + NW, ...)
        for (int h = wave; h < Gq; h += NW) {
          float m = -INFINITY;
          for (int i = lane; i < np; i += 64) m = fmaxf(m, at.sc[h * CHP + i]);
          m = wave_max(m);
          if (lane == 0) {
            const float mn = fmaxf(sm.mrun[h], m);
            sm.alpha[h] = sm.mrun[h] == -INFINITY ? 0.f : __expf(sm.mrun[h] - mn);
            sm.mrun[h] = mn;
          }
        }
        __syncthreads();
        for (int i = tid; i < Gq * np; i += NT) {
          const int h = i / np, k = i % np;
          at.sc[h * CHP + k] = __expf(at.sc[h * CHP + k] - sm.mrun[h]);
        }
        __syncthreads();
        for (int h = wave; h < Gq; h += NW) {
          float t = 0.f;
          for (int i = lane; i < np; i += 64) t += at.sc[h * CHP + i];
          t = wave_sum(t);
          if (lane == 0) sm.lsum[h] = t;
        }
        // P.V from the LDS V rows: thread = (dim pair dp, subset sb)
        {
          const int DP = hd / 2, NS = NT / DP;
          const int dp = tid % DP, sb = tid / DP;
          float acc0[MAX_GQ], acc1[MAX_GQ];
#pragma unroll
          for (int h = 0; h < MAX_GQ; ++h) acc0[h] = acc1[h] = 0.f;
          const uint8_t* vb = reinterpret_cast<const uint8_t*>(at.vbuf);
#pragma unroll 4
          for (int i = sb; i < np; i += NS) {
            float v0, v1;
            if constexpr (kAct32<WT>) {
              const float2 v2 = reinterpret_cast<const float2*>(vb + (size_t)i * rowb)[dp];
              v0 = v2.x;
              v1 = v2.y;
            } else {
              const uint32_t v2 = reinterpret_cast<const uint32_t*>(vb + (size_t)i * rowb)[dp];
              v0 = bf2f(v2 & 0xFFFF);
              v1 = bf2f(v2 >> 16);
            }
#pragma unroll
            for (int h = 0; h < MAX_GQ; ++h)
              if (h < Gq) {
                const float p = at.sc[h * CHP + i];
                acc0[h] = fmaf(p, v0, acc0[h]);
                acc1[h] = fmaf(p, v1, acc1[h]);
              }
          }
#pragma unroll
          for (int h = 0; h < MAX_GQ; ++h)
            if (h < Gq) {
              at.red[(sb * MAX_GQ + h) * hd + 2 * dp] = acc0[h];
              at.red[(sb * MAX_GQ + h) * hd + 2 * dp + 1] = acc1[h];
            }
          __syncthreads();
          for (int i = tid; i < Gq * hd; i += NT) {
            const int h = i / hd, e = i % hd;
            float t = 0.f;
            for (int k = 0; k < NS; ++k) t += at.red[(k * MAX_GQ + h) * hd + e];
            at.ocur[i] = at.ocur[i] * sm.alpha[h] + t;
          }
          __syncthreads();
          if (tid < Gq) sm.lrun[tid] = sm.lrun[tid] * sm.alpha[tid] + sm.lsum[tid];
          __syncthreads();
        }
      }
      // publish (m, l, o) of each head: slot ((h * (hd + 2) + field) * S + split);
      // l and o first, m (the field the merge polls) once they have completed
      uint64_t* dst = ks.x_part + (size_t)par * nq * (hd + 2) * S;
      for (int i = tid; i < Gq * (hd + 1); i += NT) {
        const int h = i / (hd + 1), f = 1 + i % (hd + 1);
        const float v = f == 1 ? sm.lrun[h] : at.ocur[h * hd + f - 2];
        xstore(dst + ((size_t)(h0 + h) * (hd + 2) + f) * S + as, slot(tag + 1, __float_as_uint(v)));
      }
      wait_vmem();
      __syncthreads();
      if (tid < Gq)
        xstore(dst + ((size_t)(h0 + tid) * (hd + 2)) * S + as, slot(tag + 1, __float_as_uint(sm.mrun[tid])));
    }
    if (stamp) stamp[1] = now();

    // o_proj rows of this workgroup: stage their weights before the merge waits
    const Geo go = geo<WT>(ore - orb, QD);
    auto o_rowfn = [&](int q) { return mrow<WT>(ks.o, (long long)l * H + orb + q, QD, sm.actA, sm.asumA); };
    lstage_issue<WT>(lstage(sm.so), go, 0, o_rowfn);

    // ---------------- merge the splits: this workgroup's pairs of output dims
    {
      const int pb = mpb, pe = mpe;
      const uint64_t* srcp = ks.x_part + (size_t)par * nq * (hd + 2) * S;
      int e0 = 2 * pb;
      while (e0 < 2 * pe) {  // one head at a time (uniform loop)
        const int h = e0 / hd, eh0 = e0 % hd;
        const int ne = min(2 * pe, (h + 1) * hd) - e0;  // elements of head h in range (even)
        const int n = (2 + ne) * S;
        ok = gather(
            sm, srcp, n, tag + 1,
            [&](int i) {
              const int f = i / S, s = i % S;
              const int field = f < 2 ? f : 2 + eh0 + (f - 2);
              return ((size_t)h * (hd + 2) + field) * S + s;
            },
            [=](int k, int m) { return (int)(((long long)(k + 1) * S) / m) - 1; }, S < 64 ? S : 64,  // m fields
            [&](int i, uint32_t p) { sm.u.gbuf[i] = p; }, wt);
        if (!ok) break;
        // one wave per output pair, lanes over splits: log-sum-exp merge
        for (int k = wave; k < ne / 2; k += NW) {
          float M = -INFINITY;
          for (int s = lane; s < S; s += 64) M = fmaxf(M, __uint_as_float(sm.u.gbuf[s]));
          M = wave_max(M);
          float Lsum = 0.f, O0 = 0.f, O1 = 0.f;
          for (int s = lane; s < S; s += 64) {
            const float m = __uint_as_float(sm.u.gbuf[s]);
            const float w = m == -INFINITY ? 0.f : __expf(m - M);
            Lsum = fmaf(w, __uint_as_float(sm.u.gbuf[S + s]), Lsum);
            O0 = fmaf(w, __uint_as_float(sm.u.gbuf[(2 + 2 * k) * S + s]), O0);
            O1 = fmaf(w, __uint_as_float(sm.u.gbuf[(3 + 2 * k) * S + s]), O1);
          }
          Lsum = wave_sum(Lsum);
          O0 = wave_sum(O0);
          O1 = wave_sum(O1);
          if (lane == 0) {
            const float o0 = act_round<WT>(O0 / Lsum), o1 = act_round<WT>(O1 / Lsum);
            const int e = e0 + 2 * k;
            if constexpr (kAct32<WT>) {
              put_all(ks.x_o, OSL, par, e, slot(tag + 2, __float_as_uint(o0)));
              put_all(ks.x_o, OSL, par, e + 1, slot(tag + 2, __float_as_uint(o1)));
            } else {
              put_all(ks.x_o, OSL, par, e / 2, slot(tag + 2, f2bf(o0) | (f2bf(o1) << 16)));
            }
          }
        }
        __syncthreads();
        e0 += ne;
      }
    }
    if (!ok) break;
    if (stamp) stamp[2] = now();

    // ---------------- o_proj rows + residual
    ok = gather_flat(sm, copy_of(ks.x_o, OSL, par), OSL, tag + 2,
                     [&](int i, uint32_t p) {
                       if constexpr (kAct32<WT>) {
                         act_put<WT>(sm.actA, i, __uint_as_float(p));
                       } else {
                         act_put<WT>(sm.actA, 2 * i, bf2f(p & 0xFFFF));
                         act_put<WT>(sm.actA, 2 * i + 1, bf2f(p >> 16));
                       }
                     },
                     wt);
    if (!ok) break;
    if (stamp) stamp[11] = now();
    act_sums<WT>(sm.actA, sm.asumA, QD);
    __syncthreads();
    gemv_lds<WT>(lstage(sm.so), go, true, o_rowfn, [&](int q, float v) {
      const int r = orb + q;
      put_all(ks.x_res1, H, par, r, slot(tag + 3, __float_as_uint(sm.xres[r] + v)));
    });
    if (stamp) stamp[12] = now();
    // router rows (all of them, every workgroup): stage before waiting for the residual
    const bool dense = l < ks.n_dense;
    const int lmoe = l - ks.n_dense;
    const Geo gr = geo<WT>(dense ? 0 : E_, H);
    auto r_rowfn = [&](int q) { return mrow<WT>(ks.router, (long long)lmoe * E_ + q, H, sm.actA, sm.asumA); };
    if (!dense) lstage_issue<WT>(lstage(sm.u.rt), gr, 0, r_rowfn);
    __syncthreads();
    ok = gather_flat(sm, copy_of(ks.x_res1, H, par), H, tag + 3,
                     [&](int i, uint32_t p) { sm.xres[i] = __uint_as_float(p); }, wt);
    if (!ok) break;
    if (stamp) stamp[3] = now();

    // ---------------- post-attention RMSNorm (recomputed by every workgroup)
    {
      float ss = 0.f;
      for (int e = tid; e < H; e += NT) ss += sm.xres[e] * sm.xres[e];
      ss = block_sum(sm, ss);
      const float inv = 1.0f / sqrtf(ss / (float)H + ks.eps);
      const float* g = ks.pnorm + (size_t)l * H;
      for (int e = tid; e < H; e += NT) act_put<WT>(sm.actA, e, act_round<WT>(sm.xres[e] * inv * g[e]));
      __syncthreads();
      act_sums<WT>(sm.actA, sm.asumA, H);
      __syncthreads();
    }

    int nunit, inner;  // SwiGLU elements this layer produces, and the down projection's input width
    if (dense) {
      nunit = DI_;
      inner = DI_;
    } else {
      // ------------ router (every workgroup computes all logits) and top-k
      gemv_lds<WT>(lstage(sm.u.rt), gr, true, r_rowfn, [&](int q, float v) { sm.z[q] = v; });
      __syncthreads();
      if (stamp) stamp[13] = now();
      if (tid < 64) {
        const float zl = lane < E_ ? sm.z[lane] : -INFINITY;
        float zsel = zl;
        const float zmax = wave_max(zl);
        const float den = wave_sum(lane < E_ ? __expf(zl - zmax) : 0.f);
        float wsum = 0.f;
        for (int r = 0; r < K_; ++r) {
          float bv = zsel;
          int bi = lane;
          wave_argmax(bv, bi);
          if (lane == bi) zsel = -INFINITY;
          const float w = __expf(bv - zmax) / den;
          wsum += w;
          if (lane == 0) {
            sm.sel[r] = bi;
            sm.wsel[r] = w;
          }
        }
        if (ks.renorm && lane < K_) sm.wsel[lane] = sm.wsel[lane] / wsum;
      }
      __syncthreads();
      if (W == 0 && tid < K_) {
        if (d.dbg_routes) d.dbg_routes[(size_t)l * K_ + tid] = sm.sel[tid];
        if (d.dbg_rw) d.dbg_rw[(size_t)l * K_ + tid] = sm.wsel[tid];
      }
      nunit = K_ * EI_;
      inner = EI_;
    }
    if (dense && W == 0 && tid < K_) {
      if (d.dbg_routes) d.dbg_routes[(size_t)l * K_ + tid] = -1;
      if (d.dbg_rw) d.dbg_rw[(size_t)l * K_ + tid] = 0.f;
    }
    if (stamp) stamp[4] = now();

    // ---------------- gate/up rows of this workgroup's SwiGLU elements; down rows staged too
    const int upb = dense ? dpb : xpb, upe = dense ? dpe : xpe;
    const int ue0 = 2 * upb, une = 2 * (upe - upb);
    const int drb = orb, dre = ore;
    const int K = K_;
    const int wstride = kAct32<WT> ? inner : inner / 2;  // words of one rank's h
    auto gu_rowfn = [&](int q) {
      const int u = ue0 + q / 2;
      const Mat& m = (q & 1) ? (dense ? ks.du : ks.eu) : (dense ? ks.dg : ks.eg);
      const long long row =
          dense ? (long long)l * DI_ + u : ((long long)lmoe * E_ + sm.sel[div_small(u, EI_, inv_ei)]) * EI_ + u - div_small(u, EI_, inv_ei) * EI_;
      return mrow<WT>(m, row, H, sm.actA, sm.asumA);
    };
    auto dn_rowfn = [&](int q) {
      if (dense) return mrow<WT>(ks.dd, (long long)l * H + drb + q, inner, sm.u.mlp.hbuf, sm.u.mlp.asumH);
      const int qk = div_small(q, K, inv_k);
      const int r = drb + qk, k = q - qk * K;
      return mrow<WT>(ks.ed, ((long long)lmoe * E_ + sm.sel[k]) * H + r, inner, sm.u.mlp.hbuf + k * wstride,
                      sm.u.mlp.asumH + k * (inner / 32));
    };
    const Geo ggu = geo<WT>(2 * une, H);
    const Geo gdn = geo<WT>(dense ? dre - drb : (dre - drb) * K, inner);
    lstage_issue<WT>(lstage(sm.u.mlp.gu), ggu, 0, gu_rowfn);
    lstage_issue<WT>(lstage(sm.u.mlp.dn), gdn, 0, dn_rowfn);
    gemv_lds<WT>(lstage(sm.u.mlp.gu), ggu, true, gu_rowfn, [&](int q, float v) { sm.ytmp[q] = v; });
    __syncthreads();
    if (stamp) stamp[14] = now();
    for (int k = tid; k < une / 2; k += NT) {
      float hv[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const float g = sm.ytmp[4 * k + 2 * t], u = sm.ytmp[4 * k + 2 * t + 1];
        hv[t] = act_round<WT>(g / (1.0f + __expf(-g)) * u);
      }
      const int e = ue0 + 2 * k;
      if constexpr (kAct32<WT>) {
        put_all(ks.x_h, HSLOTS, par, e, slot(tag + 4, __float_as_uint(hv[0])));
        put_all(ks.x_h, HSLOTS, par, e + 1, slot(tag + 4, __float_as_uint(hv[1])));
      } else {
        put_all(ks.x_h, HSLOTS, par, e / 2, slot(tag + 4, f2bf(hv[0]) | (f2bf(hv[1]) << 16)));
      }
    }
    // ---------------- gather the SwiGLU output, down projection + residual
    ok = gather_flat(sm, copy_of(ks.x_h, HSLOTS, par), kAct32<WT> ? nunit : nunit / 2, tag + 4,
                     [&](int i, uint32_t p) {
                       // element e of rank r lives at hbuf element r * inner + e: the same flat index
                       if constexpr (kAct32<WT>) {
                         act_put<WT>(sm.u.mlp.hbuf, i, __uint_as_float(p));
                       } else {
                         act_put<WT>(sm.u.mlp.hbuf, 2 * i, bf2f(p & 0xFFFF));
                         act_put<WT>(sm.u.mlp.hbuf, 2 * i + 1, bf2f(p >> 16));
                       }
                     },
                     wt);
    if (!ok) break;
    act_sums<WT>(sm.u.mlp.hbuf, sm.u.mlp.asumH, nunit);
    __syncthreads();
    if (stamp) stamp[5] = now();
    if (dense) {
      gemv_lds<WT>(lstage(sm.u.mlp.dn), gdn, true, dn_rowfn, [&](int q, float v) {
        const int r = drb + q;
        put_all(ks.x_res2, H, par, r, slot(tag + 5, __float_as_uint(sm.xres[r] + v)));
      });
    } else {
      gemv_lds<WT>(lstage(sm.u.mlp.dn), gdn, true, dn_rowfn, [&](int q, float v) { sm.ytmp[q] = v; });
      __syncthreads();
      for (int q = tid; q < dre - drb; q += NT) {
        float y = 0.f;
        for (int k = 0; k < K; ++k) y = fmaf(sm.wsel[k], sm.ytmp[q * K + k], y);
        const int r = drb + q;
        put_all(ks.x_res2, H, par, r, slot(tag + 5, __float_as_uint(sm.xres[r] + y)));
      }
    }
    if (stamp) stamp[15] = now();
    // next layer's QKV rows: stage before waiting for the residual
    if (l + 1 < L) lstage_issue<WT>(lstage(sm.sq), gq, 0, qkv_rowfn(l + 1));
    __syncthreads();
    ok = gather_flat(sm, copy_of(ks.x_res2, H, par), H, tag + 5,
                     [&](int i, uint32_t p) { sm.xres[i] = __uint_as_float(p); }, wt);
    if (!ok) break;
    if (stamp) stamp[6] = now();
    if (d.dbg_resid && W == 0 && l == d.dbg_resid_layer)
      for (int e = tid; e < H; e += NT) d.dbg_resid[e] = sm.xres[e];
  }

  // ---------------- final norm, lm_head, argmax
  {
    float ss = 0.f;
    for (int e = tid; e < H; e += NT) ss += sm.xres[e] * sm.xres[e];
    ss = block_sum(sm, ss);
    const float inv = 1.0f / sqrtf(ss / (float)H + ks.eps);
    // the head is bf16 (or fp32) even when the layers are int4: natural element order
    constexpr int HW = WT == W_I4 ? W_BF16 : WT;
    uint32_t* fact = sm.u.mlp.hbuf;
    for (int e = tid; e < H; e += NT) act_put<HW>(fact, e, act_round<WT>(sm.xres[e] * inv * ks.fnorm[e]));
    __syncthreads();
    const int vb = ok ? part(V_, G, W) : 0, ve = ok ? part(V_, G, W + 1) : 0;
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    const Mat lmh{ks.lmhead, nullptr};
    float* const dbg_logits = d.dbg_logits;
    const Geo gl = geo<HW>(ve - vb, H);
    Stage<4> st_l;
    gemv_run<HW, 4, true>(gl, st_l, false, [&](int q) { return mrow<HW>(lmh, vb + q, H, fact, nullptr); },
                    [&](int q, float v) {
                      const int r = vb + q;
                      if (dbg_logits) dbg_logits[r] = v;
                      if (v > bv || (v == bv && r < bi)) {
                        bv = v;
                        bi = r;
                      }
                    });
    // best of the workgroup: max logit, then lowest id
    wave_argmax(bv, bi);
    const uint32_t u = __float_as_uint(bv);
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    const unsigned long long key =
        bi == 0x7FFFFFFF ? 0ull : (((unsigned long long)ord << 32) | (0xFFFFFFFFu - (uint32_t)bi));
    if (lane == 0) sm.best[wave] = key;
    __syncthreads();
    if (tid == 0) {
      unsigned long long k = 0;
      for (int w = 0; w < NW; ++w) k = sm.best[w] > k ? sm.best[w] : k;
      __hip_atomic_fetch_max(ks.amax, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t prev = __hip_atomic_fetch_add(ks.done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      if (prev == (uint32_t)G - 1) {  // last workgroup: publish the token, reset for the next launch
        const unsigned long long fin =
            __hip_atomic_exchange(ks.amax, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ks.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        d.out_ids[d.out_idx] = (int32_t)(0xFFFFFFFFu - (uint32_t)(fin & 0xFFFFFFFFull));
        d.len[seq] = pos + 1;
        if (d.dbg_ts) d.dbg_ts[2] = now();
      }
    }
  }
  if (stamps) stamps[1] = now();
  wait_vmem();
}

__global__ void fill_kernel(uint64_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0;
}

bool shape_is_static(const KStatic& k, int grid) {
  using S = Shape2048;
  return grid == S::G && k.H == S::H && k.hd == S::HD && k.nq == S::NQ && k.nkv == S::NKV && k.V == S::V &&
         k.E == S::E && k.K == S::K && k.EI == S::EI && (k.n_dense == 0 || k.DI == S::DI);
}

hipError_t launch_decode(int wt, bool stat, const KStatic* ks, const KDyn& d, int grid, hipStream_t stream) {
  if (stat) {
    switch (wt) {
      case W_BF16: hipLaunchKernelGGL((decode_kernel<W_BF16, Shape2048>), dim3(grid), dim3(NT), 0, stream, ks, d); break;
      case W_I4: hipLaunchKernelGGL((decode_kernel<W_I4, Shape2048>), dim3(grid), dim3(NT), 0, stream, ks, d); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (wt) {
      case W_F32: hipLaunchKernelGGL((decode_kernel<W_F32, DynShape>), dim3(grid), dim3(NT), 0, stream, ks, d); break;
      case W_BF16: hipLaunchKernelGGL((decode_kernel<W_BF16, DynShape>), dim3(grid), dim3(NT), 0, stream, ks, d); break;
      default: hipLaunchKernelGGL((decode_kernel<W_I4, DynShape>), dim3(grid), dim3(NT), 0, stream, ks, d); break;
    }
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
    case W_F32: return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, decode_kernel<W_F32, DynShape>, NT, 0);
    case W_BF16: return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, decode_kernel<W_BF16, DynShape>, NT, 0);
    default: return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, decode_kernel<W_I4, DynShape>, NT, 0);
  }
}

}  // namespace flint

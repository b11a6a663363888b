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
// unique per launch, layer and phase, so no flag ever needs resetting and no
// slot needs ordering against another; buffers alternate by layer parity so a
// slot is rewritten only after every reader has consumed it.
//
// Every byte a phase reads from HBM that does not depend on the phase's input
// (weight panels, the K/V rows of the attention split, norm weights) is
// brought into LDS by direct-to-LDS DMA (global_load_lds) before the exchange
// that precedes the phase is waited for, so its latency hides behind the
// exchange; only the selected experts' weights are fetched after the routing
// decision.  GEMVs keep the lane's activation chunk in registers when every
// row of the phase shares it.
//
// Per layer the exchanges are: q/k/v -> attention partials -> merged
// attention output -> residual after o_proj -> router logits -> SwiGLU
// output -> residual after the MLP.  Every wait is bounded (1 s); a timeout latches an error
// word that every other wait also checks, so a failed step always ends.

#include <atomic>
#include <mutex>

#include "flint_device.h"

namespace flint {

// LDS words between consecutive activation chunks.  An int4 chunk (32 bf16,
// 64 B, read by one lane as four 16-byte loads) is padded to 80 B so that the
// 16 lanes served together touch all 64 banks once; fp32 / bf16 chunks are
// one 16-byte load per lane and need no padding.
template <int WT> constexpr int kChunkWords = WT == W_I4 ? 20 : 4;
// Activation value as the GEMV input: bf16-rounded unless the model is fp32.
template <int WT> __device__ __forceinline__ float act_round(float v) { return kAct32<WT> ? v : round_bf16(v); }

// ---------------------------------------------------------------- shared memory

typedef short s16x4_t __attribute__((ext_vector_type(4)));  // 4 bf16 bit patterns: a 16x16x16 MFMA operand

// Weight staging in LDS: item i of wave w is 64 lanes x 16 B at w16[(i * NW + w) * 64 + lane]
// and, for int4, the dword holding the item's scale at s32[(i * NW + w) * 64 + lane].
template <int CAP> struct StageLds {
  uint4 w16[CAP * NW * 64];
  uint32_t s32[CAP * NW * 64];
};
// The phases of a layer reuse one region: each layout is live from the DMA that
// fills it (issued after a barrier that ends the previous layout's reads) to
// the last read of its phase.
struct AttnLds {                         // QKV and attention
  StageLds<QKV_CAP> sq;                  // QKV weights (staged during the previous layer)
  uint4 kbuf[KV_LDS / 16];               // K rows of a chunk
  uint4 vbuf[KV_LDS / 16];               // V rows of a chunk
  float qs[MAX_GQ * MAX_HD];             // queries of the kv-head group, pre-scaled
  uint16_t qop[2][4 * 64 * 8];           // MFMA scores: the same as B operands (bf16 high, low parts) for
                                         // 128-dim heads: [dims / 32][lane (head + 16 * k-slice)][8]
  float kn[MAX_HD], vn[MAX_HD];          // the new token's k, v (activation-rounded)
  float sc[MAX_GQ * MAX_CHUNK_POS];      // scores of a chunk, [head][position]
  float pt[MAX_GQ * MAX_CHUNK_POS];      // probabilities of a chunk, [position][head (padded to 4 or 8)]
  float fac[MAX_GQ], mst[MAX_GQ], lst[MAX_GQ];  // per head: rescale of the running output, running max and sum
};
struct MergeLds {                        // split merge and o_proj
  StageLds<O_CAP> so;                    // o_proj weights (staged during the merge)
  uint32_t gbuf[MAX_GATHER];             // gathered attention partials
};
struct MlpLds {                          // gate/up and down
  StageLds<GU_CAP> gu;
  StageLds<DN_CAP> dn;
  uint32_t hbuf[MAX_HBUF / 32 * 20];     // SwiGLU output as the down GEMV input (room for int4 padding)
  float asumH[MAX_HBUF / 32];
};
struct HeadLds {                         // lm_head: two staging buffers (bf16 / fp32 rows: no scales)
  uint4 a[LM_CAP * NW * 64], b[LM_CAP * NW * 64];
};

struct Smem {
  KStatic ks;                            // the context, copied once per launch: its fields are read with
                                         // LDS loads, never with vector loads that would wait for the DMAs
  // arrays read or written 16 bytes at a time start on 16-byte boundaries whatever the context's size
  // (a misaligned 16-byte LDS access is split: one such layout doubled the o_proj phase)
  alignas(16) float xres[MAX_H];         // residual (every workgroup keeps all of it)
  alignas(16) uint32_t actA[MAX_QD];     // GEMV input: fp32 words or bf16 pairs (also the lm_head input)
  alignas(16) float asumA[MAX_QD / 32];  // int4: sum of each 32-element chunk of actA
  alignas(16) float gn[MAX_H];           // weights of the next RMSNorm (DMA target)
  alignas(16) float ytmp[MAX_YROWS];     // this workgroup's GEMV results of a phase
  f32x2_t rcs[MAX_QPAIRS];               // RoPE (cos, sin) of this workgroup's QKV pairs at this position
  union {
    AttnLds att;
    MergeLds mg;
    StageLds<(MAX_H / 4 + 63) / 64> rt;  // router rows of this workgroup (staged during the o_proj exchange)
    MlpLds mlp;
    HeadLds head;
  } u;
  float z[MAX_E];                        // router logits
  int sel[MAX_K];
  float wsel[MAX_K];
  float wred[NW * 2];
  unsigned long long best[NW];
  uint32_t st_base[STAMP_LAYERS];        // phase stamps (debug, thread 0 of workgroup 0): each layer's start after
  uint16_t st[STAMP_LAYERS][16];         // the step's, its 16 stamps after that (10 ns ticks); stored at the end
  int flag;                              // sticky: a wait of this workgroup failed
};

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
    const int p = WT == W_I4 ? (e >> 5) * (2 * kChunkWords<WT>) + ((e & 24) | ((e & 3) << 1) | ((e >> 2) & 1)) : e;
    reinterpret_cast<uint16_t*>(act)[p] = (uint16_t)f2bf(v);
  }
}
// Elements e, e + 1 (e even) given as a pair of bf16 bit patterns (low half first), stored as they are:
// in the int4 layout element e + 1 sits two halfwords after element e.
template <int WT> __device__ __forceinline__ void act_put2_bits(uint32_t* act, int e, uint32_t bits) {
  static_assert(!kAct32<WT>, "bf16 inputs only");
  if constexpr (WT == W_I4) {
    const int p = (e >> 5) * (2 * kChunkWords<WT>) + ((e & 24) | ((e & 3) << 1) | ((e >> 2) & 1));
    uint16_t* const a16 = reinterpret_cast<uint16_t*>(act);
    a16[p] = (uint16_t)(bits & 0xFFFFu);
    a16[p + 2] = (uint16_t)(bits >> 16);
  } else {
    act[e >> 1] = bits;
  }
}
// After act_put of n elements (and a barrier): chunk sums for the int4 bias.
template <int WT> __device__ __forceinline__ void act_sums(const uint32_t* act, float* asum, int n) {
  if constexpr (WT == W_I4) {
    for (int c = threadIdx.x; c < n / 32; c += NT) {
      const uint4* p = reinterpret_cast<const uint4*>(act + c * kChunkWords<WT>);
      asum[c] = chunk_sum(p[0], p[1], p[2], p[3]);
    }
  }
}
// RMSNorm of the residual with the weights sm.gn (brought in by this
// workgroup's DMA), as the next GEMV input actA in the layout of OW (and, with
// sums, the int4 chunk sums).  Thread t takes elements 4t .. 4t + 3 (H <= 4 NT),
// which is also the 16-byte unit of sm.gn its own wave brought in, so the
// weights need only this wave's wait; two barriers in all.  half: which half of
// sm.wred holds the wave sums (consecutive norms alternate, so no barrier is
// needed before writing them).
// later: vector memory operations this wave issued after the norm weights' DMA (they may stay in flight).
// PRE: the wave sums of squares are already in sm.wred (written by the gather that brought the residual,
// before its closing barrier), so the norm starts from them.
// WAIT = false: the caller knows the weights have landed and every wave has passed a barrier since.
template <int WT, int OW = WT, bool PRE = false, bool WAIT = true>
__device__ __forceinline__ void rmsnorm_act(Smem& sm, int H, float eps, bool sums, int later = 0, int half = 0) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if constexpr (WAIT) wait_vmem_dyn(later);
  const int e0 = 4 * tid;
  const bool mine = e0 < H;
  const float4 x = mine ? *reinterpret_cast<const float4*>(&sm.xres[e0]) : make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (!PRE) {
    float ss = x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
    ss = wave_sum(ss);
    if (lane == 0) sm.wred[half * NW + wave] = ss;
    __syncthreads();
  }
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) t += sm.wred[half * NW + w];
  const float inv = __builtin_amdgcn_rsqf(t * (1.0f / (float)H) + eps);  // the hardware reciprocal square root
  if (mine) {
    const float4 g = *reinterpret_cast<const float4*>(&sm.gn[e0]);
    const float y0 = act_round<WT>(x.x * inv * g.x), y1 = act_round<WT>(x.y * inv * g.y);
    const float y2 = act_round<WT>(x.z * inv * g.z), y3 = act_round<WT>(x.w * inv * g.w);
    act_put<OW>(sm.actA, e0, y0);
    act_put<OW>(sm.actA, e0 + 1, y1);
    act_put<OW>(sm.actA, e0 + 2, y2);
    act_put<OW>(sm.actA, e0 + 3, y3);
    if constexpr (OW == W_I4) {
      if (sums) {  // the 32 elements of chunk t / 8 belong to 8 consecutive threads
        const float cs = group_sum((y0 + y1) + (y2 + y3), 8);
        if ((tid & 7) == 0) sm.asumA[e0 >> 5] = cs;
      }
    }
  }
  __syncthreads();
}
// Bring n floats (n a multiple of 64) into sm.gn by DMA; wave w moves 1 KB units w, w + NW, ...
// Waves w0 .. NW - 1 share the work.
template <bool UNTRACKED = false>
__device__ __forceinline__ void gn_issue(Smem& sm, const float* src, int n, int w0 = 0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int units = n / 4;  // 16-byte units
  if (wave < w0) return;
  for (int gi = wave - w0; gi * 64 < units; gi += NW - w0) {
    const int unit = min(gi * 64 + lane, units - 1);
    if constexpr (UNTRACKED) dma16_untracked(src + 4 * unit, lds_offset(&sm.gn[gi * 256]));
    else dma16(src + 4 * unit, &sm.gn[gi * 256]);
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

template <int WT> __device__ __forceinline__ ActC<WT> act_chunk(const uint32_t* act, const float* asum, int c) {
  ActC<WT> r;
  if constexpr (WT == W_I4) {
    const uint4* p = reinterpret_cast<const uint4*>(act + kChunkWords<WT> * c);
    r.a[0] = p[0];
    r.a[1] = p[1];
    r.a[2] = p[2];
    r.a[3] = p[3];
    r.s = asum[c];
  } else {
    r.a[0] = *reinterpret_cast<const uint4*>(act + 4 * c);
    r.s = 0.f;
  }
  return r;
}

// Lane geometry of a GEMV over `nrows` rows of width `in`: each row is read in
// 16-byte chunks by a group of LPR lanes (64, or fewer for short rows, RPW
// rows side by side in a wave).  A wave's work is a list of NI items (row
// pass p, chunk j), staged in LDS and computed in rounds.
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
  g.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  g.sub = lane / LPR;
  g.li = lane % LPR;
  const int npass = (nrows + NW * g.RPW - 1) / (NW * g.RPW);
  g.NI = npass * g.CPL;
  return g;
}

// LDS staging: the items of a round are brought into LDS by DMA (no registers
// held, so every load of the round is in flight at once and can be issued
// long before the activation is ready), then each wave computes its own items.
struct LStage {
  uint4* w16;
  uint32_t* s32;
  int cap;
};
template <int CAP> __device__ __forceinline__ LStage lstage(StageLds<CAP>& s) { return LStage{s.w16, s.s32, CAP}; }

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

// Issue NIS items (known at compile time) starting at item k0: every chunk
// address first (any LDS reads the row function needs are batched), then the
// DMA instructions back to back.
template <int WT, int NIS, bool UNTRACKED = false, class RowFn>
__device__ __forceinline__ void lstage_issue_static(const LStage& st, const Geo& g, int k0, RowFn rowfn, int cw) {
  const uint8_t* wp[NIS];
  const uint16_t* sp[NIS];
  bool ok[NIS];
#pragma unroll
  for (int i = 0; i < NIS; ++i) {
    const int k = k0 + i, p = k / g.CPL, j = k - p * g.CPL;
    const int r = cw * g.RPW + p * NW * g.RPW + g.sub, c = g.li + j * g.LPR;
    ok[i] = r < g.nrows && c < g.C;
    const RowSrc src = rowfn(ok[i] ? r : 0);
    wp[i] = src.w + 16ll * c;
    sp[i] = WT == W_I4 ? src.s + ((c >> 1) & ~1) : nullptr;
  }
#pragma unroll
  for (int i = 0; i < NIS; ++i)
    if (ok[i]) {
      if constexpr (UNTRACKED) {
        dma16_untracked(wp[i], lds_offset(&st.w16[(i * NW + cw) * 64]));
        if constexpr (WT == W_I4) dma4_untracked(sp[i], lds_offset(&st.s32[(i * NW + cw) * 64]));
      } else {
        dma16(wp[i], &st.w16[(i * NW + cw) * 64]);
        if constexpr (WT == W_I4) dma4(sp[i], &st.s32[(i * NW + cw) * 64]);
      }
    }
}

// Round 0 of a GEMV: the static issue when its NIS items fit the capacity, else the general loop.
template <int WT, int NIS, int CAP, bool UNTRACKED = false, class RowFn>
__device__ __forceinline__ void issue_auto(const LStage& st, const Geo& g, RowFn rowfn) {
  if constexpr (NIS > 0 && NIS <= CAP) lstage_issue_static<WT, NIS, UNTRACKED>(st, g, 0, rowfn, g.wave);
  else lstage_issue<WT>(st, g, 0, rowfn);
}

// A lane's activation chunks for a phase whose rows all share one input (CPLR chunks per lane).
template <int WT, int CPLR> struct ActRegs {
  ActC<WT> c[CPLR > 0 ? CPLR : 1];
};
template <int WT, int CPLR>
__device__ __forceinline__ ActRegs<WT, CPLR> act_regs(const Geo& g, const uint32_t* act, const float* asum) {
  ActRegs<WT, CPLR> r;
  if constexpr (CPLR > 0) {
#pragma unroll
    for (int j = 0; j < CPLR; ++j) {
      const int c = g.li + j * g.LPR;
      r.c[j] = act_chunk<WT>(act, asum, c < g.C ? c : 0);
    }
  }
  return r;
}

// bf16 scale of chunk c from the staged dword holding the scales of groups (c / 2) & ~1 and + 1
__device__ __forceinline__ float chunk_scale(uint32_t sw, int c) {
  return bf2f(((c >> 1) & 1) ? (sw >> 16) : (sw & 0xFFFFu));
}
template <int WT>
__device__ __forceinline__ float item_dot(const LStage& st, int slot, int c, const ActC<WT>& a, const I4K& k4) {
  const uint4 w = st.w16[slot];
  float scale = 1.f;
  if constexpr (WT == W_I4) scale = chunk_scale(st.s32[slot], c);
  return chunk_dot<WT>(w, a, scale, k4);
}

// Sum over the wave of R rows at once (R a power of two, at most 16).  Lane
// bit 5, then bits 4, 3, 2 split the rows between lanes: each step pairs two
// partial rows, every lane keeps one of them and adds its partner lane's copy
// (permlane swaps across 32 and 16 lanes, then DPP mirrors within 16 and 8),
// so a step halves the values a lane carries; the lane bits left over are
// summed.  On return every lane holds the total of row row_of<R>(lane).
template <int R> __device__ __forceinline__ int row_of(int lane) {
  constexpr int LG = R >= 16 ? 4 : R >= 8 ? 3 : R >= 4 ? 2 : R >= 2 ? 1 : 0;
  int r = LG > 0 ? (lane >> 5) & 1 : 0;
#pragma unroll
  for (int j = 1; j < LG; ++j) r |= ((lane >> (5 - j)) & 1) << (LG - j);
  return r;
}
template <int CTRL>
__device__ __forceinline__ float keep_add(float x, float y, bool hi) {  // hi ? y + partner's y : x + partner's x
  const float keep = hi ? y : x, send = hi ? x : y;
  return keep + dpp<CTRL>(send);
}
template <int R> __device__ __forceinline__ float reduce_rows(const float (&a)[R]) {
  static_assert(R == 1 || R == 2 || R == 4 || R == 8 || R == 16, "rows per reduction");
  const int lane = threadIdx.x & 63;
  if constexpr (R == 1) {
    return wave_sum(a[0]);
  } else {
    float b[R / 2];  // lane ^ 32: lanes 0-31 keep row 2k, lanes 32-63 row 2k + 1
#pragma unroll
    for (int k = 0; k < R / 2; ++k) {
      const auto s = __builtin_amdgcn_permlane32_swap(__float_as_int(a[2 * k]), __float_as_int(a[2 * k + 1]), false, false);
      b[k] = __int_as_float(s[0]) + __int_as_float(s[1]);
    }
    if constexpr (R == 2) {
      float v = b[0];
      v += dpp<DPP_XOR1>(v);
      v += dpp<DPP_XOR2>(v);
      v += dpp<DPP_HALF_MIRROR>(v);
      v += dpp<DPP_MIRROR>(v);
      return v + swap16(v);
    } else {
      float c[R / 4];  // lane ^ 16: lanes with bit 4 clear keep b[k], set keep b[k + R / 4]
#pragma unroll
      for (int k = 0; k < R / 4; ++k) {
        const auto s = __builtin_amdgcn_permlane16_swap(__float_as_int(b[k]), __float_as_int(b[k + R / 4]), false, false);
        c[k] = __int_as_float(s[0]) + __int_as_float(s[1]);
      }
      if constexpr (R == 4) {
        float v = c[0];
        v += dpp<DPP_XOR1>(v);
        v += dpp<DPP_XOR2>(v);
        v += dpp<DPP_HALF_MIRROR>(v);
        return v + dpp<DPP_MIRROR>(v);
      } else {
        const bool h3 = lane & 8;
        float d[R / 8];  // mirror within 16 lanes (partner 15 - l): bit 3 picks the row
#pragma unroll
        for (int k = 0; k < R / 8; ++k) d[k] = keep_add<DPP_MIRROR>(c[k], c[k + R / 8], h3);
        if constexpr (R == 8) {
          float v = d[0];
          v += dpp<DPP_XOR1>(v);
          v += dpp<DPP_XOR2>(v);
          return v + dpp<DPP_HALF_MIRROR>(v);
        } else {
          const bool h2 = lane & 4;  // mirror within 8 lanes (partner 7 - l): bit 2 picks the row
          float v = keep_add<DPP_HALF_MIRROR>(d[0], d[1], h2);
          v += dpp<DPP_XOR1>(v);
          return v + dpp<DPP_XOR2>(v);
        }
      }
    }
  }
}

// Compute NIS staged items of this wave in one pass (static shapes: 64 lanes
// per row, every item valid, CPLR chunks per row, activation in registers):
// all LDS reads first, then the dot products, then one reduction for the
// wave's rows.  p0: row pass of the first item.
template <int WT, int CPLR, int NIS, class OutFn>
__device__ __forceinline__ void compute_static(const LStage& st, const Geo& g, int p0, const ActRegs<WT, CPLR>& ar,
                                               OutFn outfn) {
  static_assert(CPLR > 0 && NIS % CPLR == 0 && NIS / CPLR <= 16, "whole rows, at most 16 per wave");
  constexpr int NR = NIS / CPLR;
  constexpr int R = NR <= 1 ? 1 : NR <= 2 ? 2 : NR <= 4 ? 4 : NR <= 8 ? 8 : 16;
  const int lane = threadIdx.x & 63;
  const I4K k4 = i4k();
  uint4 w[NIS];
  uint32_t s[NIS];
#pragma unroll
  for (int i = 0; i < NIS; ++i) {
    w[i] = st.w16[(i * NW + g.wave) * 64 + lane];
    if constexpr (WT == W_I4) s[i] = st.s32[(i * NW + g.wave) * 64 + lane];
  }
  float acc[R];
#pragma unroll
  for (int p = 0; p < R; ++p) {
    acc[p] = 0.f;
    if (p < NR) {
#pragma unroll
      for (int j = 0; j < CPLR; ++j)
        acc[p] += chunk_dot<WT>(w[p * CPLR + j], ar.c[j], WT == W_I4 ? chunk_scale(s[p * CPLR + j], lane + 64 * j) : 1.f,
                                k4);
    }
  }
  const float v = reduce_rows<R>(acc);
  const int rho = row_of<R>(lane);
  if ((lane & (64 / R - 1)) == 0 && rho < NR) {
    const int r = g.wave + (p0 + rho) * NW;
    if (r < g.nrows) outfn(r, v);
  }
}

// The same for rows of one chunk per lane, item by item as the requests land (loads complete in order:
// item p has landed once no more than `later` plus the requests of the items after it are outstanding),
// so that the products of the first items overlap the arrival of the last.
template <int WT, int NIS, class OutFn>
__device__ __forceinline__ void compute_static_stream(const LStage& st, const Geo& g, const ActRegs<WT, 1>& ar,
                                                      OutFn outfn, int later) {
  static_assert(NIS <= 16, "at most 16 rows per wave");
  constexpr int R = NIS <= 1 ? 1 : NIS <= 2 ? 2 : NIS <= 4 ? 4 : NIS <= 8 ? 8 : 16;
  constexpr int PER = WT == W_I4 ? 2 : 1;  // requests per item (weights, scales)
  const int lane = threadIdx.x & 63;
  const I4K k4 = i4k();
  // this wave's items with a row (row wave + p * NW): their requests were issued, the others' not
  const int nv = g.nrows > g.wave ? min(NIS, (g.nrows - g.wave + NW - 1) / NW) : 0;
  float acc[R];
#pragma unroll
  for (int p = 0; p < R; ++p) acc[p] = 0.f;
#pragma unroll
  for (int p = 0; p < NIS; ++p) {
    if (p < nv) {
      wait_vmem_dyn(later + PER * (nv - 1 - p));
      const uint4 w = st.w16[(p * NW + g.wave) * 64 + lane];
      const float sc = WT == W_I4 ? chunk_scale(st.s32[(p * NW + g.wave) * 64 + lane], lane) : 1.f;
      acc[p] = chunk_dot<WT>(w, ar.c[0], sc, k4);
    }
  }
  const float v = reduce_rows<R>(acc);
  const int rho = row_of<R>(lane);
  if ((lane & (64 / R - 1)) == 0 && rho < NIS) {
    const int r = g.wave + rho * NW;
    if (r < g.nrows) outfn(r, v);
  }
}

// Compute NIS staged items of this wave whose activation chunk depends on the
// row (read from LDS through rowfn), any lanes per row, one chunk per lane per
// row (static shapes): loads of a batch of NB items first, then their dot
// products, a sum over each row's lanes per item.
template <int WT, int NIS, int NB, class RowFn, class OutFn>
__device__ __forceinline__ void compute_static_rows(const LStage& st, const Geo& g, RowFn rowfn, OutFn outfn) {
  static_assert(NIS % NB == 0, "whole batches");
  const int lane = threadIdx.x & 63;
  const I4K k4 = i4k();
  const int c = g.li;
#pragma unroll
  for (int b0 = 0; b0 < NIS; b0 += NB) {
    uint4 w[NB];
    uint32_t s[NB];
    ActC<WT> a[NB];
    int r[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      r[i] = g.wave * g.RPW + (b0 + i) * NW * g.RPW + g.sub;
      const int slot = ((b0 + i) * NW + g.wave) * 64 + lane;
      w[i] = st.w16[slot];
      if constexpr (WT == W_I4) s[i] = st.s32[slot];
      const RowSrc src = rowfn(r[i] < g.nrows ? r[i] : 0);
      a[i] = act_chunk<WT>(src.act, src.asum, c < g.C ? c : 0);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      float acc = 0.f;
      if (c < g.C) acc = chunk_dot<WT>(w[i], a[i], WT == W_I4 ? chunk_scale(s[i], c) : 1.f, k4);
      const float v = group_sum(acc, g.LPR);
      if (g.li == 0 && r[i] < g.nrows) outfn(r[i], v);
    }
  }
}

// A staged GEMV of the static shape whose items fit one round of NIS items per wave; later: vector
// memory operations this wave issued after the stage's DMA (they may stay in flight).
template <int WT, int CPLR, int NIS, bool STREAM = false, class RowFn, class OutFn>
__device__ __forceinline__ void gemv_static(const LStage& st, const Geo& g, bool issued, const ActRegs<WT, CPLR>& ar,
                                            RowFn rowfn, OutFn outfn, int later = 0) {
  if (!issued) lstage_issue_static<WT, NIS>(st, g, 0, rowfn, g.wave);
  if constexpr (STREAM && CPLR == 1) {
    compute_static_stream<WT, NIS>(st, g, ar, outfn, issued ? later : 0);
  } else {
    wait_vmem_dyn(issued ? later : 0);
    compute_static<WT, CPLR, NIS>(st, g, 0, ar, outfn);
  }
}

// The single-round static path when the wave's NIS items (known at compile
// time, 0 = not) fit the capacity CAP, else the general rounds.
template <int WT, int CPLR, int NIS, int CAP, bool STREAM = false, class RowFn, class OutFn>
__device__ __forceinline__ void gemv_auto(const LStage& st, const Geo& g, bool issued, const ActRegs<WT, CPLR>& ar,
                                          RowFn rowfn, OutFn outfn, int later = 0) {
  if constexpr (CPLR > 0 && NIS > 0 && NIS <= CAP && NIS / CPLR <= 16)
    gemv_static<WT, CPLR, NIS, STREAM>(st, g, issued, ar, rowfn, outfn, later);
  else
    gemv_lds<WT, CPLR>(st, g, issued, ar, rowfn, outfn);  // waits for everything (later ignored)
}

// Compute round `round` of this wave's items.  CPLR > 0: every row has CPLR
// chunks per lane, the capacity is a multiple of CPLR and the activation is in
// registers; CPLR == 0: any geometry, the activation read from LDS per item.
template <int WT, int CPLR, class RowFn, class OutFn>
__device__ __forceinline__ void lstage_compute(const LStage& st, const Geo& g, int round, float& acc,
                                               const ActRegs<WT, CPLR>& ar, RowFn rowfn, OutFn outfn) {
  const int k0 = round * st.cap;
  const int n = min(st.cap, g.NI - k0);
  const int lane = threadIdx.x & 63;
  const I4K k4 = i4k();
  if constexpr (CPLR > 0) {
    int p = k0 / CPLR;
#pragma unroll 2
    for (int i0 = 0; i0 < n; i0 += CPLR, ++p) {
      const int r = g.wave * g.RPW + p * NW * g.RPW + g.sub;
#pragma unroll
      for (int j = 0; j < CPLR; ++j) {
        const int c = g.li + j * g.LPR;
        if (r < g.nrows && c < g.C) acc += item_dot<WT>(st, ((i0 + j) * NW + g.wave) * 64 + lane, c, ar.c[j], k4);
      }
      const float v = group_sum(acc, g.LPR);
      if (g.li == 0 && r < g.nrows) outfn(r, v);
      acc = 0.f;
    }
  } else {
    int p = k0 / g.CPL, j = k0 - p * g.CPL;
#pragma unroll 2
    for (int i = 0; i < n; ++i) {
      const int r = g.wave * g.RPW + p * NW * g.RPW + g.sub, c = g.li + j * g.LPR;
      if (r < g.nrows && c < g.C) {
        const RowSrc src = rowfn(r);
        acc += item_dot<WT>(st, (i * NW + g.wave) * 64 + lane, c, act_chunk<WT>(src.act, src.asum, c), k4);
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
}

// Run a staged GEMV; `issued`: round 0 was already issued.  The activation
// must be in LDS (and, for CPLR > 0, in `ar`) before the call.
template <int WT, int CPLR, class RowFn, class OutFn>
__device__ __forceinline__ void gemv_lds(const LStage& st, const Geo& g, bool issued, const ActRegs<WT, CPLR>& ar,
                                         RowFn rowfn, OutFn outfn) {
  const int nr = (g.NI + st.cap - 1) / st.cap;
  float acc = 0.f;
  for (int b = 0; b < nr; ++b) {
    if (b > 0) wait_lds();  // this wave's reads of the previous round are done before the DMA reuses the slots
    if (b > 0 || !issued) lstage_issue<WT>(st, g, b, rowfn);
    wait_vmem();
    lstage_compute<WT, CPLR>(st, g, b, acc, ar, rowfn, outfn);
  }
}

// Streaming GEMV with two staging buffers: round b + 1 is in flight while
// round b is computed.  Static shapes only: every lane of every item valid
// (whole rows of 64 lanes, rows a multiple of the waves, items a multiple of
// CAP), so a round issues exactly CAP DMA instructions per wave (no scales)
// and the older round can be waited for with vmcnt(CAP).
template <int WT, int CPLR, int CAP, class RowFn, class OutFn>
__device__ __forceinline__ void gemv_stream(const LStage& A, const LStage& B, const Geo& g,
                                            const ActRegs<WT, CPLR>& ar, RowFn rowfn, OutFn outfn) {
  static_assert(WT != W_I4 && CPLR > 0 && CAP % CPLR == 0, "streamed GEMV: bf16 / fp32 rows, activation in registers");
  const int nr = g.NI / CAP;
  if (nr > 0) lstage_issue_static<WT, CAP>(A, g, 0, rowfn, g.wave);
  for (int b = 0; b < nr; ++b) {
    const LStage& cur = (b & 1) ? B : A;
    const LStage& nxt = (b & 1) ? A : B;
    if (b + 1 < nr) {
      wait_lds();  // this wave's reads of round b - 1 (in nxt) are done
      lstage_issue_static<WT, CAP>(nxt, g, (b + 1) * CAP, rowfn, g.wave);
      wait_vmem_n<CAP>();  // round b + 1 issued CAP loads: round b has landed
    } else {
      wait_vmem();
    }
    compute_static<WT, CPLR, CAP>(cur, g, b * (CAP / CPLR), ar, outfn);
  }
}

// ---------------------------------------------------------------- exchanges

struct Waiter {
  uint32_t* err;
  uint32_t* herr;
  int sleep;
  int sentinels;
  uint32_t limit;
  bool abort;
};
__device__ __forceinline__ void backoff(const Waiter& wt) {
  for (int z = 0; z < wt.sleep; ++z) __builtin_amdgcn_s_sleep(8);  // none by default: re-poll at once
}

// Latch an error: atomically in device memory, by a plain system-scope store
// in the host-mapped word (the host only tests it for non-zero).
__device__ __forceinline__ void raise_error(const Waiter& wt, uint32_t bits) {
  __hip_atomic_fetch_or(gp(wt.err), bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  __hip_atomic_store(gp(wt.herr), bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// True once this wait should give up: another wait has timed out, or this one
// has run for longer than the timeout (which it then reports).  t0: the clock
// when the wait began, tn: when this round of polls was issued (both read
// ahead of loads, so the clock's latency hides behind theirs).
__device__ __forceinline__ bool poll_timed_out(const Waiter& wt, uint64_t t0, uint64_t tn, uint32_t it) {
  if ((it & 15) == 0 &&
      (__hip_atomic_load(gp(wt.err), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) & ERR_TIMEOUT))
    return true;
  if (tn - t0 > wt.limit) {
    raise_error(wt, ERR_TIMEOUT);
    return true;
  }
  return false;
}

// Barrier that also makes any thread's abort the workgroup's (uniform) decision.
// The LDS flag is sticky: after a failed wait the launch only winds down.
__device__ __forceinline__ bool sync_ok(Smem& sm, Waiter& wt) {
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
// GT: threads that read slots (the first GT of the workgroup; the others only take part in the barriers,
// e.g. while their DMAs are in flight: a wave's loads complete in order, so a poll issued behind a DMA burst
// would return only after the burst).
struct NoHook {
  __device__ void operator()() const {}
};
// pre() runs in every thread just before the closing barrier (after the last put).
template <int GT = NT, class IndexFn, class SentFn, class PutFn, class PreFn = NoHook>
__device__ __forceinline__ bool gather(Smem& sm, const uint64_t* src, int n, uint32_t tag, IndexFn index, SentFn sent,
                                       int nsent, PutFn put, Waiter& wt, PreFn pre = PreFn{}) {
  static_assert(GT % 64 == 0 && GT >= 64 && GT <= NT, "whole waves poll");
  const int tid = threadIdx.x;
  if (nsent > wt.sentinels) nsent = wt.sentinels;
  if (tid < 64 && tid < nsent && !wt.abort) {  // sentinels == 0: every thread polls its own slots at once
    const uint64_t* p = src + index(sent(tid, nsent));
    const uint64_t t0 = now();
    if ((uint32_t)(xload(p) >> 32) != tag) {
      uint32_t it = 0;
      while (true) {
        backoff(wt);
        const uint64_t tn = now();
        if ((uint32_t)(xload(p) >> 32) == tag) break;
        if (poll_timed_out(wt, t0, tn, ++it)) {
          wt.abort = true;
          break;
        }
      }
    }
  }
  if (!sync_ok(sm, wt)) return false;
  for (int b0 = 0; b0 < n && tid < GT; b0 += 8 * GT) {
    const uint64_t t0 = now();
    uint64_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = b0 + tid + k * GT;
      v[k] = i < n ? xload(src + index(i)) : slot(tag, 0);
    }
    uint32_t pending = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if ((uint32_t)(v[k] >> 32) != tag) pending |= 1u << k;
    if (pending) {
      uint32_t it = 0;
      while (pending) {
        backoff(wt);
        const uint64_t tn = now();
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (pending & (1u << k)) v[k] = xload(src + index(b0 + tid + k * GT));
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if ((pending & (1u << k)) && (uint32_t)(v[k] >> 32) == tag) pending &= ~(1u << k);
        if (pending && poll_timed_out(wt, t0, tn, ++it)) {
          wt.abort = true;
          break;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = b0 + tid + k * GT;
      if (i < n) put(i, (uint32_t)v[k]);
    }
  }
  pre();
  return sync_ok(sm, wt);
}

// Gather n contiguous slots, sentinels spread evenly.
template <int GT = NT, class PutFn, class PreFn = NoHook>
__device__ __forceinline__ bool gather_flat(Smem& sm, const uint64_t* src, int n, uint32_t tag, PutFn put,
                                            Waiter& wt, PreFn pre = PreFn{}) {
  const int ns = n < 64 ? n : 64;
  return gather<GT>(
      sm, src, n, tag, [](int i) { return i; }, [=](int k, int m) { return (int)(((long long)(k + 1) * n) / m) - 1; },
      ns, put, wt, pre);
}

// Publish `count` values into a replicated exchange buffer [NCOPY][2 parities][n]:
// thread t stores value t % count of replica t / count, so neighbouring lanes
// write neighbouring slots and a wave's stores cover whole cache lines;
// val(i, idx) returns the payload of value i and sets its slot index.
template <class ValFn>
__device__ __forceinline__ void publish(uint64_t* base, int n, int par, int count, uint32_t tag, ValFn val) {
  for (int t = threadIdx.x; t < count * NCOPY; t += NT) {
    const int c = t / count, i = t - c * count;
    int idx;
    const uint32_t v = val(i, idx);
    xstore(base + (size_t)(c * 2 + par) * n + idx, slot(tag, v));
  }
}
__device__ __forceinline__ const uint64_t* copy_of(const uint64_t* base, int n, int par) {
  return base + (size_t)((xcc_id() & (NCOPY - 1)) * 2 + par) * n;
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

// Chunks per lane of a GEMV over rows of `in` elements staged CAP items at a
// time, when the shape is static and CAP holds whole rows (0: the dynamic path).
template <int WT, class SH> constexpr int cpl_fit(int in, int cap) {
  if (!SH::kStatic) return 0;
  const int C = in / kChunkElems<WT>;
  const int cpl = C >= 64 ? (C + 63) / 64 : 1;
  return cap % cpl == 0 ? cpl : 0;
}

// Items per wave of a GEMV whose workgroups own `per_wg` rows each, at cpl
// chunks per row (the last row pass of some waves may be empty: those rows
// are neither loaded nor stored).
constexpr int nis_of(int per_wg, int cpl) { return cpl > 0 && per_wg > 0 ? (per_wg + NW - 1) / NW * cpl : 0; }
constexpr int even_share(int total, int G) { return G > 0 && total % G == 0 ? total / G : 0; }

template <int WT, class SH>
__global__ void __launch_bounds__(NT, 1) decode_kernel(const KStatic* __restrict__ ksp, const KDyn d) {
  __shared__ Smem sm;
  constexpr bool SS = SH::kStatic;
  const int G = SS ? SH::G : (int)gridDim.x, W = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  static_assert(sizeof(KStatic) % 4 == 0, "context copied as words");
  for (int i = tid; i < (int)(sizeof(KStatic) / 4); i += NT)
    reinterpret_cast<uint32_t*>(&sm.ks)[i] = gp(reinterpret_cast<const uint32_t*>(ksp))[i];
  __syncthreads();
  const KStatic& ks = sm.ks;
  const int H = SS ? SH::H : ks.H, hd = SS ? SH::HD : ks.hd, nq = SS ? SH::NQ : ks.nq, nkv = SS ? SH::NKV : ks.nkv;
  const int QD = nq * hd, Gq = nq / nkv, L = ks.L;
  const int V_ = SS ? SH::V : ks.V, DI_ = SS ? SH::DI : ks.DI, E_ = SS ? SH::E : ks.E, K_ = SS ? SH::K : ks.K;
  const int EI_ = SS ? SH::EI : ks.EI;
  const int QR = (nq + 2 * nkv) * hd;                            // q, k, v rows
  const int OSL = kAct32<WT> ? QD : QD / 2;                      // slots of the merged attention output
  const int HSLOTS = ks.h_slots;                                 // slots of the SwiGLU output exchange
  Waiter wt{ks.err, ks.herr, ks.poll_sleep, ks.sentinels, ks.spin_limit, false};
  // context values used inside DMA issue loops and publishes, held in registers
  // context values stay in LDS and are read where they are used (an LDS read never waits for the vector
  // memory counter; held in registers across the layer loop they were spilled to scratch memory, and
  // each reload of a spill waited behind every store and DMA issued before it)
  const Mat &m_qkv = ks.qkv, &m_o = ks.o, &m_r = ks.router, &m_dg = ks.dg, &m_du = ks.du, &m_dd = ks.dd;
  const Mat &m_eg = ks.eg, &m_eu = ks.eu, &m_ed = ks.ed;
  const float* const& p_anorm = ks.anorm;
  const float* const& p_pnorm = ks.pnorm;
  const float* const& p_fnorm = ks.fnorm;
  // exchange buffers: the context's, or (d.xbase, the fixed scratch array shared by every model on the
  // device) the argmax counters at a fixed place in its first 128 bytes and the slots in the context's
  // layout after them
  auto rebase = [&](uint64_t* p) { return d.xbase ? d.xbase + 16 + (p - ks.x_qkv) : p; };
  uint64_t *const x_qkv = rebase(ks.x_qkv), *const x_part = rebase(ks.x_part), *const x_o = rebase(ks.x_o);
  uint64_t *const x_res1 = rebase(ks.x_res1), *const x_h = rebase(ks.x_h), *const x_res2 = rebase(ks.x_res2);
  uint64_t *const x_z = rebase(ks.x_z);
  unsigned long long* const p_amax = d.xbase ? (unsigned long long*)d.xbase : ks.amax;
  uint32_t* const p_done = d.xbase ? (uint32_t*)(d.xbase + 8) : ks.done;
  uint8_t* const kc = d.kc;
  uint8_t* const vc = d.vc;
  const int seq = d.seq, B = d.B, cap = d.cap;
  GLOBAL uint64_t* const stamps = (d.dbg_ts != nullptr && W == 0 && tid == 0) ? gp(d.dbg_ts) : nullptr;
  // chunks per lane of each GEMV of the static shape (0: dynamic geometry, activation read from LDS)
  constexpr int HW = WT == W_I4 ? W_BF16 : WT;  // the head is bf16 (or fp32) even when the layers are int4
  constexpr int CP_QKV = cpl_fit<WT, SH>(SH::H, QKV_CAP), CP_O = cpl_fit<WT, SH>(SH::NQ * SH::HD, O_CAP);
  constexpr int CP_GU = cpl_fit<WT, SH>(SH::H, GU_CAP);
  constexpr int CP_DN = cpl_fit<WT, SH>(SH::DI, DN_CAP), CP_LM = cpl_fit<HW, SH>(SH::H, LM_CAP);
  // attention scores on MFMA: bf16 cache rows of 128 dims, at most 4 query heads per kv head
  constexpr bool MFMA_QK = SS && !kAct32<WT> && SH::HD == 128 && SH::NQ / SH::NKV <= 4;
  // The static shape's weight, norm and K/V requests are made out of the compiler's sight (inline
  // assembly): the compiler cannot tell which LDS a request writes, so it would make every later LDS
  // access, and every barrier, wait for all outstanding requests; here each reader waits for its own
  // bytes explicitly (vmcnt) and the exchanges' polls go out while the requests are in flight.
  constexpr bool UT = SS;
  constexpr bool ASUM_A = WT == W_I4;  // int4 GEMVs take the chunk sums of actA from LDS
  constexpr int RCH = (MAX_H / kChunkElems<WT> + 63) / 64;  // router row chunks per lane
  // items per wave of each GEMV of the static shape (0: general rounds)
  constexpr int NI_QKV = nis_of(2 * even_share((SH::NQ + 2 * SH::NKV) * SH::HD / 2, SH::G), CP_QKV);
  constexpr int NI_O = nis_of(even_share(SH::H, SH::G), CP_O);
  // the o_proj staging lies inside the QKV staging (the start of both layouts), clear of the attention's buffers
  constexpr bool kEarlyO = SS && NI_O > 0 && NI_O <= O_CAP && CP_O > 0 && NI_O / CP_O <= 16;
  static_assert(!kEarlyO || (offsetof(MergeLds, so) == 0 && offsetof(AttnLds, sq) == 0 &&
                             sizeof(StageLds<O_CAP>) <= sizeof(StageLds<QKV_CAP>)),
                "the early o_proj rows overlap only the QKV staging");
  constexpr int NI_GUM = nis_of(4 * even_share(SH::K * SH::EI / 2, SH::G), CP_GU);
  constexpr int NI_GUD = nis_of(4 * even_share(SH::DI / 2, SH::G), CP_GU);
  constexpr int NI_DND = nis_of(even_share(SH::H, SH::G), CP_DN);
  // MoE down: K rows per output row, one chunk per lane (rows of expert_inter fit one lane group)
  constexpr int C_DN = SS ? SH::EI / kChunkElems<WT> : 0;
  constexpr int RPW_DN = C_DN > 0 && C_DN <= 32 ? (C_DN <= 16 ? (C_DN <= 8 ? 8 : 4) : 2) : 1;
  constexpr int NI_DNM = SS && C_DN > 0 && C_DN <= 64 && (even_share(SH::H, SH::G) * SH::K) % (NW * RPW_DN) == 0
                             ? even_share(SH::H, SH::G) * SH::K / (NW * RPW_DN)
                             : 0;

  // token and position of this step (every workgroup makes the same choice)
  int tok = gp(d.tokens)[d.tok_idx];
  const int pos = gp(d.len)[seq];
  if (pos < 0 || pos >= cap) {
    if (W == 0 && tid == 0) raise_error(wt, ERR_POS);
    return;
  }
  if (tok < 0 || tok >= V_) {
    if (W == 0 && tid == 0) raise_error(wt, ERR_TOKEN);
    tok = 0;
  }
  if (W == 0 && tid == 0) gp(d.hist)[(size_t)seq * cap + pos] = tok;  // the cache's token record
  // stamps stay in LDS until the step ends: a store among the layers' counted DMA waits (or a wait that also
  // covers a store) would change what the stamps measure
  const uint64_t t_start = stamps ? now() : 0, c_start = stamps ? __builtin_amdgcn_s_memtime() : 0;
  if (tid == 0) sm.flag = 0;

  const int T = pos + 1;
  const int S = nkv > 0 ? G / nkv : 0;  // attention splits per kv head
  const int aj = W / S, as = W % S;  // attention work: kv head aj, split as
  const bool attn = aj < nkv;
  const int t0 = attn ? part(T, S, as) : 0, t1 = attn ? part(T, S, as + 1) : 0;
  const float qscale = 1.0f / sqrtf((float)hd);
  const int ebytes = kAct32<WT> ? 4 : 2;
  const int rowb = hd * ebytes;                 // bytes of one cached K or V row
  const int CHP = KV_LDS / rowb;                // positions per attention chunk
  // A split one chunk plus at most TAIL_POS positions long (contexts just past 64 x 128 positions) has its
  // tail's K/V rows requested right after the QKV products, into the part of the QKV staging that the
  // early o_proj rows leave free, and takes the tail as a ninth block of 16 positions in the same pass
  // as the chunk (scored by wave 0, its probabilities after the block maxima and sums in the score
  // buffer, one more K-step of the P.V): no second chunk.
  constexpr int TAIL_POS = 16, TAIL_OFF = (int)sizeof(StageLds<O_CAP>);
  static_assert(offsetof(AttnLds, sq) == 0 && TAIL_OFF + 2 * TAIL_POS * 256 <= (int)sizeof(StageLds<QKV_CAP>),
                "the tail's K and V rows fit between the early o_proj rows and the K buffer");
  const bool tail_pre = MFMA_QK && kEarlyO && attn && t1 - t0 > CHP && t1 - t0 - CHP <= TAIL_POS;
  uint4* const ktail = reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(&sm.u.att) + TAIL_OFF);
  uint4* const vtail = ktail + TAIL_POS * 16;
  const size_t kvstride = (size_t)cap * hd;     // elements per (layer, seq, kv head)
  bool ok = true;  // false once a wait failed: skip to the argmax hand-off so the launch still ends cleanly

  // QKV rows of this workgroup: RoPE pairs (i, i + hd/2) stay together
  const int half = hd / 2, NPAIR = QR / 2;
  const int qpb = part(NPAIR, G, W), qpe = part(NPAIR, G, W + 1);
  const Geo gq = geo<WT>(2 * (qpe - qpb), H);
  auto qkv_rowfn = [&](int l) {
    return [&, l](int q) {
      const int u = qpb + q / 2, head = u / half, i = u % half;
      return mrow<WT>(m_qkv, (long long)l * QR + head * hd + i + (q & 1) * half, H, sm.actA, sm.asumA);
    };
  };
  // this workgroup's shares of every other phase (the same in every layer)
  const int orb = part(H, G, W), ore = part(H, G, W + 1);               // o_proj and down rows
  const int mpb = part(QD / 2, G, W), mpe = part(QD / 2, G, W + 1);     // merged output dim pairs
  const int dpb = part(DI_ / 2, G, W), dpe = part(DI_ / 2, G, W + 1);  // dense SwiGLU pairs
  const int xpb = part(K_ * EI_ / 2, G, W), xpe = part(K_ * EI_ / 2, G, W + 1);  // expert pairs
  const float inv_ei = 1.0f / (float)EI_, inv_k = 1.0f / (float)K_;
  // QKV weights of layer l and the K and / or V rows of its first attention chunk (into the shared region)
  auto issue_qkv = [&](int l) { issue_auto<WT, NI_QKV, QKV_CAP, UT>(lstage(sm.u.att.sq), gq, qkv_rowfn(l)); };
  auto issue_kv_front = [&](int l, bool k, bool v) {
    if (!attn || t1 <= t0) return;
    const size_t cb = (((size_t)l * B + seq) * nkv + aj) * kvstride * ebytes;
    const int np0 = min(CHP, t1 - t0);
    if constexpr (MFMA_QK) {  // V rows swizzled like K: the transposing operand reads are conflict-free
      if (k) k_issue_mfma<UT>(sm.u.att.kbuf, kc + cb, t0, np0);
      if (v) k_issue_mfma<UT>(sm.u.att.vbuf, vc + cb, t0, np0);
    } else {
      if (k) kv_issue(sm.u.att.kbuf, kc + cb, t0, np0, rowb);
      if (v) kv_issue(sm.u.att.vbuf, vc + cb, t0, np0, rowb);
    }
  };
  // The MoE layers' down products request the next layer's QKV rows and the K rows of its first chunk
  // (their LDS overlaps only the gate/up staging, dead by then) without the compiler seeing the requests,
  // so that the products' LDS reads do not wait for them: the chip serves them while the products run,
  // and only the V rows (over the down staging) wait for the products to end.  The QKV products and the
  // attention wait for every request (vmcnt(0)) before they read their rows.
  static_assert(offsetof(AttnLds, kbuf) + sizeof(AttnLds::kbuf) <= sizeof(StageLds<GU_CAP>) &&
                    offsetof(AttnLds, sq) + sizeof(AttnLds::sq) <= sizeof(StageLds<GU_CAP>) &&
                    offsetof(MlpLds, gu) == 0,
                "the QKV staging and the K rows overlap only the gate/up staging");
  // Elsewhere a layer's first attention chunk is requested at the end of the layer before, ahead of the
  // residual exchange's polls; every wait that follows is a full one (no later loads left in flight).
  const int kv_later = 0;

  issue_qkv(0);
  issue_kv_front(0, true, true);
  gn_issue<UT>(sm, p_anorm, H);
  float ss0 = 0.f;  // the first input norm's sum of squares, as the residual gathers keep it for later ones
  for (int e = tid; e < H; e += NT) {  // embedding row -> residual
    float v;
    if constexpr (kAct32<WT>)
      v = gp(reinterpret_cast<const float*>(ks.embed))[(long long)tok * H + e];
    else
      v = bf2f(gp(reinterpret_cast<const uint16_t*>(ks.embed))[(long long)tok * H + e]);
    sm.xres[e] = v;
    ss0 = fmaf(v, v, ss0);
  }
  ss0 = wave_sum(ss0);
  if (lane == 0) sm.wred[wave] = ss0;
  for (int q2 = tid; q2 < qpe - qpb; q2 += NT)  // RoPE of this workgroup's pairs at this position
    sm.rcs[q2] = *(GLOBAL const f32x2_t*)(d.rope + (size_t)pos * half + (qpb + q2) % half);
  wait_vmem();
  __syncthreads();

  for (int l = 0; l < L; ++l) {
    const uint32_t tag = d.epoch + (uint32_t)l * 8u;
    const int par = l & 1;
    uint16_t* const stamp = stamps && l < STAMP_LAYERS ? sm.st[l] : nullptr;
    const uint64_t lbase = stamp ? now() : 0;
    if (stamp) sm.st_base[l] = (uint32_t)(lbase - t_start);
    auto stampit = [&](int k) {
      if (stamp) stamp[k] = (uint16_t)(now() - lbase);
    };
    const size_t cbase = (((size_t)l * B + seq) * nkv + (attn ? aj : 0)) * kvstride;
    const uint8_t* const kbase = kc + cbase * ebytes;
    const uint8_t* const vbase = vc + cbase * ebytes;
    const bool dense = l < ks.n_dense;
    const int lmoe = l - ks.n_dense;
    bool front_early = false;  // the next layer's QKV and K rows were requested during the down products

    const Geo go = geo<WT>(ore - orb, QD);  // o_proj rows of this workgroup
    auto o_rowfn = [&](int q) { return mrow<WT>(m_o, (long long)l * H + orb + q, QD, sm.actA, sm.asumA); };

    // ---------------- input RMSNorm (recomputed by every workgroup)
    // static shape: this norm's weights were requested before the previous layer's down products, which
    // waited for every request of each wave (the first layer's, before the loop), so the norm need not wait
    // for the residual's publish or the requests issued since
    rmsnorm_act<WT, WT, true, !SS>(sm, H, ks.eps, ASUM_A, kv_later);
    stampit(0);

    // ---------------- QKV rows (staged during the previous layer), RoPE, publish, KV append
    {
      const auto ar = act_regs<WT, CP_QKV>(gq, sm.actA, sm.asumA);
      gemv_auto<WT, CP_QKV, NI_QKV, QKV_CAP>(lstage(sm.u.att.sq), gq, true, ar, qkv_rowfn(l),
                                             [&](int q, float v) { sm.ytmp[q] = v; }, kv_later);
    }
    __syncthreads();
    // the static shape requests its o_proj rows now, over the QKV staging every wave has finished reading,
    // out of the compiler's sight: the chip serves them long before the merge, whose exchange then waits
    // for no weights, and nothing before the o_proj products reads them (the attention's wait for its
    // chunk covers them as well)
    if constexpr (kEarlyO) lstage_issue_static<WT, NI_O, true>(lstage(sm.u.mg.so), go, 0, o_rowfn, go.wave);
    if constexpr (MFMA_QK) {
      if (tail_pre) {  // the new token's rows among them are replaced from the exchange before use
        k_issue_mfma<true>(ktail, kbase, t0 + CHP, t1 - t0 - CHP);
        k_issue_mfma<true>(vtail, vbase, t0 + CHP, t1 - t0 - CHP);
      }
    }
    stampit(1);
    for (int q2 = tid; q2 < qpe - qpb; q2 += NT) {  // RoPE on q and k heads: pairs (i, i + hd/2)
      const int head = (qpb + q2) / half;
      if (head < nq + nkv) {
        const f32x2_t cs = sm.rcs[q2];
        const float y0 = sm.ytmp[2 * q2], y1 = sm.ytmp[2 * q2 + 1];
        sm.ytmp[2 * q2] = y0 * cs.x - y1 * cs.y;
        sm.ytmp[2 * q2 + 1] = y1 * cs.x + y0 * cs.y;
      }
    }
    __syncthreads();
    publish(x_qkv, QR, par, 2 * (qpe - qpb), tag + 0, [&](int q, int& idx) {
      const int u = qpb + q / 2, head = u / half;
      idx = head * hd + u % half + (q & 1) * half;
      return __float_as_uint(sm.ytmp[q]);
    });
    for (int q = tid; q < 2 * (qpe - qpb); q += NT) {  // append K (after RoPE) and V at this position
      const int u = qpb + q / 2, head = u / half, i = u % half + (q & 1) * half;
      if (head >= nq) {
        const bool isk = head < nq + nkv;
        const int j = isk ? head - nq : head - nq - nkv;
        const size_t off = (((size_t)l * B + seq) * nkv + j) * kvstride + (size_t)pos * hd + i;
        uint8_t* base = isk ? kc : vc;
        if constexpr (kAct32<WT>) gp(reinterpret_cast<float*>(base))[off] = sm.ytmp[q];
        else gp(reinterpret_cast<uint16_t*>(base))[off] = (uint16_t)f2bf(sm.ytmp[q]);
      }
    }
    gn_issue<UT>(sm, p_pnorm + (size_t)l * H, H);  // post-attention norm weights, read after the o_proj exchange
    stampit(2);

    // ---------------- attention partial over positions [t0, t1) of kv head aj
    if (attn) {
      const int h0 = aj * Gq;
      AttnLds& at = sm.u.att;
      if (t0 < t1) {
        const uint64_t* src = copy_of(x_qkv, QR, par);
        // polls go out once this wave's stores (q/k/v, the K/V append) and requests have completed: in
        // alternating runs that beats polling behind them here and in the merge, the merged-output and the
        // residual exchanges, while the exchanges behind a weight burst (router logits, SwiGLU, residual
        // after the MoE) do better polling behind the burst
        wait_vmem();
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
              if (i < nqs) {
                at.qs[i] = v * qscale;
                if constexpr (MFMA_QK) {  // query dim d of head h goes to lane 16 ((d / 8) % 4) + h, slot d % 8
                  const float qv = v * qscale;
                  const uint32_t hb = f2bf(qv);
                  const int h = i >> 7, dd = i & 127;
                  const int idx = ((dd >> 5) * 64 + ((dd >> 3) & 3) * 16 + h) * 8 + (dd & 7);
                  at.qop[0][idx] = (uint16_t)hb;
                  at.qop[1][idx] = (uint16_t)f2bf(qv - bf2f(hb));
                }
              }
              else if (i < nqs + hd) at.kn[i - nqs] = act_round<WT>(v);
              else at.vn[i - nqs - hd] = act_round<WT>(v);
            },
            wt);
        if constexpr (MFMA_QK)  // the operand lanes of heads Gq .. 15 are zero
          for (int idx = tid; idx < 4 * 64 * 8; idx += NT)
            if (((idx >> 3) & 15) >= Gq) at.qop[0][idx] = at.qop[1][idx] = 0;
      } else {
        ok = sync_ok(sm, wt);
      }
      if (!ok) break;
      stampit(3);
      // running output: every wave accumulates all heads over its positions (lane: DPV dims)
      constexpr int DPVM = MAX_HD / 64;
      const int DPV = hd / 64, PST = Gq <= 4 ? 4 : 8;
      float o[MAX_GQ][DPVM];
#pragma unroll
      for (int h = 0; h < MAX_GQ; ++h)
#pragma unroll
        for (int e = 0; e < DPVM; ++e) o[h][e] = 0.f;
      // MFMA path: wave w holds O^T for dims 16 w .. 16 w + 15: lane 16 g + i has dims 16 w + 4 g + j
      // (j = 0..3) of head i
      f32x4_t o4 = {0.f, 0.f, 0.f, 0.f};
      // MFMA path: the probabilities as the B operand of O^T += V^T P^T, bf16 high parts then low parts:
      // K-step kk, lane 16 g + h, element j holds P[h][16 kk + 4 g + j] (zero past the chunk and for the
      // heads Gq .. 15)
      uint16_t* const pb = reinterpret_cast<uint16_t*>(at.pt);
      constexpr int PB_HALF = MAX_CHUNK_POS / 2 / 16 * 64 * 4;  // 128 positions per chunk at head_dim 128
      float* const bmax = at.sc;                 // MFMA path: [wave][head] block maxima, then block sums
      float* const bsum = at.sc + NW * MAX_GQ;
      float sv[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};  // MFMA path: this lane's scores of the chunk
      float st8[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};  // and of the tail block (wave 0)
      float alpha_r = 0.f;                       // MFMA path: rescale of the running output for head lane % 16
      if (tid < Gq) {
        at.mst[tid] = -INFINITY;
        at.lst[tid] = 0.f;
      }
      const int nt = tail_pre ? t1 - t0 - CHP : 0;  // positions of the tail block (MFMA path)
      uint16_t* const pb8 = reinterpret_cast<uint16_t*>(at.sc + 2 * NW * MAX_GQ);  // its probabilities
      for (int c0 = t0; c0 < t1 - nt; c0 += CHP) {
        const int np = min(CHP, t1 - c0);
        uint4* const kb = at.kbuf;
        uint4* const vbm = at.vbuf;
        if (c0 != t0) {  // later chunks (long contexts): load now
          __syncthreads();  // every wave is done with the previous chunk
          if constexpr (MFMA_QK) {
            k_issue_mfma<UT>(at.kbuf, kbase, c0, np);
            k_issue_mfma<UT>(at.vbuf, vbase, c0, np);
          } else {
            kv_issue(at.kbuf, kbase, c0, np, rowb);
            kv_issue(at.vbuf, vbase, c0, np, rowb);
          }
        }
        wait_vmem();
        __syncthreads();
        // the new token's row: k, v from the exchange replace what the DMA read
        if (nt > 0 && pos >= c0 + np && pos < c0 + np + nt) {  // in the tail block (MFMA path)
          for (int e = tid; e < hd; e += NT) {
            reinterpret_cast<uint16_t*>(ktail)[k_slot(pos - c0 - np, e >> 3) * 8 + (e & 7)] = (uint16_t)f2bf(at.kn[e]);
            reinterpret_cast<uint16_t*>(vtail)[k_slot(pos - c0 - np, e >> 3) * 8 + (e & 7)] = (uint16_t)f2bf(at.vn[e]);
          }
          __syncthreads();
        }
        if (pos >= c0 && pos < c0 + np) {
          uint8_t* kr = reinterpret_cast<uint8_t*>(at.kbuf) + (size_t)(pos - c0) * rowb;
          uint8_t* vr = reinterpret_cast<uint8_t*>(at.vbuf) + (size_t)(pos - c0) * rowb;
          for (int e = tid; e < hd; e += NT) {
            if constexpr (kAct32<WT>) {
              reinterpret_cast<float*>(kr)[e] = at.kn[e];
              reinterpret_cast<float*>(vr)[e] = at.vn[e];
            } else {
              if constexpr (MFMA_QK) {  // the rows' units are swizzled by the position
                reinterpret_cast<uint16_t*>(kb)[k_slot(pos - c0, e >> 3) * 8 + (e & 7)] = (uint16_t)f2bf(at.kn[e]);
                reinterpret_cast<uint16_t*>(vbm)[k_slot(pos - c0, e >> 3) * 8 + (e & 7)] = (uint16_t)f2bf(at.vn[e]);
              } else {
                reinterpret_cast<uint16_t*>(kr)[e] = (uint16_t)f2bf(at.kn[e]);
                reinterpret_cast<uint16_t*>(vr)[e] = (uint16_t)f2bf(at.vn[e]);
              }
            }
          }
          __syncthreads();
        }
        if constexpr (MFMA_QK) {
          // scores on MFMA: D[position][head] = K[16 positions x 32 dims] . Q^T[32 dims x 16 heads], the
          // query split into bf16 high and low parts (q = hi + lo to about 16 bits) so the product keeps
          // fp32-level accuracy; lane L supplies head L % 16 (zero past Gq) and gets positions
          // (L / 16) * 4 + r of the block
          const int n = lane & 15;
          bf16x8_t qh[4], ql[4];
#pragma unroll
          for (int sk = 0; sk < 4; ++sk) {
            qh[sk] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(&at.qop[0][(sk * 64 + lane) * 8]));
            ql[sk] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(&at.qop[1][(sk * 64 + lane) * 8]));
          }
          // a chunk holds at most 128 positions here: wave w scores block w of 16 positions and keeps them in
          // registers (-inf for positions past the chunk and heads past Gq); each block's maximum per head
          // meets the others' in LDS
          const int b = wave;
#pragma unroll
          for (int r = 0; r < 4; ++r) sv[r] = -INFINITY;
          if (b * 16 < np) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sk = 0; sk < 4; ++sk) {
              const bf16x8_t a =
                  __builtin_bit_cast(bf16x8_t, kb[k_slot(b * 16 + (lane & 15), sk * 4 + (lane >> 4))]);
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qh[sk], acc, 0, 0, 0);
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ql[sk], acc, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) sv[r] = (n < Gq && b * 16 + (lane >> 4) * 4 + r < np) ? acc[r] : -INFINITY;
          }
          float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
          if (nt > 0 && wave == 0) {  // the tail block
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sk = 0; sk < 4; ++sk) {
              const bf16x8_t a = __builtin_bit_cast(bf16x8_t, ktail[k_slot(lane & 15, sk * 4 + (lane >> 4))]);
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qh[sk], acc, 0, 0, 0);
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ql[sk], acc, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) st8[r] = (n < Gq && (lane >> 4) * 4 + r < nt) ? acc[r] : -INFINITY;
            bm = fmaxf(bm, fmaxf(fmaxf(st8[0], st8[1]), fmaxf(st8[2], st8[3])));
          }
          bm = fmaxf(bm, swap16(bm));
          bm = fmaxf(bm, swap32(bm));
          if (lane < Gq) bmax[wave * MAX_GQ + lane] = bm;
        } else {
        // scores: LPK lanes read one K row (16 B each), RPI rows per wave instruction
          constexpr int DPL = kAct32<WT> ? 4 : 8;  // dims per lane
          const int LPK = rowb / 16, RPI = 64 / LPK;
          const int seg = lane % LPK, rsub = lane / LPK;
          const int ninstr = (np + RPI - 1) / RPI;
          for (int hg = 0; hg < Gq; hg += 4) {
            float qv[4][DPL];
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
              for (int e = 0; e < DPL; ++e) qv[a][e] = hg + a < Gq ? at.qs[(hg + a) * hd + seg * DPL + e] : 0.f;
            for (int it = wave; it < ninstr; it += NW) {
              const uint4 kr = at.kbuf[it * 64 + lane];
              float kf[DPL];
              if constexpr (kAct32<WT>) {
                kf[0] = __uint_as_float(kr.x);
                kf[1] = __uint_as_float(kr.y);
                kf[2] = __uint_as_float(kr.z);
                kf[3] = __uint_as_float(kr.w);
              } else {
                const uint32_t kw[4] = {kr.x, kr.y, kr.z, kr.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                  kf[2 * k] = bf2f(kw[k] & 0xFFFFu);
                  kf[2 * k + 1] = bf2f(kw[k] >> 16);
                }
              }
              const int row = it * RPI + rsub;
#pragma unroll
              for (int a = 0; a < 4; ++a) {
                float t = 0.f;
#pragma unroll
                for (int e = 0; e < DPL; ++e) t = fmaf(qv[a][e], kf[e], t);
                t = group_sum(t, LPK);
                if (seg == a && hg + a < Gq && row < np) at.sc[(hg + a) * CHP + row] = t;
              }
            }
          }
        }
        __syncthreads();
        if constexpr (MFMA_QK) {
          // softmax from the registers: every wave finds each head's maximum over the blocks, writes its
          // block's probabilities as the B operand of the P.V below (lane 16 g + i, K-step = block, element r:
          // P[i][16 b + 4 g + r], bf16 high and low parts) and its block's sum per head
          const int i = lane & 15;
          float mc = -INFINITY;
#pragma unroll
          for (int w = 0; w < NW; ++w) mc = fmaxf(mc, bmax[w * MAX_GQ + (i < Gq ? i : 0)]);
          const float mo = i < Gq ? at.mst[i] : -INFINITY;
          const float mn = fmaxf(mo, mc);
          alpha_r = mo == -INFINITY ? 0.f : __expf(mo - mn);
          float ls = 0.f;
          if (wave * 16 < np) {
            s16x4_t ph, pl;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float pr = i < Gq ? __expf(sv[r] - mn) : 0.f;
              const uint32_t hb = f2bf(pr);
              ph[r] = (short)hb;
              pl[r] = (short)f2bf(pr - bf2f(hb));
              ls += pr;
            }
            *reinterpret_cast<s16x4_t*>(pb + (wave * 64 + lane) * 4) = ph;
            *reinterpret_cast<s16x4_t*>(pb + PB_HALF + (wave * 64 + lane) * 4) = pl;
          }
          if (nt > 0 && wave == 0) {
            s16x4_t ph, pl;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float pr = i < Gq ? __expf(st8[r] - mn) : 0.f;
              const uint32_t hb = f2bf(pr);
              ph[r] = (short)hb;
              pl[r] = (short)f2bf(pr - bf2f(hb));
              ls += pr;
            }
            *reinterpret_cast<s16x4_t*>(pb8 + lane * 4) = ph;
            *reinterpret_cast<s16x4_t*>(pb8 + 256 + lane * 4) = pl;
          }
          ls += swap16(ls);
          ls += swap32(ls);
          if (lane < Gq) bsum[wave * MAX_GQ + lane] = ls;
          __syncthreads();
          if (tid < Gq) {  // the running maximum and sum of head tid (lane tid of wave 0 holds its values)
            float t = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) t += bsum[w * MAX_GQ + tid];
            at.mst[tid] = mn;
            at.lst[tid] = at.lst[tid] * alpha_r + t;
          }
        }
        // softmax, one wave per head: probabilities to pt, the running max / sum and rescale factor to LDS
        for (int h = wave; !MFMA_QK && h < Gq; h += NW) {
          const float* sh = at.sc + h * CHP;
          float mc = -INFINITY;
          for (int i = lane; i < np; i += 64) mc = fmaxf(mc, sh[i]);
          mc = wave_max(mc);
          const float mo = at.mst[h];
          const float mn = fmaxf(mo, mc);
          const float alpha = mo == -INFINITY ? 0.f : __expf(mo - mn);
          float ls = 0.f;
          for (int i = lane; i < np; i += 64) {
            const float pr = __expf(sh[i] - mn);
            if constexpr (MFMA_QK) {
              const uint32_t hb = f2bf(pr);
              const int idx = ((i >> 4) * 64 + ((i >> 2) & 3) * 16 + h) * 4 + (i & 3);
              pb[idx] = (uint16_t)hb;
              pb[PB_HALF + idx] = (uint16_t)f2bf(pr - bf2f(hb));
            } else {
              at.pt[i * PST + h] = pr;
            }
            ls += pr;
          }
          ls = wave_sum(ls);
          if (lane == 0) {
            at.fac[h] = alpha;
            at.mst[h] = mn;
            at.lst[h] = at.lst[h] * alpha + ls;
          }
        }
        if (!MFMA_QK && Gq < PST)  // padding heads of pt stay zero
          for (int i = tid; i < np * (PST - Gq); i += NT) at.pt[(i / (PST - Gq)) * PST + Gq + i % (PST - Gq)] = 0.f;
        if (!MFMA_QK) __syncthreads();
        if constexpr (MFMA_QK) {
          // O^T += V^T P^T on v_mfma_f32_16x16x16_bf16 (P as bf16 high and low parts): the A operand (16 dims
          // x 16 positions) comes from the swizzled V rows through the transposing LDS read, this lane
          // passing position 16 kk + 4 g + i / 4, dims 16 w + 4 (i % 4) .. + 3
          const int g = lane >> 4, i = lane & 15;
#pragma unroll
          for (int j = 0; j < 4; ++j) o4[j] *= alpha_r;
          const uint8_t* vlb = reinterpret_cast<const uint8_t*>(vbm);
          const int u = 2 * wave + ((i & 3) >> 1);
          const int nk = (np + 15) / 16;
          // four K-steps at a time: their operand reads are issued together, then their products
          for (int k0 = 0; k0 < nk; k0 += 4) {
            s16x4_t vt[4], ph[4], pl[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int kk = min(k0 + q, nk - 1);  // past the last K-step: a repeated read, not used
              const int row = 16 * kk + 4 * g + (i >> 2);
              vt[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) s16x4_t*)(vlb + row * 256 + ((u ^ (row & 15)) * 16) + (i & 1) * 8));
              ph[q] = *reinterpret_cast<const s16x4_t*>(pb + (kk * 64 + lane) * 4);
              pl[q] = *reinterpret_cast<const s16x4_t*>(pb + PB_HALF + (kk * 64 + lane) * 4);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int kk = k0 + q;
              if (kk < nk) {
                if (16 * kk + 16 > np) {  // rows past the chunk may hold anything: their zero probabilities
#pragma unroll                            // must not meet a NaN
                  for (int j = 0; j < 4; ++j)
                    if (16 * kk + 4 * g + j >= np) vt[q][j] = 0;
                }
                o4 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt[q], ph[q], o4, 0, 0, 0);
                o4 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt[q], pl[q], o4, 0, 0, 0);
              }
            }
          }
          if (nt > 0) {  // the tail block: one more K-step, V rows from the tail buffer
            const int row = 4 * g + (i >> 2);
            const uint8_t* vtb = reinterpret_cast<const uint8_t*>(vtail);
            s16x4_t vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4_t*)(vtb + row * 256 + ((u ^ (row & 15)) * 16) + (i & 1) * 8));
            const s16x4_t ph = *reinterpret_cast<const s16x4_t*>(pb8 + lane * 4);
            const s16x4_t pl = *reinterpret_cast<const s16x4_t*>(pb8 + 256 + lane * 4);
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (4 * g + j >= nt) vt[j] = 0;
            o4 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, ph, o4, 0, 0, 0);
            o4 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, pl, o4, 0, 0, 0);
          }
          continue;
        }
        // P.V: wave w takes positions w, w + NW, ...; all heads at once
#pragma unroll
        for (int h = 0; h < MAX_GQ; ++h) {
          const float f = h < Gq ? at.fac[h] : 0.f;
#pragma unroll
          for (int e = 0; e < DPVM; ++e) o[h][e] *= f;
        }
        const uint8_t* vb = reinterpret_cast<const uint8_t*>(at.vbuf);
#pragma unroll 4
        for (int i = wave; i < np; i += NW) {
          float pr[MAX_GQ];
          const float4 p0 = *reinterpret_cast<const float4*>(at.pt + i * PST);
          pr[0] = p0.x;
          pr[1] = p0.y;
          pr[2] = p0.z;
          pr[3] = p0.w;
          if (PST == 8) {
            const float4 p1 = *reinterpret_cast<const float4*>(at.pt + i * PST + 4);
            pr[4] = p1.x;
            pr[5] = p1.y;
            pr[6] = p1.z;
            pr[7] = p1.w;
          } else {
            pr[4] = pr[5] = pr[6] = pr[7] = 0.f;
          }
          float v[DPVM];
          const uint8_t* row = vb + (size_t)i * rowb;
          if constexpr (kAct32<WT>) {
            if (DPV == 2) {
              const float2 v2 = reinterpret_cast<const float2*>(row)[lane];
              v[0] = v2.x;
              v[DPVM - 1] = v2.y;
            } else {
              v[0] = reinterpret_cast<const float*>(row)[lane];
            }
          } else {
            if (DPV == 2) {
              const uint32_t v2 = reinterpret_cast<const uint32_t*>(row)[lane];
              v[0] = bf2f(v2 & 0xFFFFu);
              v[DPVM - 1] = bf2f(v2 >> 16);
            } else {
              v[0] = bf2f(reinterpret_cast<const uint16_t*>(row)[lane]);
            }
          }
#pragma unroll
          for (int h = 0; h < MAX_GQ; ++h)
            if (h < PST)
#pragma unroll
              for (int e = 0; e < DPVM; ++e)
                if (e < DPV) o[h][e] = fmaf(pr[h], v[e], o[h][e]);
        }
      }
      uint64_t* dst = x_part + (size_t)par * nq * (hd + 2) * S + ((size_t)aj * S + as) * Gq * (hd + 2);
      if constexpr (MFMA_QK) {
        // each wave holds whole dims (16 w .. 16 w + 15 of every head): it publishes them from registers,
        // lane 16 h + d taking dim 16 w + d of head h (from lane 16 (d / 4) + h, element d % 4) so that
        // each head's 16 dims go out as one contiguous run
        const int h = lane >> 4, d = lane & 15, src = 16 * (d >> 2) + h;
        float v = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float t = __int_as_float(__builtin_amdgcn_ds_bpermute(src * 4, __float_as_int(o4[j])));
          if ((d & 3) == j) v = t;
        }
        if (h < Gq) xstore(dst + (size_t)h * (hd + 2) + 2 + 16 * wave + d, slot(tag + 1, __float_as_uint(v)));
        if (tid < 2 * Gq) {
          const int hh = tid >> 1;
          const float mlv = (tid & 1) ? at.lst[hh] : at.mst[hh];
          xstore(dst + (size_t)hh * (hd + 2) + (tid & 1), slot(tag + 1, __float_as_uint(mlv)));
        }
      }
      // sum the waves' outputs (the K rows are dead: their buffer holds the partial sums)
      float* red = reinterpret_cast<float*>(at.kbuf);
      if constexpr (!MFMA_QK) {
        __syncthreads();
#pragma unroll
        for (int h = 0; h < MAX_GQ; ++h)
          if (h < Gq)
#pragma unroll
            for (int e = 0; e < DPVM; ++e)
              if (e < DPV) red[(wave * MAX_GQ + h) * hd + lane * DPV + e] = o[h][e];
        __syncthreads();
        // publish (m, l, o) of each head of this split, contiguous: slot ((split * Gq + h) * (hd + 2) + field)
        // of the kv head's block; every slot is tagged
        for (int idx = tid; idx < Gq * hd; idx += NT) {
          const int h = idx / hd, e = idx % hd;
          float t = 0.f;
#pragma unroll
          for (int w = 0; w < NW; ++w) t += red[(w * MAX_GQ + h) * hd + e];
          xstore(dst + (size_t)h * (hd + 2) + 2 + e, slot(tag + 1, __float_as_uint(t)));
        }
        if (tid < 2 * Gq) {
          const int h = tid >> 1;
          const float v = (tid & 1) ? at.lst[h] : at.mst[h];
          xstore(dst + (size_t)h * (hd + 2) + (tid & 1), slot(tag + 1, __float_as_uint(v)));
        }
      }
    }
    stampit(4);

    // elsewhere the o_proj rows of this workgroup are staged before the merge waits
    __syncthreads();  // the attention layout of the shared region is dead
    if constexpr (!kEarlyO) issue_auto<WT, NI_O, O_CAP, UT>(lstage(sm.u.mg.so), go, o_rowfn);

    // ---------------- merge the splits: this workgroup's pairs of output dims
    {
      constexpr int MNF = SS ? 2 + 2 * (SH::NQ * SH::HD / 2 / SH::G) : 1;  // fields gathered per split
      static_assert(!SS || ((SH::NQ * SH::HD / 2) % SH::G == 0 && (SH::HD / 2) % ((MNF - 2) / 2) == 0),
                    "the static shape merges whole runs of dims inside one head");
      const int pb = mpb, pe = mpe;
      const uint64_t* srcp = x_part + (size_t)par * nq * (hd + 2) * S;
      wait_vmem();  // polls once this wave's stores (the attention partials) have completed
      int e0 = 2 * pb;
      while (e0 < 2 * pe) {  // one head at a time (uniform loop)
        const int h = e0 / hd, eh0 = e0 % hd;
        const int ne = min(2 * pe, (h + 1) * hd) - e0;  // elements of head h in range (even)
        const int nf = 2 + ne, n = nf * S;  // gathered as [split][m, l, this range of o]
        const float inv_nf = 1.0f / (float)nf;
        const size_t hblk = (size_t)(h / Gq) * S * Gq * (hd + 2) + (size_t)(h % Gq) * (hd + 2);
        ok = gather(
            sm, srcp, n, tag + 1,
            [&](int i) {
              // the static shape: every workgroup merges one whole run of MNF - 2 dims of one head, so the
              // field count is a constant and the division a multiply
              const int sp = SS ? i / MNF : div_small(i, nf, inv_nf), f = i - sp * nf;
              return hblk + (size_t)sp * Gq * (hd + 2) + (f < 2 ? f : 2 + eh0 + (f - 2));
            },
            [=](int k, int m) { return (((k + 1) * S) / m - 1) * nf; }, S < 64 ? S : 64,  // m fields
            [&](int i, uint32_t p) { sm.u.mg.gbuf[i] = p; }, wt);
        if (!ok) break;
        // one wave per output pair, lanes over splits: log-sum-exp merge
        for (int k = wave; k < ne / 2; k += NW) {
          float M = -INFINITY;
          for (int s = lane; s < S; s += 64) M = fmaxf(M, __uint_as_float(sm.u.mg.gbuf[s * nf]));
          M = wave_max(M);
          float Lsum = 0.f, O0 = 0.f, O1 = 0.f;
          for (int s = lane; s < S; s += 64) {
            const uint32_t* gs = sm.u.mg.gbuf + s * nf;
            const float m = __uint_as_float(gs[0]);
            const float w = m == -INFINITY ? 0.f : __expf(m - M);
            Lsum = fmaf(w, __uint_as_float(gs[1]), Lsum);
            O0 = fmaf(w, __uint_as_float(gs[2 + 2 * k]), O0);
            O1 = fmaf(w, __uint_as_float(gs[3 + 2 * k]), O1);
          }
          Lsum = wave_sum(Lsum);
          O0 = wave_sum(O0);
          O1 = wave_sum(O1);
          if (lane == 0) {
            sm.ytmp[e0 - 2 * pb + 2 * k] = act_round<WT>(O0 / Lsum);
            sm.ytmp[e0 - 2 * pb + 2 * k + 1] = act_round<WT>(O1 / Lsum);
          }
        }
        __syncthreads();
        e0 += ne;
      }
      if (ok) {  // publish the merged dims: fp32 one per slot, else a bf16 pair
        const int nv = 2 * (pe - pb);
        if constexpr (kAct32<WT>)
          publish(x_o, OSL, par, nv, tag + 2, [&](int i, int& idx) {
            idx = 2 * pb + i;
            return __float_as_uint(sm.ytmp[i]);
          });
        else
          publish(x_o, OSL, par, nv / 2, tag + 2, [&](int i, int& idx) {
            idx = pb + i;
            return f2bf(sm.ytmp[2 * i]) | (f2bf(sm.ytmp[2 * i + 1]) << 16);
          });
      }
    }
    if (!ok) break;
    stampit(5);

    // ---------------- o_proj rows + residual
    wait_vmem();  // polls once this wave's stores (the merged dims) have completed
    ok = gather_flat(sm, copy_of(x_o, OSL, par), OSL, tag + 2,
                     [&](int i, uint32_t p) {
                       if constexpr (kAct32<WT>) {
                         act_put<WT>(sm.actA, i, __uint_as_float(p));
                       } else {
                         act_put2_bits<WT>(sm.actA, 2 * i, p);
                       }
                     },
                     wt);
    if (!ok) break;
    stampit(6);
    if constexpr (ASUM_A) {
      act_sums<WT>(sm.actA, sm.asumA, QD);
      __syncthreads();
    }
    {
      const auto ar = act_regs<WT, CP_O>(go, sm.actA, sm.asumA);
      gemv_auto<WT, CP_O, NI_O, O_CAP>(lstage(sm.u.mg.so), go, true, ar, o_rowfn, [&](int q, float v) { sm.ytmp[q] = v; });
    }
    __syncthreads();
    publish(x_res1, H, par, ore - orb, tag + 3, [&](int q, int& idx) {
      idx = orb + q;
      return __float_as_uint(sm.xres[orb + q] + sm.ytmp[q]);
    });
    stampit(7);
    // router rows of this workgroup (one wave per row): the first row of each wave is staged before
    // the wait for the residual (chunk lane + 64 j of the row in item j)
    const int rbb = dense ? 0 : part(E_, G, W), rbe = dense ? 0 : part(E_, G, W + 1);
    const int RC = H / kChunkElems<WT>;  // chunks of one router row
    const LStage rst = lstage(sm.u.rt);
    auto router_issue = [&](int r) {
      const RowSrc src = mrow<WT>(m_r, (long long)lmoe * E_ + r, H, nullptr, nullptr);
#pragma unroll
      for (int j = 0; j < RCH; ++j) {
        const int c = lane + 64 * j < RC ? lane + 64 * j : 0;
        if constexpr (UT) {
          dma16_untracked(src.w + 16ll * c, lds_offset(&rst.w16[(j * NW + wave) * 64]));
          if constexpr (WT == W_I4) dma4_untracked(src.s + ((c >> 1) & ~1), lds_offset(&rst.s32[(j * NW + wave) * 64]));
        } else {
          dma16(src.w + 16ll * c, &rst.w16[(j * NW + wave) * 64]);
          if constexpr (WT == W_I4) dma4(src.s + ((c >> 1) & ~1), &rst.s32[(j * NW + wave) * 64]);
        }
      }
    };
    wait_vmem();  // likewise (the o_proj rows); the router rows are requested after it, ahead of the polls
    if (rbb + wave < rbe) router_issue(rbb + wave);
    // the gathered residual's squares are summed on the way in: the post-attention norm starts from them
    float ss1 = 0.f;
    ok = gather_flat(
        sm, copy_of(x_res1, H, par), H, tag + 3,
        [&](int i, uint32_t p) {
          const float v = __uint_as_float(p);
          sm.xres[i] = v;
          ss1 = fmaf(v, v, ss1);
        },
        wt,
        [&]() {
          ss1 = wave_sum(ss1);
          if (lane == 0) sm.wred[NW + wave] = ss1;
        });
    if (!ok) break;
    stampit(8);

    // ---------------- post-attention RMSNorm (recomputed by every workgroup)
    rmsnorm_act<WT, WT, true>(sm, H, ks.eps, ASUM_A, 0, 1);
    stampit(9);

    int nunit, inner;  // SwiGLU elements this layer produces, and the down projection's input width
    if (dense) {
      nunit = DI_;
      inner = DI_;
      if (W == 0 && tid < K_) {
        if (d.dbg_routes) gp(d.dbg_routes)[(size_t)l * K_ + tid] = -1;
        if (d.dbg_rw) gp(d.dbg_rw)[(size_t)l * K_ + tid] = 0.f;
      }
    } else {
      // ------------ router: each of its rows computed by one workgroup, the logits exchanged; top-k
      {
        const I4K k4 = i4k();
        for (int r = rbb + wave, it = 0; r < rbe; r += NW, ++it) {
          if (it > 0) {  // more rows than waves (small grids): this wave's reads of the slots are done
            wait_lds();
            router_issue(r);
          }
          wait_vmem();
          float acc = 0.f;
#pragma unroll
          for (int j = 0; j < RCH; ++j) {
            const int c = lane + 64 * j;
            if (c < RC) acc += item_dot<WT>(rst, (j * NW + wave) * 64 + lane, c, act_chunk<WT>(sm.actA, sm.asumA, c), k4);
          }
          acc = wave_sum(acc);
          if (lane < NCOPY) xstore(x_z + (size_t)(lane * 2 + par) * E_ + r, slot(tag + 6, __float_as_uint(acc)));
        }
      }
      ok = gather_flat(sm, copy_of(x_z, E_, par), E_, tag + 6, [&](int i, uint32_t p) { sm.z[i] = __uint_as_float(p); },
                       wt);
      if (!ok) break;
      if (d.dbg_z && W == 0)
        for (int e = tid; e < E_; e += NT) gp(d.dbg_z)[(size_t)l * E_ + e] = sm.z[e];
      stampit(10);
      // top-k by rank, in every wave (identical results; a wave reads only its own writes):
      // lane e counts the experts that beat it (larger logit, or equal logit and lower index)
      {
        const float zl = lane < E_ ? sm.z[lane] : -INFINITY;
        const uint32_t u = __float_as_uint(zl);
        const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
        const uint64_t key = lane < E_ ? (((uint64_t)ord << 32) | (uint32_t)(63 - lane)) : 0ull;
        const uint32_t khi = (uint32_t)(key >> 32), klo = (uint32_t)key;
        // wave w compares against experts 16 w .. 16 w + 15; the partial counts meet in LDS (the SwiGLU
        // buffer is unused until the SwiGLU exchange)
        int* rk = reinterpret_cast<int*>(sm.u.mlp.hbuf);
        int part = 0;
#pragma unroll
        for (int jj = 0; jj < MAX_E / NW; ++jj) {
          const int j = wave * (MAX_E / NW) + jj;
          const uint64_t kj = ((uint64_t)__builtin_amdgcn_readlane(khi, j) << 32) | __builtin_amdgcn_readlane(klo, j);
          part += j < E_ && kj > key;
        }
        rk[wave * 64 + lane] = part;
        // the softmax needs no ranks: it runs while the other waves finish their counts
        const float zmax = wave_max(zl);
        const float pe = lane < E_ ? __expf(zl - zmax) : 0.f;
        const float den = wave_sum(pe);
        const float w = pe / den;
        __syncthreads();
        int rank = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) rank += rk[w * 64 + lane];
        const float wsum = ks.renorm ? wave_sum(lane < E_ && rank < K_ ? w : 0.f) : 1.f;
        if (lane < E_ && rank < K_) {
          sm.sel[rank] = lane;
          sm.wsel[rank] = ks.renorm ? w / wsum : w;
        }
        wait_lds();
        __builtin_amdgcn_wave_barrier();
      }
      if (W == 0 && tid < K_) {
        if (d.dbg_routes) gp(d.dbg_routes)[(size_t)l * K_ + tid] = sm.sel[tid];
        if (d.dbg_rw) gp(d.dbg_rw)[(size_t)l * K_ + tid] = sm.wsel[tid];
      }
      nunit = K_ * EI_;
      inner = EI_;
      stampit(11);
    }

    // ---------------- gate/up rows of this workgroup's SwiGLU elements
    const int upb = dense ? dpb : xpb, upe = dense ? dpe : xpe;
    const int ue0 = 2 * upb, une = 2 * (upe - upb);
    const int drb = orb, dre = ore;
    const int K = K_;
    const int wstride = inner / kChunkElems<WT> * kChunkWords<WT>;  // words of one rank's h
    // this workgroup's units are contiguous: unless they span more than two experts, the selected
    // experts of the first and the next rank are all a row needs
    const Mat& mg = dense ? m_dg : m_eg;
    const Mat& mu = dense ? m_du : m_eu;
    const int gk0 = dense ? 0 : div_small(ue0, EI_, inv_ei);
    const bool two = !dense && une <= EI_;
    const int gsel0 = dense ? 0 : sm.sel[gk0], gsel1 = (!dense && gk0 + 1 < K_) ? sm.sel[gk0 + 1] : gsel0;
    const int gub = (gk0 + 1) * EI_;  // first unit of the next rank
    auto gu_rowfn = [&](int q) {
      const int u = ue0 + q / 2;
      long long row;
      if (dense) {
        row = (long long)l * DI_ + u;
      } else if (two) {
        const bool nx = u >= gub;
        row = ((long long)lmoe * E_ + (nx ? gsel1 : gsel0)) * EI_ + u - (nx ? gub : gub - EI_);
      } else {
        const int k = div_small(u, EI_, inv_ei);
        row = ((long long)lmoe * E_ + sm.sel[k]) * EI_ + u - k * EI_;
      }
      return mrow<WT>((q & 1) ? mu : mg, row, H, sm.actA, sm.asumA);
    };
    auto dn_rowfn = [&](int q) {
      if (dense) return mrow<WT>(m_dd, (long long)l * H + drb + q, inner, sm.u.mlp.hbuf, sm.u.mlp.asumH);
      const int qk = div_small(q, K, inv_k);
      const int r = drb + qk, k = q - qk * K;
      return mrow<WT>(m_ed, ((long long)lmoe * E_ + sm.sel[k]) * H + r, inner, sm.u.mlp.hbuf + k * wstride,
                      sm.u.mlp.asumH + k * (inner / 32));
    };
    // the static MoE down visits its rows expert by expert: geometry row rp is output row rp % R8 of
    // rank rp / R8 (R8 = rows per workgroup), so every item of a wave reads one expert
    const int R8 = dre - drb;
    auto dn_rowfn_x = [&](int rp) {
      const int k = rp / R8, r = drb + rp - k * R8;
      return mrow<WT>(m_ed, ((long long)lmoe * E_ + sm.sel[k]) * H + r, inner, sm.u.mlp.hbuf + k * wstride,
                      sm.u.mlp.asumH + k * (inner / 32));
    };
    const Geo ggu = geo<WT>(2 * une, H);
    const Geo gdn = geo<WT>(dense ? dre - drb : (dre - drb) * K, inner);
    if (dense) issue_auto<WT, NI_GUD, GU_CAP, UT>(lstage(sm.u.mlp.gu), ggu, gu_rowfn);
    else issue_auto<WT, NI_GUM, GU_CAP, UT>(lstage(sm.u.mlp.gu), ggu, gu_rowfn);
    {
      const auto ar = act_regs<WT, CP_GU>(ggu, sm.actA, sm.asumA);
      auto out = [&](int q, float v) { sm.ytmp[q] = v; };
      if (dense) gemv_auto<WT, CP_GU, NI_GUD, GU_CAP>(lstage(sm.u.mlp.gu), ggu, true, ar, gu_rowfn, out);
      else gemv_auto<WT, CP_GU, NI_GUM, GU_CAP, true>(lstage(sm.u.mlp.gu), ggu, true, ar, gu_rowfn, out);
    }
    __syncthreads();
    // SwiGLU of this workgroup's units: fp32 one value per slot, else a bf16 pair of adjacent units
    if constexpr (kAct32<WT>)
      publish(x_h, HSLOTS, par, une, tag + 4, [&](int k, int& idx) {
        const float g = sm.ytmp[2 * k], u = sm.ytmp[2 * k + 1];
        idx = ue0 + k;
        return __float_as_uint(g / (1.0f + __expf(-g)) * u);
      });
    else
      publish(x_h, HSLOTS, par, une / 2, tag + 4, [&](int k, int& idx) {
        uint32_t hv[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const float g = sm.ytmp[4 * k + 2 * t], u = sm.ytmp[4 * k + 2 * t + 1];
          hv[t] = f2bf(g / (1.0f + __expf(-g)) * u);
        }
        idx = ue0 / 2 + k;
        return hv[0] | (hv[1] << 16);
      });
    // the down weights and the next norm's weights load during the SwiGLU exchange
    if (dense) issue_auto<WT, NI_DND, DN_CAP, UT>(lstage(sm.u.mlp.dn), gdn, dn_rowfn);
    else if constexpr (NI_DNM > 0 && NI_DNM <= DN_CAP) lstage_issue_static<WT, NI_DNM, UT>(lstage(sm.u.mlp.dn), gdn, 0, dn_rowfn_x, gdn.wave);
    else lstage_issue<WT>(lstage(sm.u.mlp.dn), gdn, 0, dn_rowfn);
    gn_issue<UT>(sm, l + 1 < L ? p_anorm + (size_t)(l + 1) * H : p_fnorm, H);
    stampit(12);
    // ---------------- gather the SwiGLU output, down projection + residual
    ok = gather_flat(sm, copy_of(x_h, HSLOTS, par), kAct32<WT> ? nunit : nunit / 2, tag + 4,
                     [&](int i, uint32_t p) {
                       // element e of rank r lives at hbuf element r * inner + e: the same flat index
                       if constexpr (kAct32<WT>) {
                         act_put<WT>(sm.u.mlp.hbuf, i, __uint_as_float(p));
                       } else {
                         act_put2_bits<WT>(sm.u.mlp.hbuf, 2 * i, p);
                       }
                     },
                     wt);
    if (!ok) break;
    act_sums<WT>(sm.u.mlp.hbuf, sm.u.mlp.asumH, nunit);
    __syncthreads();
    stampit(13);
    if (dense) {
      const auto ar = act_regs<WT, CP_DN>(gdn, sm.u.mlp.hbuf, sm.u.mlp.asumH);
      gemv_auto<WT, CP_DN, NI_DND, DN_CAP>(lstage(sm.u.mlp.dn), gdn, true, ar, dn_rowfn,
                                           [&](int q, float v) { sm.ytmp[q] = v; });
    } else {
      auto out = [&](int q, float v) { sm.ytmp[q] = v; };
      if constexpr (NI_DNM > 0 && NI_DNM <= DN_CAP) {
        wait_vmem();
        if constexpr (MFMA_QK) {
          if (l + 1 < L && attn && t0 < t1) {
            issue_qkv(l + 1);
            const size_t cb = (((size_t)(l + 1) * B + seq) * nkv + aj) * kvstride * ebytes;
            k_issue_mfma<true>(sm.u.att.kbuf, kc + cb, t0, min(CHP, t1 - t0));
            front_early = true;
          }
        }
        compute_static_rows<WT, NI_DNM, NI_DNM % 3 == 0 ? 3 : 1>(lstage(sm.u.mlp.dn), gdn, dn_rowfn_x,
                                                                 [&](int rp, float v) {
                                                                   const int k = rp / R8;
                                                                   sm.ytmp[(rp - k * R8) * K + k] = v;
                                                                 });
      } else {
        const ActRegs<WT, 0> none{};
        gemv_lds<WT, 0>(lstage(sm.u.mlp.dn), gdn, true, none, dn_rowfn, out);
      }
    }
    __syncthreads();
    publish(x_res2, H, par, dre - drb, tag + 5, [&](int q, int& idx) {
      idx = drb + q;
      float y;
      if (dense) {
        y = sm.ytmp[q];
      } else {
        y = 0.f;
        for (int k = 0; k < K; ++k) y = fmaf(sm.wsel[k], sm.ytmp[q * K + k], y);
      }
      return __float_as_uint(sm.xres[drb + q] + y);
    });
    // the shared region is free: the next layer's QKV weights load during the exchange; its first
    // attention chunk after it (the exchange's loads would otherwise return only after the chunk)
    if (l + 1 < L) {
      if (!front_early) issue_qkv(l + 1);
      issue_kv_front(l + 1, !front_early, true);
    }
    stampit(14);
    float ss2 = 0.f;  // likewise for the next input norm (or the final norm)
    ok = gather_flat(
        sm, copy_of(x_res2, H, par), H, tag + 5,
        [&](int i, uint32_t p) {
          const float v = __uint_as_float(p);
          sm.xres[i] = v;
          ss2 = fmaf(v, v, ss2);
        },
        wt,
        [&]() {
          ss2 = wave_sum(ss2);
          if (lane == 0) sm.wred[wave] = ss2;
        });
    if (!ok) break;
    stampit(15);
    if (d.dbg_resid && W == 0)
      for (int e = tid; e < H; e += NT) gp(d.dbg_resid)[(size_t)l * H + e] = sm.xres[e];
  }

  // ---------------- final norm (its weights are in sm.gn), lm_head, argmax
  {
    __syncthreads();
    rmsnorm_act<WT, HW, true>(sm, H, ks.eps, false);
    const int vb = ok ? part(V_, G, W) : 0, ve = ok ? part(V_, G, W + 1) : 0;
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    const Mat lmh{ks.lmhead, nullptr};
    float* const dbg_logits = d.dbg_logits;
    const Geo gl = geo<HW>(ve - vb, H);
    auto lm_rowfn = [&](int q) { return mrow<HW>(lmh, vb + q, H, sm.actA, nullptr); };
    // debug logits wait in LDS: a global store inside the streamed loop would upset its load count
    auto lm_out = [&](int q, float v) {
      const int r = vb + q;
      if (dbg_logits) {
        if (q < MAX_YROWS) sm.ytmp[q] = v;
        else gp(dbg_logits)[r] = v;
      }
      if (v > bv || (v == bv && r < bi)) {
        bv = v;
        bi = r;
      }
    };
    const auto ar = act_regs<HW, CP_LM>(gl, sm.actA, nullptr);
    static_assert(!SS || (SH::V % SH::G == 0 && ((SH::V / SH::G) / NW * CP_LM) % LM_CAP == 0 &&
                          (SH::H / kChunkElems<HW>) % 64 == 0),
                  "the streamed lm_head needs whole rows in every lane and whole rounds");
    if constexpr (CP_LM > 0)
      gemv_stream<HW, CP_LM, LM_CAP>(LStage{sm.u.head.a, nullptr, LM_CAP}, LStage{sm.u.head.b, nullptr, LM_CAP}, gl, ar,
                                     lm_rowfn, lm_out);
    else
      gemv_lds<HW, 0>(LStage{sm.u.head.a, nullptr, LM_CAP}, gl, false, ar, lm_rowfn, lm_out);
    if (dbg_logits) {
      __syncthreads();
      for (int q = tid; q < min(ve - vb, MAX_YROWS); q += NT) gp(dbg_logits)[vb + q] = sm.ytmp[q];
    }
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
      __hip_atomic_fetch_max(gp(p_amax), k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t prev = __hip_atomic_fetch_add(gp(p_done), 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_SYSTEM);
      if (prev == (uint32_t)G - 1) {  // last workgroup: publish the token, reset for the next launch
        const unsigned long long fin =
            __hip_atomic_exchange(gp(p_amax), 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(gp(p_done), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // a wait of this step gave up (some layers were not computed): the step leaves the length as it
        // was and writes -1 in place of an id; the host reports the error once and re-reads the lengths
        const bool failed = (__hip_atomic_load(gp(ks.err), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) & ERR_TIMEOUT) != 0;
        gp(d.out_ids)[d.out_idx] = failed ? -1 : (int32_t)(0xFFFFFFFFu - (uint32_t)(fin & 0xFFFFFFFFull));
        if (!failed) gp(d.len)[seq] = pos + 1;
        if (d.dbg_ts) gp(d.dbg_ts)[2] = now();
      }
    }
  }
  if (stamps) {
    stamps[1] = now();
    stamps[0] = t_start;
    stamps[3] = c_start;
    stamps[4] = __builtin_amdgcn_s_memtime();
    for (int l = 0; l < L && l < STAMP_LAYERS; ++l)
      for (int j = 0; j < 16; ++j) stamps[(size_t)(l + 1) * 16 + j] = t_start + sm.st_base[l] + sm.st[l][j];
  }
  wait_vmem();
}

// ---------------------------------------------------------------- the non-allocating entry point's scratch

// Exchange slots and argmax counters of flint_decode_step_noalloc, for callers that cannot allocate device
// memory: a fixed array in the library's device image (each GPU holds its own copy for the life of the
// process).  Host code never passes the array's name to a kernel (on the host it only stands for the
// symbol): its device address is looked up once per device and that address is passed.
static __device__ __align__(256) uint64_t scratch[NOALLOC_SCRATCH_WORDS];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_na_mutex;
uint64_t* g_na_ptr[MAX_DEVICES];
std::atomic<uint64_t> g_na_launches[MAX_DEVICES];
}  // namespace

hipError_t noalloc_scratch(int dev, hipStream_t stream, uint64_t** ptr) {
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_na_mutex);
  if (!g_na_ptr[dev]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    // every slot starts untagged and the argmax counters at zero
    e = launch_fill((uint64_t*)p, NOALLOC_SCRATCH_WORDS, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return e;
    g_na_ptr[dev] = (uint64_t*)p;
  }
  *ptr = g_na_ptr[dev];
  return hipSuccess;
}

uint64_t noalloc_next_launch(int dev) { return g_na_launches[dev].fetch_add(1); }

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

// Batched greedy decode for gfx950 (MI355X): up to 16 sequences per pass.
//
// The page "Flint Inference on Apple Silicon: rec Megakernel and Tempo9
// Compared" (section 4) sets per-token GEMVs, which suit one client, against
// tiled and grouped contractions once several clients decode together.  Here
// every weight tile is read once per pass and multiplied against all the
// sequences' activations on MFMA: v_mfma_f32_16x16x32_bf16 takes 16 weight
// rows x 32 inputs and 32 inputs x 16 sequences.  int4 weights are unpacked
// to bf16 in registers and each 64-input group's scale multiplies that
// group's fp32 products, so the arithmetic matches the dequantised weights.
//
// A pass is a sequence of ordinary kernels per layer, on one stream:
//   input norm -> QKV (RoPE, K/V append) -> attention splits over each
//   sequence's own length -> split merge -> o_proj -> post norm, router and
//   top-k -> gate/up of the selected experts (grouped by expert over the
//   union of the sequences' picks) -> down and combine.
// Kernels that would need a grid-wide sum (o_proj and down over input chunks
// or expert chunks) write partial sums that the next norm kernel adds to the
// residual, so no kernel waits for another workgroup.  The head's argmax uses
// packed (logit, id) atomic maxima per sequence; the last workgroup to finish
// publishes the ids and advances the lengths, as the persistent kernel does.

#include "flint_device.h"

namespace flint {
namespace {

constexpr int BNT = 512, BNW = BNT / 64;
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// Position of element e in a GEMM input row: int4 models store each group of
// 8 as (0, 4, 1, 5, 2, 6, 3, 7), the order in which a word of 8 codes unpacks.
template <int WT> __device__ __forceinline__ int act_pos(int e) {
  return WT == W_I4 ? (e & ~7) | ((e & 3) << 1) | ((e >> 2) & 1) : e;
}
__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }
// inputs per 1 KB chunk of a tile of the tiled weights
template <int WT> constexpr int kChunkIn = WT == W_I4 ? 128 : 32;
__device__ __forceinline__ f32x4_t mfma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 8 int4 codes (element i in bits 4i .. 4i + 3) as the bf16 values 128 + u, in the order (0, 4, 1, 5, 2, 6, 3, 7)
__device__ __forceinline__ bf16x8_t unpack8(uint32_t q, const I4K& k4) {
  return as_bf16x8(make_uint4((q & k4.m) | k4.mag, ((q >> 4) & k4.m) | k4.mag, ((q >> 8) & k4.m) | k4.mag,
                              ((q >> 12) & k4.m) | k4.mag));
}
__device__ __forceinline__ void latch(const BArgs& a, uint32_t bits) {
  __hip_atomic_fetch_or(gp(a.err), bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  __hip_atomic_store(gp(a.herr), bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Row of the matrix at row m (< 16) of tile T: rows in order, or, for the fused QKV rows of heads of rope_hd
// dims, 8 rotate-half pairs of one head (rows i0 + m and rope_hd/2 + i0 + m), so that a row and its RoPE
// partner meet in one MFMA result.
__host__ __device__ __forceinline__ long long tile_row(long long T, int m, int rope_hd) {
  if (rope_hd == 0) return T * 16 + m;
  const int tph = rope_hd / 16, half = rope_hd / 2, i0 = (int)(T % tph) * 8;
  return T / tph * rope_hd + (m < 8 ? i0 + m : half + i0 + m - 8);
}

// Tiled weights of the batched path: tile T (16 rows), chunk c, lane L hold, at ((T * C + c) * 64 + L) * 16,
// the 16 bytes that lane L feeds to the MFMAs of chunk c: row tile_row(T, L % 16), k-slice L / 16.
//   int4 (C = in / 128): inputs (2c + h) * 64 + (L / 16) * 16 + j * 8 + [0, 8) in dword 2h + j (h, j < 2);
//   bf16 (C = in / 32): inputs c * 32 + (L / 16) * 8 + [0, 8).
// A wave's load of one chunk of one tile is then 1 KB of contiguous memory.
template <int WT>
__global__ void tile_weights_kernel(const uint8_t* w, uint8_t* dst, size_t rows, int in, int rope_hd) {
  const int C = WT == W_I4 ? in / 128 : in / 32;
  const size_t total = rows / 16 * (size_t)C * 64;
  for (size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += (size_t)gridDim.x * blockDim.x) {
    const int L = (int)(u & 63), kg = L >> 4;
    const size_t tc = u >> 6, T = tc / C;
    const int c = (int)(tc - T * C);
    const long long r = tile_row((long long)T, L & 15, rope_hd);
    uint4 v;
    if constexpr (WT == W_I4) {
      const uint8_t* row = w + r * (in / 2);
      const uint32_t* pa = reinterpret_cast<const uint32_t*>(row + (2 * c) * 32 + kg * 8);
      const uint32_t* pb = reinterpret_cast<const uint32_t*>(row + (2 * c + 1) * 32 + kg * 8);
      v = make_uint4(gp(pa)[0], gp(pa)[1], gp(pb)[0], gp(pb)[1]);
    } else {
      v = ld16(w + (r * in + c * 32 + kg * 8) * 2);
    }
    *(GLOBAL u32x4_t*)(dst + u * 16) = u32x4_t{v.x, v.y, v.z, v.w};
  }
}

// One int4 chunk (128 inputs) of one tile: wv = this lane's 16 bytes of the tiled weights, sa / sb = the
// scales of its 4 rows for the chunk's two groups, b = this lane's inputs of the chunk.
__device__ __forceinline__ void i4_chunk(f32x4_t& acc, uint4 wv, u32x2_t sa, u32x2_t sb, const uint4 (&b)[4],
                                         const I4K& k4, bf16x8_t bias) {
  f32x4_t da = {0.f, 0.f, 0.f, 0.f}, db = {0.f, 0.f, 0.f, 0.f};
  da = mfma(unpack8(wv.x, k4), as_bf16x8(b[0]), da);
  da = mfma(unpack8(wv.y, k4), as_bf16x8(b[1]), da);
  da = mfma(bias, as_bf16x8(b[0]), da);
  da = mfma(bias, as_bf16x8(b[1]), da);
  db = mfma(unpack8(wv.z, k4), as_bf16x8(b[2]), db);
  db = mfma(unpack8(wv.w, k4), as_bf16x8(b[3]), db);
  db = mfma(bias, as_bf16x8(b[2]), db);
  db = mfma(bias, as_bf16x8(b[3]), db);
  acc[0] = fmaf(bf2f(sa.x & 0xFFFFu), da[0], fmaf(bf2f(sb.x & 0xFFFFu), db[0], acc[0]));
  acc[1] = fmaf(bf2f(sa.x >> 16), da[1], fmaf(bf2f(sb.x >> 16), db[1], acc[1]));
  acc[2] = fmaf(bf2f(sa.y & 0xFFFFu), da[2], fmaf(bf2f(sb.y & 0xFFFFu), db[2], acc[2]));
  acc[3] = fmaf(bf2f(sa.y >> 16), da[3], fmaf(bf2f(sb.y >> 16), db[3], acc[3]));
}
__device__ __forceinline__ bf16x8_t bias136() {  // bf16 -136 in every element
  return as_bf16x8(make_uint4(0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u));
}
// This lane's inputs of int4 chunk c (both groups, both 32-input halves), or zeros for a null column.
__device__ __forceinline__ void i4_inputs(uint4 (&b)[4], const uint16_t* col, int c, int kg) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    b[q] = col ? ld16(col + (2 * c + (q >> 1)) * 64 + kg * 16 + (q & 1) * 8) : make_uint4(0u, 0u, 0u, 0u);
}

// acc[t] += W[tile t] . x over the chunks [c0, c1) (int4: 128 inputs, bf16: 32) for 16 sequence columns,
// the input operand of a chunk loaded once for all NT tiles.  tile_of(t): the tile's index in m.wt;
// rowmap(t, m): its rows (for the int4 scales; rows rowmap(t, 4 k) .. + 3 are consecutive from a
// multiple of 4).  Lane L accumulates rows (L / 16) * 4 + r of column L % 16 (`col`: that sequence's
// input row, null for a zero column).  int4: codes enter as 128 + u, two MFMAs with the constant -136 as
// the weight operand remove the offset, then each row's group scale (four rows in one 8-byte load of the
// regrouped scales) multiplies the group's fp32 result.  Every load of U chunks is issued first.
template <int WT, int NT, int UF = 0, class TileOf, class RowMap>
__device__ __forceinline__ void mma_tiles(f32x4_t (&acc)[NT], const Mat& m, int in, TileOf tile_of, RowMap rowmap,
                                          const uint16_t* col, int c0, int c1) {
  const int lane = threadIdx.x & 63, kg = lane >> 4, G = in / 64;
  const int C = in / kChunkIn<WT>;
  const uint8_t* tp[NT];
  const uint16_t* s4[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    tp[t] = m.wt + ((size_t)tile_of(t) * C * 64 + lane) * 16;
    if constexpr (WT == W_I4) s4[t] = m.s4 + (size_t)(rowmap(t, 4 * kg) >> 2) * G * 4;
  }
  const I4K k4 = i4k();
  const bf16x8_t bias = bias136();
  constexpr int U = UF ? UF : (WT == W_I4 ? (NT >= 4 ? 2 : 4) : (NT >= 4 ? 4 : 8));
  constexpr int NB = WT == W_I4 ? 4 : 1;  // 16-byte input loads per chunk
  for (int c = c0; c < c1; c += U) {
    uint4 wv[U][NT], b[U][NB];
    u32x2_t sa[U][NT], sb[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c + u >= c1) break;
      const int cc = c + u;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        wv[u][t] = ld16(tp[t] + (size_t)cc * 1024);
        if constexpr (WT == W_I4) {
          sa[u][t] = *(GLOBAL const u32x2_t*)(s4[t] + (size_t)(2 * cc) * 4);
          sb[u][t] = *(GLOBAL const u32x2_t*)(s4[t] + (size_t)(2 * cc + 1) * 4);
        }
      }
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        const int e = WT == W_I4 ? (2 * cc + (q >> 1)) * 64 + kg * 16 + (q & 1) * 8 : cc * 32 + kg * 8;
        b[u][q] = col ? ld16(col + e) : make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c + u >= c1) break;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if constexpr (WT == W_I4) {
          i4_chunk(acc[t], wv[u][t], sa[u][t], sb[u][t], b[u], k4, bias);
        } else {
          acc[t] = mfma(as_bf16x8(wv[u][t]), as_bf16x8(b[u][0]), acc[t]);
        }
      }
    }
  }
}

// Sum of the workgroup's 8 wave tiles, returned in wave 0 (other waves get their own tile back).
__device__ __forceinline__ f32x4_t sum_waves(f32x4_t acc, f32x4_t* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  red[wave * 64 + lane] = acc;
  __syncthreads();
  if (wave == 0)
#pragma unroll
    for (int w = 1; w < BNW; ++w) acc += red[w * 64 + lane];
  return acc;
}

__device__ __forceinline__ float bsum(float v, float* wred) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) wred[wave] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < BNW; ++w) t += wred[w];
  return t;
}

enum { NORM_EMBED = 0, NORM_INPUT = 1, NORM_POST = 2, NORM_FINAL = 3 };

// Cache sequence and position of column n of the pass (decode: sequence cseq[n] at its length;
// prefill: sequence seq0 at its length + n); n may differ between lanes (selects over the kernel
// argument arrays, no loads).
__device__ __forceinline__ int col_seq(const BArgs& a, int n) {
  if (a.prefill) return a.seq0;
  int q = 0;
#pragma unroll
  for (int m = 0; m < BT; ++m) q = n == m ? a.cseq[m] : q;
  return q;
}
// Position of column n; n may differ between lanes (a select over the kernel argument array, no load).
__device__ __forceinline__ int col_pos(const BArgs& a, int n) {
  int p = 0;
#pragma unroll
  for (int m = 0; m < BT; ++m) p = n == m ? a.pos[m] : p;
  return p;
}

// Partial sums cross workgroups (and XCDs) through memory: written with system-scope stores, which go
// through the writer's L2, and read back with system-scope loads, which do not take a stale line from the
// reader's L2.
__device__ __forceinline__ void pstore(float* p, float v) {
  __hip_atomic_store(gp(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ float pload(const float* p) {
  return __hip_atomic_load(gp(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// The last of the NP workgroups that wrote partial sums for rows [r0, r0 + nr) adds them to the residual
// (in partial order, so the result does not depend on which workgroup is last) and re-arms the counter.
// Called by the whole workgroup after its partial rows are stored (pstore).
template <int NP>
__device__ __forceinline__ void fold_parts(const BArgs& a, const float* parts, uint32_t* cnt, int r0, int nr) {
  __shared__ int last;
  wait_vmem();  // this thread's partial stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(gp(cnt), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = prev == (uint32_t)NP - 1;
    if (last) __hip_atomic_store(gp(cnt), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!last) return;
  for (int idx = threadIdx.x; idx < nr * a.B; idx += BNT) {
    const int n = idx / nr, r = r0 + idx - n * nr;
    float v[NP + 1];
    v[0] = gp(a.x)[(size_t)n * a.H + r];
#pragma unroll
    for (int p = 0; p < NP; ++p) v[p + 1] = pload(parts + ((size_t)p * BT + n) * a.H + r);
    float t = v[0];
#pragma unroll
    for (int p = 0; p < NP; ++p) t += v[p + 1];
    gp(a.x)[(size_t)n * a.H + r] = t;
  }
}

// RMSNorm of one sequence's residual (grid: one workgroup per sequence); the normalised row becomes the
// next GEMM input.  NORM_POST of a MoE layer also computes the router logits and the top-k.
template <int WT>
__global__ void __launch_bounds__(BNT) bk_norm(const BArgs a, int l, int mode) {
  __shared__ __attribute__((aligned(16))) uint16_t an[MAX_H];
  __shared__ float z[MAX_E];
  __shared__ int rk[BNW][64];
  __shared__ float wred[BNW];
  const int n = blockIdx.x, seq = col_seq(a, n), tid = threadIdx.x, H = a.H;
  const int lane = tid & 63, wave = tid >> 6, E = a.E, lm = l - a.n_dense;
  float* xg = a.x + (size_t)n * H;
  // router rows of this wave (e = wave + 8 i; lanes over 16-byte chunks), loaded before the norm so that
  // their latency overlaps it
  constexpr int CE = WT == W_I4 ? 32 : 8;               // inputs per 16-byte chunk
  constexpr int RPW = MAX_E / BNW, CPL = (MAX_H / CE + 63) / 64;
  const int C = H / CE;
  const bool route = mode == NORM_POST && l >= a.n_dense;
  uint4 rw[RPW][CPL];
  uint32_t rs[RPW][CPL];  // int4: the 32-bit word holding the chunk's bf16 scale (groups 2k, 2k + 1)
  if (route) {  // no conditions around the loads (indices clamped), so all of them are in flight at once
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int e = min(wave + BNW * i, E - 1), c = min(lane + 64 * j, C - 1);
        rw[i][j] = ld16(a.router.w + ((long long)lm * E + e) * row_bytes<WT>(H) + 16ll * c);
        if constexpr (WT == W_I4)
          rs[i][j] = gp(reinterpret_cast<const uint32_t*>(a.router.s))[(((long long)lm * E + e) * (H / 64) + c / 2) >> 1];
      }
  }
  // the residual row (layer 0: the embedding row; later: complete, the last o_proj / down workgroup of each
  // row block having added the partial sums) and the norm weights, every load in flight at once
  constexpr int EPT = MAX_H / BNT;
  const float* g = mode == NORM_POST ? a.pnorm + (size_t)l * H : (mode == NORM_FINAL ? a.fnorm : a.anorm + (size_t)l * H);
  float xv[EPT], gv[EPT];
  if (mode == NORM_EMBED) {
    int tok = gp(a.tokens)[a.prefill ? a.tok0 + n : n];
    if (tok < 0 || tok >= a.V) {
      if (tid == 0) latch(a, ERR_TOKEN);
      tok = 0;
    }
    if (tid == 0) gp(a.hist)[(size_t)seq * a.cap + (a.prefill ? a.p0 + n : col_pos(a, n))] = tok;
    const uint16_t* er = reinterpret_cast<const uint16_t*>(a.embed) + (size_t)tok * H;
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const int e = tid + k * BNT;
      xv[k] = e < H ? bf2f(gp(er)[e]) : 0.f;
      gv[k] = e < H ? gp(g)[e] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < EPT; ++k)
      if (tid + k * BNT < H) gp(xg)[tid + k * BNT] = xv[k];
  } else {
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const int e = tid + k * BNT;
      xv[k] = e < H ? gp(xg)[e] : 0.f;
      gv[k] = e < H ? gp(g)[e] : 0.f;
    }
  }
  // the residual after layer l - 1 is complete at layer l's input norm (after the last layer: the final norm)
  if (a.dbg_resid && (mode == NORM_INPUT || mode == NORM_FINAL) && (mode == NORM_FINAL || l > 0)) {
    const int lr = mode == NORM_FINAL ? a.L - 1 : l - 1;
#pragma unroll
    for (int k = 0; k < EPT; ++k)
      if (tid + k * BNT < H) gp(a.dbg_resid)[((size_t)seq * a.L + lr) * H + tid + k * BNT] = xv[k];
  }
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < EPT; ++k) ss += xv[k] * xv[k];
  ss = bsum(ss, wred);
  const float inv = 1.0f / sqrtf(ss / (float)H + a.eps);
  uint16_t* ag = a.act + (size_t)n * a.astride;
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int e = tid + k * BNT;
    if (e >= H) break;
    const uint16_t v = (uint16_t)f2bf(xv[k] * inv * gv[k]);
    const int p = mode == NORM_FINAL ? e : act_pos<WT>(e);  // the lm_head is bf16: natural order
    an[p] = v;
    gp(ag)[p] = v;
  }
  if (mode != NORM_POST) return;
  if (l < a.n_dense) {  // dense layer: no routing
    if (a.dbg_z && tid < E) gp(a.dbg_z)[((size_t)seq * a.L + l) * E + tid] = 0.f;
    if (tid < a.K) {
      if (a.dbg_routes) gp(a.dbg_routes)[((size_t)seq * a.L + l) * a.K + tid] = -1;
      if (a.dbg_rw) gp(a.dbg_rw)[((size_t)seq * a.L + l) * a.K + tid] = 0.f;
    }
    return;
  }

  // router logits from the staged rows: each lane's activation chunks read once for all its rows
  __syncthreads();
  const I4K k4 = i4k();
  float racc[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) racc[i] = 0.f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = lane + 64 * j;
    if (c >= C) break;
    ActC<WT> x;
    if constexpr (WT == W_I4) {
      const uint4* p = reinterpret_cast<const uint4*>(an + 32 * c);
      x.a[0] = p[0];
      x.a[1] = p[1];
      x.a[2] = p[2];
      x.a[3] = p[3];
      x.s = chunk_sum(x.a[0], x.a[1], x.a[2], x.a[3]);
    } else {
      x.a[0] = *reinterpret_cast<const uint4*>(an + 8 * c);
      x.s = 0.f;
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i)
      racc[i] += chunk_dot<WT>(rw[i][j], x, WT == W_I4 ? bf2f(((c >> 1) & 1) ? rs[i][j] >> 16 : rs[i][j] & 0xFFFFu) : 1.f, k4);
  }
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const float v = wave_sum(racc[i]);
    const int e = wave + BNW * i;
    if (lane == 0 && e < E) z[e] = v;
  }
  __syncthreads();
  // top-k by rank (larger logit first, equal logits: lower index first): wave w counts the experts
  // 8 w .. 8 w + 7 that beat lane e's, the counts meet in LDS; weights: softmax over all experts
  const float zl = lane < E ? z[lane] : -INFINITY;
  if (a.dbg_z && wave == 0 && lane < E) gp(a.dbg_z)[((size_t)seq * a.L + l) * E + lane] = zl;
  {
    int part = 0;
#pragma unroll
    for (int jj = 0; jj < MAX_E / BNW; ++jj) {
      const int j = wave * (MAX_E / BNW) + jj;
      const float zj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(zl), j));
      part += j < E && (zj > zl || (zj == zl && j < lane));
    }
    rk[wave][lane] = part;
  }
  __syncthreads();
  if (wave != 0) return;
  int rank = 0;
#pragma unroll
  for (int w = 0; w < BNW; ++w) rank += rk[w][lane];
  const float zmax = wave_max(zl);
  const float pe = lane < E ? __expf(zl - zmax) : 0.f;
  const float w = pe / wave_sum(pe);
  const bool pick = lane < E && rank < a.K;
  const float wsum = wave_sum(pick ? w : 0.f);
  if (pick) {
    const float wr = a.renorm ? w / wsum : w;
    gp(a.sel)[n * a.K + rank] = lane;
    gp(a.wsel)[n * a.K + rank] = wr;
    if (a.dbg_routes) gp(a.dbg_routes)[((size_t)seq * a.L + l) * a.K + rank] = lane;
    if (a.dbg_rw) gp(a.dbg_rw)[((size_t)seq * a.L + l) * a.K + rank] = wr;
  }
}

// QKV rows, RoPE, K/V append.  Workgroup t: 8 rotate-half pairs of one head (rows i0 + m and
// hd/2 + i0 + m, m < 8), so a row and its RoPE partner sit in lanes L and L ^ 32 of the result.
template <int WT>
__global__ void __launch_bounds__(BNT) bk_qkv(const BArgs a, int l) {
  __shared__ f32x4_t red[BNW * 64];
  const int t = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hd = a.hd, half = hd / 2, tph = hd / 16;
  const int hh = t / tph, i0 = (t % tph) * 8;
  const int QR = (a.nq + 2 * a.nkv) * hd;
  auto rowmap = [&](int, int m) -> long long { return (long long)l * QR + hh * hd + (m < 8 ? i0 + m : half + i0 + m - 8); };
  const int C = a.H / kChunkIn<WT>, n = lane & 15, kg = lane >> 4;
  const uint16_t* col = n < a.B ? a.act + (size_t)n * a.astride : nullptr;
  f32x4_t acc[1] = {{0.f, 0.f, 0.f, 0.f}};
  auto tile_of = [&](int) -> long long { return (long long)l * (QR / 16) + t; };  // tiled with rope_hd = hd
  mma_tiles<WT, 1>(acc, a.qkv, a.H, tile_of, rowmap, col, part(C, BNW, wave), part(C, BNW, wave + 1));
  const f32x4_t sum = sum_waves(acc[0], red);
  if (wave != 0) return;
  float y[4] = {sum[0], sum[1], sum[2], sum[3]};
  const int pos = n < a.B ? col_pos(a, n) : 0;
  if (hh < a.nq + a.nkv) {  // RoPE on q and k heads: (y_i, y_{i + hd/2}) rotated by the angle of pair i
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = swap32(y[r]);
    if (n < a.B) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const f32x2_t cs = *(GLOBAL const f32x2_t*)(a.rope + (size_t)pos * half + i0 + 4 * (kg & 1) + r);
        y[r] = kg < 2 ? y[r] * cs.x - p[r] * cs.y : y[r] * cs.x + p[r] * cs.y;
      }
    }
  }
  if (n >= a.B) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * kg + r, d = m < 8 ? i0 + m : half + i0 + m - 8;
    if (hh < a.nq) {
      gp(a.q)[(size_t)n * a.nq * hd + hh * hd + d] = y[r];
    } else {
      const bool isk = hh < a.nq + a.nkv;
      const int j = isk ? hh - a.nq : hh - a.nq - a.nkv;
      const size_t off = ((((size_t)l * a.Bc + col_seq(a, n)) * a.nkv + j) * a.cap + pos) * hd + d;
      gp(reinterpret_cast<uint16_t*>(isk ? a.kc : a.vc))[off] = (uint16_t)f2bf(y[r]);
    }
  }
}

// Attention of the batched path: a workgroup of ATT_NW waves takes ATT_P cached positions of one (column,
// kv head); wave w takes the chunks of ATT_C positions w, w + ATT_NW, ... and keeps its own online softmax,
// with the K and V rows of a chunk loaded straight into registers one chunk ahead of the math, so the loop
// has no barrier.  One exchange through LDS at the end folds the waves into the split's partial.
constexpr int ATT_NW = 4, ATT_NT = ATT_NW * 64, ATT_K = ATT_P / (ATT_NW * ATT_C);  // chunks per wave
static_assert(ATT_C == 16 && ATT_K * ATT_NW * ATT_C == ATT_P, "attention split shape");

// Rows of one chunk: k[sk] is the A operand of v_mfma_f32_16x16x32_bf16 for dims sk * 32 .. + 32 (lane L:
// position c0 + L % 16, dims sk * 32 + (L / 16) * 8 .. + 8); v[r] holds dims (L % 16) * 8 .. + 8 of position
// c0 + (L / 16) * 4 + r, the position whose score lands in element r of lane L's score fragment.  Positions
// past tl re-read row tl.
struct AttChunk {
  uint4 k[4], v[4];
};
__device__ __forceinline__ void att_load(AttChunk& c, const uint8_t* kbase, const uint8_t* vbase, int c0, int tl,
                                         int lane) {
  const size_t pk = min(c0 + (lane & 15), tl);
#pragma unroll
  for (int sk = 0; sk < 4; ++sk) c.k[sk] = ld16(kbase + pk * 256 + sk * 64 + (lane >> 4) * 16);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const size_t pv = min(c0 + (lane >> 4) * 4 + r, tl);
    c.v[r] = ld16(vbase + pv * 256 + (lane & 15) * 16);
  }
}

// Attention of one split: kv head j of one column over cached positions [t0, t1) (t0 < t1) of the cache
// slice at kbase / vbase, for the Gq query heads at qcol (fp32, head-major): scores on MFMA (the query split
// into bf16 high and low parts), online softmax, P.V on the vector units.  Writes (m, l, o) of each query
// head to dst + h * hstep.
__device__ __forceinline__ void attn_split(const BArgs& a, const uint8_t* const kbase, const uint8_t* const vbase,
                                           const float* qcol, int t0, int t1, float* const dst, size_t hstep) {
  __shared__ __align__(16) float ow[ATT_NW][4][128];
  __shared__ float mw[ATT_NW][4], lw[ATT_NW][4];
  __shared__ uint4 qop[4][2][64];  // [dims / 32][high, low][lane]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tl = t1 - 1, hd = 128, Gq = a.nq / a.nkv;
  AttChunk buf[2];
  att_load(buf[0], kbase, vbase, t0 + wave * ATT_C, tl, lane);
  // the query as MFMA B operands (lane: head L % 16, dims (L / 16) * 8 ..), bf16 high and low parts, built by
  // wave 0 into LDS
  const int hcol = lane & 15, grp = lane >> 4;
  if (wave == 0) {
    const float* qp = qcol + (size_t)min(hcol, Gq - 1) * hd + grp * 8;
    const float qm = hcol < Gq ? 1.0f / sqrtf((float)hd) : 0.f;
#pragma unroll
    for (int sk = 0; sk < 4; ++sk) {
      const f32x4_t x0 = *(GLOBAL const f32x4_t*)(qp + sk * 32), x1 = *(GLOBAL const f32x4_t*)(qp + sk * 32 + 4);
      uint32_t hw[4], lw4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t hb[2], lb[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const float qv = (2 * e + u < 4 ? x0[2 * e + u] : x1[2 * e + u - 4]) * qm;
          hb[u] = f2bf(qv);
          lb[u] = f2bf(qv - bf2f(hb[u]));
        }
        hw[e] = hb[0] | hb[1] << 16;
        lw4[e] = lb[0] | lb[1] << 16;
      }
      qop[sk][0][lane] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      qop[sk][1][lane] = make_uint4(lw4[0], lw4[1], lw4[2], lw4[3]);
    }
  }
  __syncthreads();
  float m = -INFINITY, lsum = 0.f;  // running max and sum of head hcol
  float o[4][8];                    // head h, dims hcol * 8 + e, over this lane's positions
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
#pragma unroll
  for (int k = 0; k < ATT_K; ++k) {
    const int c0 = t0 + (k * ATT_NW + wave) * ATT_C;
    if (k + 1 < ATT_K) att_load(buf[(k + 1) & 1], kbase, vbase, c0 + ATT_NW * ATT_C, tl, lane);
    if (c0 < t1) {
      const AttChunk& c = buf[k & 1];
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};  // D[position][head]
#pragma unroll
      for (int sk = 0; sk < 4; ++sk) {
        acc = mfma(as_bf16x8(c.k[sk]), as_bf16x8(qop[sk][0][lane]), acc);
        acc = mfma(as_bf16x8(c.k[sk]), as_bf16x8(qop[sk][1][lane]), acc);
      }
      float sv[4], mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sv[r] = c0 + grp * 4 + r < t1 ? acc[r] : -INFINITY;
        mx = fmaxf(mx, sv[r]);
      }
      mx = fmaxf(mx, swap16(mx));
      mx = fmaxf(mx, swap32(mx));
      const float mn = fmaxf(m, mx);  // finite: position c0 is in range
      const float alpha = __expf(m - mn);
      float p[4], ps = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = __expf(sv[r] - mn);
        ps += p[r];
      }
      ps += swap16(ps);
      ps += swap32(ps);
      lsum = lsum * alpha + ps;
      m = mn;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float ah = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), h));
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] *= ah;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t w4[4] = {c.v[r].x, c.v[r].y, c.v[r].z, c.v[r].w};
        float vv[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vv[2 * e] = bf2f(w4[e] & 0xFFFFu);
          vv[2 * e + 1] = bf2f(w4[e] >> 16);
        }
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const float ph =
              __int_as_float(__builtin_amdgcn_ds_bpermute(((lane & 48) + h) * 4, __float_as_int(p[r])));
#pragma unroll
          for (int e = 0; e < 8; ++e) o[h][e] = fmaf(ph, vv[e], o[h][e]);
        }
      }
    }
  }
  // fold the four lane groups (their positions), then the waves
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[h][e] += swap16(o[h][e]);
      o[h][e] += swap32(o[h][e]);
    }
  if (lane < 16)
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      *reinterpret_cast<float4*>(&ow[wave][h][lane * 8]) = make_float4(o[h][0], o[h][1], o[h][2], o[h][3]);
      *reinterpret_cast<float4*>(&ow[wave][h][lane * 8 + 4]) = make_float4(o[h][4], o[h][5], o[h][6], o[h][7]);
    }
  if (lane < 4) {
    mw[wave][lane] = m;
    lw[wave][lane] = lsum;
  }
  __syncthreads();
  for (int idx = tid; idx < Gq * hd; idx += ATT_NT) {
    const int h = idx / hd, e = idx % hd;
    float M = mw[0][h];  // wave 0 always has position t0
#pragma unroll
    for (int w = 1; w < ATT_NW; ++w) M = fmaxf(M, mw[w][h]);
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < ATT_NW; ++w) t += __expf(mw[w][h] - M) * ow[w][h][e];
    gp(dst)[h * hstep + 2 + e] = t;
  }
  if (tid < Gq) {
    float M = mw[0][tid];
#pragma unroll
    for (int w = 1; w < ATT_NW; ++w) M = fmaxf(M, mw[w][tid]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < ATT_NW; ++w) L += __expf(mw[w][tid] - M) * lw[w][tid];
    gp(dst)[tid * hstep] = M;
    gp(dst)[tid * hstep + 1] = L;
  }
}

// Attention of (split s, kv head j, column n) over positions [s P, min(s P + P, pos + 1)) of the column's
// own cache (the new token's K/V already appended).  The grid holds only real splits: workgroup x is split
// x - asp[n] of column n.
__global__ void __launch_bounds__(ATT_NT) bk_attn(const BArgs a, int l) {
  const int j = blockIdx.y, hd = 128, Gq = a.nq / a.nkv;
  int n = 0;
  while (n + 1 < a.B && a.asp[n + 1] <= (int)blockIdx.x) ++n;
  const int s = blockIdx.x - a.asp[n];
  const int T = a.pos[n] + 1, t0 = s * ATT_P;  // t0 < T: the host counts ceil(T / P) splits
  const size_t cb = (((size_t)l * a.Bc + col_seq(a, n)) * a.nkv + j) * (size_t)a.cap * hd * 2;
  attn_split(a, a.kc + cb, a.vc + cb, a.q + (size_t)n * a.nq * hd + (size_t)j * Gq * hd, t0, min(t0 + ATT_P, T),
             a.part + (((size_t)n * a.nq + (size_t)j * Gq) * a.nsmax + s) * (hd + 2), (size_t)a.nsmax * (hd + 2));
}

// Merge of the ns splits at p (one query head of one column): o = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M)
// l_s, written in bf16 to out[act_pos(d)] (the o_proj input).  Thread d owns dim d; the splits are taken MB
// at a time with every load of a block (m, l and o of each split) issued before any is used, and the
// blocks are folded by the running-max rule.
template <int WT, int MB = 32>
__device__ __forceinline__ void merge_head(const float* p, int ns, int hd, uint16_t* out) {
  const int d = threadIdx.x;
  float M = -INFINITY, L = 0.f, O = 0.f;
  for (int s0 = 0; s0 < ns; s0 += MB) {
    float m[MB], lv[MB], o[MB];
#pragma unroll
    for (int u = 0; u < MB; ++u) {  // past the last split: re-read it with weight 0
      const float* q = p + (size_t)min(s0 + u, ns - 1) * (hd + 2);
      m[u] = gp(q)[0];
      lv[u] = gp(q)[1];
      o[u] = gp(q)[2 + d];
    }
    float mb = M;
#pragma unroll
    for (int u = 0; u < MB; ++u) mb = s0 + u < ns ? fmaxf(mb, m[u]) : mb;
    const float sc = __expf(M - mb);  // M = -inf on the first block: 0
    L *= sc;
    O *= sc;
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const float w = s0 + u < ns ? __expf(m[u] - mb) : 0.f;
      L = fmaf(w, lv[u], L);
      O = fmaf(w, o[u], O);
    }
    M = mb;
  }
  gp(out)[act_pos<WT>(d)] = (uint16_t)f2bf(O / L);
}
template <int WT>
__global__ void __launch_bounds__(128) bk_merge(const BArgs a) {
  const int h = blockIdx.x, n = blockIdx.y, hd = a.hd, ns = a.asp[n + 1] - a.asp[n];
  const float* p = a.part + ((size_t)n * a.nq + h) * a.nsmax * (hd + 2);
  uint16_t* out = a.act + (size_t)n * a.astride + h * hd;
  if (ns <= 16) merge_head<WT, 16>(p, ns, hd, out);  // shorter sequences: blocks of 16 splits (fewer padded loads)
  else merge_head<WT, 32>(p, ns, hd, out);
}

// o_proj rows t*16 .. t*16 + 15 over input chunk kc: partial sums, added to the residual by the next norm.
template <int WT>
__global__ void __launch_bounds__(BNT) bk_oproj(const BArgs a, int l) {
  __shared__ f32x4_t red[BNW * 64];
  const int t = blockIdx.x, kc = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int QD = a.nq * a.hd, C = QD / kChunkIn<WT>, cb = part(C, OKC, kc), ce = part(C, OKC, kc + 1);
  const int n = lane & 15, kg = lane >> 4;
  auto rowmap = [&](int, int m) -> long long { return (long long)l * a.H + t * 16 + m; };
  auto tile_of = [&](int) -> long long { return ((long long)l * a.H >> 4) + t; };
  const uint16_t* col = n < a.B ? a.act + (size_t)n * a.astride : nullptr;
  f32x4_t acc[1] = {{0.f, 0.f, 0.f, 0.f}};
  mma_tiles<WT, 1>(acc, a.o, QD, tile_of, rowmap, col, cb + part(ce - cb, BNW, wave), cb + part(ce - cb, BNW, wave + 1));
  const f32x4_t sum = sum_waves(acc[0], red);
  if (wave == 0 && n < a.B)
#pragma unroll
    for (int r = 0; r < 4; ++r) pstore(a.opart + ((size_t)kc * BT + n) * a.H + t * 16 + 4 * kg + r, sum[r]);
  fold_parts<OKC>(a, a.opart, a.cnt + t, t * 16, 16);
}

// One item of a 4-tile contraction: four 16-row tiles (rows row0 .. row0 + 63) x one input chunk (int4:
// 128 inputs, bf16: 32), this lane's inputs of its sequence column (zeroed at use when !use; the address
// stays valid either way) and the column's weight.  int4: s = the four rows' scales of the chunk's two
// groups, one 16-byte load (the regrouped scales hold 4 rows x 1 group in 8 bytes, groups in order).
template <int WT>
struct TileItem {
  static constexpr int NB = WT == W_I4 ? 4 : 1;
  uint4 w[4], s[4], b[NB];
  float wn;
  bool use;
};

// Issue every load of one item (chunk cc of the in-input rows row0 ..) with no conditions, so the loads of
// several items are in flight together.
template <int WT>
__device__ __forceinline__ void item_issue(TileItem<WT>& it, const Mat& m, int in, long long row0, int cc,
                                           const uint16_t* col, bool use, float wn, int kg, int lane) {
  const int C = in / kChunkIn<WT>, G = in / 64;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    it.w[q] = ld16(m.wt + ((size_t)((row0 >> 4) + q) * C * 64 + lane) * 16 + (size_t)cc * 1024);
    if constexpr (WT == W_I4) it.s[q] = ld16(m.s4 + (size_t)((row0 + q * 16 + 4 * kg) >> 2) * G * 4 + 8 * cc);
  }
#pragma unroll
  for (int q = 0; q < TileItem<WT>::NB; ++q) {
    const int x = WT == W_I4 ? (2 * cc + (q >> 1)) * 64 + kg * 16 + (q & 1) * 8 : cc * 32 + kg * 8;
    it.b[q] = ld16(col + x);
  }
  it.wn = wn;
  it.use = use;
}

// acc += the item's four tiles . inputs per sequence column; WEIGHTED: each column's product times wn.
template <int WT, bool WEIGHTED>
__device__ __forceinline__ void item_math(f32x4_t (&acc)[4], const TileItem<WT>& it, const I4K& k4, bf16x8_t bias) {
  uint4 b[TileItem<WT>::NB];
#pragma unroll
  for (int q = 0; q < TileItem<WT>::NB; ++q) b[q] = it.use ? it.b[q] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f32x4_t d = WEIGHTED ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc[q];
    if constexpr (WT == W_I4) {
      const uint4 sv = it.s[q];
      const u32x2_t sa = {sv.x, sv.y}, sb = {sv.z, sv.w};
      i4_chunk(d, it.w[q], sa, sb, b, k4, bias);
    } else {
      d = mfma(as_bf16x8(it.w[q]), as_bf16x8(b[0]), d);
    }
    if constexpr (WEIGHTED) {
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[q][r] = fmaf(it.wn, d[r], acc[q][r]);
    } else {
      acc[q] = d;
    }
  }
}

// Items k = 0 .. nk - 1 of this wave through a ring of D (3 or 4): item k + D - 1 is issued before the
// math of item k (past the last, the last again, so the loads carry no condition).  issue(it, k) loads
// item k, math(it, k) consumes it.
template <int WT, int D, class Issue, class Math>
__device__ __forceinline__ void item_ring(int nk, Issue issue, Math math) {
  static_assert(D == 3 || D == 4, "ring of 3 or 4 items");
  if (nk <= 0) return;
  auto clamp = [&](int k) { return k < nk ? k : nk - 1; };
  TileItem<WT> x[D];
#pragma unroll
  for (int i = 0; i < D - 1; ++i) issue(x[i], clamp(i));
  for (int k = 0;;) {
#pragma unroll
    for (int i = 0; i < D; ++i) {  // slot i holds item k; slot (i + D - 1) % D takes item k + D - 1
      issue(x[(i + D - 1) % D], clamp(k + D - 1));
      math(x[i], k);
      if (++k >= nk) return;
    }
  }
}

// Gate and up rows t*64 .. t*64 + 63 of expert e (dense layers: of the dense MLP) for the sequences that
// selected it, then SwiGLU into h[sequence][slot * expert_inter + row].  Every wave computes all eight
// 16-row tiles (gate 0-3, up 4-7) over its eighth of the inputs; the partial tiles meet in LDS.
template <int WT>
__global__ void __launch_bounds__(BNT) bk_gateup(const BArgs a, int l) {
  __shared__ f32x4_t red[BNW * 8 * 64];  // the waves' partial tiles [wave][tile][lane]
  __shared__ int slot[BT];
  const int t = blockIdx.x, e = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool dense = l < a.n_dense;
  if (tid < BT) slot[tid] = dense && tid < a.B ? 0 : -1;
  __syncthreads();
  if (!dense && tid < a.B * a.K && gp(a.sel)[tid] == e) slot[tid / a.K] = tid % a.K;  // one load per thread
  __syncthreads();
  bool any = false;
#pragma unroll
  for (int i = 0; i < BT; ++i) any |= slot[i] >= 0;
  if (!any) return;  // no sequence picked this expert
  const int n = lane & 15;
  const Mat& Mg = dense ? a.dg : a.eg;
  const Mat& Mu = dense ? a.du : a.eu;
  const long long base = dense ? (long long)l * a.DI : ((long long)(l - a.n_dense) * a.E + e) * a.EI;
  const uint16_t* col = slot[n] >= 0 ? a.act + (size_t)n * a.astride : nullptr;
  const int C = a.H / kChunkIn<WT>, c0 = part(C, BNW, wave), c1 = part(C, BNW, wave + 1);
  {
    f32x4_t acc[4];
    // gate tiles, then up tiles (same rows; the two matrices share the layout)
#pragma unroll
    for (int mat = 0; mat < 2; ++mat) {
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      auto rowmap = [&](int q, int m) -> long long { return base + t * 64 + q * 16 + m; };
      auto tile_of = [&](int q) -> long long { return (base >> 4) + t * 4 + q; };
      // one chunk per load round keeps the kernel within two workgroups per compute unit
      mma_tiles<WT, 4, 1>(acc, mat ? Mu : Mg, a.H, tile_of, rowmap, col, c0, c1);
#pragma unroll
      for (int q = 0; q < 4; ++q) red[(wave * 8 + mat * 4 + q) * 64 + lane] = acc[q];
    }
  }
  __syncthreads();
  const int inner = dense ? a.DI : a.EI;
  for (int idx = tid; idx < 64 * BT; idx += BNT) {
    const int q = idx >> 6, rr = idx & 63, sl = slot[q];
    if (sl < 0) continue;
    const int tile = rr >> 4, m = rr & 15, ln = (m >> 2) * 16 + q, r = m & 3;
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int w = 0; w < BNW; ++w) {
      g += red[(w * 8 + tile) * 64 + ln][r];
      u += red[(w * 8 + 4 + tile) * 64 + ln][r];
    }
    const int ei = sl * inner + t * 64 + rr;
    gp(a.h)[(size_t)q * a.hstride + act_pos<WT>(ei)] = (uint16_t)f2bf(g / (1.0f + __expf(-g)) * u);
  }
}

// Down rows t*64 .. t*64 + 63 (four 16-row tiles), partial sums of workgroup c, added to the residual by the
// last of the row block's workgroups (every workgroup writes its partial rows, zeros included).
// Dense (grid.y = DKC): the pairs of 64-input groups of input chunk c.  MoE (grid.y = DKM): the row block's
// items are (picked expert in index order, pair of input chunks); workgroup c takes items c, c + DKM, ...
// and its wave w every BNW-th of those, loading the next item while the MFMAs run on the current one; each
// product is weighted per sequence by its routing weight (zero for sequences that did not pick the expert).
constexpr int DN_RING = 3;  // items in flight per wave in the MoE down projection
template <int WT>
__global__ void __launch_bounds__(BNT) bk_down(const BArgs a, int l) {
  __shared__ f32x4_t red[BNW][4][64];
  __shared__ float wtab[MAX_E][BT];        // routing weight of (expert, sequence), 0: not picked
  __shared__ signed char stab[MAX_E][BT];  // slot of the expert in the sequence's top-k, -1: not picked
  __shared__ int elist[MAX_E];             // picked experts in index order
  __shared__ unsigned long long emask;
  const int t = blockIdx.x, c = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, kg = lane >> 4;
  const bool dense = l < a.n_dense;
  f32x4_t acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (dense) {
    // items of 256 inputs (int4: two chunks, bf16: eight)
    constexpr int IC = 256 / kChunkIn<WT>;
    const int NI = a.DI / 256, ib = part(NI, DKC, c), ie = part(NI, DKC, c + 1);
    auto rowmap = [&](int q, int m) -> long long { return (long long)l * a.H + t * 64 + q * 16 + m; };
    auto tile_of = [&](int q) -> long long { return ((long long)l * a.H >> 4) + t * 4 + q; };
    const uint16_t* col = n < a.B ? a.h + (size_t)n * a.hstride : nullptr;
    for (int i = ib + wave; i < ie; i += BNW) mma_tiles<WT, 4>(acc, a.dd, a.DI, tile_of, rowmap, col, i * IC, (i + 1) * IC);
  } else {
    if (tid == 0) emask = 0ull;
    for (int i = tid; i < MAX_E * BT; i += BNT) {
      (&wtab[0][0])[i] = 0.f;
      (&stab[0][0])[i] = -1;
    }
    __syncthreads();
    if (tid < a.B * a.K) {
      const int e = gp(a.sel)[tid], q = tid / a.K;
      stab[e][q] = (signed char)(tid - q * a.K);
      wtab[e][q] = gp(a.wsel)[tid];
      atomicOr(&emask, 1ull << e);
    }
    __syncthreads();
    const unsigned long long mk = emask;
    if (tid < MAX_E && ((mk >> tid) & 1ull)) elist[__builtin_popcountll(mk & ((1ull << tid) - 1ull))] = tid;
    __syncthreads();
    const int NI = a.EI / kChunkIn<WT>, total = __builtin_popcountll(mk) * NI, lm = l - a.n_dense;
    // this wave's items are c + DKM (w + BNW k)
    const int wu = __builtin_amdgcn_readfirstlane(wave), j0 = c + DKM * wu, jstep = DKM * BNW;
    const I4K k4 = i4k();
    const bf16x8_t bias = bias136();
    item_ring<WT, DN_RING>(
        j0 < total ? (total - j0 + jstep - 1) / jstep : 0,
        [&](TileItem<WT>& it, int k) {
          const int jj = j0 + k * jstep, r = jj / NI, e = elist[r], sl = stab[e][n];
          item_issue<WT>(it, a.ed, a.EI, ((long long)lm * a.E + e) * a.H + t * 64, jj - r * NI,
                         a.h + (size_t)n * a.hstride + (size_t)(sl > 0 ? sl : 0) * a.EI, sl >= 0, wtab[e][n], kg, lane);
        },
        [&](const TileItem<WT>& it, int) { item_math<WT, true>(acc, it, k4, bias); });
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) red[wave][q][lane] = acc[q];
  __syncthreads();
  // 64 rows x 16 sequences: thread -> (row, sequence)
  for (int idx = tid; idx < 64 * BT; idx += BNT) {
    const int q = idx >> 6, rr = idx & 63;
    if (q >= a.B) continue;
    const int tile = rr >> 4, m = rr & 15, ln = (m >> 2) * 16 + q, r = m & 3;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < BNW; ++w) v += red[w][tile][ln][r];
    pstore(a.dpart + ((size_t)c * BT + q) * a.H + t * 64 + rr, v);
  }
  if (dense) fold_parts<DKC>(a, a.dpart, a.cnt + a.H / 16 + t, t * 64, 64);
  else fold_parts<DKM>(a, a.dpart, a.cnt + a.H / 16 + t, t * 64, 64);
}

// lm_head (bf16) rows of this workgroup in 16-row tiles; wave w computes four tiles over half of the
// inputs (waves w and w + 4 share tiles), the halves meet in LDS.  Per sequence the largest logit (lowest
// id on ties) goes into a packed atomic maximum; the last workgroup publishes the ids.
__global__ void __launch_bounds__(BNT) bk_head(const BArgs a) {
  __shared__ f32x4_t red[BNW][4][64];
  __shared__ float bv_s[4][BT];
  __shared__ int bi_s[4][BT];
  const int W = blockIdx.x, G = gridDim.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, kg = lane >> 4, ntl = a.V / 16;
  const int tb = part(ntl, G, W), te = part(ntl, G, W + 1);
  const Mat lm{a.lmhead, nullptr, nullptr, a.lmt};
  const uint16_t* col = n < a.B ? a.act + (size_t)n * a.astride : nullptr;
  const int half = wave >> 2, grp = wave & 3, NC = a.H / kChunkIn<W_BF16>;
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int t0 = tb; t0 < te; t0 += 16) {  // 16 tiles per round: wave group grp takes tiles t0 + 4 grp .. + 3
    f32x4_t acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto tile_of = [&](int q) -> long long { return min(t0 + 4 * grp + q, te - 1); };
    auto rowmap = [&](int q, int m) -> long long { return tile_of(q) * 16 + m; };
    mma_tiles<W_BF16, 4>(acc, lm, a.H, tile_of, rowmap, col, half ? NC / 2 : 0, half ? NC : NC / 2);
    __syncthreads();  // the previous round's reads of red are done
#pragma unroll
    for (int q = 0; q < 4; ++q) red[wave][q][lane] = acc[q];
    __syncthreads();
    if (half == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int tl = t0 + 4 * grp + q;
        if (tl >= te) break;
        const f32x4_t v = acc[q] + red[wave + 4][q][lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = tl * 16 + 4 * kg + r;
          if (a.dbg_logits && n < a.B) gp(a.dbg_logits)[(size_t)col_seq(a, n) * a.V + row] = v[r];
          if (v[r] > bv || (v[r] == bv && row < bi)) {
            bv = v[r];
            bi = row;
          }
        }
      }
    }
  }
  if (half == 0) {
    // lanes n, n + 16, n + 32, n + 48 hold the same sequence
#define FLINT_BEST(MOVV, MOVI)              \
  {                                         \
    const float ov = MOVV;                  \
    const int oi = MOVI;                    \
    if (ov > bv || (ov == bv && oi < bi)) { \
      bv = ov;                              \
      bi = oi;                              \
    }                                       \
  }
    FLINT_BEST(swap16(bv), swap16i(bi))
    FLINT_BEST(swap32(bv), swap32i(bi))
#undef FLINT_BEST
    if (lane < BT) {
      bv_s[grp][lane] = bv;
      bi_s[grp][lane] = bi;
    }
  }
  __syncthreads();
  if (tid == 0) {
    for (int q = 0; q < a.B; ++q) {
      float v = -INFINITY;
      int id = 0x7FFFFFFF;
      for (int w = 0; w < 4; ++w)
        if (bv_s[w][q] > v || (bv_s[w][q] == v && bi_s[w][q] < id)) {
          v = bv_s[w][q];
          id = bi_s[w][q];
        }
      if (id == 0x7FFFFFFF) continue;  // no rows in this workgroup
      const uint32_t u = __float_as_uint(v);
      const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
      const unsigned long long key = ((unsigned long long)ord << 32) | (0xFFFFFFFFu - (uint32_t)id);
      __hip_atomic_fetch_max(gp(a.amax + q), key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const uint32_t prev = __hip_atomic_fetch_add(gp(a.done), 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == (uint32_t)G - 1) {  // last workgroup: publish the ids, advance the lengths, reset
      for (int q = 0; q < a.B; ++q) {
        const unsigned long long fin = __hip_atomic_exchange(gp(a.amax + q), 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int32_t id = (int32_t)(0xFFFFFFFFu - (uint32_t)(fin & 0xFFFFFFFFull));
        if (!a.prefill) {
          gp(a.out_ids)[q] = id;
          gp(a.len)[col_seq(a, q)] += 1;
        } else if (q == a.B - 1) {  // prefill: the id after the last prompt token of the pass
          gp(a.out_ids)[0] = id;
          gp(a.len)[a.seq0] += a.lenadd;
        }
      }
      __hip_atomic_store(gp(a.done), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Scales regrouped by four rows for the batched contractions.
__global__ void regroup_scales_kernel(const uint16_t* s, uint16_t* s4, size_t rows, int G) {
  const size_t total = rows * (size_t)G;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i / G, g = i - r * G;
    s4[((r >> 2) * G + g) * 4 + (r & 3)] = s[i];
  }
}

// ---------------------------------------------------------------- prefill of long chunks
// A chunk of n > BT prompt tokens of one sequence: the contractions run over 64 tokens per workgroup so
// that every weight byte loaded feeds 64 tokens; attention runs on MFMA per block of 16 tokens and split of
// cached positions, merged per token; the experts run on the tokens that picked them, grouped by expert.

constexpr int PF_T = 64;     // tokens per contraction workgroup
constexpr int PF_W = 8;      // its waves, each one 16-row weight tile against the 64 tokens
constexpr int PF_NT = PF_W * 64;
constexpr int PF_DI = 16 / PF_W;  // input loads (4 token rows of 256 bytes each) per wave and 128 inputs
constexpr int PF_SC = 2;     // 128-input halves per stage
constexpr int PF_PB = 512;   // columns per attention batch (bounds the partial-result buffer)
enum { PF_QKV = 0, PF_ADD = 1, PF_SWIGLU = 2, PF_DOWNG = 3 };

struct PfJob {
  Mat m, m2;           // weights; m2: the up matrix of a SwiGLU job (waves 2 and 3)
  long long tile0;     // first 16-row tile of the job's rows (grouped jobs: of expert 0 of the layer)
  long long etiles;    // grouped jobs: tiles per expert
  int K;               // inputs, a multiple of 128
  const uint16_t* A;   // input rows, bf16 in GEMM input order
  int lda;
  int M;               // input rows of an ungrouped job
  int grouped;         // 0: rows 0 .. M-1; 1: the token row of each list entry; 2: one input row per list entry
  int l;               // layer
  uint16_t* hout;      // SwiGLU output rows
  int ldh;
};

// Output tile (16 PF_W rows x 64 tokens) of one job.  Wave w owns weight tile w (SwiGLU: gate tiles in the
// first half of the waves, the matching up tiles in the second) and all four 16-token tiles; the tokens'
// inputs go to LDS 256 inputs per stage (two halves of 128; direct-to-LDS loads of 256 contiguous bytes per
// token row, spread over the waves), double-buffered against the MFMAs of the previous stage, and each
// wave's weight chunks and scales are loaded into registers one stage ahead.  int4: the codes are unpacked once per stage for the
// four token tiles; arithmetic as in the batched path (codes 128 + u, the constant -136 operand, the group
// scale on each group's fp32 result).
template <int WT, int EPI>
__global__ void __launch_bounds__(PF_NT) pf_gemm(const BArgs a, const PfJob j) {
  __shared__ uint4 abuf[2][PF_SC][PF_T * 16];  // [buffer][half][token][16-byte unit ^ (token & 15)] of 128 inputs
  __shared__ f32x4_t upx[PF_W / 2][4][64];  // SwiGLU: the up tiles' results
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 15, kg = lane >> 4;
  const int rb = blockIdx.x;
  int r0, r1, e = 0;  // input rows (list entries of grouped jobs) [r0, r1) of this token block
  if (j.grouped) {
    if ((int)blockIdx.y >= gp(a.nblk)[0]) return;
    const int32_t* bk = a.blk + 3 * blockIdx.y;
    e = gp(bk)[0];
    r0 = gp(bk)[1];
    r1 = min(r0 + PF_T, gp(bk)[2]);
  } else {
    r0 = blockIdx.y * PF_T;
    r1 = min(r0 + PF_T, j.M);
  }
  // load i of wave w brings token rows 4 (w PF_DI + i) .. + 3 of the block, 256 contiguous bytes each:
  // this lane's row 4 (w PF_DI + i) + L / 16 (rows past r1 repeat the last one), 16-byte unit L % 16
  const uint16_t* ap[PF_DI];
#pragma unroll
  for (int k = 0; k < PF_DI; ++k) {
    const int ri = min(r0 + 4 * (wave * PF_DI + k) + kg, r1 - 1);
    const int arow = j.grouped == 1 ? (gp(a.lst)[ri] >> 3) : ri;
    ap[k] = j.A + (size_t)arow * j.lda + (n ^ ((4 * (wave * PF_DI + k) + kg) & 15)) * 8;
  }
  constexpr bool SWI = EPI == PF_SWIGLU;
  constexpr int HW = PF_W / 2;  // SwiGLU: gate tiles in waves 0 .. HW - 1, up tiles in the others
  const Mat& M = SWI && wave >= HW ? j.m2 : j.m;
  const long long T = j.tile0 + (long long)e * j.etiles + (SWI ? rb * HW + wave % HW : rb * PF_W + wave);
  const int C = j.K / kChunkIn<WT>, S = j.K / 128, G = j.K / 64;
  const uint8_t* wp = M.wt + ((size_t)T * C * 64 + lane) * 16;
  const long long srow = EPI == PF_QKV ? tile_row(T, 4 * kg, a.hd) : T * 16 + 4 * kg;  // rows 4 kg .. + 3
  const uint16_t* sp = WT == W_I4 ? M.s4 + (size_t)(srow >> 2) * G * 4 : nullptr;
  constexpr int NW4 = WT == W_I4 ? 1 : 4;  // weight chunks per stage
  // stage s: halves PF_SC s + h of 128 inputs; a half past the last (K / 128 odd) re-reads the last one, so
  // that the loads carry no condition, and is not used
  const int NS = (S + PF_SC - 1) / PF_SC;
  auto half_of = [&](int s, int h) { return min(PF_SC * s + h, S - 1); };
  auto issue = [&](int s, uint4 (*buf)[PF_T * 16]) {
#pragma unroll
    for (int h = 0; h < PF_SC; ++h)
#pragma unroll
      for (int k = 0; k < PF_DI; ++k) dma16(ap[k] + (size_t)half_of(s, h) * 128, &buf[h][4 * (wave * PF_DI + k) * 16]);
  };
  // the MFMA input operand of token tile t, 32-input slice q: token 16 t + n, 16-byte unit
  // int4: (q / 2) * 8 + 2 kg + (q & 1) (groups of 64 in the code order); bf16: 4 q + kg
  auto bop = [&](const uint4* buf, int t, int q) -> bf16x8_t {
    const int u = WT == W_I4 ? (q >> 1) * 8 + 2 * kg + (q & 1) : 4 * q + kg;
    return as_bf16x8(buf[(16 * t + n) * 16 + (u ^ n)]);
  };
  uint4 wc[PF_SC][NW4], wn[PF_SC][NW4], sc[PF_SC], sn[PF_SC];
  auto wload = [&](int s, uint4 (&w)[PF_SC][NW4], uint4 (&sv)[PF_SC]) {
#pragma unroll
    for (int h = 0; h < PF_SC; ++h) {
      const int hs = half_of(s, h);
#pragma unroll
      for (int q = 0; q < NW4; ++q) w[h][q] = ld16(wp + (size_t)(NW4 * hs + q) * 1024);
      if constexpr (WT == W_I4) sv[h] = ld16(sp + (size_t)(2 * hs) * 4);
      else sv[h] = make_uint4(0u, 0u, 0u, 0u);
    }
  };
  f32x4_t acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const I4K k4 = i4k();
  const bf16x8_t bias = bias136();
  wload(0, wc, sc);
  issue(0, abuf[0]);
  for (int s = 0; s < NS; ++s) {
    int later = 0;
    if (s + 1 < NS) {
      wload(s + 1, wn, sn);
      issue(s + 1, abuf[(s + 1) & 1]);
      later = PF_SC * (NW4 + (WT == W_I4 ? 1 : 0) + PF_DI);
    }
    wait_vmem_dyn(later);  // stage s has landed (every wave's part of it, after the barrier)
    __syncthreads();
#pragma unroll
    for (int h = 0; h < PF_SC; ++h) {
    if (PF_SC * s + h >= S) break;  // the re-read half past the last
    const uint4* buf = abuf[s & 1][h];
    if constexpr (WT == W_I4) {
      const bf16x8_t c0 = unpack8(wc[h][0].x, k4), c1 = unpack8(wc[h][0].y, k4), c2 = unpack8(wc[h][0].z, k4),
                     c3 = unpack8(wc[h][0].w, k4);
      const uint4 sv = sc[h];
      const float sa[4] = {bf2f(sv.x & 0xFFFFu), bf2f(sv.x >> 16), bf2f(sv.y & 0xFFFFu), bf2f(sv.y >> 16)};
      const float sb[4] = {bf2f(sv.z & 0xFFFFu), bf2f(sv.z >> 16), bf2f(sv.w & 0xFFFFu), bf2f(sv.w >> 16)};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf16x8_t b0 = bop(buf, t, 0), b1 = bop(buf, t, 1), b2 = bop(buf, t, 2), b3 = bop(buf, t, 3);
        f32x4_t da = {0.f, 0.f, 0.f, 0.f}, db = {0.f, 0.f, 0.f, 0.f};
        da = mfma(bias, b0, da);
        da = mfma(bias, b1, da);
        db = mfma(bias, b2, db);
        db = mfma(bias, b3, db);
        da = mfma(c0, b0, da);
        da = mfma(c1, b1, da);
        db = mfma(c2, b2, db);
        db = mfma(c3, b3, db);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][r] = fmaf(sa[r], da[r], fmaf(sb[r], db[r], acc[t][r]));
      }
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[t] = mfma(as_bf16x8(wc[h][q]), bop(buf, t, q), acc[t]);
    }
    }
    __syncthreads();  // every wave is done with this buffer before stage s + 2 is loaded into it
#pragma unroll
    for (int h = 0; h < PF_SC; ++h) {
#pragma unroll
      for (int q = 0; q < NW4; ++q) wc[h][q] = wn[h][q];
      sc[h] = sn[h];
    }
  }
  // epilogue: lane holds rows 4 kg .. 4 kg + 3 of its tile for token n of each token tile
  if constexpr (EPI == PF_SWIGLU) {
    if (wave >= HW)
#pragma unroll
      for (int t = 0; t < 4; ++t) upx[wave - HW][t][lane] = acc[t];
    __syncthreads();
    if (wave >= HW) return;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int rr = r0 + t * 16 + n;
      if (rr >= r1) continue;
      const f32x4_t u = upx[wave][t][lane];
      uint16_t* hr = j.hout + (size_t)rr * j.ldh;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float g = acc[t][r];
        gp(hr)[act_pos<WT>(rb * 16 * HW + wave * 16 + 4 * kg + r)] = (uint16_t)f2bf(g / (1.0f + __expf(-g)) * u[r]);
      }
    }
  } else if constexpr (EPI == PF_ADD) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int rr = r0 + t * 16 + n;
      if (rr >= r1) continue;
      f32x4_t* xp = reinterpret_cast<f32x4_t*>(a.x + (size_t)rr * a.H + rb * 16 * PF_W + wave * 16 + 4 * kg);
      gp(xp)[0] = gp(xp)[0] + acc[t];
    }
  } else if constexpr (EPI == PF_DOWNG) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int rr = r0 + t * 16 + n;
      if (rr >= r1) continue;
      const int ent = gp(a.lst)[rr];
      f32x4_t* yp = reinterpret_cast<f32x4_t*>(a.y + ((size_t)(ent >> 3) * a.K + (ent & 7)) * a.H +
                                                rb * 16 * PF_W + wave * 16 + 4 * kg);
      gp(yp)[0] = acc[t];
    }
  } else {  // PF_QKV: RoPE on q and k heads (partner rows in lane ^ 32), q kept in fp32, K/V appended
    const int hd = a.hd, half = hd / 2, tph = hd / 16;
    const int tl = (int)(T - j.tile0), hh = tl / tph, i0 = (tl % tph) * 8;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int rr = min(r0 + t * 16 + n, r1 - 1), pos = a.p0 + rr;
      float y[4] = {acc[t][0], acc[t][1], acc[t][2], acc[t][3]};
      if (hh < a.nq + a.nkv) {
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pr[r] = swap32(y[r]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const f32x2_t cs = *(GLOBAL const f32x2_t*)(a.rope + (size_t)pos * half + i0 + 4 * (kg & 1) + r);
          y[r] = kg < 2 ? y[r] * cs.x - pr[r] * cs.y : y[r] * cs.x + pr[r] * cs.y;
        }
      }
      if (r0 + t * 16 + n >= r1) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * kg + r, d = m < 8 ? i0 + m : half + i0 + m - 8;
        if (hh < a.nq) {
          gp(a.q)[((size_t)rr * a.nq + hh) * hd + d] = y[r];
        } else {
          const bool isk = hh < a.nq + a.nkv;
          const int jh = isk ? hh - a.nq : hh - a.nq - a.nkv;
          const size_t off = ((((size_t)j.l * a.Bc + a.seq0) * a.nkv + jh) * a.cap + pos) * hd + d;
          gp(reinterpret_cast<uint16_t*>(isk ? a.kc : a.vc))[off] = (uint16_t)f2bf(y[r]);
        }
      }
    }
  }
}

// Expert e's entries (token << 3 | slot) in token order at the sum of the earlier experts' counts, and its
// blocks of up to 64 entries in the block table after the earlier experts' blocks.  Every workgroup copies
// the chunk's picks into LDS (one byte each) and counts all experts itself (LDS atomics: the counts do not
// depend on their order), so no other kernel precedes it; then each wave writes the entries of its quarter
// of the picks, after the earlier quarters' (two passes over LDS, no barrier inside them).
constexpr int PF_MAXNK = 4096 * MAX_K;  // picks of the largest chunk
__global__ void __launch_bounds__(256) pf_fill(const BArgs a, int n) {
  __shared__ uint8_t ssel[PF_MAXNK];
  __shared__ int cnt[MAX_E];
  __shared__ int wc[4];
  __shared__ int base[2];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nk = n * a.K;
  if (tid < MAX_E) cnt[tid] = 0;
  __syncthreads();
  for (int i0 = 0; i0 < nk; i0 += 256 * 8) {  // eight loads in flight per thread (clamped, unconditional)
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = gp(a.sel)[min(i0 + u * 256 + tid, nk - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * 256 + tid;
      if (i < nk) {
        ssel[i] = (uint8_t)v[u];
        atomicAdd(&cnt[v[u]], 1);
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    const int c = lane < a.E ? cnt[lane] : 0, nb = (c + PF_T - 1) / PF_T;
    const int off = (int)wave_sum(lane < e ? (float)c : 0.f), boff = (int)wave_sum(lane < e ? (float)nb : 0.f);
    const int tot = (int)wave_sum((float)nb);
    if (lane == 0) {
      base[0] = off;
      base[1] = boff;
      if (e == 0) gp(a.nblk)[0] = tot;
    }
    if (lane == e)
      for (int b = 0; b < nb; ++b) {
        gp(a.blk)[3 * (boff + b)] = e;
        gp(a.blk)[3 * (boff + b) + 1] = off + b * PF_T;
        gp(a.blk)[3 * (boff + b) + 2] = off + c;
      }
  }
  // wave w: picks [q0, q1); first its count, then its entries after the earlier waves'
  const int q = (nk + 3) / 4, q0 = min(wave * q, nk), q1 = min(q0 + q, nk);
  int mine = 0;
  for (int i0 = q0; i0 < q1; i0 += 64) {
    const int i = i0 + lane;
    mine += __popcll(__ballot(i < q1 && ssel[min(i, nk - 1)] == e));
  }
  if (lane == 0) wc[wave] = mine;
  __syncthreads();
  int pos = base[0];
  for (int w = 0; w < wave; ++w) pos += wc[w];
  for (int i0 = q0; i0 < q1; i0 += 64) {
    const int i = i0 + lane;
    const bool m = i < q1 && ssel[min(i, nk - 1)] == e;
    const unsigned long long bal = __ballot(m);
    if (m) gp(a.lst)[pos + __popcll(bal & ((1ull << lane) - 1ull))] = ((i / a.K) << 3) | (i % a.K);
    pos += __popcll(bal);
  }
}

// x[t] += sum over slots k (in order) of wsel[t][k] y[t][k].
__global__ void __launch_bounds__(256) pf_combine(const BArgs a) {
  const int t = blockIdx.x;
  for (int r = threadIdx.x * 4; r < a.H; r += 1024) {
    f32x4_t* xp = reinterpret_cast<f32x4_t*>(a.x + (size_t)t * a.H + r);
    f32x4_t v = gp(xp)[0];
    for (int k = 0; k < a.K; ++k)
      v += gp(a.wsel)[t * a.K + k] * gp(reinterpret_cast<const f32x4_t*>(a.y + ((size_t)t * a.K + k) * a.H + r))[0];
    gp(xp)[0] = v;
  }
}

// Prefill attention, flash style: workgroup (query block b of FA_Q tokens, key split s of P positions (a
// multiple of FA_KS, at least ATT_P), kv head j); wave w is query head j Gq + w over the block's tokens, in FA_SB sub-blocks of 16 whose
// dependency chains interleave and which share every K and V operand read.  Scores are computed
// transposed, S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (K as the A operand, the query's bf16 high and low
// parts as B), so that a lane holds 4 keys of one query row: the online softmax of a row stays in its lane
// group, and the probabilities are already the B operand of O^T += V^T P^T on v_mfma_f32_16x16x16_bf16
// (high and low parts again).  V^T comes from row-major V in LDS through the transposing LDS read
// (ds_read_b64_tr_b16); V's 16-byte units are XOR-swizzled by row so that those reads spread over the
// banks.  K and V go to LDS 64 keys at a time, double-buffered.  Writes the split's (m, l, o) per token and
// head; a token's splits past its own causal range are written but never merged.
constexpr int FA_SB = 2, FA_Q = 16 * FA_SB, FA_KS = 64;
typedef short s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4_t mfma16(s16x4_t a, s16x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__global__ void __launch_bounds__(256, 2) pf_fattn(const BArgs a, int l, int c0, int c1, int P) {
  __shared__ uint4 kl[2][FA_KS * 16];  // [chunk of 16 keys][dims / 32][lane]: the A operand of S^T
  __shared__ uint4 vl[2][FA_KS * 16];  // [key][16-byte unit ^ (key & 15)]
  const int b = blockIdx.x, s = blockIdx.y, j = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, i = lane & 15, g = lane >> 4;
  const int t0 = c0 + b * FA_Q, tq1 = min(t0 + FA_Q, c1);
  const int k0 = s * P, kend = a.p0 + tq1;  // keys [0, kend) are visible to some token of the block
  if (t0 >= c1 || k0 >= kend) return;
  const int k1 = min(k0 + P, kend), hd = 128, Gq = a.nq / a.nkv;
  const size_t cb = (((size_t)l * a.Bc + a.seq0) * a.nkv + j) * (size_t)a.cap * hd * 2;
  const uint8_t* const kb = a.kc + cb;
  const uint8_t* const vb = a.vc + cb;
  auto issue = [&](int ks, int buf) {  // keys [ks, ks + 64), past k1 re-reading k1 - 1: 8 loads per wave
#pragma unroll
    for (int q = wave; q < 16; q += 4) {
      const int c = q >> 2, sk = q & 3, key = min(ks + 16 * c + i, k1 - 1);
      dma16(kb + (size_t)key * 256 + sk * 64 + g * 16, &kl[buf][q * 64]);
    }
#pragma unroll
    for (int q = wave; q < 16; q += 4) {
      const int row = 4 * q + g, key = min(ks + row, k1 - 1);
      dma16(vb + (size_t)key * 256 + (i ^ (row & 15)) * 16, &vl[buf][q * 64]);
    }
  };
  issue(k0, 0);
  // this wave's query rows as B operands of S^T: sub-block sb is token t0 + 16 sb + i, dims 32 sk + 8 g .. + 8,
  // high and low parts
  const bool act = wave < Gq;
  const int head = j * Gq + min(wave, Gq - 1);
  const float qm = 1.0f / sqrtf((float)hd);
  bf16x8_t qh[FA_SB][4], ql[FA_SB][4];
  int qpos[FA_SB];
#pragma unroll
  for (int sb = 0; sb < FA_SB; ++sb) {
    const int tq = min(t0 + 16 * sb + i, tq1 - 1);
    qpos[sb] = a.p0 + t0 + 16 * sb + i;
    const float* qp = a.q + ((size_t)tq * a.nq + head) * hd + g * 8;
#pragma unroll
    for (int sk = 0; sk < 4; ++sk) {
      const f32x4_t x0 = *(GLOBAL const f32x4_t*)(qp + sk * 32), x1 = *(GLOBAL const f32x4_t*)(qp + sk * 32 + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float qv = (e < 4 ? x0[e] : x1[e - 4]) * qm;
        const uint32_t hb = f2bf(qv);
        qh[sb][sk][e] = __builtin_bit_cast(__bf16, (uint16_t)hb);
        ql[sb][sk][e] = __builtin_bit_cast(__bf16, (uint16_t)f2bf(qv - bf2f(hb)));
      }
    }
  }
  float m[FA_SB], lsum[FA_SB];  // of query row i of each sub-block
  f32x4_t o[FA_SB][8];          // O^T: dims 16 db + 4 g + r of query row i
#pragma unroll
  for (int sb = 0; sb < FA_SB; ++sb) {
    m[sb] = -INFINITY;
    lsum[sb] = 0.f;
#pragma unroll
    for (int db = 0; db < 8; ++db) o[sb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const int nst = (k1 - k0 + FA_KS - 1) / FA_KS;
  for (int st = 0; st < nst; ++st) {
    const int ks = k0 + st * FA_KS, buf = st & 1;
    int later = 0;
    if (st + 1 < nst) {
      issue(ks + FA_KS, buf ^ 1);
      later = 8;
    }
    wait_vmem_dyn(later);
    __syncthreads();
    if (act) {
      const uint8_t* vlb = reinterpret_cast<const uint8_t*>(vl[buf]);
      for (int c = 0; c < FA_KS / 16; ++c) {
        const int kc0 = ks + 16 * c;
        if (kc0 >= k1) break;
        f32x4_t sc[FA_SB];  // S^T: keys kc0 + 4 g + r, query row i
#pragma unroll
        for (int sb = 0; sb < FA_SB; ++sb) sc[sb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sk = 0; sk < 4; ++sk) {
          const bf16x8_t kop = as_bf16x8(kl[buf][(c * 4 + sk) * 64 + lane]);
#pragma unroll
          for (int sb = 0; sb < FA_SB; ++sb) {
            sc[sb] = mfma(kop, qh[sb][sk], sc[sb]);
            sc[sb] = mfma(kop, ql[sb][sk], sc[sb]);
          }
        }
        float alpha[FA_SB];
        s16x4_t ph[FA_SB], pl[FA_SB];
#pragma unroll
        for (int sb = 0; sb < FA_SB; ++sb) {
          float sv[4], mx = -INFINITY;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int kp = kc0 + 4 * g + r;
            sv[r] = kp < k1 && kp <= qpos[sb] ? sc[sb][r] : -INFINITY;
            mx = fmaxf(mx, sv[r]);
          }
          mx = fmaxf(mx, swap16(mx));
          mx = fmaxf(mx, swap32(mx));
          const float mn = fmaxf(m[sb], mx), mref = mn == -INFINITY ? 0.f : mn;
          alpha[sb] = __expf(m[sb] - mref);
          float p[4], ps = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            p[r] = __expf(sv[r] - mref);
            ps += p[r];
          }
          ps += swap16(ps);
          ps += swap32(ps);
          lsum[sb] = lsum[sb] * alpha[sb] + ps;
          m[sb] = mn;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t hb = f2bf(p[r]);
            ph[sb][r] = (short)hb;
            pl[sb][r] = (short)f2bf(p[r] - bf2f(hb));
          }
        }
        // V^T operand of dims 16 db .. + 16: this lane passes key row 16 c + 4 g + i / 4, dims 16 db + 4 (i & 3)
        const int row = 16 * c + 4 * g + (i >> 2);
#pragma unroll
        for (int sb = 0; sb < FA_SB; ++sb) {
          if (__builtin_amdgcn_ballot_w64(alpha[sb] != 1.0f)) {  // some row's running max moved (else x 1)
#pragma unroll
            for (int db = 0; db < 8; ++db) o[sb][db] *= alpha[sb];
          }
        }
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const int u = 2 * db + ((i & 3) >> 1);
          const s16x4_t vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4_t*)(vlb + row * 256 + ((u ^ (row & 15)) * 16) + (i & 1) * 8));
#pragma unroll
          for (int sb = 0; sb < FA_SB; ++sb) {
            o[sb][db] = mfma16(vt, ph[sb], o[sb][db]);
            o[sb][db] = mfma16(vt, pl[sb], o[sb][db]);
          }
        }
      }
    }
    __syncthreads();  // every wave is done with this buffer before it is refilled
  }
  if (!act) return;
#pragma unroll
  for (int sb = 0; sb < FA_SB; ++sb) {
    const int t = t0 + 16 * sb + i;
    if (t >= tq1) continue;
    float* dst = a.part + (((size_t)(t - c0) * a.nq + head) * a.nsmax + s) * (hd + 2);
#pragma unroll
    for (int db = 0; db < 8; ++db) *(GLOBAL f32x4_t*)(dst + 2 + 16 * db + 4 * g) = o[sb][db];
    if (g == 0) {
      gp(dst)[0] = m[sb];
      gp(dst)[1] = lsum[sb];
    }
  }
}
template <int WT, int MB>
__global__ void __launch_bounds__(128) pf_merge(const BArgs a, int c0, int P) {
  const int h = blockIdx.x, n = c0 + blockIdx.y, hd = a.hd;
  merge_head<WT, MB>(a.part + ((size_t)blockIdx.y * a.nq + h) * a.nsmax * (hd + 2), (a.p0 + n + P) / P, hd,
                 a.act + (size_t)n * a.astride + h * hd);
}

// Key split of a prefill attention call over keys [0, kmax) with `groups` (query block, kv head) pairs:
// about FA_SPLITS splits per pair (enough workgroups to fill the chip), never shorter than ATT_P keys (the
// split count the partial buffer is sized for) and in whole FA_KS stages.  Longer splits write and merge
// fewer partials.
constexpr int FA_WG = 512;
inline int fa_split(int kmax, int groups) {
  const int want = std::max(1, (FA_WG + groups - 1) / groups);
  const int p = (kmax + want - 1) / want;
  return std::max(ATT_P, (p + FA_KS - 1) / FA_KS * FA_KS);
}

template <int WT> hipError_t run_prefill(const BArgs& a0, int n, hipStream_t st) {
  BArgs a = a0;
  a.B = n;
  a.prefill = 1;
  a.tok0 = 0;
  const int QR = (a.nq + 2 * a.nkv) * a.hd, QD = a.nq * a.hd, TB = (n + PF_T - 1) / PF_T;
  const int NBM = (n * a.K + PF_T - 1) / PF_T + a.E;
  const Mat none{};
  for (int l = 0; l < a.L; ++l) {
    hipLaunchKernelGGL(bk_norm<WT>, dim3(n), dim3(BNT), 0, st, a, l, l == 0 ? (int)NORM_EMBED : (int)NORM_INPUT);
    const PfJob jq{a.qkv, none, (long long)l * (QR / 16), 0, a.H, a.act, a.astride, n, 0, l, nullptr, 0};
    hipLaunchKernelGGL((pf_gemm<WT, PF_QKV>), dim3(QR / (16 * PF_W), TB), dim3(PF_NT), 0, st, a, jq);
    for (int c0 = 0; c0 < n; c0 += PF_PB) {
      const int c1 = std::min(n, c0 + PF_PB);
      const int nb = (c1 - c0 + FA_Q - 1) / FA_Q, P = fa_split(a.p0 + c1, nb * a.nkv);
      hipLaunchKernelGGL(pf_fattn, dim3(nb, (a.p0 + c1 + P - 1) / P, a.nkv), dim3(256), 0, st, a, l, c0, c1, P);
      if ((a.p0 + c1 + P - 1) / P <= 8)  // splits merged 8 at a time (every load of a block is issued at once)
        hipLaunchKernelGGL((pf_merge<WT, 8>), dim3(a.nq, c1 - c0), dim3(a.hd), 0, st, a, c0, P);
      else
        hipLaunchKernelGGL((pf_merge<WT, 32>), dim3(a.nq, c1 - c0), dim3(a.hd), 0, st, a, c0, P);
    }
    const PfJob jo{a.o, none, (long long)l * (a.H / 16), 0, QD, a.act, a.astride, n, 0, l, nullptr, 0};
    hipLaunchKernelGGL((pf_gemm<WT, PF_ADD>), dim3(a.H / (16 * PF_W), TB), dim3(PF_NT), 0, st, a, jo);
    hipLaunchKernelGGL(bk_norm<WT>, dim3(n), dim3(BNT), 0, st, a, l, (int)NORM_POST);
    if (l < a.n_dense) {
      const PfJob jg{a.dg, a.du, (long long)l * (a.DI / 16), 0, a.H, a.act, a.astride, n, 0, l, a.h, a.DI};
      hipLaunchKernelGGL((pf_gemm<WT, PF_SWIGLU>), dim3(a.DI / (8 * PF_W), TB), dim3(PF_NT), 0, st, a, jg);
      const PfJob jd{a.dd, none, (long long)l * (a.H / 16), 0, a.DI, a.h, a.DI, n, 0, l, nullptr, 0};
      hipLaunchKernelGGL((pf_gemm<WT, PF_ADD>), dim3(a.H / (16 * PF_W), TB), dim3(PF_NT), 0, st, a, jd);
    } else {
      const long long lm = l - a.n_dense;
      hipLaunchKernelGGL(pf_fill, dim3(a.E), dim3(256), 0, st, a, n);
      const PfJob jg{a.eg, a.eu, lm * a.E * (a.EI / 16), a.EI / 16, a.H, a.act, a.astride, 0, 1, l, a.h, a.EI};
      hipLaunchKernelGGL((pf_gemm<WT, PF_SWIGLU>), dim3(a.EI / (8 * PF_W), NBM), dim3(PF_NT), 0, st, a, jg);
      const PfJob jd{a.ed, none, lm * a.E * (a.H / 16), a.H / 16, a.EI, a.h, a.EI, 0, 2, l, nullptr, 0};
      hipLaunchKernelGGL((pf_gemm<WT, PF_DOWNG>), dim3(a.H / (16 * PF_W), NBM), dim3(PF_NT), 0, st, a, jd);
      hipLaunchKernelGGL(pf_combine, dim3(n), dim3(256), 0, st, a);
    }
  }
  // the last token: final norm, lm_head, argmax; the length advances by n
  BArgs f = a;
  f.B = 1;
  f.x = a.x + (size_t)(n - 1) * a.H;
  f.lenadd = n;
  hipLaunchKernelGGL(bk_norm<WT>, dim3(1), dim3(BNT), 0, st, f, a.L, (int)NORM_FINAL);
  hipLaunchKernelGGL(bk_head, dim3(std::min(256, a.V / 16)), dim3(BNT), 0, st, f);
  return hipGetLastError();
}

template <int WT> hipError_t run_pass(const BArgs& a, hipStream_t st) {
  const int QR = (a.nq + 2 * a.nkv) * a.hd;
  for (int l = 0; l < a.L; ++l) {
    hipLaunchKernelGGL(bk_norm<WT>, dim3(a.B), dim3(BNT), 0, st, a, l, l == 0 ? (int)NORM_EMBED : (int)NORM_INPUT);
    hipLaunchKernelGGL(bk_qkv<WT>, dim3(QR / 16), dim3(BNT), 0, st, a, l);
    hipLaunchKernelGGL(bk_attn, dim3(a.asp[a.B], a.nkv), dim3(ATT_NT), 0, st, a, l);
    hipLaunchKernelGGL(bk_merge<WT>, dim3(a.nq, a.B), dim3(a.hd), 0, st, a);
    hipLaunchKernelGGL(bk_oproj<WT>, dim3(a.H / 16, OKC), dim3(BNT), 0, st, a, l);
    hipLaunchKernelGGL(bk_norm<WT>, dim3(a.B), dim3(BNT), 0, st, a, l, (int)NORM_POST);
    const bool dense = l < a.n_dense;
    hipLaunchKernelGGL(bk_gateup<WT>, dense ? dim3(a.DI / 64, 1) : dim3(a.EI / 64, a.E), dim3(BNT), 0, st, a, l);
    hipLaunchKernelGGL(bk_down<WT>, dim3(a.H / 64, dense ? DKC : DKM), dim3(BNT), 0, st, a, l);
  }
  hipLaunchKernelGGL(bk_norm<WT>, dim3(a.B), dim3(BNT), 0, st, a, a.L, (int)NORM_FINAL);
  hipLaunchKernelGGL(bk_head, dim3(std::min(256, a.V / 16)), dim3(BNT), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_batch_pass(int wt, const BArgs& a, hipStream_t stream) {
  return wt == W_I4 ? run_pass<W_I4>(a, stream) : run_pass<W_BF16>(a, stream);
}

hipError_t launch_prefill(int wt, const BArgs& a, int n, hipStream_t stream) {
  return wt == W_I4 ? run_prefill<W_I4>(a, n, stream) : run_prefill<W_BF16>(a, n, stream);
}

size_t prefill_part_floats(int nq, int nsmax, int hd) { return (size_t)PF_PB * nq * nsmax * (hd + 2); }

hipError_t launch_tile_weights(int wt, const uint8_t* w, uint8_t* dst, size_t rows, int in, int rope_hd,
                               hipStream_t stream) {
  const size_t units = rows / 16 * (size_t)(wt == W_I4 ? in / 128 : in / 32) * 64;
  const int blocks = (int)std::min<size_t>((units + 255) / 256, 65536);
  if (wt == W_I4)
    hipLaunchKernelGGL(tile_weights_kernel<W_I4>, dim3(blocks), dim3(256), 0, stream, w, dst, rows, in, rope_hd);
  else
    hipLaunchKernelGGL(tile_weights_kernel<W_BF16>, dim3(blocks), dim3(256), 0, stream, w, dst, rows, in, rope_hd);
  return hipGetLastError();
}

hipError_t launch_regroup_scales(const uint16_t* s, uint16_t* s4, size_t rows, int G, hipStream_t stream) {
  const size_t total = rows * (size_t)G;
  const int blocks = (int)std::min<size_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(regroup_scales_kernel, dim3(blocks), dim3(256), 0, stream, s, s4, rows, G);
  return hipGetLastError();
}

}  // namespace flint

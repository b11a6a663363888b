// Device helpers shared by the kernels of the library (gfx950): scalar
// conversions, memory-scope accesses, wait counters, direct-to-LDS DMA and
// wave-level reductions.
#pragma once
#include "flint_internal.h"

namespace flint {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((address_space(3))) void lds_void;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// Every device pointer the kernel dereferences is cast to the global address
// space: generic (flat) accesses would also count against the LDS wait counter.
#define GLOBAL __attribute__((address_space(1)))
template <class T> __device__ __forceinline__ GLOBAL T* gp(T* p) { return (GLOBAL T*)p; }
// 16 bytes from global memory into registers.
__device__ __forceinline__ uint4 ld16(const void* p) {
  const u32x4_t v = *(GLOBAL const u32x4_t*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}

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
  return __hip_atomic_load(gp(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void xstore(uint64_t* p, uint64_t v) {
  __hip_atomic_store(gp(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
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
// s_waitcnt vmcnt(N): all but this wave's N most recent vector memory operations have completed
// (also a compiler barrier: LDS reads of bytes that requests out of the compiler's sight wrote stay after it)
template <int N> __device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_vmem() { wait_vmem_n<0>(); }
// vmcnt(n) for a run-time n (waits for everything when n is outside 0..15)
__device__ __forceinline__ void wait_vmem_dyn(int n) {
  switch (n) {
    case 1: wait_vmem_n<1>(); break;
    case 2: wait_vmem_n<2>(); break;
    case 3: wait_vmem_n<3>(); break;
    case 4: wait_vmem_n<4>(); break;
    case 5: wait_vmem_n<5>(); break;
    case 6: wait_vmem_n<6>(); break;
    case 7: wait_vmem_n<7>(); break;
    case 8: wait_vmem_n<8>(); break;
    case 9: wait_vmem_n<9>(); break;
    case 10: wait_vmem_n<10>(); break;
    case 11: wait_vmem_n<11>(); break;
    case 12: wait_vmem_n<12>(); break;
    case 13: wait_vmem_n<13>(); break;
    case 14: wait_vmem_n<14>(); break;
    case 15: wait_vmem_n<15>(); break;
    default: wait_vmem_n<0>(); break;
  }
}
// wait until this wave's LDS operations have completed (lgkmcnt(0))
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }
__device__ __forceinline__ void dma16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)l, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, void* l) { __builtin_amdgcn_global_load_lds(g, (lds_void*)l, 4, 0, 0); }
// The same 16-byte request written as inline assembly, so that the compiler does not see it: the compiler
// cannot tell which LDS a request writes, and after one it makes every later LDS access wait for all
// outstanding requests.  The caller waits for this one itself (vmcnt) before anything reads its bytes.
// M0 (the LDS address) is an input the compiler sets; one wait state separates that write from the request.
// LDS byte address of a generic pointer into LDS: its low 32 bits (the shared aperture sits above them)
__device__ __forceinline__ uint32_t lds_offset(const void* l) { return (uint32_t)(uintptr_t)l; }
__device__ __forceinline__ void dma16_untracked(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "{m0}"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}
__device__ __forceinline__ void dma4_untracked(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" : : "v"(g), "{m0}"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}

template <int WT> constexpr bool kAct32 = (WT == W_F32);
template <int WT> constexpr int kChunkElems = WT == W_F32 ? 4 : (WT == W_BF16 ? 8 : 32);
template <int WT> __device__ __forceinline__ long long row_bytes(int in) {
  return WT == W_F32 ? 4ll * in : (WT == W_BF16 ? 2ll * in : in / 2);
}
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
// int4 unpack constants held in VGPRs: with them in registers one v_and_or_b32
// turns a shifted word into two bf16 values (a VOP3 operand cannot be a literal).
struct I4K {
  uint32_t m, mag;
};
__device__ __forceinline__ I4K i4k() {
  I4K k;
  asm volatile("v_mov_b32 %0, 0xf000f" : "=v"(k.m));
  asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(k.mag));
  return k;
}


// ---------------------------------------------------------------- int4 / bf16 chunk dot products

// Sum of the 32 bf16 values of an int4 activation chunk (one fixed order).
__device__ __forceinline__ float chunk_sum(uint4 x0, uint4 x1, uint4 x2, uint4 x3) {
  const uint32_t w[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                          x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int k = 0; k < 16; k += 2) {
    s0 += bf2f(w[k] & 0xFFFFu) + bf2f(w[k] >> 16);
    s1 += bf2f(w[k + 1] & 0xFFFFu) + bf2f(w[k + 1] >> 16);
  }
  return s0 + s1;
}

// One lane's activation chunk: 4 fp32, 8 bf16 or (int4 weights) 32 bf16 and their sum.
template <int WT> struct ActC {
  uint4 a[WT == W_I4 ? 4 : 1];
  float s;
};

// Dot product of one 16-byte weight chunk with the matching activation chunk.
template <int WT>
__device__ __forceinline__ float chunk_dot(uint4 w, const ActC<WT>& x, float scale, const I4K& k4) {
  if constexpr (WT == W_F32) {
    const uint4 a = x.a[0];
    float acc = __uint_as_float(w.x) * __uint_as_float(a.x);
    acc = fmaf(__uint_as_float(w.y), __uint_as_float(a.y), acc);
    acc = fmaf(__uint_as_float(w.z), __uint_as_float(a.z), acc);
    return fmaf(__uint_as_float(w.w), __uint_as_float(a.w), acc);
  } else if constexpr (WT == W_BF16) {
    const uint4 a = x.a[0];
    float acc = dot2(w.x, a.x, 0.f);
    acc = dot2(w.y, a.y, acc);
    acc = dot2(w.z, a.z, acc);
    return dot2(w.w, a.w, acc);
  } else {
    // nibble n of a word becomes bf16 (128 + n) via 0x4300 | n; the chunk sum
    // of the activation removes the 128 + 8 offset: sum (u - 8) a = sum (128 + u) a - 136 sum a
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint4 a = x.a[k];
      const uint32_t q = ww[k];
      a0 = dot2((q & k4.m) | k4.mag, a.x, a0);
      a1 = dot2(((q >> 4) & k4.m) | k4.mag, a.y, a1);
      a0 = dot2(((q >> 8) & k4.m) | k4.mag, a.z, a0);
      a1 = dot2(((q >> 12) & k4.m) | k4.mag, a.w, a1);
    }
    return scale * ((a0 + a1) - 136.0f * x.s);
  }
}

// ---------------------------------------------------------------- attention data

// Rows [c0, c0 + np) of one (layer, sequence, kv head) cache slice into LDS,
// 1 KB per wave instruction; lanes past the end re-read the last 16 bytes.
__device__ __forceinline__ void kv_issue(uint4* buf, const uint8_t* base, int c0, int np, int rowb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint8_t* src = base + (size_t)c0 * rowb;
  const int units = np * rowb / 16;
  for (int gi = wave; gi * 64 < units; gi += NW) {
    const int unit = min(gi * 64 + lane, units - 1);
    dma16(src + (size_t)unit * 16, &buf[gi * 64]);
  }
}

// K rows [c0, c0 + np) (np <= 128) of one bf16 cache slice with head_dim 128,
// row-major in LDS (256 B per position) with the 16-byte units of position p
// XOR-swizzled by p % 16: unit u of row p sits at slot p * 16 + (u ^ (p % 16)).
// Each wave instruction reads 1 KB of contiguous cache (4 whole rows); the
// swizzle makes the MFMA operand reads (16 rows, one unit each) conflict-free.
// Rows past the end repeat the last one.
__device__ __forceinline__ int k_slot(int p, int u) { return p * 16 + (u ^ (p & 15)); }
template <bool UNTRACKED = false>
__device__ __forceinline__ void k_issue_mfma(uint4* buf, const uint8_t* base, int c0, int np) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ni = (np * 16 + 63) / 64;
  const uint32_t lb = lds_offset(buf);
  for (int gi = wave; gi < ni; gi += NW) {
    const int sl = gi * 64 + lane, p = sl >> 4, pr = min(p, np - 1);
    const int u = (sl & 15) ^ (p & 15);
    if constexpr (UNTRACKED) dma16_untracked(base + (size_t)(c0 + pr) * 256 + u * 16, lb + (uint32_t)gi * 1024u);
    else dma16(base + (size_t)(c0 + pr) * 256 + u * 16, &buf[gi * 64]);
  }
}

}  // namespace flint

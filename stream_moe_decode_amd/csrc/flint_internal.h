// Internal interface between the host runtime and the persistent decode kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flint {

constexpr int NT = 512;                 // threads per workgroup (8 waves of 64: two per SIMD)
constexpr int NW = NT / 64;             // waves per workgroup
constexpr int MAX_H = 2048;             // residual width
constexpr int MAX_QD = 2048;            // n_q_heads * head_dim
constexpr int MAX_HBUF = 6144;          // dense_inter, or top_k * expert_inter (bf16 elements; fp32: half)
constexpr int MAX_E = 64;               // experts (top-k runs inside one wave)
constexpr int MAX_K = 8;                // top_k
constexpr int MAX_GQ = 8;               // query heads per kv head
constexpr int MAX_HD = 128;             // head_dim
constexpr int MAX_YROWS = 1024;         // GEMV results a workgroup keeps per phase
constexpr int MAX_QPAIRS = 64;          // RoPE pairs of the QKV rows one workgroup owns
constexpr int MAX_GATHER = 4096;        // 32-bit words of the merge gather buffer
constexpr int KV_LDS = 32768;           // bytes of K (and of V) rows per attention chunk
constexpr int MAX_CHUNK_POS = KV_LDS / 128;  // positions per chunk for the smallest row (64 bf16)
constexpr int NCOPY = 8;                // replicas of broadcast exchanges (one per XCD)
// LDS weight staging, in items (one 16-byte chunk per lane of a wave) per wave
constexpr int QKV_CAP = 2, O_CAP = 1, GU_CAP = 6, DN_CAP = 3, LM_CAP = 8;
constexpr int TAGS_PER_LAUNCH = 1024;   // exchange tags one launch may use
constexpr int STAMP_LAYERS = 56;        // layers whose phase stamps the debug output records
constexpr uint32_t SPIN_TIMEOUT = 100000000u;  // default wait bound: 1 s of the 100 MHz wall clock

enum { W_F32 = 0, W_BF16 = 1, W_I4 = 2 };
enum { ERR_TIMEOUT = 1u, ERR_TOKEN = 2u, ERR_POS = 4u };

struct Mat {
  const uint8_t* w;      // row-major [rows][in] (fp32 / bf16) or int4 codes [rows][in/2]
  const uint16_t* s;     // int4 only: bf16 scales [rows][in/64]
  const uint16_t* s4;    // int4, batched path: the same scales as [rows/4][in/64][4] (4 rows per 8 bytes)
  const uint8_t* wt;     // batched path: the weights in 16-row tiles of 1 KB MFMA operand chunks (see tile_map)
};

// Per-context constants, kept in device memory for the kernel's lifetime.
struct KStatic {
  int H, nq, nkv, hd, V, L, n_dense, DI, E, K, EI, renorm;
  float eps;
  int S;                 // attention splits per kv head (grid / n_kv_heads)
  int qkv_rows, o_slots, h_slots;
  int poll_sleep;        // s_sleep(8) repetitions between polls of a stale slot
  int sentinels;         // slots polled by wave 0 before the bulk read (0: none, up to 64)
  uint32_t spin_limit;   // a wait gives up after this many ticks of the 100 MHz wall clock (fills the
                         // padding before the pointers: the fields after it keep their offsets)
  const uint8_t* embed;
  const uint8_t* lmhead;
  const float* fnorm;
  const float* anorm;
  const float* pnorm;
  Mat qkv, o, dg, du, dd, router, eg, eu, ed;
  uint64_t* x_qkv;       // [NCOPY][2][qkv_rows]            q/k/v after RoPE (fp32)
  uint64_t* x_part;      // [2][nq][hd + 2][S]              attention partials (fp32)
  uint64_t* x_o;         // [NCOPY][2][o_slots]             merged attention output
  uint64_t* x_res1;      // [NCOPY][2][H]                   residual after o_proj (fp32)
  uint64_t* x_h;         // [NCOPY][2][h_slots]             SwiGLU output
  uint64_t* x_res2;      // [NCOPY][2][H]                   residual after the MLP (fp32)
  uint64_t* x_z;         // [NCOPY][2][E]                   router logits (fp32)
  uint32_t* err;         // device error word
  uint32_t* herr;        // host-mapped error word
  unsigned long long* amax;  // packed argmax key
  uint32_t* done;        // workgroups finished with lm_head
};

// Per-launch arguments (passed by value).
struct KDyn {
  uint8_t* kc;           // KV cache [L][B][nkv][cap][hd] in the activation type
  uint8_t* vc;
  int B, cap;
  const float2* rope;    // [cap][hd/2] (cos, sin)
  int32_t* len;          // [B] device lengths
  const int32_t* tokens;
  int tok_idx, seq;
  int32_t* hist;         // [B][cap] token consumed at each position
  int32_t* out_ids;
  int out_idx;
  uint32_t epoch;
  float* dbg_logits;
  int32_t* dbg_routes;
  float* dbg_rw;
  float* dbg_resid;      // [n_layers][H] residual after each layer of this sequence
  uint64_t* dbg_ts;
  float* dbg_z;          // [n_layers][n_experts] router logits of this sequence
  uint64_t* xbase;       // null: the context's exchange buffer; else the fixed scratch array of the
                         // non-allocating entry point: argmax counters in words 0 and 8, the context's slot
                         // layout from word 16
};

// Batched decode: up to BT sequences per pass go through a sequence of
// ordinary kernels per layer whose contractions run on MFMA with the
// sequences as the 16 columns.
constexpr int BT = 16;                  // sequences per pass (MFMA columns)
constexpr int ATT_P = 256;              // cached positions per attention split of the batched path
constexpr int ATT_C = 16;               // positions per chunk of a split (one MFMA score tile)
constexpr int MAX_SPLITS = 1024;        // attention splits per sequence (max_tokens <= ATT_P * MAX_SPLITS)
constexpr int OKC = 2;                  // o_proj input chunks (partial sums added by the next norm)
constexpr int DKC = 16;                 // dense down input chunks (partial-sum buffers)
constexpr int DKM = 8;                  // MoE down workgroups per 64-row block (<= DKC)

struct BArgs {
  // model
  int H, nq, nkv, hd, V, L, n_dense, DI, E, K, EI, renorm;
  float eps;
  const uint8_t* embed;
  const uint8_t* lmhead;
  const uint8_t* lmt;    // lm_head in the tiled layout
  const float* fnorm;
  const float* anorm;
  const float* pnorm;
  Mat qkv, o, dg, du, dd, router, eg, eu, ed;
  // this pass: columns n < B are the cache's sequences cseq[n] (of Bc), each at its own length, with
  // tokens[n] and out_ids[n] their token and next id; or (prefill) B consecutive prompt tokens
  // tokens[tok0 ..] of sequence seq0 at positions len[seq0] ..,
  // the greedy id after the last one written to out_ids[0]
  int B, seq0, Bc, cap, prefill, tok0;
  int cseq[BT];
  // position of column n (its sequence's length, or len + n in prefill), taken from the host's mirror of
  // the lengths so that no kernel waits on a load to know it; asp[n] = attention splits of columns 0 .. n - 1
  int pos[BT];
  int asp[BT + 1];
  uint8_t* kc;           // [L][Bc][nkv][cap][hd] bf16
  uint8_t* vc;
  const float2* rope;    // [cap][hd/2] (cos, sin)
  int32_t* len;          // [Bc]
  const int32_t* tokens; // [Bc]
  int32_t* out_ids;      // [Bc]
  uint32_t* err;         // device error word
  uint32_t* herr;        // host-mapped error word
  // scratch of the pass (device, owned by the cache)
  float* x;              // [BT][H] residual
  uint16_t* act;         // [BT][astride] bf16 GEMM input (int4 models: 8-element groups permuted)
  int astride;
  float* q;              // [BT][nq * hd] queries after RoPE
  float* part;           // [BT][nq][nsmax][hd + 2] attention partials (m, l, o)
  int nsmax;
  float* opart;          // [OKC][BT][H]
  float* dpart;          // [DKC][BT][H]
  uint16_t* h;           // [BT][hstride] SwiGLU output (same layout rule as act)
  int hstride;
  int32_t* sel;          // [BT][K] selected experts
  float* wsel;           // [BT][K] their weights
  // prefill of a chunk of n > BT tokens of sequence seq0 at positions p0 .. p0 + n - 1 (the buffers above then
  // hold n rows); the head adds lenadd to the length (batched prefill passes: B)
  int p0, lenadd;
  int32_t* hist;         // [Bc][cap] token consumed at each position (written at the embedding)
  float* y;              // [n][K][H] expert down products per (token, slot)
  int32_t* lst;          // [n K] (token << 3 | slot), grouped by expert in expert order, tokens ascending
  int32_t* ecnt;         // [E] entries per expert
  int32_t* blk;          // [n K / 64 + E][3] token blocks: (expert, first entry, end of the expert's entries)
  int32_t* nblk;         // [1] token blocks in use
  unsigned long long* amax;  // [BT] packed argmax keys
  uint32_t* done;        // workgroups finished with lm_head
  uint32_t* cnt;         // [H/16 + H/64] workgroups finished per o_proj row tile, then per down row block
  // debug outputs (indexed by cache sequence), or null
  float* dbg_logits;
  int32_t* dbg_routes;
  float* dbg_rw;
  float* dbg_resid;      // [Bc][L][H] residual after each layer
  float* dbg_z;
};

// Enqueue one batched decode pass (every layer and the head) on `stream`.
hipError_t launch_batch_pass(int wt, const BArgs& a, hipStream_t stream);
// Prefill of n (BT < n <= 4096) tokens of sequence a.seq0 at positions a.p0 .. through the long-chunk
// kernels; a's buffers hold n rows (a.part: prefill_part_floats floats).
hipError_t launch_prefill(int wt, const BArgs& a, int n, hipStream_t stream);
size_t prefill_part_floats(int nq, int nsmax, int hd);

// Measurement helpers (flint_micro.hip).
hipError_t launch_micro_read(const void* p, size_t bytes, uint32_t* sink, int blocks, hipStream_t st);
hipError_t launch_micro_exchange(unsigned long long* slots, int workgroups, int rounds, uint32_t* err, hipStream_t st,
                                 bool xcd);
hipError_t launch_micro_empty(hipStream_t st);
// s4[((r / 4) * G + g) * 4 + r % 4] = s[r * G + g] for r < rows (a multiple of 4), g < G.
hipError_t launch_regroup_scales(const uint16_t* s, uint16_t* s4, size_t rows, int G, hipStream_t stream);
// Copy a [rows][in] weight matrix into the tiled layout of the batched path (rows a multiple of 16).  Tile
// T holds rows tile_row(T, m), m < 16: the rows in order (rope_hd == 0), or, for the fused QKV rows of
// rope_hd-dim heads, 8 rotate-half pairs per tile (rows i0 + m and rope_hd/2 + i0 + m of one head).
hipError_t launch_tile_weights(int wt, const uint8_t* w, uint8_t* dst, size_t rows, int in, int rope_hd,
                               hipStream_t stream);

// True if the compile-time 2048-wide shape (and a 256-workgroup grid) matches.
bool shape_is_static(const KStatic& k, int grid);
// Launch the persistent kernel for weight type wt on `stream` (stat: the compile-time shape).
hipError_t launch_decode(int wt, bool stat, const KStatic* ks, const KDyn& d, int grid, hipStream_t stream);
// The fixed exchange scratch of the non-allocating decode entry point: NOALLOC_SCRATCH_WORDS 64-bit words
// per device (4 MiB).  noalloc_scratch finds this device's copy (device `dev`, current) once per device,
// clears it once on `stream` and returns its address; noalloc_next_launch counts the launches that use it.
constexpr size_t NOALLOC_SCRATCH_WORDS = 512 * 1024;
hipError_t noalloc_scratch(int dev, hipStream_t stream, uint64_t** ptr);
uint64_t noalloc_next_launch(int dev);
// Zero `n` 64-bit words with a fill kernel.
hipError_t launch_fill(uint64_t* p, size_t n, hipStream_t stream);
// Static LDS bytes of the persistent kernel.
int kernel_lds_bytes(int wt);
// Co-resident workgroups per CU of the persistent kernel.
hipError_t kernel_occupancy(int wt, int* per_cu);

}  // namespace flint

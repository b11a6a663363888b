/*
 * flint.h -- C ABI of the MI355X (gfx950) decode library.
 *
 * The library runs one greedy decode step of a top-k mixture-of-experts
 * transformer as ONE persistent HIP kernel per step: input RMSNorm, QKV
 * projection, RoPE, KV-cache append, attention over the resident cache,
 * o_proj, post-attention RMSNorm, router and top-k selection, expert
 * gate/up/SiLU/down (a dense SwiGLU MLP on the first n_dense_layers layers),
 * final norm, lm_head and argmax.  This is the operator list of one decode
 * step given in section 2 of the page "Flint Inference on Apple Silicon: rec
 * Megakernel and Tempo9 Compared" (49 layers, 2048-wide residual, top-6,
 * layers 0 and 1 dense, the whole step inside a single dispatch whose groups
 * synchronise through device-scope atomics only where data crosses groups).
 *
 * Conventions for every entry point:
 *  - Every call returns an int status (FLINT_OK or one of the FLINT_E* codes
 *    below).  On failure flint_last_error() returns a message for the calling
 *    thread; no output is written and no work is enqueued.
 *  - "device" pointers point to GPU memory of the device that was current at
 *    flint_decode_init; "host" pointers to CPU memory.
 *  - Work is enqueued on the HIP stream given at init and is asynchronous:
 *    outputs are valid once the stream has completed (flint_sync).
 *  - One flint_ctx serves one stream; calls on a ctx and on its flint_kv
 *    objects are not thread-safe.  Free every flint_kv before its ctx.
 */
#ifndef FLINT_H
#define FLINT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ status */
#define FLINT_OK 0
#define FLINT_EINVAL 1       /* bad argument or configuration */
#define FLINT_ENOMEM 2       /* device or host allocation failed */
#define FLINT_EHIP 3         /* a HIP runtime call failed */
#define FLINT_ECAPACITY 4    /* KV cache has no room for the new positions */
#define FLINT_ETIMEOUT 5     /* a cross-workgroup wait inside the kernel timed out (see flint_set_wait_limit) */
#define FLINT_ENORESIDENT 6  /* the device cannot hold the persistent grid */
#define FLINT_EDEVICE 7      /* the kernel flagged bad device data (token id out of range) */

/* ------------------------------------------------------------- configuration */
#define FLINT_W_F32 0        /* fp32 weights, fp32 activations and KV cache */
#define FLINT_W_BF16 1       /* bf16 weights, bf16 GEMV inputs and KV cache, fp32 accumulate */
#define FLINT_W_INT4G64 2    /* int4 group-64 weights (bf16 scales); embedding and lm_head bf16;
                                activations and KV cache as for FLINT_W_BF16 */

typedef struct flint_config {
  int32_t n_layers;        /* layers, e.g. 49 */
  int32_t n_dense_layers;  /* the first n_dense_layers layers use a dense SwiGLU MLP (e.g. 2) */
  int32_t hidden;          /* residual width H (multiple of 64, <= 2048) */
  int32_t n_q_heads;       /* query heads (n_q_heads * head_dim <= 2048) */
  int32_t n_kv_heads;      /* key/value heads; n_q_heads % n_kv_heads == 0, group <= 8 */
  int32_t head_dim;        /* 64 or 128 */
  int32_t vocab;           /* rows of the embedding and of lm_head */
  int32_t dense_inter;     /* intermediate width of the dense MLP (multiple of 64, <= 6144) */
  int32_t n_experts;       /* experts per MoE layer (<= 64) */
  int32_t top_k;           /* experts chosen per token (<= 8, top_k * expert_inter <= 6144) */
  int32_t expert_inter;    /* intermediate width of one expert (multiple of 64) */
  int32_t weight_type;     /* FLINT_W_*; it also fixes the activation type (there is no separate
                              act_type): fp32 weights run fp32 activations and an fp32 cache, bf16 and
                              int4 weights bf16 GEMV inputs and a bf16 cache with fp32 accumulation */
  int32_t router_renorm;   /* 0: weight = softmax probability over all experts; 1: renormalised
                              over the top_k selected */
  int32_t grid;            /* persistent workgroups; 0 = one per compute unit */
  float rope_theta;        /* RoPE base, e.g. 1e4 */
  float rms_eps;           /* RMSNorm epsilon, e.g. 1e-6 */
} flint_config;

/* One linear layer: row-major [out][in] weights.  For FLINT_W_INT4G64 `w`
 * holds uint8 codes [out][in / 2] (element 2j in the low nibble of byte j,
 * stored as q + 8, q in [-8, 7]) and `scales` bf16 [out][in / 64]; the weight
 * is scales[r][c / 64] * q.  Otherwise `w` is fp32 or bf16 [out][in] and
 * `scales` is ignored. */
typedef struct flint_mat {
  const void* w;
  const void* scales;
} flint_mat;

/* Device pointers in canonical layout, borrowed only for the duration of
 * flint_decode_init: the library copies what it needs and the caller may free
 * its buffers after the call returns.  Stacked tensors put the layer (and then
 * the expert) index first. */
typedef struct flint_weights {
  const void* embed;       /* [vocab][hidden], fp32 for FLINT_W_F32 else bf16 */
  const void* lm_head;     /* [vocab][hidden], same dtype as embed */
  const float* final_norm; /* [hidden] fp32 */
  const float* attn_norm;  /* [n_layers][hidden] fp32 */
  const float* post_norm;  /* [n_layers][hidden] fp32 */
  flint_mat qkv;           /* [n_layers][(n_q + 2 n_kv) head_dim][hidden]: q heads, then k heads, then v heads;
                              each head's head_dim rows in rotate-half order (pairs i, i + head_dim/2) */
  flint_mat o;             /* [n_layers][hidden][n_q head_dim] */
  flint_mat dense_gate;    /* [n_dense_layers][dense_inter][hidden] */
  flint_mat dense_up;      /* [n_dense_layers][dense_inter][hidden] */
  flint_mat dense_down;    /* [n_dense_layers][hidden][dense_inter] */
  flint_mat router;        /* [n_layers - n_dense_layers][n_experts][hidden] */
  flint_mat exp_gate;      /* [n_layers - n_dense_layers][n_experts][expert_inter][hidden] */
  flint_mat exp_up;        /* [n_layers - n_dense_layers][n_experts][expert_inter][hidden] */
  flint_mat exp_down;      /* [n_layers - n_dense_layers][n_experts][hidden][expert_inter] */
} flint_weights;

typedef struct flint_ctx flint_ctx;
typedef struct flint_kv flint_kv;

/* Optional outputs of flint_decode_step_debug (device pointers; NULL = skip).
 * They come from the same kernel as flint_decode_step. */
typedef struct flint_debug {
  float* logits;        /* [batch][vocab] fp32 logits of the step */
  int32_t* routes;      /* [batch][n_layers][top_k] selected experts, descending router logit;
                           -1 on dense layers */
  float* route_w;       /* [batch][n_layers][top_k] expert weights */
  float* resid;         /* [batch][n_layers][hidden] fp32 residual after every layer */
  uint64_t* phase_ts;   /* [n_layers + 1][16] wall-clock stamps (100 MHz) of workgroup 0 at
                           phase boundaries, for sequence 0.  Row 0: start, end, argmax published,
                           then the shader clock counter (s_memtime) at start and at end.
                           Row l + 1 (layer l, the first 56 layers), in order: 0 input norm, 1 QKV, 2 q/k/v published,
                           3 q gathered, 4 attention partial published, 5 splits merged, 6 merged
                           output gathered, 7 o_proj published, 8 residual gathered, 9 post norm,
                           10 router, 11 top-k (10 and 11 are 0 on dense layers), 12 SwiGLU
                           published, 13 SwiGLU gathered, 14 MLP residual published, 15 gathered.
                           The persistent kernel only (several sequences: not written) */
  float* router_logits; /* [batch][n_layers][n_experts] router logits (0 on dense layers) */
} flint_debug;

/* ------------------------------------------------------------- entry points */

/*
 * Create a context for the decode step of section 2 of "Flint Inference on
 * Apple Silicon: rec Megakernel and Tempo9 Compared" (the model whose layers
 * that section lists, here any size within the limits of flint_config):
 * validate cfg, query the device, copy the weights into
 * library-owned device memory and allocate the kernel's scratch.  hip_stream
 * is a hipStream_t (NULL = the default stream) on which all later work of
 * this ctx is enqueued.  Synchronises hip_stream before returning.
 * Errors: FLINT_EINVAL (cfg or weights), FLINT_ENOMEM, FLINT_EHIP,
 * FLINT_ENORESIDENT (fewer co-resident workgroups than the grid).
 */
int flint_decode_init(const flint_config* cfg, const flint_weights* w, void* hip_stream, flint_ctx** out);

/* Destroy a context (synchronises its stream).  NULL is accepted. */
int flint_decode_free(flint_ctx* ctx);

/*
 * Allocate the resident KV cache that decode attends over (section 2 of "Flint
 * Inference on Apple Silicon: rec Megakernel and Tempo9 Compared": the step
 * appends the new token's K/V and attends over every cached position; section 1
 * keeps that cache across turns of one session) for `batch` sequences of up
 * to max_tokens positions:
 * per layer K and V of [batch][n_kv_heads][max_tokens][head_dim] in the
 * activation type (fp32 for FLINT_W_F32, else bf16), zero-filled, plus the
 * per-sequence lengths (all 0) on the device with a host mirror.  The
 * library owns this memory.  Errors: FLINT_EINVAL, FLINT_ENOMEM, FLINT_EHIP.
 */
int flint_kv_alloc(flint_ctx* ctx, int32_t batch, int32_t max_tokens, flint_kv** out);
int flint_kv_free(flint_kv* kv);

/* Set (host array [batch]) the sequence lengths.  Shrinking a length is a
 * rollback: positions at and past it are ignored and later overwritten.
 * Errors: FLINT_EINVAL if a length is outside [0, max_tokens]. */
int flint_kv_set_lengths(flint_kv* kv, const int32_t* lengths);

/* Copy the device lengths into a host array [batch] (synchronises the stream). */
int flint_kv_get_lengths(flint_kv* kv, int32_t* lengths);

/*
 * The token ids a sequence's cache holds: tokens[p] for p < n <= len[seq] is
 * the token consumed at position p (by flint_decode_step*, flint_prefill_chunk),
 * -1 for positions whose K/V were written otherwise (flint_kv_layer_ptrs).
 * Host output; synchronizes the context's stream.  Errors: FLINT_EINVAL,
 * FLINT_EHIP.
 */
int flint_kv_tokens(flint_kv* kv, int32_t seq, int32_t* tokens, int32_t n);

/*
 * Prefix reuse within one sequence: *matched = the number of leading entries of
 * the host array tokens[0 .. n-1] equal to the sequence's cached tokens (at
 * most len[seq]).  The caller keeps that prefix with flint_kv_set_lengths
 * (rollback truncates; generated tokens that were consumed are part of the
 * cache) and prefills the rest, the single-session prompt cache of "Flint
 * Inference on Apple Silicon: rec Megakernel and Tempo9 Compared", section 1.
 * Synchronizes the context's stream.  Errors: FLINT_EINVAL, FLINT_EHIP.
 */
int flint_kv_prefix_match(flint_kv* kv, int32_t seq, const int32_t* tokens, int32_t n, int32_t* matched);

/* Device pointers to layer `layer`'s K and V ([batch][n_kv][max_tokens][head_dim]),
 * e.g. to load a resident cache.  Errors: FLINT_EINVAL. */
int flint_kv_layer_ptrs(flint_kv* kv, int32_t layer, void** k, void** v);

/*
 * One greedy decode step, the operator list of section 2 of "Flint Inference
 * on Apple Silicon: rec Megakernel and Tempo9 Compared" (input RMSNorm, QKV,
 * RoPE, KV append, attention, o_proj, post-attention RMSNorm, router and
 * top-k, experts or the dense MLP, final norm, lm_head, argmax), for every
 * sequence b of kv: consume the device token
 * tokens[b] at position len[b], append its K/V, write the argmax token id to
 * out_ids[b] (device) and increment len[b].  tokens and out_ids may alias,
 * so out_ids can be fed back as the next step's tokens without a host round
 * trip.  One or two sequences: the persistent kernel per sequence.  Three or
 * more (the environment variable FLINT_BATCH_MIN, read at flint_decode_init,
 * changes the threshold) on bf16 / int4 models with 128-dim heads: passes of up
 * to 16 sequences on the batched MFMA path,
 * which on the first such cache makes the context's tiled weight copies (the
 * "batch-16 ragged" step of the pages' concurrent-client workload, section 4
 * of "Flint Inference on Apple Silicon: rec Megakernel and Tempo9 Compared").
 * Errors: FLINT_EINVAL, FLINT_ENOMEM, FLINT_ECAPACITY (len[b] + 1 > max_tokens,
 * from the host mirror), FLINT_EHIP, and FLINT_ETIMEOUT / FLINT_EDEVICE latched
 * by an earlier step (reported once, then cleared).
 */
int flint_decode_step(flint_ctx* ctx, const int32_t* tokens, flint_kv* kv, int32_t* out_ids);

/*
 * One greedy decode step for the n distinct sequences seqs[0 .. n-1] (host
 * array, 1 <= n <= batch) of kv and no other: sequence seqs[i] consumes the
 * device token tokens[i] at position len[seqs[i]], appends its K/V, gets its
 * argmax id in out_ids[i] (device; may alias tokens) and len[seqs[i]] += 1.
 * Sequences may join, leave and come back between calls (each keeps its own
 * cache), the continuous-batching use of the batch-16 step of "Flint Inference
 * on Apple Silicon: rec Megakernel and Tempo9 Compared", section 4.  Three or
 * more sequences take the batched path (when the cache has one), one or two the
 * persistent kernel per sequence.  Errors: FLINT_EINVAL (NULL pointer, n out of range,
 * a sequence out of range or listed twice), FLINT_ECAPACITY, FLINT_EHIP, and
 * errors latched by an earlier step.
 */
int flint_decode_step_seqs(flint_ctx* ctx, flint_kv* kv, const int32_t* seqs, int32_t n, const int32_t* tokens,
                           int32_t* out_ids);

/*
 * flint_decode_step for callers that cannot allocate device memory at call
 * time (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): every sequence of kv runs the persistent kernel, whose
 * exchange slots and argmax counters live in a fixed 4 MiB array of the
 * library's device image instead of the context's buffer.  The call allocates
 * nothing (the array's device address is found once per device by
 * flint_decode_init).  Every call on a GPU shares that GPU's array: calls
 * that overlap on one GPU (other streams, other contexts, other threads)
 * race and give undefined results.  Same arguments, outputs and errors as
 * flint_decode_step, plus FLINT_EINVAL if the model needs more than the
 * array's 4 MiB of exchange scratch (the 49-layer 2048-wide shape needs
 * about 3.5 MB) and FLINT_EHIP if the array was not found at init.
 */
int flint_decode_step_noalloc(flint_ctx* ctx, const int32_t* tokens, flint_kv* kv, int32_t* out_ids);

/* flint_decode_step with the optional outputs of `dbg` (may be NULL). */
int flint_decode_step_debug(flint_ctx* ctx, const int32_t* tokens, flint_kv* kv, int32_t* out_ids,
                            const flint_debug* dbg);

/*
 * Chunked prefill (section 1 of "Flint Inference on Apple Silicon: rec
 * Megakernel and Tempo9 Compared" prefills prompts in chunks of 4,096 tokens):
 * the decode step's operators applied to a block of known tokens.
 * Process n (1 <= n <= 4096) known device tokens of sequence seq at positions
 * len[seq] .. len[seq] + n - 1 (causal attention over the cache and the
 * chunk), append their K/V, write the greedy id after the last position to
 * out_id[0] (device) and add n to len[seq].  bf16 / int4 models with 128-dim
 * heads: up to 16 tokens as one batched MFMA pass; longer chunks layer by layer
 * over all n tokens (MFMA contractions over 64 tokens per workgroup, experts
 * run on the tokens that picked them, attention per 16 tokens and split of
 * 256 cached positions).  The first call makes the tiled weight copies and the
 * cache's scratch; the first long chunk on a cache allocates the long-chunk
 * scratch, sized for 4,096 tokens (about 0.5 GB for the 49-layer shape at
 * 9,300 positions), held until flint_kv_free.  Other models: one persistent
 * launch per token.  Errors: FLINT_EINVAL, FLINT_ENOMEM, FLINT_ECAPACITY,
 * FLINT_EHIP.
 */
int flint_prefill_chunk(flint_ctx* ctx, flint_kv* kv, int32_t seq, const int32_t* tokens, int32_t n,
                        int32_t* out_id);

/*
 * Measurement helpers (outside the decode path; each synchronizes the
 * context's stream and allocates and frees its own device memory), the
 * microbenchmarks that "Flint Inference on Apple Silicon: rec Megakernel and
 * Tempo9 Compared" reports beside its decode numbers (section 3):
 *  - flint_micro_stream_read: GB/s of reading `bytes` (>= 1 MiB) of device
 *    memory once per launch, `reps` launches (the practical HBM ceiling);
 *  - flint_micro_exchange: microseconds per round of an all-to-all exchange
 *    among `workgroups` (2 .. compute units) co-resident workgroups through
 *    tagged system-scope slots written in 8 replicas (one per XCD) and read
 *    all at once, as the decode kernel hands data between workgroups;
 *    FLINT_ETIMEOUT if a bounded wait ran out;
 *  - flint_micro_exchange_xcd: the same round confined to each XCD: workgroup
 *    w exchanges with the workgroups of its XCD only (w mod 8, where the
 *    dispatcher places it), through device-scope slots that stay in that
 *    XCD's L2; `workgroups` a multiple of 8, at least 16;
 *  - flint_micro_launch: microseconds per back-to-back empty kernel launch.
 * Errors: FLINT_EINVAL, FLINT_ENOMEM, FLINT_EHIP (and FLINT_ETIMEOUT above).
 */
int flint_micro_stream_read(flint_ctx* ctx, size_t bytes, int32_t reps, float* gbps);
int flint_micro_exchange(flint_ctx* ctx, int32_t workgroups, int32_t rounds, float* us_per_round);
int flint_micro_exchange_xcd(flint_ctx* ctx, int32_t workgroups, int32_t rounds, float* us_per_round);
int flint_micro_launch(flint_ctx* ctx, int32_t launches, float* us_per_launch);

/* Wait for the ctx stream; report and clear a latched device error. */
int flint_sync(flint_ctx* ctx);

/*
 * Bound every cross-workgroup wait of the persistent kernel by `microseconds`
 * (0 restores the default of one second; bounds above 42.9 s are clamped to it).  The kernel's workgroups hand data to
 * each other through spin-waits that assume the whole grid is resident at once
 * (the condition section 2 of "Flint Inference on Apple Silicon: rec Megakernel
 * and Tempo9 Compared" notes for device-scope spin barriers); a wait that runs
 * past the bound gives up and every workgroup of the step winds down and exits.
 * Such a step, and every step queued behind it before the error is reported,
 * writes -1 in place of its id, leaves its sequence's length unchanged and may
 * have written part of the K/V at that position (the next step at that
 * position overwrites it).  The next call on the ctx (or flint_sync) reports
 * FLINT_ETIMEOUT once and re-reads the lengths of the ctx's caches.
 * Synchronizes the ctx's stream.  Errors: FLINT_EINVAL, FLINT_EHIP.
 */
int flint_set_wait_limit(flint_ctx* ctx, uint32_t microseconds);

/* Launch shape of the persistent kernel. */
int flint_device_info(flint_ctx* ctx, int32_t* grid, int32_t* block, int32_t* lds_bytes);

/* Message of the last failing call on this thread ("" if none). */
const char* flint_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* FLINT_H */

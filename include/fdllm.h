/*
 * fdllm.h -- C ABI of the Fast-dLLM decoding hot path on AMD MI355X (gfx950).
 *
 * One denoising step of a masked-diffusion LLM decoded block by block: the
 * active block's queries attend bidirectionally (no causal mask) over an
 * approximate KV cache, and the step ends with confidence-aware parallel
 * unmasking. Sources (cited by page title and section):
 *   [commentary] "Fast-dLLM: Training-free Acceleration of Diffusion LLM by
 *                Enabling KV Cache and Parallel Decoding", paper-graph-ui page,
 *                sections 3.2, 3.4.2, 3.4.3, 3.4.4;
 *   [README]     NVlabs/Fast-dLLM GitHub README, "Parameter descriptions"
 *                (gen_length, steps, block_size, use_cache, dual cache,
 *                threshold).
 *
 * Conventions
 *   - Every pointer named d_* is device memory on the current HIP device;
 *     other pointers are host memory. The library never takes ownership of
 *     caller memory and never frees it.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call except fdllm_decode only enqueues work and returns without
 *     synchronising.
 *   - Token ids are int32, masked flags uint8 (1 = still masked). A sequence
 *     x of batch b is row-major [batch][seq_len].
 *   - Weights and the KV cache have the model's storage dtype (FDLLM_F32 or
 *     FDLLM_BF16; bf16 = raw uint16 bit pattern). Activations (hidden states,
 *     queries, attention outputs) are float32; with bf16 weights the float32
 *     operand of every matrix product is fed to the bf16 matrix cores as two
 *     bf16 terms (hi + lo). Accumulation is float32.
 *   - Errors: a negative fdllm_status; fdllm_last_error() returns a
 *     thread-local message for the last failing call on this thread. No C++
 *     exception crosses this boundary. On error nothing was enqueued unless
 *     the status is FDLLM_EHIP.
 */
#ifndef FDLLM_H
#define FDLLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t fdllm_status;
#define FDLLM_OK 0
#define FDLLM_EINVAL (-1)   /* a parameter is out of range */
#define FDLLM_ESHAPE (-2)   /* a shape the kernels do not support */
#define FDLLM_EDTYPE (-3)   /* unknown dtype */
#define FDLLM_ENOTSUP (-4)  /* device is not gfx950 */
#define FDLLM_EHIP (-5)     /* a HIP runtime call failed (message has hipGetErrorString) */
#define FDLLM_EBUDGET (-6)  /* a block still had masked positions after its step budget */
#define FDLLM_ENUMERIC (-7) /* reserved: no call returns it (NaN logits are handled, see below) */

typedef enum fdllm_dtype { FDLLM_F32 = 0, FDLLM_BF16 = 1 } fdllm_dtype;

/* Model shape. Pre-norm transformer: RMSNorm -> q,k,v projections with
 * rotate-half RoPE at absolute positions -> bidirectional grouped-query
 * attention -> output projection + residual -> RMSNorm -> SwiGLU FFN +
 * residual; final RMSNorm, untied LM head, logits multiplied by logit_scale.
 * Supported: head_dim in {64, 128}; d_model % 256 == 0 and d_model <= 8192;
 * n_heads % n_kv_heads == 0; (n_heads * head_dim) % 128 == 0; ffn_dim % 128
 * == 0; vocab % 16 == 0; 0 <= mask_id < vocab. */
typedef struct fdllm_model_config {
  int32_t n_layers;
  int32_t d_model;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t ffn_dim;
  int32_t vocab;
  int32_t mask_id;
  int32_t dtype;       /* fdllm_dtype */
  int32_t max_seq_len; /* largest sequence length (prompt + gen) to be used */
  float rope_theta;
  float norm_eps;
  float logit_scale;
} fdllm_model_config;

typedef struct fdllm_model fdllm_model; /* opaque host handle */
typedef struct fdllm_cache fdllm_cache; /* opaque host handle */

/* How a step picks the masked positions it commits ([commentary] 3.4.3;
 * see fdllm_confidence_unmask for each rule). tau: the threshold rule
 * (finite). factor > 0: the factor rule instead. topk > 0: the fixed top-K
 * baseline instead. sampling != 0: stochastic tau-leaping ([commentary]
 * 3.4.1) instead of all three, its draws keyed by seed. */
typedef struct fdllm_select_params {
  float tau;
  float factor;
  int32_t topk;
  int32_t sampling;
  uint32_t seed;
} fdllm_select_params;

/* Decode settings, as the README's decode parameters:
 * gen_length L (multiple of block_size B), steps (multiple of K = L/B; each
 * block gets T = steps/K denoising steps), use_cache, dual_cache (DualCache;
 * requires use_cache; otherwise PrefixCache), threshold tau (finite; tau > 1
 * commits exactly one token per step) and factor f (finite, >= 0; f > 0
 * selects by the factor strategy of [commentary] 3.4.3 instead of the
 * threshold, see fdllm_confidence_unmask) and refresh_interval r (>= 0;
 * [commentary] Table 10's policy: with use_cache, step t of a block runs a
 * full forward that rebuilds the cache when t % r == 0, not only at t = 0;
 * 0 keeps one rebuild per block), topk (>= 0; > 0 selects the fixed
 * top-K baseline), sampling and seed (stochastic tau-leaping; see
 * fdllm_select_params and fdllm_confidence_unmask). */
typedef struct fdllm_decode_params {
  int32_t gen_length;
  int32_t steps;
  int32_t block_size;
  int32_t use_cache;
  int32_t dual_cache;
  float threshold;
  float factor;
  int32_t refresh_interval; /* r > 0: also rebuild the cache at steps t % r == 0 of a block */
  int32_t topk;             /* > 0: fixed top-K selection instead of threshold / factor */
  int32_t sampling;         /* != 0: stochastic tau-leaping instead of a confidence rule */
  uint32_t seed;            /* key of the sampling draws (sequence b uses key (seed, b)) */
} fdllm_decode_params;

/* Per-call statistics of fdllm_decode (host struct filled by the call). */
#define FDLLM_STATS_BLOCKS 1024
#define FDLLM_STATS_STEPS 4096
typedef struct fdllm_decode_stats {
  int32_t nfe;             /* model forwards run (refreshes + cached + full) */
  int32_t refreshes;       /* full forwards that rebuilt the cache (block starts and refresh-interval steps) */
  int32_t cached_steps;    /* forwards over the cache */
  int32_t full_steps;      /* uncached full forwards after the first of a block */
  int32_t max_steps_block; /* most steps any block needed */
  int32_t committed;       /* tokens committed (== batch * gen_length) */
  int32_t steps_per_block[FDLLM_STATS_BLOCKS]; /* first min(K, FDLLM_STATS_BLOCKS) blocks */
  /* tokens committed by each forward, summed over the batch, in decode
   * order: the first min(nfe, FDLLM_STATS_STEPS) forwards ([commentary]
   * Figure 7 plots this count over a generation); it sums to committed when
   * nfe <= FDLLM_STATS_STEPS */
  int32_t commits_per_step[FDLLM_STATS_STEPS];
} fdllm_decode_stats;

/* ---- lifetime and sizing ------------------------------------------------ */

/* Library version string (static storage). */
const char* fdllm_version(void);

/* Message of the last failing call on this thread ("" if none). */
const char* fdllm_last_error(void);

/* Bytes of device memory fdllm_model_create needs for the packed weights. */
fdllm_status fdllm_model_packed_bytes(const fdllm_model_config* cfg, size_t* bytes);

/* Creates a model: copies the raw weights into `d_packed` (caller-allocated,
 * fdllm_model_packed_bytes bytes, 256-byte aligned) in the kernels' layout and
 * builds the RoPE table. `d_weights` is a host array of device pointers in
 * this order: embed [vocab][d]; then per layer: attn_norm [d], wq [Hq*D][d],
 * wk [Hkv*D][d], wv [Hkv*D][d], wo [d][Hq*D], ffn_norm [d], w_gate [F][d],
 * w_up [F][d], w_down [d][F]; then final_norm [d], lm_head [vocab][d].
 * Matrices are [out][in] row-major in the model dtype. The raw weights are
 * only read (on `stream`) and may be freed once the stream has passed this
 * call. `d_packed` must outlive the model. */
fdllm_status fdllm_model_create(const fdllm_model_config* cfg, const void* const* d_weights,
                                void* d_packed, size_t packed_bytes, void* stream,
                                fdllm_model** out);
fdllm_status fdllm_model_destroy(fdllm_model* model);

/* Bytes of device memory for the KV cache plus the working buffers of
 * batch sequences of up to max_seq rows (max_seq <= cfg max_seq_len). */
fdllm_status fdllm_cache_bytes(const fdllm_model* model, int32_t batch, int32_t max_seq,
                               size_t* bytes);

/* Of fdllm_cache_bytes, the bytes that are working buffers rather than
 * K/V: activations, split-K and attention partials, tickets, LM-head
 * statistics, counters. The cache arena holds both, K/V first. */
fdllm_status fdllm_workspace_bytes(const fdllm_model* model, int32_t batch, int32_t max_seq,
                                   size_t* bytes);

/* Creates a cache in caller memory `d_mem` (fdllm_cache_bytes bytes, 256-byte
 * aligned); clears its counters on `stream`. With ncap = max_seq rounded up to
 * a multiple of 32, layer l's K [batch][Hkv][ncap][D] and V, in the tile
 * layout described at fdllm_block_attention, [batch][Hkv][ncap / 32][D][32]
 * (model dtype) come first in the buffer, in layer
 * order, each at a 256-byte aligned offset; the working buffers follow. One
 * cache serves one stream at a time. */
fdllm_status fdllm_cache_create(const fdllm_model* model, int32_t batch, int32_t max_seq,
                                void* d_mem, size_t bytes, void* stream, fdllm_cache** out);
fdllm_status fdllm_cache_destroy(fdllm_cache* cache);

/* ---- the hot path -------------------------------------------------------- */

/* Cache refresh ([commentary] 3.4.2 "Block-Wise Generation Scheme" and 3.4.4
 * "Cache Initialization"): a full forward over rows [0, seq_len) of each of
 * the `batch` sequences in d_x [batch][seq_len], no attention mask. Rewrites
 * every layer's K and V for all seq_len rows and writes the final-normed
 * hidden states of the block rows [blk_start, blk_start + blk_len) to
 * d_hidden_blk, float32 [batch][blk_len][d_model], 16-byte aligned
 * (FDLLM_EINVAL otherwise). With use_cache off the same call is the uncached
 * (vanilla) forward. */
fdllm_status fdllm_cache_refresh(fdllm_model* model, fdllm_cache* cache, const int32_t* d_x,
                                 int32_t batch, int32_t seq_len, int32_t blk_start,
                                 int32_t blk_len, void* d_hidden_blk, void* stream);

/* Cached forward of rows [row_start, row_end) ([commentary] 3.4.2
 * "PrefixCache": row_end = seq_len, the block and the suffix are recomputed;
 * "DualCache": row_end = blk_start + blk_len, only the block is). Fresh q, k, v
 * are computed for those rows at their absolute positions and their K/V are
 * written into the cache in place (rows in the range are always recomputed
 * before they are read, so this equals using them for this step only); every
 * query attends over all seq_len cached rows. Requires blk_start == row_start
 * and a prior fdllm_cache_refresh of this cache at the same batch/seq_len.
 * Writes the final-normed hidden of the block rows to d_hidden_blk (float32,
 * 16-byte aligned, FDLLM_EINVAL otherwise). */
fdllm_status fdllm_block_forward(fdllm_model* model, fdllm_cache* cache, const int32_t* d_x,
                                 int32_t batch, int32_t seq_len, int32_t row_start,
                                 int32_t row_end, int32_t blk_start, int32_t blk_len,
                                 void* d_hidden_blk, void* stream);

/* Standalone block attention ([commentary] 3.4.2: the block's queries attend to
 * every cached key, no mask). q and o [batch][q_rows][hq][head_dim]; k
 * [batch][hkv][kv_len][head_dim]; v in the value cache's tile layout: per
 * (sequence, kv head) ceil(kv_len / 32) tiles, tile t a contiguous
 * [head_dim][32] block holding keys 32t .. 32t + 31, logical key k of the
 * tile at column 8 * ((k % 16) / 4) + 4 * (k / 16) + k % 4 (entries past
 * kv_len are read but ignored). This is the layout the cache keeps V in;
 * values held as plain rows [batch][hkv][kv_len][head_dim] are converted
 * once by fdllm_tile_values. Query head h uses kv head h / (hq / hkv). o =
 * softmax(q k^T * scale) v, rounded to dtype. d_lse (may be NULL): float32
 * [batch][q_rows][hq], the natural log of sum_k exp(scale q.k) of each query
 * row and head (what a caller needs to merge this result with attention over
 * further keys). d_workspace (may be NULL, then one workgroup per (sequence,
 * head, 32-query tile)) holds split partials; it must be zero-filled once
 * before its first use and is left reusable. kv_len must be a multiple of 4. */
fdllm_status fdllm_block_attention_workspace(int32_t batch, int32_t q_rows, int32_t hq,
                                             int32_t head_dim, int32_t kv_len, size_t* bytes);
fdllm_status fdllm_block_attention(const void* d_q, const void* d_k, const void* d_v, void* d_o,
                                   float* d_lse, int32_t batch, int32_t q_rows, int32_t hq,
                                   int32_t hkv, int32_t head_dim, int32_t kv_len, int32_t dtype,
                                   float scale, void* d_workspace, size_t workspace_bytes,
                                   void* stream);

/* Converts values held as plain rows, d_v [batch][hkv][kv_len][head_dim],
 * into the tile layout fdllm_block_attention and the cache use, d_vt
 * [batch][hkv][ceil(kv_len / 32)][head_dim][32] (columns as described at
 * fdllm_block_attention; entries past kv_len are zero). dtype FDLLM_F32 or
 * FDLLM_BF16, head_dim 64 or 128. Enqueued on `stream`; d_v and d_vt must
 * not overlap. */
fdllm_status fdllm_tile_values(const void* d_v, void* d_vt, int32_t batch, int32_t hkv,
                               int32_t kv_len, int32_t head_dim, int32_t dtype, void* stream);

/* Confidence-aware parallel unmasking fused with the LM head ([commentary]
 * 3.4.3 "The Core Idea", "Threshold Strategy", "Factor Strategy"). For each
 * sequence i and block position j in [0, blk_len): z = logit_scale * hidden
 * W_lm^T (d_hidden_blk float32 [batch][blk_len][d_model], 16-byte aligned,
 * FDLLM_EINVAL otherwise) over the whole vocabulary, c = max softmax(z) = 1 / sum exp(z - max
 * z), a = argmax z (lowest id on ties). Among the positions still masked in
 * d_masked [batch][seq_len] at [blk_start, blk_start + blk_len), with
 * factor == 0 every one with c >= tau is committed; with factor > 0 the n
 * most confident are, n the largest count with (n + 1) * (1 - c_(n)) <
 * factor where c_(1) >= c_(2) >= ... are the masked confidences (evaluated
 * in float32; tau is then unused); with topk > 0 (the fixed top-K
 * baseline; tau and factor unused) the topk most confident are (all of them
 * when fewer are masked). For these three, if fewer than q = max(1,
 * ceil(U / (steps_per_block - step_in_block))) are (U = masked count), the q
 * most confident are (lower position first on equal confidence). Committed positions get x = a and flag
 * 0 in d_x / d_masked. With rule->sampling (stochastic tau-leaping,
 * [commentary] 3.4.1 "The Reverse Generation Process"): a linear schedule
 * over the block's steps_per_block steps fills each masked position with
 * probability 1 / (steps_per_block - step_in_block), with a token drawn from
 * softmax(z) by Gumbel-max (argmax of z + G); every draw comes from
 * Philox-4x64-10 with key (seed, sequence) and counter (v / 4, position,
 * step_in_block, 1) for the noise of ids v..v+3 (u = ((w >> 41) + 0.5) *
 * 2^-23, G = -log(-log u) in float32) and (0, position, step_in_block, 2)
 * for the fill decision (u = (w >> 11) * 2^-53 against the probability in
 * float64); committed positions take the drawn token. Outputs (each may be
 * NULL): d_conf, d_argmax [batch][blk_len] (conf of unmasked positions is
 * also reported), d_counts [batch][2] = {committed this call, still masked
 * in the block}, d_logits [batch][blk_len][vocab] float32 (debug dump). */
fdllm_status fdllm_confidence_unmask(fdllm_model* model, fdllm_cache* cache,
                                     const void* d_hidden_blk, int32_t* d_x, uint8_t* d_masked,
                                     int32_t batch, int32_t seq_len, int32_t blk_start,
                                     int32_t blk_len, const fdllm_select_params* rule,
                                     int32_t step_in_block, int32_t steps_per_block, float* d_conf,
                                     int32_t* d_argmax, int32_t* d_counts, float* d_logits,
                                     void* stream);

/* The same selection taking logits directly: d_logits [batch][blk_len][vocab]
 * in `dtype` (no logit scale applied; vocab a multiple of 8). Only rows still
 * masked are read. NaN logits count as -inf; +inf logits share the
 * probability mass equally (a row whose maximum is +inf gets confidence
 * 1 / (number of +inf entries) and the first of them as argmax). A row with
 * no finite or +inf logit gets confidence 0 and argmax -1. The call does not
 * synchronise. d_workspace holds per-row partial statistics (no initial
 * contents needed); query its size with fdllm_unmask_logits_workspace. */
fdllm_status fdllm_unmask_logits_workspace(int32_t batch, int32_t blk_len, int32_t vocab,
                                           size_t* bytes);
fdllm_status fdllm_confidence_unmask_logits(const void* d_logits, int32_t dtype, int32_t* d_x,
                                            uint8_t* d_masked, int32_t batch, int32_t seq_len,
                                            int32_t blk_start, int32_t blk_len, int32_t vocab,
                                            const fdllm_select_params* rule,
                                            int32_t step_in_block, int32_t steps_per_block,
                                            float* d_conf,
                                            int32_t* d_argmax, int32_t* d_counts,
                                            void* d_workspace, size_t workspace_bytes,
                                            void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops that must not call hipMalloc, harnesses that forbid
 * it): fdllm_confidence_unmask_logits with the same arguments and results
 * but no workspace. Its per-(row, chunk) statistics live in a fixed scratch
 * array inside the library, one copy per GPU, held until the process ends;
 * the call allocates nothing. At most FDLLM_NOALLOC_UNMASK_ENTRIES entries:
 * batch * blk_len * ceil(vocab / 16384) must not exceed it (FDLLM_EINVAL
 * otherwise). Every call on a GPU uses that GPU's one scratch array, so
 * calls that overlap on one GPU (other streams, other host threads) race
 * and must not be issued; consecutive calls on one stream are safe. The
 * scratch needs no initial contents. */
#define FDLLM_NOALLOC_UNMASK_ENTRIES 16384
fdllm_status fdllm_confidence_unmask_logits_noalloc(
    const void* d_logits, int32_t dtype, int32_t* d_x, uint8_t* d_masked, int32_t batch,
    int32_t seq_len, int32_t blk_start, int32_t blk_len, int32_t vocab,
    const fdllm_select_params* rule, int32_t step_in_block, int32_t steps_per_block, float* d_conf,
    int32_t* d_argmax, int32_t* d_counts, void* stream);

/* Block-wise decoding ([commentary] 3.2 information flow and 3.4.4 "The
 * Integrated Algorithm"). d_x [batch][prompt_len + gen_length] holds the
 * prompt followed by mask ids, d_masked the matching flags (1 on the
 * generated positions); both are updated in place to the decoded result.
 * For every block k (s = prompt_len + k*B): one cache refresh whose block
 * logits drive step 0, then cached forwards (PrefixCache rows [s, N),
 * DualCache rows [s, s+B)) or, with use_cache off, full forwards, each
 * followed by fdllm_confidence_unmask, until the block has no masked position
 * (at most T steps). Synchronises `stream` once per step to read the 8-byte
 * per-sequence counters, and at the end. With batch > 1 a block ends when
 * every sequence's block is done; finished sequences commit nothing. */
fdllm_status fdllm_decode(fdllm_model* model, fdllm_cache* cache, int32_t* d_x, uint8_t* d_masked,
                          int32_t batch, int32_t prompt_len, const fdllm_decode_params* params,
                          fdllm_decode_stats* stats, void* stream);

/* ---- K/V drift diagnostics ([commentary] 3.4.2 "The Empirical Justification:
 * Cosine Similarity of KV Activations") ----------------------------------- */

/* Device pointers to layer `layer`'s K and V inside the cache (layouts as
 * described at fdllm_cache_create) and the cache's row capacity ncap, so a
 * caller can snapshot them (K: batch * Hkv * ncap * D elements, V the same
 * count) and compare snapshots with fdllm_kv_cosine. The pointers stay valid
 * for the cache's lifetime; the cache's calls overwrite what they point at. */
fdllm_status fdllm_cache_kv(const fdllm_cache* cache, int32_t layer, void** d_k, void** d_v,
                            int32_t* ncap);

/* Per-token cosine similarity between two K/V snapshots a and b of one layer
 * (the measurement behind the approximate cache: how far a token's keys and
 * values move between two decoding steps). K [batch][n_kv_heads][cap][D];
 * V in the tile layout, [batch][n_kv_heads][ceil(cap / 32)][D][32]. For each
 * sequence s and row r in [row0, row1): d_cos[(s * (row1 - row0) + r - row0)
 * * 2 + 0] = cos(K_a, K_b) over the token's n_kv_heads * D key values, and
 * [... + 1] the same for V; cos = <a, b> / (|a| |b|) accumulated in float32,
 * 0 when either vector is all zero. Enqueued on `stream`. */
fdllm_status fdllm_kv_cosine(const void* d_k_a, const void* d_v_a, const void* d_k_b,
                             const void* d_v_b, int32_t batch, int32_t n_kv_heads, int32_t cap,
                             int32_t head_dim, int32_t row0, int32_t row1, int32_t dtype,
                             float* d_cos, void* stream);

/* ---- instrumentation (not part of the method) --------------------------- */

/* When enabled, every kernel launch the cache's calls enqueue is bracketed by
 * a pair of hipEvents on the launch stream, keyed by kernel variant (e.g.
 * "gemm_swiglu_bm64", "attention", "gemm_lmhead_bm32"), together with the
 * launch's algorithmic bytes (weights, activations and cache rows it must
 * move at least once) and algorithmic FLOPs (2 per multiply-add of the
 * mathematical product; the extra MFMA work of splitting float32
 * activations into two bf16 terms is not counted). Adds two event records
 * per launch. */
fdllm_status fdllm_cache_profile_enable(fdllm_cache* cache, int32_t enable);

/* Restricts the timing to launches of one kernel variant (variant NULL or ""
 * times every launch), and of those to every stride-th launch, so that the
 * events perturb a timed run less. Resets the launch counter. */
fdllm_status fdllm_cache_profile_select(fdllm_cache* cache, const char* variant, int32_t stride);

/* Peak rates for the per-launch floor the timer also sums: with both > 0,
 * every timed launch adds max(bytes / hbm_bytes_per_s, flops / flops_per_s)
 * (its time at the roofline of whichever resource bounds it) to its
 * variant's floor; 0 turns the floor off (the default). */
fdllm_status fdllm_cache_profile_peaks(fdllm_cache* cache, double hbm_bytes_per_s,
                                       double flops_per_s);

/* Waits for the recorded events and writes one text line per kernel variant,
 * "name launches total_ms total_bytes total_flops floor_ms", into buf
 * (NUL-terminated; EINVAL if len is too small). reset != 0 clears the totals
 * afterwards. */
fdllm_status fdllm_cache_profile_read(fdllm_cache* cache, char* buf, size_t len, int32_t reset);

/* Streaming read of d_buf (bytes a multiple of 16): up to 8 workgroups per
 * CU stride over the buffer in 16-byte loads, and each writes one float (a
 * checksum of what it read) to d_out; fdllm_stream_read_blocks gives the
 * number of floats d_out must hold. The HBM read rate this kernel reaches is
 * the measured ceiling the other kernels' rates are compared with. */
fdllm_status fdllm_stream_read_blocks(size_t bytes, int32_t* blocks);
fdllm_status fdllm_stream_read(const void* d_buf, size_t bytes, float* d_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FDLLM_H */

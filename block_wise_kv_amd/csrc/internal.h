// Internal launch interface between the C-ABI host code and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fdllm {

constexpr int kNT = 256;      // GEMM output-feature tile (4 waves x 4 fragments x 16)
constexpr int kMaxSsqTiles = 32;  // RMSNorm partial sums per row a normed GEMM reads (K <= 8192)
constexpr int kGateUp = 128;  // gate/up interleave unit: each 256-row tile = 128 gate + 128 up rows
constexpr int kMaxBlock = 64; // largest block_size the unmask kernels handle (one lane per position)

enum Dtype { kF32 = 0, kBF16 = 1 };

inline size_t dtype_bytes(int dt) { return dt == kBF16 ? 2 : 4; }
__host__ __device__ inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// ---- weight packing -------------------------------------------------------
enum PackMode { kPackPlain = 0, kPackQKV = 1, kPackGateUp = 2 };
// Packs a [N][K] matrix (or the concatenation / interleave named by mode) into
// MFMA fragment order, rows padded with zeros to a multiple of kNT.
size_t packed_matrix_bytes(int dt, int64_t n_rows, int64_t k);
hipError_t pack_matrix(int dt, int mode, const void* src0, const void* src1, const void* src2,
                       int64_t n0, int64_t n1, int64_t n2, int64_t k, int head_dim, void* dst,
                       hipStream_t st);

// ---- GEMM: out = X W^T with a fused epilogue -------------------------------
enum EpiMode { kEpiQKV = 0, kEpiResid = 1, kEpiSwiGLU = 2, kEpiLMHead = 3 };

struct EpiParams {
  // rows of the stacked activation matrix: row m belongs to sequence m / rows_per_seq
  // at absolute position row0 + m % rows_per_seq
  int rows_per_seq = 1, row0 = 0;
  // QKV: q -> q_out float32 [M][Hq*D]; k -> k_cache [b][Hkv][ncap][D]; v -> vt_cache
  // [b][Hkv][ncap/32][D][32] in the value cache's tile layout (vtile_off); the
  // cache in the model dtype
  void* q_out = nullptr;
  void* k_cache = nullptr;
  void* vt_cache = nullptr;
  int ncap = 0, n_heads = 0, n_kv_heads = 0, head_dim = 0;
  const float2* rope = nullptr;  // [max_pos][D/2] (cos, sin)
  // residual: h [M][N] += out; ssq_out [N/kNT][M] = per-tile row sum of squares of new h
  float* h = nullptr;
  float* ssq_out = nullptr;
  // residual: when xs_next is set, also (h * gain_next) in the split
  // activation layout with N / 32 slots per row block: the next GEMM's input
  char* xs_next = nullptr;
  const void* gain_next = nullptr;
  // SwiGLU: act in the split activation layout, (N / 2) / 32 slots per row block
  void* act = nullptr;
  // LM head: stats [M][n_tiles] (max, argmax, sumexp), with sampling also
  // sstats [M][n_tiles] (best z + G, its id); optional fp32 logits dump [M][N]
  float logit_scale = 1.f;
  float4* stats = nullptr;
  float2* sstats = nullptr;
  float* logits = nullptr;
  int* final_ticket = nullptr;
  // selection (LM head, run by the last workgroup)
  int32_t* x = nullptr;
  uint8_t* masked = nullptr;
  int batch = 0, seq_len = 0, blk_start = 0, blk_len = 0, step = 0, steps_per_block = 1;
  float tau = 0.f;
  float factor = 0.f;  // > 0: factor rule instead of the threshold
  int topk = 0;        // > 0: fixed top-K instead of either
  int sampling = 0;    // != 0: stochastic tau-leaping instead of a confidence rule
  uint32_t seed = 0;   // key of the sampling draws
  float* conf_out = nullptr;
  int32_t* argmax_out = nullptr;
  int32_t* counts_out = nullptr;
};

struct GemmProblem {
  int dt = kBF16;
  int mode = kEpiResid;
  // X of the layer projections (every mode but the LM head): the split
  // activation layout, K / 32 slots per 16-row block, rows padded past
  // the last row any tile height reads; with norm = true it already holds x * gain and the
  // epilogue applies the row factor rsqrt(sum_t ssq[t][m] / K + eps).
  // X of the LM head: float32 [M][K] (row stride ldx), normalised on the
  // fly when norm = true: x * rsqrt(sum_t ssq[t][m] / K + eps) * gain.
  const void* x = nullptr;
  int ldx = 0;
  bool norm = false;
  const float* ssq = nullptr;
  int ssq_tiles = 0;
  const void* gain = nullptr;
  float eps = 1e-5f;
  const void* w = nullptr;  // packed
  int M = 0, N = 0, K = 0;  // N: logical output features (packed rows padded to kNT)
  EpiParams ep;
};

struct GemmScratch {
  float* part = nullptr;   // partial tiles
  size_t part_elems = 0;
  int* tickets = nullptr;  // one per output tile
  int n_tickets = 0;
};

// Workgroup tiling chosen for a problem (exposed so scratch can be sized).
struct GemmPlan {
  int bm, kc, m_tiles, n_tiles, splits, k_per_split;
  size_t part_elems() const { return (size_t)m_tiles * n_tiles * splits * bm * kNT; }
  int tiles() const { return m_tiles * n_tiles; }
};
GemmPlan plan_gemm(int dt, int M, int N, int K, int mode);
hipError_t launch_gemm(const GemmProblem& p, const GemmScratch& s, hipStream_t st);

// ---- other kernels ------------------------------------------------------------
// h[m][:] = embed[x[seq(m)][row0 + m % R]]; ssq[t][m] partial sums of squares per kNT cols;
// xs = h * gain in the split activation layout (d / 32 slots per row block).
hipError_t launch_embed(int dt, const int32_t* x, int seq_len, int batch, int row0, int rows,
                        const void* embed, int d, float* h, float* ssq, int vocab,
                        const void* gain, void* xs, hipStream_t st);
// hidden[b][j][:] = rmsnorm(h[b*R + off + j]) * gain, float32.
hipError_t launch_final_norm(int dt, const float* h, const float* ssq, int d, int batch, int rows,
                             int off, int blk_len, const void* gain, float eps, void* hidden,
                             hipStream_t st);

// Value rows [b][Hkv][kv_len][D] -> the value cache's tile layout
// [b][Hkv][ceil(kv_len / 32)][D][32] (vtile_off), zero past kv_len.
hipError_t launch_tile_values(int dt, const void* v, void* vt, int batch, int hkv, int kv_len, int D,
                              hipStream_t st);
// Streaming read of `bytes` (a multiple of 16) from buf: one float per
// workgroup into out (the sum of the words read, so the loads are kept).
int stream_read_blocks(size_t bytes);
hipError_t launch_stream_read(const void* buf, size_t bytes, float* out, hipStream_t st);

// Per-token cosine similarity of two K/V snapshots in the cache layout (K
// [b][Hkv][cap][D], V in the tile layout); out [b][nrows][2] (K, V).
hipError_t launch_kv_cosine(int dt, const void* ka, const void* va, const void* kb, const void* vb,
                            int batch, int hkv, int cap, int D, int row0, int nrows, float* out,
                            hipStream_t st);

// Block attention over a cache laid out as K [b][Hkv][ncap][D], V in the tile
// layout [b][Hkv][ncap/32][D][32] (vtile_off).
struct AttnProblem {
  int dt = kBF16;           // cache (k, v) element type
  int qdt = kBF16;          // q and o element type (float32 queries split in two bf16 terms)
  const void* q = nullptr;  // [b][rows][Hq][D]
  void* o = nullptr;        // same layout as q, or with xs_out the split activation layout
  bool xs_out = false;      // o as the next GEMM's split input ([b * rows][Hq * D])
  const void* k = nullptr;   // [b][Hkv][ncap][D]
  const void* vt = nullptr;  // [b][Hkv][ceil(ncap / 32)][D][32], tile layout (vtile_off)
  int batch = 0, rows = 0, hq = 0, hkv = 0, d = 0, kv_len = 0, ncap = 0;
  float scale = 1.f;
  float* part = nullptr;    // split partials
  int* tickets = nullptr;
  int splits = 1;
  float* lse = nullptr;     // optional [b][rows][Hq]: natural log of sum_k exp(scale q.k)
};
constexpr int kAttnSplitTarget = 192;  // workgroups the attention split planner aims for
int plan_attention_splits(int batch, int rows, int hq, int kv_len);
size_t attention_part_floats(int batch, int rows, int hq, int d, int splits);
int attention_tickets(int batch, int rows, int hq);
hipError_t launch_attention(const AttnProblem& p, hipStream_t st);

// Logits-in confidence unmask.
int unmask_chunks(int vocab);
// Selection rule arguments of the host API (the device-side SelectRule in
// select.h carries the same fields).
struct SelectRuleArgs {
  float tau = 0.9f;
  float factor = 0.f;
  int topk = 0;
  int sampling = 0;
  uint32_t seed = 0;
};
// stats holds [batch*blk_len][chunks] float4 followed by as many float2
// (sampling statistics).
// The allocation-free variant's fixed scratch: at most this many (row,
// chunk) statistics entries, and the current device's address of it (looked
// up once per device with hipGetSymbolAddress).
constexpr int kStaticUnmaskEntries = 16384;
hipError_t unmask_static_scratch(float4** out);
hipError_t launch_unmask_logits(int dt, const void* logits, int32_t* x, uint8_t* masked, int batch,
                                int seq_len, int blk_start, int blk_len, int vocab,
                                const SelectRuleArgs& rule, int step, int steps_per_block,
                                float* conf, int32_t* argmax, int32_t* counts, float4* stats,
                                hipStream_t st);

}  // namespace fdllm

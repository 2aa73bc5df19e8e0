// Weight packing and the projection GEMMs of the transformer forward:
// out[m][n] = sum_k X[m][k] W[n][k], with W streamed from HBM in MFMA
// fragment order and the float32 activations X staged through LDS (for bf16
// weights as two bf16 terms, hi + lo, so the product keeps ~16 significant
// bits of X; float32 weights use float32 MFMA), split along K when the output
// tile count alone cannot fill 256 CUs, and a fused epilogue that works on
// the accumulator registers directly:
//   QKV     rotate-half RoPE at absolute positions on q and k; q to a buffer,
//           k and v written straight into the layer's KV cache rows
//   Resid   residual add into the float32 stream h plus per-tile row sums of
//           squares, from which the next GEMM applies RMSNorm on the fly
//   SwiGLU  silu(gate) * up
//   LMHead  logits * scale reduced to per-tile (max, argmax, sum exp); the
//           last workgroup merges all tiles and runs the threshold selection
// Packed rows are permuted so that the operands an epilogue combines (the two
// halves a RoPE rotation pairs, a gate row and its up row) sit in the same
// lane. Cross-workgroup merges (split-K sums, vocabulary tiles) use a
// completion ticket and a fixed merge order, so results do not depend on
// scheduling.
#include <cmath>
#include <map>
#include <tuple>

#include "common.h"
#include "internal.h"
#include "select.h"

namespace fdllm {

// ---------------------------------------------------------------------------
// Layout of a 256-row output tile: tile column c belongs to wave c / 64,
// fragment (c % 64) / 16, fragment row c % 16.
//
// QKV: within each head, packed head-local row p maps to feature d(p) =
//   (p / 64) * (D / 4) + ((p / 16) & 1) * 16 + ((p / 32) & 1) * (D / 2) + p % 16,
// so fragments f and f + 2 of a wave hold the rotation partners d and d + D/2.
__host__ __device__ __forceinline__ int qkv_feature(int p, int D) {
  return (p >> 6) * (D >> 2) + ((p >> 4) & 1) * 16 + ((p >> 5) & 1) * (D >> 1) + (p & 15);
}
// gate/up: packed row n -> (feature, is_up); even fragments gate, odd up.
__host__ __device__ __forceinline__ int gateup_feature(int64_t n, bool* is_up) {
  int64_t t = n / kNT;
  int c = (int)(n % kNT);
  int w = c >> 6, f = (c >> 4) & 3, r = c & 15;
  *is_up = (f & 1) != 0;
  return (int)(t * kGateUp + w * 32 + (f >> 1) * 16 + r);
}

// Packing: element (n, k) of the (permuted) [N][K] matrix goes to lane
// (n % 16) + 16 * ((k % 32) / 8), slot k % 8 of fragment (n % 64) / 16 of
// slab n / 64 of step k / 32; storage order [step][slab][fragment][lane][slot].
// A wave owns one 64-row slab, so each of its steps reads one contiguous
// 4-fragment block (4 KB of bf16), and the waves working on the same steps
// at the same time read adjacent blocks, which spreads them over all HBM
// channels instead of camping on the channel of a common slab offset.
template <typename E>
__global__ void pack_kernel(int mode, const E* __restrict__ s0, const E* __restrict__ s1,
                            const E* __restrict__ s2, int64_t n0, int64_t n1, int64_t n2,
                            int64_t K, int64_t n_pad, int head_dim, E* __restrict__ dst) {
  const int64_t KB = K / 32;
  const int64_t total = n_pad / 16 * KB * 64;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n_slabs = n_pad / 64;
    const int lane = (int)(e % 64);
    const int fr = (int)((e / 64) % 4);
    const int64_t slab = (e / 256) % n_slabs;
    const int64_t kb = e / (256 * n_slabs);
    const int64_t n = slab * 64 + fr * 16 + (lane & 15);
    const int64_t k = kb * 32 + 8 * (lane >> 4);
    const E* src = nullptr;
    if (mode == kPackPlain) {
      if (n < n0) src = s0 + n * K;
    } else if (mode == kPackQKV) {
      const E* base = nullptr;
      int64_t rel = 0;
      if (n < n0) { base = s0; rel = n; }
      else if (n < n0 + n1) { base = s1; rel = n - n0; }
      else if (n < n0 + n1 + n2) { base = s2; rel = n - n0 - n1; }
      if (base) {
        int64_t head = rel / head_dim;
        int p = (int)(rel % head_dim);
        src = base + (head * head_dim + qkv_feature(p, head_dim)) * K;
      }
    } else {  // gate/up, n0 = ffn_dim
      bool up;
      int feat = gateup_feature(n, &up);
      if (feat < n0) src = (up ? s1 : s0) + (int64_t)feat * K;
    }
    E* d = dst + e * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) d[j] = src ? src[k + j] : (E)0;
  }
}

size_t packed_matrix_bytes(int dt, int64_t n_rows, int64_t k) {
  return (size_t)round_up(n_rows, kNT) * (size_t)k * dtype_bytes(dt);
}

hipError_t pack_matrix(int dt, int mode, const void* src0, const void* src1, const void* src2,
                       int64_t n0, int64_t n1, int64_t n2, int64_t k, int head_dim, void* dst,
                       hipStream_t st) {
  int64_t rows = mode == kPackQKV ? n0 + n1 + n2 : (mode == kPackGateUp ? 2 * n0 : n0);
  int64_t n_pad = round_up(rows, kNT);
  int64_t total = n_pad / 16 * (k / 32) * 64;
  int grid = (int)std::min<int64_t>((total + 255) / 256, 65536);
  if (dt == kBF16)
    hipLaunchKernelGGL(pack_kernel<uint16_t>, dim3(grid), dim3(256), 0, st, mode,
                       (const uint16_t*)src0, (const uint16_t*)src1, (const uint16_t*)src2, n0, n1,
                       n2, k, n_pad, head_dim, (uint16_t*)dst);
  else
    hipLaunchKernelGGL(pack_kernel<float>, dim3(grid), dim3(256), 0, st, mode, (const float*)src0,
                       (const float*)src1, (const float*)src2, n0, n1, n2, k, n_pad, head_dim,
                       (float*)dst);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// GEMM kernel. Workgroup = 4 waves; output tile BM rows x kNT features; wave w
// owns tile columns [w*64, w*64+64) as 4 fragments. Its W fragments for one K
// chunk (KC/32 steps) stay in flight in registers while the previous chunk is
// multiplied; X chunks are double-buffered in LDS.
constexpr int kWN = 4;

// K chunk per tile height: deeper weight prefetch for the skinniest tiles; the
// tall tiles' double-buffered X chunks fill most of the 160 KB of LDS.
constexpr int gemm_kc(int bm) { return bm <= 32 ? 256 : 128; }
constexpr int gemm_occupancy(int bm) { return bm <= 64 ? 2 : 1; }  // workgroups per CU

// X operand of one MFMA step: bf16 weights take X as hi + lo bf16 terms (two
// MFMAs); float32 weights take X as float32.
template <typename T> struct XFrag;
template <> struct XFrag<BF16> { FragBF hi, lo; };
template <> struct XFrag<F32> { FragF32 v; };

__device__ __forceinline__ void mma_x(f32x4_t& acc, const FragBF& w, const XFrag<BF16>& x) {
  mma(acc, w, x.hi);
  mma(acc, w, x.lo);
}
__device__ __forceinline__ void mma_x(f32x4_t& acc, const FragF32& w, const XFrag<F32>& x) {
  mma(acc, w, x.v);
}

// An X fragment slot in LDS is two 1 KB blocks (64 lanes x 16 B): hi / lo
// bf16 terms, or elements 0-3 / 4-7 of the float32 fragment.
__device__ __forceinline__ void load_xfrag(XFrag<BF16>& x, const char* slot, int lane) {
  x.hi.v = *(const uint4*)(slot + lane * 16);
  x.lo.v = *(const uint4*)(slot + 1024 + lane * 16);
}
__device__ __forceinline__ void load_xfrag(XFrag<F32>& x, const char* slot, int lane) {
  x.v.lo = *(const float4*)(slot + lane * 16);
  x.v.hi = *(const float4*)(slot + 1024 + lane * 16);
}

// LM head, last workgroup: merges the vocabulary tiles' statistics of rows
// wv, wv + 4, ... (row m by wave m % 4) in tile order within a lane, then by a
// fixed butterfly across lanes, and leaves each row's 1 / sum, argmax and
// sampled id in LDS. The statistics are read with coherent loads that miss the
// L2, so a lane issues its tiles of kR rows (kB per row) together and merges
// each row's in tile order. Indices past the last tile re-read it and are not
// merged: a select, not a branch, so the loads stay batched. The sampling
// statistics are read only when sampling; without them a lane has the
// registers for four rows at a time, which halves the load round trips and
// lets four rows' butterflies interleave.
template <bool kSamp>
__device__ __forceinline__ void lm_merge_rows(const EpiParams& e, int M, int n_tiles, int wv, int lane,
                                              float* s_c, int* s_a, int* s_tok) {
  constexpr int kB = 8, kR = kSamp ? 2 : 4;
  const auto rs = agent_rsrc(e.stats);    // uniform resources, the row and
  const auto rss = agent_rsrc(e.sstats);  // tile in the per-lane offset
  for (int mb = wv; mb < M; mb += 4 * kR) {
    SoftStat st[kR];
    SampStat ss[kR];
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      st[r] = stat_empty();
      ss[r] = samp_empty();
    }
    for (int t0 = lane; t0 < n_tiles; t0 += 64 * kB) {
      f32x4_t s4[kR][kB];
      f32x2_t s2[kR][kB];
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int m = min(mb + 4 * r, M - 1);
#pragma unroll
        for (int q = 0; q < kB; ++q) {
          const int t = m * n_tiles + min(t0 + 64 * q, n_tiles - 1);
          s4[r][q] = ld_agent4(rs, t * 16);
          if constexpr (kSamp) s2[r][q] = ld_agent2(rss, t * 8);
        }
      }
#pragma unroll
      for (int r = 0; r < kR; ++r)
#pragma unroll
        for (int q = 0; q < kB; ++q) {
          const bool live = t0 + 64 * q < n_tiles;
          const SoftStat a = stat_merge(st[r], SoftStat{s4[r][q][0], __float_as_int(s4[r][q][1]), s4[r][q][2]});
          st[r].m = live ? a.m : st[r].m;
          st[r].a = live ? a.a : st[r].a;
          st[r].s = live ? a.s : st[r].s;
          if constexpr (kSamp) {
            const SampStat b = samp_merge(ss[r], SampStat{s2[r][q][0], __float_as_int(s2[r][q][1])});
            ss[r].m = live ? b.m : ss[r].m;
            ss[r].a = live ? b.a : ss[r].a;
          }
        }
    }
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const int m = mb + 4 * r;
      const SoftStat t = stat_wave_reduce(st[r]);
      const SampStat u = kSamp ? samp_wave_reduce(ss[r]) : ss[r];
      if (lane == 0 && m < M && m < kMaxBlock * 4) {
        s_c[m] = 1.f / t.s;
        s_a[m] = t.a;
        s_tok[m] = u.a;
      }
    }
  }
}

template <typename T, int BM, int KC>
struct GemmLds {
  static constexpr int FB = FragInfo<T>::kBytes;  // W fragment bytes per lane
  static constexpr int MT = BM / 16;
  static constexpr int KS = KC / 32;
  static constexpr int kSlot = 2048;               // bytes of one X fragment slot
  static constexpr int kBufBytes = MT * KS * kSlot;
};

// Stages a BM x KC chunk of the float32 activations into LDS fragment slots,
// optionally applying RMSNorm (x * rinv[row] * gain[k]) on the way.
template <typename T, int BM, int KC, bool NORM>
struct XStager {
  using E = typename T::store_t;
  using L = GemmLds<T, BM, KC>;
  static constexpr int kGroupsPerRow = KC / 8;
  static constexpr int kGroups = BM * kGroupsPerRow / 256;  // 8-element groups per thread
  static_assert(BM * kGroupsPerRow % 256 == 0, "tile too small for one pass");
  float v[kGroups][8];
  uint4 gain[NORM ? kGroups : 1][sizeof(E) * 8 / 16];  // raw norm gains of each group

  // Every thread issues the same loads on every chunk (rows past M read the
  // last row and are zeroed), so the compiler's in-order load counting can
  // wait for exactly the loads each step needs. The norm gains are loaded
  // here too, so that staging never waits on a load younger than the
  // weight prefetch.
  // Group gi is lane gi % 64 of fragment slot gi / 64 (slot = row block *
  // KS + step): row 16 * (slot / KS) + lane % 16, k group 4 * (slot % KS) +
  // lane / 16. A wave thus writes one slot's 1 KB contiguously (no LDS bank
  // conflicts) and reads 128 contiguous bytes of each of 16 rows.
  __device__ __forceinline__ static void group_of(int gi, int& r, int& kg) {
    const int slot = gi >> 6, l = gi & 63;
    r = 16 * (slot / L::KS) + (l & 15);
    kg = 4 * (slot % L::KS) + (l >> 4);
  }

  __device__ __forceinline__ void load(const GemmProblem& p, int m0, int kc0, int tid) {
#pragma unroll
    for (int i = 0; i < kGroups; ++i) {
      int r, kg;
      group_of(tid + i * 256, r, kg);
      int m = m0 + r, k = kc0 + 8 * kg;
      const float4* src = (const float4*)((const float*)p.x + (size_t)min(m, p.M - 1) * p.ldx + k);
      float4 a = src[0];  // rows past M are zeroed by their row scale in store()
      float4 b = src[1];
      v[i][0] = a.x; v[i][1] = a.y; v[i][2] = a.z; v[i][3] = a.w;
      v[i][4] = b.x; v[i][5] = b.y; v[i][6] = b.z; v[i][7] = b.w;
      if constexpr (NORM) {
        const uint4* g = (const uint4*)((const E*)p.gain + k);
#pragma unroll
        for (int q = 0; q < (int)(sizeof(E) * 8 / 16); ++q) gain[i][q] = g[q];
      }
    }
  }

  __device__ __forceinline__ void store(char* buf, const GemmProblem& p, const float* rinv,
                                        int kc0, int tid) {
#pragma unroll
    for (int i = 0; i < kGroups; ++i) {
      const int gi = tid + i * 256;
      int r, kg;
      group_of(gi, r, kg);
      char* slot = buf + (gi >> 6) * L::kSlot + (gi & 63) * 16;
      // row scale: the RMSNorm factor (1 without norm), 0 for rows past M
      const float s = rinv[r];
      float o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = v[i][j] * s;
      if constexpr (NORM) {
        const E* g = (const E*)&gain[i][0];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = o[j] * T::to_f(g[j]);
      }
      if constexpr (sizeof(E) == 2) {
        uint4 hi, lo;
        split_bf16x8(o, hi, lo);
        *(uint4*)slot = hi;
        *(uint4*)(slot + 1024) = lo;
      } else {
        *(float4*)slot = *(float4*)&o[0];
        *(float4*)(slot + 1024) = *(float4*)&o[4];
      }
    }
  }
};

// Stages the BM x KC chunk at rows m0, columns k0 of a split activation
// matrix into the LDS fragment slots: the chunk is MT row blocks of KS
// contiguous 2 KB slots in both places, so thread t copies 16-byte pieces
// t, t + 256, ... (one slot's 2 KB is 128 consecutive pieces), through
// registers: load() issues the reads, store() writes LDS.
template <typename T, int BM, int KC>
struct XSStager {
  using L = GemmLds<T, BM, KC>;
  static constexpr int kPieces = L::MT * L::KS * 128;
  static constexpr int kPer = kPieces / 256;
  static_assert(kPieces % 256 == 0, "chunk too small for one pass");
  u32x4_t v[kPer];
  __device__ __forceinline__ void load(const char* xs, int kslots, int m0, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int q = tid + 256 * i, slot = q >> 7;
      const int a = slot / L::KS, j = slot % L::KS;
      v[i] = *(const u32x4_t*)(xs + ((size_t)((m0 >> 4) + a) * kslots + (k0 >> 5) + j) * 2048 +
                             (q & 127) * 16);
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) *(u32x4_t*)(lds + (tid + 256 * i) * 16) = v[i];
  }
};

__device__ __forceinline__ float silu(float x) { return x / (1.f + __expf(-x)); }

template <typename T>
__device__ __forceinline__ void store4(void* base, size_t idx, float a, float b, float c, float d) {
  using E = typename T::store_t;
  E* p = (E*)base + idx;
  if constexpr (sizeof(E) == 2) {
    *(uint2*)p = make_uint2(f2bf2(a, b), f2bf2(c, d));
  } else {
    *(float4*)p = make_float4(a, b, c, d);
  }
}

// Weight fragments: read once (non-temporal) when a single row tile covers M;
// with several row tiles, the tiles of one weight slab run back to back on
// one XCD and re-read it from that XCD's L2, so the loads keep it there.
template <bool SHARED, typename F>
__device__ __forceinline__ void load_w(F& f, const void* p) {
  if constexpr (SHARED)
    load_frag_cached(f, p);
  else
    load_frag(f, p);
}

// Tiles up to 64 rows fit two workgroups per CU (<= 256 registers per lane).
template <typename T, int BM, int KC, int MODE, bool NORM, bool SHARED>
__global__ __launch_bounds__(256, gemm_occupancy(BM)) void gemm_kernel(GemmProblem p, GemmPlan pl,
                                                                      GemmScratch sc) {
  using F = typename Frag<T>::type;
  using L = GemmLds<T, BM, KC>;
  constexpr int MT = L::MT, KS = L::KS, FB = L::FB;
  __shared__ __align__(16) char xs[2][L::kBufBytes];  // X chunks, double-buffered
  __shared__ float s_rinv[BM];  // per-row scale applied while staging X
  __shared__ float s_ssq[256];  // RMSNorm partial sums of split activations
  __shared__ float4 s_red[4][BM];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int w = xcd_remap(blockIdx.x, gridDim.x);
  const int mt = w % pl.m_tiles;
  w /= pl.m_tiles;
  const int split = w % pl.splits;
  const int nt = w / pl.splits;
  const int m0 = mt * BM, n0 = nt * kNT;
  const int k0 = split * pl.k_per_split;
  const int k1 = min(p.K, k0 + pl.k_per_split);
  const int nchunks = max(0, k1 - k0) / KC;

  // Layer projections read activations already split into their operand
  // slots (a plain copy into LDS); the LM head stages float32 rows,
  // splitting and normalising them on the way.
  constexpr bool kXS = MODE != kEpiLMHead;
  if constexpr (!kXS) {
    if (tid < BM) {
      const int m = m0 + tid;
      float scale = 0.f;
      if (m < p.M) {
        scale = 1.f;
        if constexpr (NORM) {
          float s = 0.f;
          for (int t = 0; t < p.ssq_tiles; ++t) s += p.ssq[(size_t)t * p.M + m];
          scale = rsqrtf(s / (float)p.K + p.eps);
        }
      }
      s_rinv[tid] = scale;
    }
    __syncthreads();
  }
  // Split activations with RMSNorm take the row factor in the epilogue. Its
  // partial sums of squares are loaded here, ahead of the operand loads, so
  // no wait for them delays the first chunk: thread tid takes row tid % BM
  // and tiles tid / BM + i * (256 / BM), and leaves their sum in s_ssq[tid].
  constexpr int kRowThr = 256 / BM;
  constexpr int kSsqPer = (kXS && NORM) ? (kMaxSsqTiles + kRowThr - 1) / kRowThr : 1;
  float ssq_part[kSsqPer];
  if constexpr (kXS && NORM) {
    const int m = min(m0 + tid % BM, p.M - 1);
#pragma unroll
    for (int i = 0; i < kSsqPer; ++i) {
      const int t = tid / BM + i * kRowThr;
      // 48-row tiles: threads past kRowThr * BM take no tile (256 % 48 != 0)
      ssq_part[i] = (t < p.ssq_tiles && tid < kRowThr * BM) ? p.ssq[(size_t)t * p.M + m] : 0.f;
    }
  }

  // this wave's slab from step k0 / 32: step j, fragment f at
  // wbase + (j * n_slabs * 4 + f) * 64 * FB
  const int n_slabs = pl.n_tiles * (kNT / 64);
  const size_t step_bytes = (size_t)n_slabs * kWN * 64 * FB;
  const char* wbase = (const char*)p.w + (size_t)(k0 / 32) * step_bytes +
                      (size_t)(n0 / 64 + wv) * kWN * 64 * FB + (size_t)lane * FB;

  f32x4_t acc[MT][kWN];
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int f = 0; f < kWN; ++f) acc[a][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // K range of this workgroup: nchunks whole chunks of KC (K and the split
  // length are multiples of KC). W fragments of the next chunk are loaded
  // while the current one is multiplied; X chunks are double-buffered in LDS.
  XStager<T, BM, KC, NORM> xst;
  XSStager<T, BM, KC> xss;
  F wbuf[KS][kWN];
  // Program order is pinned (sched_barrier): step j's multiplies, then the
  // refill of its registers with step j of the next chunk. Left alone, the
  // scheduler hoists all refills above the multiplies, which doubles the
  // weight registers and makes the first multiply wait for the refills.
  // Tiles of 48 rows and more (bf16) read the X fragments of step j + 1
  // from LDS before the multiplies of step j, so their latency hides behind
  // those multiplies (the 16- and 32-row tiles have no registers to spare;
  // 48-row tiles measured ~2 % faster with it, 210 VGPRs).
  constexpr bool kPipeX = sizeof(typename T::store_t) == 2 && MT >= 3;
  auto mul_chunk = [&](const char* xb, bool refill, int next_step0) {
    XFrag<T> xf[2][MT];
    if constexpr (kPipeX)
#pragma unroll
      for (int a = 0; a < MT; ++a) load_xfrag(xf[0][a], xb + a * KS * L::kSlot, lane);
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      if constexpr (kPipeX) {
        if (j + 1 < KS)
#pragma unroll
          for (int a = 0; a < MT; ++a)
            load_xfrag(xf[(j + 1) & 1][a], xb + (a * KS + j + 1) * L::kSlot, lane);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int a = 0; a < MT; ++a)
#pragma unroll
          for (int f = 0; f < kWN; ++f) mma_x(acc[a][f], wbuf[j][f], xf[j & 1][a]);
      } else {
#pragma unroll
        for (int a = 0; a < MT; ++a) {
          load_xfrag(xf[0][a], xb + (a * KS + j) * L::kSlot, lane);
#pragma unroll
          for (int f = 0; f < kWN; ++f) mma_x(acc[a][f], wbuf[j][f], xf[0][a]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (refill)
#pragma unroll
        for (int f = 0; f < kWN; ++f)
          load_w<SHARED>(wbuf[j][f], wbase + (size_t)(next_step0 + j) * step_bytes + f * 64 * FB);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Either way the next chunk's reads are in flight during the current
  // chunk's multiplies.
  const int kslots = p.K >> 5;
  const char* xsrc = (const char*)p.x;
  if (nchunks > 0) {
    if constexpr (kXS)
      xss.load(xsrc, kslots, m0, k0, tid);
    else
      xst.load(p, m0, k0, tid);
#pragma unroll
    for (int j = 0; j < KS; ++j)
#pragma unroll
      for (int f = 0; f < kWN; ++f)
        load_w<SHARED>(wbuf[j][f], wbase + (size_t)j * step_bytes + f * 64 * FB);
    if constexpr (kXS && NORM) {
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < kSsqPer; ++i) sum += ssq_part[i];
      s_ssq[tid] = sum;
    }
    if constexpr (kXS)
      xss.store(xs[0], tid);
    else
      xst.store(xs[0], p, s_rinv, k0, tid);
    __syncthreads();
    for (int c = 0; c + 1 < nchunks; ++c) {
      const int kn = k0 + (c + 1) * KC;
      if constexpr (kXS)
        xss.load(xsrc, kslots, m0, kn, tid);
      else
        xst.load(p, m0, kn, tid);
      mul_chunk(xs[c & 1], true, (c + 1) * KS);
      if constexpr (kXS)
        xss.store(xs[(c + 1) & 1], tid);
      else
        xst.store(xs[(c + 1) & 1], p, s_rinv, kn, tid);
      __syncthreads();
    }
    mul_chunk(xs[(nchunks - 1) & 1], false, 0);
  } else if constexpr (kXS && NORM) {
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < kSsqPer; ++i) sum += ssq_part[i];
    s_ssq[tid] = sum;
    __syncthreads();
  }

  // ---- split-K: partials in register order, summed in split order ----
  // The residual epilogue's h rows are loaded by the summing workgroup
  // together with the partial tiles, not after them.
  float4 hpre[MODE == kEpiResid ? MT : 1][kWN];
  bool have_h = false;
  if (pl.splits > 1) {
    constexpr int kPer = MT * kWN * 64 * 16;  // bytes per wave per split
    const size_t tile = (size_t)(mt * pl.n_tiles + nt);
    const auto rs = agent_rsrc((const char*)sc.part + tile * pl.splits * 4 * kPer);
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
      for (int f = 0; f < kWN; ++f)
        st_agent4(rs, (split * 4 + wv) * kPer + ((a * kWN + f) * 64 + lane) * 16, acc[a][f]);
    if (!last_arrival(sc.tickets + tile, pl.splits)) return;
    if constexpr (MODE == kEpiResid) {
#pragma unroll
      for (int a = 0; a < MT; ++a) {
        const int m = m0 + 16 * a + (lane & 15);
#pragma unroll
        for (int f = 0; f < kWN; ++f)
          if (m < p.M)
            hpre[a][f] = *(const float4*)(p.ep.h + (size_t)m * p.N + n0 + wv * 64 + 4 * (lane >> 4) + 16 * f);
      }
      have_h = true;
    }
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
      for (int f = 0; f < kWN; ++f) acc[a][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // splits summed in order 0, 1, 2, ...: one split's whole tile in flight
    // at a time
    for (int s = 0; s < pl.splits; ++s) {
      f32x4_t t[MT][kWN];
#pragma unroll
      for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int f = 0; f < kWN; ++f)
          t[a][f] = ld_agent4(rs, (s * 4 + wv) * kPer + ((a * kWN + f) * 64 + lane) * 16);
#pragma unroll
      for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int f = 0; f < kWN; ++f) acc[a][f] += t[a][f];
    }
  }

  // ---- epilogue on the accumulators: element (a, f, i) is output row
  //      m0 + 16a + (lane & 15), tile column wv*64 + 16f + 4(lane >> 4) + i ----
  if constexpr (kXS && NORM) {
    // the split input held x * gain: apply the RMSNorm row factor now
#pragma unroll
    for (int a = 0; a < MT; ++a) {
      const int r0 = 16 * a + (lane & 15);
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < kRowThr; ++j) ss += s_ssq[r0 + j * BM];
      const float r = rsqrtf(ss / (float)p.K + p.eps);
#pragma unroll
      for (int f = 0; f < kWN; ++f) acc[a][f] *= r;
    }
  }
  const EpiParams& e = p.ep;
  const int rl = lane & 15, g4 = 4 * (lane >> 4);
  const int cw = wv * 64 + g4;  // tile column of fragment 0, element 0

  if constexpr (MODE == kEpiQKV) {
    const int D = e.head_dim, qd = e.n_heads * D, kvd = e.n_kv_heads * D;
#pragma unroll
    for (int a = 0; a < MT; ++a) {
      const int m = m0 + 16 * a + rl;
      if (m >= p.M) continue;
      const int seq = m / e.rows_per_seq, pos = e.row0 + m % e.rows_per_seq;
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int n = n0 + cw + 16 * f;  // packed row of element 0; partner at fragment f + 2
        if (n >= p.N) continue;
        const bool is_q = n < qd, is_k = !is_q && n < qd + kvd;
        const int rel = is_q ? n : (is_k ? n - qd : n - qd - kvd);
        const int hd = rel / D;
        const int d1 = qkv_feature(rel % D, D);  // d1 < D/2, partner d1 + D/2
        const int d2 = d1 + D / 2;
        f32x4_t x1 = acc[a][f], x2 = acc[a][f + 2];
        float o1[4], o2[4];
        if (is_q || is_k) {
          const float2* cs = e.rope + (size_t)pos * (D / 2) + d1;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float2 t = cs[i];
            o1[i] = x1[i] * t.x - x2[i] * t.y;
            o2[i] = x2[i] * t.x + x1[i] * t.y;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) { o1[i] = x1[i]; o2[i] = x2[i]; }
        }
        if (is_q) {
          size_t b = (size_t)m * qd + (size_t)hd * D;
          store4<F32>(e.q_out, b + d1, o1[0], o1[1], o1[2], o1[3]);
          store4<F32>(e.q_out, b + d2, o2[0], o2[1], o2[2], o2[3]);
        } else if (is_k) {
          size_t b = (((size_t)seq * e.n_kv_heads + hd) * e.ncap + pos) * D;
          store4<T>(e.k_cache, b + d1, o1[0], o1[1], o1[2], o1[3]);
          store4<T>(e.k_cache, b + d2, o2[0], o2[1], o2[2], o2[3]);
        } else {
          using E = typename T::store_t;
          E* vt = (E*)e.vt_cache + ((size_t)seq * e.n_kv_heads + hd) * D * e.ncap;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            vt[vtile_off(pos, d1 + i, D)] = T::from_f(o1[i]);
            vt[vtile_off(pos, d2 + i, D)] = T::from_f(o2[i]);
          }
        }
      }
    }
  } else if constexpr (MODE == kEpiResid) {
#pragma unroll
    for (int a = 0; a < MT; ++a) {
      const int m = m0 + 16 * a + rl;
      float ss = 0.f;
      if (m < p.M) {
#pragma unroll
        for (int f = 0; f < kWN; ++f) {
          const int n = n0 + cw + 16 * f;
          float4* hp = (float4*)(e.h + (size_t)m * p.N + n);
          float4 hv = have_h ? hpre[a][f] : *hp;
          hv.x += acc[a][f][0]; hv.y += acc[a][f][1]; hv.z += acc[a][f][2]; hv.w += acc[a][f][3];
          *hp = hv;
          ss += hv.x * hv.x + hv.y * hv.y + hv.z * hv.z + hv.w * hv.w;
          if (e.xs_next) {
            using E = typename T::store_t;
            const E* g = (const E*)e.gain_next + n;
            XSplit<T>::store4(e.xs_next, p.N >> 5, m, n, hv.x * T::to_f(g[0]), hv.y * T::to_f(g[1]),
                              hv.z * T::to_f(g[2]), hv.w * T::to_f(g[3]));
          }
        }
      }
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      if (lane < 16) s_red[wv][16 * a + lane].x = ss;
    }
    __syncthreads();
    if (tid < BM && m0 + tid < p.M)
      e.ssq_out[(size_t)nt * p.M + m0 + tid] =
          ((s_red[0][tid].x + s_red[1][tid].x) + s_red[2][tid].x) + s_red[3][tid].x;
  } else if constexpr (MODE == kEpiSwiGLU) {
    const int F_ = p.N / 2;
#pragma unroll
    for (int a = 0; a < MT; ++a) {
      const int m = m0 + 16 * a + rl;
      if (m >= p.M) continue;
#pragma unroll
      for (int f = 0; f < kWN; f += 2) {
        const int feat = nt * kGateUp + wv * 32 + (f >> 1) * 16 + g4;
        if (feat >= F_) continue;
        f32x4_t g = acc[a][f], u = acc[a][f + 1];
        XSplit<T>::store4((char*)e.act, F_ >> 5, m, feat, silu(g[0]) * u[0], silu(g[1]) * u[1],
                          silu(g[2]) * u[2], silu(g[3]) * u[3]);
      }
    }
  } else {  // LM head
    // with sampling, also the best z + G of the row's tile (Gumbel-max draw,
    // philox.h); its (score, id) rides in the spare half of s_red
    __shared__ float2 s_samp[4][BM];
#pragma unroll
    for (int a = 0; a < MT; ++a) {
      const int m = m0 + 16 * a + rl;
      SoftStat st = stat_empty();
      SampStat ss = samp_empty();
      if (m < p.M) {
        const int seq = m / e.blk_len, pos = e.blk_start + m % e.blk_len;
#pragma unroll
        for (int f = 0; f < kWN; ++f) {
          const int n = n0 + cw + 16 * f;  // a multiple of 4
          U64x4 r{};
          if (e.sampling)
            r = philox4x64((uint64_t)(n >> 2), (uint64_t)pos, (uint64_t)e.step, 1, e.seed,
                           (uint64_t)seq);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (n + i < p.N) {
              float z = acc[a][f][i] * e.logit_scale;
              stat_push(st, z, n + i);
              if (e.sampling) {
                const float sc = z + gumbel_of(r.w[i]);
                if (sc > ss.m) ss = SampStat{sc, n + i};  // ids increase within the lane
              }
              if (e.logits) e.logits[(size_t)m * p.N + n + i] = z;
            }
          }
        }
      }
      st = stat_merge(st, stat_shfl_xor(st, 16));
      st = stat_merge(st, stat_shfl_xor(st, 32));
      if (lane < 16) s_red[wv][16 * a + lane] = make_float4(st.m, __int_as_float(st.a), st.s, 0.f);
      if (e.sampling) {
        ss = samp_merge(ss, samp_shfl_xor(ss, 16));
        ss = samp_merge(ss, samp_shfl_xor(ss, 32));
        if (lane < 16) s_samp[wv][16 * a + lane] = make_float2(ss.m, __int_as_float(ss.a));
      }
    }
    __syncthreads();
    if (tid < BM && m0 + tid < p.M) {
      SoftStat st = stat_empty();
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float4 s4 = s_red[q][tid];
        st = stat_merge(st, SoftStat{s4.x, __float_as_int(s4.y), s4.z});
      }
      // buffer resources from the (uniform) base pointers, the row in the
      // per-lane offset: a resource built from a per-lane address makes the
      // compiler wrap each access in a loop over the distinct lanes
      st_agent4(agent_rsrc(e.stats), ((m0 + tid) * pl.n_tiles + nt) * 16,
                f32x4_t{st.m, __int_as_float(st.a), st.s, 0.f});
      if (e.sampling) {
        SampStat ss = samp_empty();
#pragma unroll
        for (int q = 0; q < 4; ++q) ss = samp_merge(ss, SampStat{s_samp[q][tid].x, __float_as_int(s_samp[q][tid].y)});
        st_agent2(agent_rsrc(e.sstats), ((m0 + tid) * pl.n_tiles + nt) * 8,
                  f32x2_t{ss.m, __int_as_float(ss.a)});
      }
    }
    // Every vocabulary tile has its row statistics: the last workgroup merges
    // them in tile order and runs the selection of every sequence.
    if (!last_arrival(e.final_ticket, pl.m_tiles * pl.n_tiles)) return;
    __shared__ float s_c[kMaxBlock * 4];
    __shared__ int s_a[kMaxBlock * 4];
    __shared__ int s_tok[kMaxBlock * 4];
    if (e.sampling)
      lm_merge_rows<true>(e, p.M, pl.n_tiles, wv, lane, s_c, s_a, s_tok);
    else
      lm_merge_rows<false>(e, p.M, pl.n_tiles, wv, lane, s_c, s_a, s_tok);
    __syncthreads();
    SelectRule rule;
    rule.tau = e.tau;
    rule.factor = e.factor;
    rule.topk = e.topk;
    rule.sampling = e.sampling;
    rule.seed = e.seed;
    for (int b = wv; b < e.batch; b += 4) {
      const int m = b * e.blk_len + lane;
      const float myc = lane < e.blk_len ? s_c[m] : 0.f;
      const int mya = lane < e.blk_len ? s_a[m] : 0;
      const int mytok = lane < e.blk_len ? s_tok[m] : 0;
      select_and_commit(lane, myc, mya, mytok, e.x + (size_t)b * e.seq_len,
                        e.masked + (size_t)b * e.seq_len, b, e.blk_start, e.blk_len, rule, e.step,
                        e.steps_per_block, e.conf_out ? e.conf_out + b * e.blk_len : nullptr,
                        e.argmax_out ? e.argmax_out + b * e.blk_len : nullptr,
                        e.counts_out ? e.counts_out + 2 * b : nullptr);
    }
  }
}

// ---------------------------------------------------------------------------
// Tile height and K split from a cost model of the busiest CU. Workgroups are
// dealt round-robin over 256 CUs, so the busiest CU runs ceil(W / 256) of
// them. Three rates bound the kernel: that many workgroups' matrix-core work
// at the main loop's sustained MFMA rate for the tile height, their bytes at
// one CU's streaming rate, and the weights streamed once from HBM. They are
// combined as a 6-norm rather than a plain maximum: when the HBM term leads,
// a plan whose workgroups each stream less still finishes sooner (measured:
// 4 splits beat 3 for the 32-row QKV projection, 8 beat 6 for the down
// projection). Each round of resident workgroups adds a start-up (first
// loads, staging, epilogue); a split adds the last workgroup's ordered read
// of every partial tile and, for the whole launch, the float32 partial tiles
// written and read back beyond the first 32 MB, which the 256 MB last-level
// cache absorbs (at 768 rows and more that traffic alone decides against a
// second split). The rate constants are least-squares fits (in log time) to
// every tile height and split of the four layer projections of the
// LLaDA-8B- and Dream-7B-shaped models at 32..768 rows, timed on MI355X;
// with the norm and the partial-traffic term, the plans it picks for those
// projections at 32..1280 rows sum to within 1.1% of the best measured plans
// over the LLaDA Prefix, LLaDA Dual and Dream Dual decodes. Rules the
// measurements show directly: 32-row tiles beat 16-row ones for wide
// outputs, 32-row tiles with 3-5 splits beat 64-row ones for the 4096- and
// 3584-wide outputs up to 160 rows (and one 32-row split the 24576-wide
// gate/up at 160 rows, where 64-row tiles leave a third of the last tile
// empty), and 128-row tiles win nowhere up to 768 rows.
static GemmPlan plan_gemm_uncached(int dt, int M, int N, int K) {
  const double kHbm = 5.03e12;    // weight stream rate
  const double kCuBw = 67.8e9;    // one CU's streaming rate
  const double kPeak = dt == kBF16 ? 2.5e15 : 157e12;
  const double kRound = 10.7e-6;  // start-up of one round of resident workgroups
  const double kReduceBw = 46.3e9;
  const double kLlcPart = 32e6;   // partial-tile bytes the last-level cache absorbs
  const double es = dt == kBF16 ? 2 : 4;
  const double mul = dt == kBF16 ? 2 : 1;  // bf16: X enters as hi + lo terms
  const int nt = (N + kNT - 1) / kNT;
  GemmPlan best{};
  double best_t = 1e30;
  for (int bm : {16, 32, 48, 64, 128}) {
    if (bm > 16 && M <= bm / 2) continue;         // tile mostly empty
    if (bm < 48 && M > 160) continue;             // short tiles re-read the weights too often
    // 48-row tiles: measured faster than 64-row ones only between 160 and
    // 768 rows (their tile counts round better there); slower at 128 and at
    // the 1280-row refresh, level at 160
    if (bm == 48 && (M <= 160 || M > 768)) continue;
    if (bm == 16 && M > 16 && N >= 8192) continue;
    if (bm == 128 && M <= 768) continue;
    const int kc = gemm_kc(bm);
    if (K % kc) continue;
    const int occ = gemm_occupancy(bm);
    // sustained fraction of the MFMA peak in the main loop
    const double eff =
        bm == 128 ? 0.427 : (bm == 64 ? 0.456 : (bm == 48 ? 0.43 : (bm == 32 ? 0.291 : 0.198)));
    const int mt = (M + bm - 1) / bm;
    const double rows = std::min(bm, M);
    const double t_hbm = ((double)N * K * es + (double)M * K * 4.0) / kHbm;
    for (int s = 1; s <= std::min(48, K / kc); ++s) {
      const int kps = (int)round_up((K + s - 1) / s, kc);
      if ((K + kps - 1) / kps != s) continue;
      const int wgs = mt * nt * s;
      const double per_cu = std::ceil(wgs / 256.0);
      const double rounds = std::ceil(wgs / (256.0 * occ));
      const double flops = 2.0 * rows * kNT * kps * mul;
      const double bytes = kNT * (double)kps * es + rows * kps * 4.0;
      const double t_mma = per_cu * flops / (kPeak / 256 * eff);
      const double t_cu = per_cu * bytes / kCuBw;
      const double t_red =
          s > 1 ? s * (double)bm * kNT * 4.0 / kReduceBw +
                      std::max(0.0, wgs * (double)bm * kNT * 4.0 - kLlcPart) * 2.0 / kHbm
                : 0.0;
      const double t6 = std::pow(t_mma, 6.0) + std::pow(t_cu, 6.0) + std::pow(t_hbm, 6.0);
      const double t = std::pow(t6, 1.0 / 6.0) + rounds * kRound + t_red;
      if (t < best_t) {
        best_t = t;
        best.bm = bm;
        best.kc = kc;
        best.m_tiles = mt;
        best.n_tiles = nt;
        best.splits = s;
        best.k_per_split = kps;
      }
    }
  }
  return best;
}

// A plan depends on the shape only, and a decode asks for the same few shapes
// at every step, so plans are kept per host thread.
GemmPlan plan_gemm(int dt, int M, int N, int K, int mode) {
  (void)mode;
  thread_local std::map<std::tuple<int, int, int, int>, GemmPlan> memo;
  const auto key = std::make_tuple(dt, M, N, K);
  auto it = memo.find(key);
  if (it != memo.end()) return it->second;
  const GemmPlan pl = plan_gemm_uncached(dt, M, N, K);
  memo.emplace(key, pl);
  return pl;
}

template <typename T, int BM, int MODE, bool NORM>
static hipError_t launch_t(const GemmProblem& p, const GemmPlan& pl, const GemmScratch& s,
                           hipStream_t st) {
  constexpr int KC = gemm_kc(BM);
  int grid = pl.m_tiles * pl.n_tiles * pl.splits;
  if (pl.m_tiles > 1)
    hipLaunchKernelGGL((gemm_kernel<T, BM, KC, MODE, NORM, true>), dim3(grid), dim3(256), 0, st, p, pl, s);
  else
    hipLaunchKernelGGL((gemm_kernel<T, BM, KC, MODE, NORM, false>), dim3(grid), dim3(256), 0, st, p, pl, s);
  return hipGetLastError();
}

template <typename T, int MODE, bool NORM>
static hipError_t launch_bm(const GemmProblem& p, const GemmPlan& pl, const GemmScratch& s,
                            hipStream_t st) {
  switch (pl.bm) {
    case 16: return launch_t<T, 16, MODE, NORM>(p, pl, s, st);
    case 32: return launch_t<T, 32, MODE, NORM>(p, pl, s, st);
    case 48: return launch_t<T, 48, MODE, NORM>(p, pl, s, st);
    case 64: return launch_t<T, 64, MODE, NORM>(p, pl, s, st);
    default: return launch_t<T, 128, MODE, NORM>(p, pl, s, st);
  }
}

template <typename T>
static hipError_t launch_mode(const GemmProblem& p, const GemmPlan& pl, const GemmScratch& s,
                              hipStream_t st) {
  switch (p.mode) {
    case kEpiQKV: return launch_bm<T, kEpiQKV, true>(p, pl, s, st);
    case kEpiResid: return launch_bm<T, kEpiResid, false>(p, pl, s, st);
    case kEpiSwiGLU: return launch_bm<T, kEpiSwiGLU, true>(p, pl, s, st);
    default: return launch_bm<T, kEpiLMHead, false>(p, pl, s, st);
  }
}

hipError_t launch_gemm(const GemmProblem& p, const GemmScratch& s, hipStream_t st) {
  GemmPlan pl = plan_gemm(p.dt, p.M, p.N, p.K, p.mode);
  if ((p.mode == kEpiQKV || p.mode == kEpiSwiGLU) && (p.ssq_tiles < 1 || p.ssq_tiles > kMaxSsqTiles))
    return hipErrorInvalidValue;
  if ((pl.splits > 1 && pl.part_elems() > s.part_elems) || pl.tiles() > s.n_tickets)
    return hipErrorInvalidValue;
  return p.dt == kBF16 ? launch_mode<BF16>(p, pl, s, st) : launch_mode<F32>(p, pl, s, st);
}

}  // namespace fdllm

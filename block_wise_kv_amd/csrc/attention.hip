// Block attention over a KV cache, no mask ([commentary] 3.4.2: the active
// block's queries attend to every cached key, prefix and suffix alike).
//
// One workgroup owns one (sequence, query head, 32-query tile, KV split):
// 8 waves for the bf16 cache at head size 128, 4 otherwise. The workgroup
// stages its queries once in LDS, already in MFMA fragment order; waves take
// interleaved 32-key tiles of the split, so they stream adjacent cache
// memory. Per tile a wave computes
// S^T = K Q^T (keys x queries) on MFMA with K fragments loaded straight from
// the cache rows, updates a running max / sum per query (online softmax in
// the exp2 domain), and accumulates O^T += V^T P^T, where V^T comes from the
// value cache's tile layout (each 32-key tile a contiguous [D][32] block,
// keys ordered so a lane's operand is one 16-byte load) and P^T is the
// exponentiated S^T tile reused in place as the B operand. P is split into a bf16 high part and a
// bf16 remainder (two MFMAs), so the product keeps ~16 significant bits
// instead of bf16's 8. Waves merge through LDS, splits through a completion
// ticket, both in fixed order.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace fdllm {

constexpr int kAttnQ = 32;     // queries per workgroup
constexpr int kAttnKeys = 32;  // keys per wave iteration

// V^T operand of O^T += V^T P^T: row d of the tile starting at key0, the 8
// keys 4g..4g+3 and 16+4g..16+4g+3 (columns 8g..8g+7 of the tile layout,
// one contiguous run), zero past kv_len.
template <typename T> struct AttnIO;
template <> struct AttnIO<BF16> {
  static __device__ __forceinline__ FragBF load_vt(const uint16_t* row, int key0, int g,
                                                   int kv_len, bool full) {
    FragBF f;
    f.v = *(const uint4*)(row + 8 * g);
    if (!full) {
      uint32_t w[4] = {f.v.x, f.v.y, f.v.z, f.v.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = key0 + (j < 4 ? 4 * g + j : 16 + 4 * g + j - 4);
        if (key >= kv_len) w[j >> 1] &= (j & 1) ? 0x0000ffffu : 0xffff0000u;
      }
      f.v = make_uint4(w[0], w[1], w[2], w[3]);
    }
    return f;
  }
};
template <> struct AttnIO<F32> {
  static __device__ __forceinline__ FragF32 load_vt(const float* row, int key0, int g, int kv_len,
                                                    bool full) {
    FragF32 f;
    f.lo = *(const float4*)(row + 8 * g);
    f.hi = *(const float4*)(row + 8 * g + 4);
    if (!full) {
      float t[8] = {f.lo.x, f.lo.y, f.lo.z, f.lo.w, f.hi.x, f.hi.y, f.hi.z, f.hi.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = key0 + (j < 4 ? 4 * g + j : 16 + 4 * g + j - 4);
        if (key >= kv_len) t[j] = 0.f;
      }
      f.lo = make_float4(t[0], t[1], t[2], t[3]);
      f.hi = make_float4(t[4], t[5], t[6], t[7]);
    }
    return f;
  }
};

// Query operand of S^T = K Q^T. With a bf16 cache and float32 queries the
// query is split into hi + lo bf16 terms (two MFMAs).
template <typename T, typename Q> struct QOp;
template <> struct QOp<BF16, BF16> {
  FragBF f;
  __device__ __forceinline__ void load(const uint16_t* p) { f.v = *(const uint4*)p; }
  __device__ __forceinline__ void zero() { f.v = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void mul(f32x4_t& acc, const FragBF& k) const { mma(acc, k, f); }
};
template <> struct QOp<BF16, F32> {
  FragBF hi, lo;
  __device__ __forceinline__ void load(const float* p) {
    float4 a = ((const float4*)p)[0], b = ((const float4*)p)[1];
    float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    split_bf16x8(v, hi.v, lo.v);
  }
  __device__ __forceinline__ void zero() { hi.v = lo.v = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void mul(f32x4_t& acc, const FragBF& k) const {
    mma(acc, k, hi);
    mma(acc, k, lo);
  }
};
template <> struct QOp<F32, F32> {
  FragF32 f;
  __device__ __forceinline__ void load(const float* p) {
    f.lo = ((const float4*)p)[0];
    f.hi = ((const float4*)p)[1];
  }
  __device__ __forceinline__ void zero() { f.lo = f.hi = make_float4(0, 0, 0, 0); }
  __device__ __forceinline__ void mul(f32x4_t& acc, const FragF32& k) const { mma(acc, k, f); }
};

// P^T operand of O^T += V^T P^T, built once per tile and query half: element
// j is key 4g+j (j<4) / 16+4g+j-4 (j>=4), matching load_vt. With a bf16
// cache P enters as hi + lo bf16 terms (two MFMAs).
template <typename T> struct POp;
template <> struct POp<BF16> {
  FragBF hi, lo;
  __device__ __forceinline__ void set(const float* p) { split_bf16x8(p, hi.v, lo.v); }
  __device__ __forceinline__ void mul(f32x4_t& acc, const FragBF& v) const {
    mma(acc, v, hi);
    mma(acc, v, lo);
  }
};
template <> struct POp<F32> {
  FragF32 f;
  __device__ __forceinline__ void set(const float* p) {
    f.lo = make_float4(p[0], p[1], p[2], p[3]);
    f.hi = make_float4(p[4], p[5], p[6], p[7]);
  }
  __device__ __forceinline__ void mul(f32x4_t& acc, const FragF32& v) const { mma(acc, v, f); }
};

// Waves per workgroup: 8 for the bf16 cache at D = 128 (the decode shapes),
// whose per-wave state then fits two waves per SIMD; 4 otherwise.
template <typename T, int D>
constexpr int attn_waves() { return (sizeof(typename T::store_t) == 2 && D == 128) ? 8 : 4; }

template <typename T, typename Q, int D>
__global__ __launch_bounds__((64 * attn_waves<T, D>())) void attn_kernel(AttnProblem p) {
  using E = typename T::store_t;   // cache element
  using QE = typename Q::store_t;  // query / output element
  using F = typename Frag<T>::type;
  constexpr int NW = attn_waves<T, D>();
  constexpr int NT = 64 * NW;  // threads
  constexpr int DS = D / 32;  // contraction steps of q.k
  constexpr int DF = D / 16;  // 16-dim output fragments
  constexpr int LD = D + 4;   // padded LDS row
  __shared__ float s_o[NW][16][LD];
  __shared__ float s_m[NW][kAttnQ], s_l[NW][kAttnQ];
  __shared__ float s_fm[kAttnQ], s_fl[kAttnQ];
  // the query operand of the workgroup's 32 queries, staged once in fragment
  // order: entry (c, s, lane) is what lane `lane` feeds the MFMA for query
  // half c and contraction step s
  __shared__ QOp<T, Q> s_q[2 * DS * 64];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int rl = lane & 15, g = lane >> 4;
  const int group = p.hq / p.hkv;
  const int qtiles = (p.rows + kAttnQ - 1) / kAttnQ;
  const int inner = group * qtiles;
  int w = xcd_remap(blockIdx.x, gridDim.x);
  const int in_ = w % inner;
  w /= inner;
  const int split = w % p.splits;
  w /= p.splits;
  const int kvh = w % p.hkv;
  const int b = w / p.hkv;
  const int h = kvh * group + in_ / qtiles;
  const int qt = in_ % qtiles;
  const int item = (b * p.hq + h) * qtiles + qt;

  const QE* qbase = (const QE*)p.q;
  const size_t qrow = (size_t)p.hq * D;
  for (int e = tid; e < 2 * DS * 64; e += NT) {
    const int a = e / (DS * 64), s = (e / 64) % DS, l = e % 64;
    const int q = qt * kAttnQ + a * 16 + (l & 15);
    QOp<T, Q> op;
    if (q < p.rows)
      op.load(qbase + ((size_t)b * p.rows + q) * qrow + (size_t)h * D + s * 32 + 8 * (l >> 4));
    else
      op.zero();
    s_q[e] = op;
  }

  const E* kb = (const E*)p.k + ((size_t)b * p.hkv + kvh) * p.ncap * D;
  const int vcap = (int)round_up(p.ncap, kAttnKeys);  // keys per value block, whole tiles
  const E* vb = (const E*)p.vt + ((size_t)b * p.hkv + kvh) * D * vcap;
  const float sl2 = p.scale * 1.4426950408889634f;

  // key range of this split, in whole tiles
  const int per = (int)round_up((p.kv_len + p.splits - 1) / p.splits, kAttnKeys * 4);
  const int kbeg = split * per, kend = min(p.kv_len, kbeg + per);

  float mrun[2] = {-INFINITY, -INFINITY}, lrun[2] = {0.f, 0.f};
  f32x4_t o[DF][2];
#pragma unroll
  for (int df = 0; df < DF; ++df) o[df][0] = o[df][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // K fragments of the tile's 32 keys (rows past kv_len clamped, their scores
  // masked below) and V^T fragments (zero past kv_len). FULL (a compile-time
  // tag): the tile lies inside kv_len, so no masking code at all.
  auto load_tile = [&](auto full_tag, F (&kf)[2][DS], F (&vf)[DF], int key0) {
    constexpr bool FULL = decltype(full_tag)::value;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int krow = FULL ? key0 + a * 16 + rl : min(key0 + a * 16 + rl, p.kv_len - 1);
#pragma unroll
      for (int s = 0; s < DS; ++s)
        load_frag(kf[a][s], kb + (size_t)krow * D + s * 32 + 8 * g);
    }
    const E* vtile = vb + (size_t)(key0 / kAttnKeys) * D * kAttnKeys;
#pragma unroll
    for (int df = 0; df < DF; ++df)
      vf[df] = AttnIO<T>::load_vt(vtile + (df * 16 + rl) * kAttnKeys, key0, g, p.kv_len, FULL);
  };
  // Online softmax with a lazily moved reference maximum: P = 2^(s - m_ref)
  // with m_ref moved (and O, l rescaled) only when a tile's maximum exceeds it
  // by more than kSlack, so most tiles leave the accumulators to the MFMAs
  // alone; P stays below 2^kSlack, which the hi/lo split of P carries at the
  // same relative precision.
  constexpr float kSlack = 8.f;
  auto tile = [&](auto full_tag, const F (&kf)[2][DS], const F (&vf)[DF], int key0) {
    constexpr bool FULL = decltype(full_tag)::value;
    f32x4_t st[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int c = 0; c < 2; ++c) st[a][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const QOp<T, Q> qv = s_q[(c * DS + s) * 64 + lane];
#pragma unroll
        for (int a = 0; a < 2; ++a) qv.mul(st[a][c], kf[a][s]);
      }

#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float sv[8];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = st[a][c][i] * sl2;
          if (!FULL && key0 + a * 16 + 4 * g + i >= p.kv_len) x = -INFINITY;
          sv[a * 4 + i] = x;
        }
      float tm = sv[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) tm = fmaxf(tm, sv[j]);
      tm = fmaxf(tm, __shfl_xor(tm, 16));
      tm = fmaxf(tm, __shfl_xor(tm, 32));
      const bool move = tm > mrun[c] + kSlack;  // always when m_ref is still -inf
      if (__ballot(move)) {
        const float mnew = move ? tm : mrun[c];
        const float alpha = mnew == mrun[c] ? 1.f : __builtin_amdgcn_exp2f(mrun[c] - mnew);
        lrun[c] *= alpha;
#pragma unroll
        for (int df = 0; df < DF; ++df) o[df][c] *= alpha;
        mrun[c] = mnew;
      }
      // keys masked so far leave m_ref at -inf; their s are -inf too
      const float mref = mrun[c] == -INFINITY ? 0.f : mrun[c];
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        sv[j] = __builtin_amdgcn_exp2f(sv[j] - mref);
        ps += sv[j];
      }
      lrun[c] += ps;
      POp<T> pf;
      pf.set(sv);
#pragma unroll
      for (int df = 0; df < DF; ++df) pf.mul(o[df][c], vf[df]);
    }
  };
  using Full = std::integral_constant<bool, true>;
  using Part = std::integral_constant<bool, false>;
  auto load_any = [&](F (&kf)[2][DS], F (&vf)[DF], int key0) {
    if (key0 + kAttnKeys <= p.kv_len) load_tile(Full{}, kf, vf, key0);
    else load_tile(Part{}, kf, vf, key0);
  };
  auto tile_any = [&](const F (&kf)[2][DS], const F (&vf)[DF], int key0) {
    if (key0 + kAttnKeys <= p.kv_len) tile(Full{}, kf, vf, key0);
    else tile(Part{}, kf, vf, key0);
  };

  // Waves take interleaved 32-key tiles; the next tile of a wave is loaded
  // while the current one is multiplied (two register buffers, alternated
  // by an unrolled pair of steps).
  __syncthreads();  // the staged queries
  constexpr int kStride = NW * kAttnKeys;
  if constexpr (NW == 8) {
    // two waves per SIMD: one tile buffer each, the other wave's loads and
    // multiplies overlap a wave's own
    for (int key0 = kbeg + wv * kAttnKeys; key0 < kend; key0 += kStride) {
      F kf[2][DS], vf[DF];
      load_any(kf, vf, key0);
      tile_any(kf, vf, key0);
    }
  } else {
  F kfa[2][DS], vfa[DF], kfb[2][DS], vfb[DF];
  int key0 = kbeg + wv * kAttnKeys;
  if (key0 < kend) load_any(kfa, vfa, key0);
  while (key0 < kend) {
    if (key0 + kStride < kend) load_any(kfb, vfb, key0 + kStride);
    tile_any(kfa, vfa, key0);
    key0 += kStride;
    if (key0 >= kend) break;
    if (key0 + kStride < kend) load_any(kfa, vfa, key0 + kStride);
    tile_any(kfb, vfb, key0);
    key0 += kStride;
  }
  }

  // ---- merge the 4 waves (per 16-query half), then the splits ----
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    lrun[c] += __shfl_xor(lrun[c], 16);
    lrun[c] += __shfl_xor(lrun[c], 32);
    if (g == 0) {
      s_m[wv][c * 16 + rl] = mrun[c];
      s_l[wv][c * 16 + rl] = lrun[c];
    }
  }
  __syncthreads();
  if (tid < kAttnQ) {
    float M = s_m[0][tid];
#pragma unroll
    for (int q = 1; q < NW; ++q) M = fmaxf(M, s_m[q][tid]);
    float L = 0.f;
#pragma unroll
    for (int q = 0; q < NW; ++q)
      L += (s_m[q][tid] == -INFINITY) ? 0.f : exp2f(s_m[q][tid] - M) * s_l[q][tid];
    s_fm[tid] = M;
    s_fl[tid] = L;
  }
  __syncthreads();

  constexpr int kPerThr = D * 16 / NT;  // output dims per thread in a 16-query pass
  const int cq = tid / (D / kPerThr), cd = (tid % (D / kPerThr)) * kPerThr;
  // row m's dims cd .. cd + kPerThr - 1 of head h, times inv: the plain
  // layout, or the split activation layout of the next GEMM's input
  auto store_out = [&](int m, const float* acc, float inv) {
    if (p.xs_out) {
      float v[kPerThr];
#pragma unroll
      for (int j = 0; j < kPerThr; ++j) v[j] = acc[j] * inv;
      const int kslots = (p.hq * D) >> 5, k = h * D + cd;
      if constexpr (kPerThr == 8)
        XSplit<T>::store8((char*)p.o, kslots, m, k, v);
      else
        XSplit<T>::store4((char*)p.o, kslots, m, k, v[0], v[1], v[2], v[3]);
    } else {
      QE* dst = (QE*)p.o + (size_t)m * qrow + (size_t)h * D + cd;
#pragma unroll
      for (int j = 0; j < kPerThr; ++j) dst[j] = Q::from_f(acc[j] * inv);
    }
  };
  // log-sum-exp of the scaled scores of row m (max M and sum L in the exp2
  // domain): ln(L) + M ln 2
  auto store_lse = [&](int m, float M, float L) {
    p.lse[(size_t)m * p.hq + h] = (M + __log2f(L)) * 0.6931471805599453f;
  };
  float* part = p.part;
  const size_t item_floats = (size_t)p.splits * kAttnQ * (D + 2);
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int df = 0; df < DF; ++df)
      *(float4*)&s_o[wv][rl][df * 16 + 4 * g] =
          make_float4(o[df][c][0], o[df][c][1], o[df][c][2], o[df][c][3]);
    __syncthreads();
    const int q = c * 16 + cq;
    const float M = s_fm[q];
    float coef[NW];
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) coef[ww] = (s_m[ww][q] == -INFINITY) ? 0.f : exp2f(s_m[ww][q] - M);
    float acc[kPerThr];
#pragma unroll
    for (int j = 0; j < kPerThr; ++j) {
      float v = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) v += coef[ww] * s_o[ww][cq][cd + j];
      acc[j] = v;
    }
    if (p.splits == 1) {
      const int qg = qt * kAttnQ + q;
      if (qg < p.rows) {
        const float inv = s_fl[q] > 0.f ? 1.f / s_fl[q] : 0.f;
        store_out(b * p.rows + qg, acc, inv);
        if (p.lse && cd == 0) store_lse(b * p.rows + qg, M, s_fl[q]);
      }
    } else {
      float* pi = part + (size_t)item * item_floats + (size_t)split * kAttnQ * (D + 2);
      const auto rs = agent_rsrc(pi);
#pragma unroll
      for (int j = 0; j < kPerThr; j += 4)
        st_agent4(rs, (q * D + cd + j) * 4, f32x4_t{acc[j], acc[j + 1], acc[j + 2], acc[j + 3]});
      if (cd == 0) {
        st_agent(pi + kAttnQ * D + q, M);
        st_agent(pi + kAttnQ * D + kAttnQ + q, s_fl[q]);
      }
    }
    __syncthreads();
  }
  if (p.splits == 1) return;

  if (!last_arrival(p.tickets + item, p.splits)) return;
  // Splits merged in split order: every split's max first, then its sum and
  // output rows, four splits' loads in flight at a time (indices past the
  // last split re-read it and are not added).
  const float* pi = part + (size_t)item * item_floats;
  const size_t sstride = (size_t)kAttnQ * (D + 2);
  const auto rs = agent_rsrc(pi);
  for (int c = 0; c < 2; ++c) {
    const int q = c * 16 + cq;
    const int qg = qt * kAttnQ + q;
    float L = 0.f, acc[kPerThr];
#pragma unroll
    for (int j = 0; j < kPerThr; ++j) acc[j] = 0.f;
    constexpr int kOne = 8;
    if (p.splits <= kOne) {
      // every split's max, sum and output rows in one batch of loads (the
      // decode shapes run 1-8 splits); same order of accumulation as below
      float ms[kOne], ls[kOne];
      f32x4_t v[kOne][kPerThr / 4];
#pragma unroll
      for (int u = 0; u < kOne; ++u) {
        const int s = min(u, p.splits - 1);
        ms[u] = ld_agent(pi + s * sstride + kAttnQ * D + q);
        ls[u] = ld_agent(pi + s * sstride + kAttnQ * D + kAttnQ + q);
#pragma unroll
        for (int j = 0; j < kPerThr; j += 4)
          v[u][j / 4] = ld_agent4(rs, (int)((s * sstride + (size_t)q * D + cd + j) * 4));
      }
      float M = -INFINITY;
#pragma unroll
      for (int u = 0; u < kOne; ++u)
        if (u < p.splits) M = fmaxf(M, ms[u]);
#pragma unroll
      for (int u = 0; u < kOne; ++u) {
        if (u >= p.splits) break;
        const float cf = (ms[u] == -INFINITY) ? 0.f : exp2f(ms[u] - M);
        L += cf * ls[u];
#pragma unroll
        for (int j = 0; j < kPerThr; ++j) acc[j] += cf * v[u][j / 4][j % 4];
      }
      if (qg < p.rows) {
        const float inv = L > 0.f ? 1.f / L : 0.f;
        store_out(b * p.rows + qg, acc, inv);
        if (p.lse && cd == 0) store_lse(b * p.rows + qg, M, L);
      }
      continue;
    }
    float M = -INFINITY;
    for (int s = 0; s < p.splits; ++s) M = fmaxf(M, ld_agent(pi + s * sstride + kAttnQ * D + q));
    constexpr int kU = 4;
    for (int s0 = 0; s0 < p.splits; s0 += kU) {
      float ms[kU], ls[kU];
      f32x4_t v[kU][kPerThr / 4];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int s = min(s0 + u, p.splits - 1);
        ms[u] = ld_agent(pi + s * sstride + kAttnQ * D + q);
        ls[u] = ld_agent(pi + s * sstride + kAttnQ * D + kAttnQ + q);
#pragma unroll
        for (int j = 0; j < kPerThr; j += 4)
          v[u][j / 4] = ld_agent4(rs, (int)((s * sstride + (size_t)q * D + cd + j) * 4));
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (s0 + u >= p.splits) break;
        const float cf = (ms[u] == -INFINITY) ? 0.f : exp2f(ms[u] - M);
        L += cf * ls[u];
#pragma unroll
        for (int j = 0; j < kPerThr; ++j) acc[j] += cf * v[u][j / 4][j % 4];
      }
    }
    if (qg < p.rows) {
      const float inv = L > 0.f ? 1.f / L : 0.f;
      store_out(b * p.rows + qg, acc, inv);
      if (p.lse && cd == 0) store_lse(b * p.rows + qg, M, L);
    }
  }
}

// Splits of the key range: about kAttnSplitTarget workgroups (one per CU
// for three quarters of the CUs), down to one 32-key tile per four waves;
// never more than ceil(kAttnSplitTarget / items), so items * splits <
// kAttnSplitTarget + items (the scratch bound). Each split costs a float32
// partial output written through to the coherence point, a ticket and a
// merge, so the count stays low. Measured with the 8-wave kernel on cold
// caches: the 32-row decode shapes (32 or 28 items, 768-1280 keys) run
// fastest at 6 splits (13.8 us at 768 keys, against 14.9 at 4 and 19.6 at
// one), 128 rows at 2, and 256 items and more at one split.
int plan_attention_splits(int batch, int rows, int hq, int kv_len) {
  const int items = batch * hq * ((rows + kAttnQ - 1) / kAttnQ);
  int s = (kAttnSplitTarget + items - 1) / items;
  int maxs = std::max(1, kv_len / (4 * kAttnKeys));  // at least one tile per four waves
  return std::max(1, std::min(s, maxs));
}

size_t attention_part_floats(int batch, int rows, int hq, int d, int splits) {
  const size_t items = (size_t)batch * hq * ((rows + kAttnQ - 1) / kAttnQ);
  return items * splits * kAttnQ * (d + 2);
}

int attention_tickets(int batch, int rows, int hq) {
  return batch * hq * ((rows + kAttnQ - 1) / kAttnQ);
}

template <typename T, typename Q, int D>
static hipError_t launch_t(const AttnProblem& p, hipStream_t st) {
  const int qtiles = (p.rows + kAttnQ - 1) / kAttnQ;
  const int grid = p.batch * p.hq * qtiles * p.splits;
  hipLaunchKernelGGL((attn_kernel<T, Q, D>), dim3(grid), dim3(64 * attn_waves<T, D>()), 0, st, p);
  return hipGetLastError();
}

template <typename T, typename Q>
static hipError_t launch_d(const AttnProblem& p, hipStream_t st) {
  return p.d == 128 ? launch_t<T, Q, 128>(p, st) : launch_t<T, Q, 64>(p, st);
}

hipError_t launch_attention(const AttnProblem& p, hipStream_t st) {
  if (p.rows <= 0 || p.batch <= 0) return hipSuccess;
  if (p.dt == kBF16)
    return p.qdt == kBF16 ? launch_d<BF16, BF16>(p, st) : launch_d<BF16, F32>(p, st);
  if (p.qdt != kF32) return hipErrorInvalidValue;
  return launch_d<F32, F32>(p, st);
}

}  // namespace fdllm

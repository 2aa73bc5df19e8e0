// C ABI of the Fast-dLLM hot path: model and cache objects, the per-layer
// forward sequence, the confidence-unmask step and the block-wise decoding
// loop ([commentary] 3.2 information flow, 3.4.4 "The Integrated
// Algorithm"). All compute runs in the HIP kernels; this file validates,
// sizes, carves caller memory and enqueues.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "fdllm.h"
#include "internal.h"

using namespace fdllm;

namespace {

thread_local std::string g_err;

fdllm_status fail(fdllm_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define HIP_TRY(expr)                                                                    \
  do {                                                                                   \
    hipError_t e_ = (expr);                                                              \
    if (e_ != hipSuccess)                                                                \
      return fail(FDLLM_EHIP, "%s failed: %s (%s:%d)", #expr, hipGetErrorString(e_),     \
                  __FILE__, __LINE__);                                                   \
  } while (0)

// Sequential carving of a caller buffer in 256-byte aligned pieces.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  void* take(size_t bytes) {
    off = (size_t)round_up((int64_t)off, 256);
    void* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  }
};

fdllm_status check_config(const fdllm_model_config* c) {
  if (!c) return fail(FDLLM_EINVAL, "config is NULL");
  if (c->dtype != FDLLM_F32 && c->dtype != FDLLM_BF16) return fail(FDLLM_EDTYPE, "dtype %d", c->dtype);
  if (c->n_layers < 1 || c->d_model < 1 || c->n_heads < 1 || c->n_kv_heads < 1 || c->ffn_dim < 1 ||
      c->vocab < 1 || c->max_seq_len < 1)
    return fail(FDLLM_EINVAL, "model sizes must be positive");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(FDLLM_ESHAPE, "head_dim must be 64 or 128 (got %d)", c->head_dim);
  if (c->d_model % 256 || c->d_model > 256 * kMaxSsqTiles)
    return fail(FDLLM_ESHAPE, "d_model must be a multiple of 256, at most %d", 256 * kMaxSsqTiles);
  if (c->n_heads % c->n_kv_heads) return fail(FDLLM_ESHAPE, "n_heads must be a multiple of n_kv_heads");
  if (c->ffn_dim % kGateUp) return fail(FDLLM_ESHAPE, "ffn_dim must be a multiple of %d", kGateUp);
  if ((c->n_heads * c->head_dim) % 128)
    return fail(FDLLM_ESHAPE, "n_heads * head_dim must be a multiple of 128");
  if (c->vocab % 16) return fail(FDLLM_ESHAPE, "vocab must be a multiple of 16");
  if (c->mask_id < 0 || c->mask_id >= c->vocab) return fail(FDLLM_EINVAL, "mask_id out of range");
  if (!std::isfinite(c->rope_theta) || c->rope_theta <= 0 || !std::isfinite(c->norm_eps) ||
      c->norm_eps <= 0 || !std::isfinite(c->logit_scale))
    return fail(FDLLM_EINVAL, "rope_theta, norm_eps and logit_scale must be finite and positive");
  return FDLLM_OK;
}

fdllm_status check_device() {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  HIP_TRY(hipGetDeviceProperties(&prop, dev));
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(FDLLM_ENOTSUP, "device %d is %s, kernels are built for gfx950", dev, prop.gcnArchName);
  return FDLLM_OK;
}

struct Layer {
  void *attn_norm, *qkv, *wo, *ffn_norm, *gateup, *down;
};

}  // namespace

struct fdllm_model {
  fdllm_model_config cfg;
  int dt;
  size_t es;
  void* embed;
  std::vector<Layer> layers;
  void* final_norm;
  void* lm;
  float2* rope;
  std::vector<float2> rope_host;
  int qd() const { return cfg.n_heads * cfg.head_dim; }
  int kvd() const { return cfg.n_kv_heads * cfg.head_dim; }
};

// Optional launch timing: a pair of hipEvents on the launch stream around
// every kernel launch, keyed by kernel variant, with the launch's algorithmic
// bytes (what the kernel must move at least once).
struct Profiler {
  struct Pending {
    std::string name;
    hipEvent_t a, b;
    double bytes, flops;
  };
  struct Acc {
    long launches = 0;
    double ms = 0, bytes = 0, flops = 0, floor_ms = 0;
  };
  bool on = false;
  double peak_bw = 0, peak_flops = 0;  // when both set: per-launch floor max(bytes/bw, flops/peak)
  std::string only;     // when non-empty, only launches of this variant are timed
  int stride = 1;       // ... and of those only every stride-th
  long seen = 0;        // launches of the selected variant so far
  std::vector<hipEvent_t> pool;
  std::vector<Pending> pending;
  std::map<std::string, Acc> acc;
  hipEvent_t get() {
    if (pool.empty()) {
      hipEvent_t e = nullptr;
      (void)hipEventCreate(&e);
      return e;
    }
    hipEvent_t e = pool.back();
    pool.pop_back();
    return e;
  }
  // Folds every completed pair into the totals (the caller has synchronised).
  hipError_t harvest() {
    for (auto& p : pending) {
      hipError_t e = hipEventSynchronize(p.b);
      if (e != hipSuccess) return e;
      float ms = 0;
      e = hipEventElapsedTime(&ms, p.a, p.b);
      if (e != hipSuccess) return e;
      Acc& a = acc[p.name];
      a.launches++;
      a.ms += ms;
      a.bytes += p.bytes;
      a.flops += p.flops;
      if (peak_bw > 0 && peak_flops > 0)
        a.floor_ms += 1e3 * std::max(p.bytes / peak_bw, p.flops / peak_flops);
      pool.push_back(p.a);
      pool.push_back(p.b);
    }
    pending.clear();
    return hipSuccess;
  }
  ~Profiler() {
    for (auto& p : pending) {
      (void)hipEventDestroy(p.a);
      (void)hipEventDestroy(p.b);
    }
    for (auto e : pool) (void)hipEventDestroy(e);
  }
};

struct ProfScope {
  Profiler* p;
  hipStream_t st;
  std::string name;
  double bytes, flops;
  hipEvent_t a = nullptr;
  ProfScope(Profiler* prof, hipStream_t s, std::string n, double b, double f = 0.0)
      : p(prof && prof->on ? prof : nullptr), st(s), name(std::move(n)), bytes(b), flops(f) {
    if (p && !p->only.empty()) {
      if (name != p->only || (p->seen++ % p->stride) != 0) p = nullptr;
    }
    if (p) {
      a = p->get();
      (void)hipEventRecord(a, st);
    }
  }
  ~ProfScope() {
    if (p) {
      hipEvent_t b = p->get();
      (void)hipEventRecord(b, st);
      p->pending.push_back({name, a, b, bytes, flops});
    }
  }
};

struct fdllm_cache {
  const fdllm_model* model;
  Profiler prof;
  int batch, ncap;
  std::vector<void*> k, vt;
  float* h;
  float* ssq;
  // q float32; attn, act, xs_a (QKV input), xs_ffn (gate/up input): split
  // activation layout, rows padded past the last row any GEMM tile reads
  void *q, *attn, *act, *xs_a, *xs_ffn, *hidden;
  GemmScratch gs;
  int* lm_final_ticket;
  float* attn_part;
  int* attn_tickets;
  float4* lm_stats;
  float2* lm_sstats;
  int32_t* counts;
  float* conf;
  int32_t* argmax;
  int32_t* host_counts;  // pinned
};

namespace {

// Sizes (and, when base != nullptr, pointers) of the packed model.
size_t carve_model(const fdllm_model_config& c, fdllm_model* m, void* base) {
  const int dt = c.dtype == FDLLM_BF16 ? kBF16 : kF32;
  const size_t es = dtype_bytes(dt);
  const int64_t d = c.d_model, qd = (int64_t)c.n_heads * c.head_dim,
                kvd = (int64_t)c.n_kv_heads * c.head_dim, F = c.ffn_dim, V = c.vocab;
  Carver cv(base);
  void* embed = cv.take((size_t)V * d * es);
  std::vector<Layer> layers(c.n_layers);
  for (auto& L : layers) {
    L.attn_norm = cv.take(d * es);
    L.qkv = cv.take(packed_matrix_bytes(dt, qd + 2 * kvd, d));
    L.wo = cv.take(packed_matrix_bytes(dt, d, qd));
    L.ffn_norm = cv.take(d * es);
    L.gateup = cv.take(packed_matrix_bytes(dt, 2 * F, d));
    L.down = cv.take(packed_matrix_bytes(dt, d, F));
  }
  void* fnorm = cv.take(d * es);
  void* lm = cv.take(packed_matrix_bytes(dt, V, d));
  void* rope = cv.take((size_t)c.max_seq_len * (c.head_dim / 2) * sizeof(float2));
  if (m) {
    m->embed = embed;
    m->layers = layers;
    m->final_norm = fnorm;
    m->lm = lm;
    m->rope = (float2*)rope;
  }
  return cv.off;
}

// Largest GEMM scratch any forward of up to max_rows rows needs.
void gemm_scratch_need(const fdllm_model_config& c, int max_rows, int max_lm_rows, size_t* part,
                       int* tickets) {
  const int dt = c.dtype == FDLLM_BF16 ? kBF16 : kF32;
  const int d = c.d_model, qd = c.n_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim,
            F = c.ffn_dim;
  struct S { int N, K, mode; } shapes[] = {{qd + 2 * kvd, d, kEpiQKV}, {d, qd, kEpiResid},
                                           {2 * F, d, kEpiSwiGLU}, {d, F, kEpiResid}};
  size_t p = 0;
  int t = 0;
  for (int M = 1; M <= max_rows; ++M)
    for (auto& s : shapes) {
      GemmPlan pl = plan_gemm(dt, M, s.N, s.K, s.mode);
      if (pl.splits > 1) p = std::max(p, pl.part_elems());
      t = std::max(t, pl.tiles());
    }
  for (int M = 1; M <= max_lm_rows; ++M) {
    GemmPlan pl = plan_gemm(dt, M, c.vocab, d, kEpiLMHead);
    if (pl.splits > 1) p = std::max(p, pl.part_elems());
    t = std::max(t, pl.tiles());
  }
  *part = p;
  *tickets = t;
}

size_t carve_cache(const fdllm_model* m, int batch, int max_seq, fdllm_cache* c, void* base) {
  const fdllm_model_config& cf = m->cfg;
  const int ncap = (int)round_up(max_seq, 32);
  const size_t es = m->es;
  const int64_t d = cf.d_model, D = cf.head_dim, Hkv = cf.n_kv_heads;
  const int64_t rows = (int64_t)batch * ncap;
  Carver cv(base);
  std::vector<void*> k(cf.n_layers), vt(cf.n_layers);
  for (int l = 0; l < cf.n_layers; ++l) {
    k[l] = cv.take((size_t)batch * Hkv * ncap * D * es);
    vt[l] = cv.take((size_t)batch * Hkv * D * ncap * es);
  }
  // the tallest GEMM tile (128 rows), and 48-row tiles, whose last tile
  // may reach up to 47 rows past M
  const int64_t rows_pad = round_up(rows, 128) + 64;
  float* h = (float*)cv.take(rows * d * 4);
  float* ssq = (float*)cv.take((d / 256) * rows * 4);
  void* q = cv.take(rows * m->qd() * 4);
  void* attn = cv.take(rows_pad * m->qd() * 4);
  void* act = cv.take(rows_pad * cf.ffn_dim * 4);
  void* xs_a = cv.take(rows_pad * d * 4);
  void* xs_ffn = cv.take(rows_pad * d * 4);
  void* hidden = cv.take((size_t)batch * kMaxBlock * d * 4);
  size_t part_elems;
  int n_tickets;
  gemm_scratch_need(cf, (int)rows, batch * kMaxBlock, &part_elems, &n_tickets);
  float* part = (float*)cv.take(part_elems * 4);
  // tickets: GEMM tiles, the LM-head final ticket, attention items -- one
  // contiguous range so creation clears them with one fill
  const int a_tickets = attention_tickets(batch, ncap, cf.n_heads);
  int* tickets = (int*)cv.take((size_t)(n_tickets + 1 + a_tickets) * 4);
  // split partials: items * splits <= items * ceil(T / items) < T + items
  // (T = kAttnSplitTarget) for any batch <= this cache's batch and any row
  // count <= ncap
  const size_t a_part = (size_t)(kAttnSplitTarget + a_tickets) * 32 * (D + 2);
  float* attn_part = (float*)cv.take(a_part * 4);
  const int lm_tiles = (int)((cf.vocab + kNT - 1) / kNT);
  float4* lm_stats = (float4*)cv.take((size_t)batch * kMaxBlock * lm_tiles * sizeof(float4));
  float2* lm_sstats = (float2*)cv.take((size_t)batch * kMaxBlock * lm_tiles * sizeof(float2));
  int32_t* counts = (int32_t*)cv.take((size_t)batch * 2 * 4);
  float* conf = (float*)cv.take((size_t)batch * kMaxBlock * 4);
  int32_t* argmax = (int32_t*)cv.take((size_t)batch * kMaxBlock * 4);
  if (c) {
    c->model = m;
    c->batch = batch;
    c->ncap = ncap;
    c->k = k;
    c->vt = vt;
    c->h = h;
    c->ssq = ssq;
    c->q = q;
    c->attn = attn;
    c->act = act;
    c->xs_a = xs_a;
    c->xs_ffn = xs_ffn;
    c->hidden = hidden;
    c->gs.part = part;
    c->gs.part_elems = part_elems;
    c->gs.tickets = tickets;
    c->gs.n_tickets = n_tickets;
    c->lm_final_ticket = tickets + n_tickets;
    c->attn_tickets = tickets + n_tickets + 1;
    c->attn_part = attn_part;
    c->lm_stats = lm_stats;
    c->lm_sstats = lm_sstats;
    c->counts = counts;
    c->conf = conf;
    c->argmax = argmax;
  }
  return cv.off;
}

size_t ticket_bytes(const fdllm_cache* c) {
  return (size_t)(c->gs.n_tickets + 1 + attention_tickets(c->batch, c->ncap, c->model->cfg.n_heads)) * 4;
}

const char* kEpiNames[] = {"qkv", "resid", "swiglu", "lmhead"};

// Algorithmic bytes of one GEMM launch: weights once, X once, outputs once.
double gemm_bytes(const fdllm_model* m, const GemmProblem& g) {
  const double es = (double)m->es;
  double b = (double)g.N * g.K * es + (double)g.M * g.K * 4.0;
  switch (g.mode) {
    case kEpiQKV: b += (double)g.M * (m->qd() * 4.0 + 2.0 * m->kvd() * es); break;
    case kEpiResid: b += 2.0 * g.M * g.N * 4.0; break;
    case kEpiSwiGLU: b += (double)g.M * (g.N / 2) * 4.0; break;
    default: break;
  }
  return b;
}

std::string gemm_name(const GemmProblem& g) {
  GemmPlan pl = plan_gemm(g.dt, g.M, g.N, g.K, g.mode);
  return std::string("gemm_") + kEpiNames[g.mode] + "_bm" + std::to_string(pl.bm);
}

hipError_t run_gemm(fdllm_cache* c, const GemmProblem& g, hipStream_t st) {
  ProfScope ps(&c->prof, st, gemm_name(g), gemm_bytes(c->model, g), 2.0 * g.M * g.N * g.K);
  return launch_gemm(g, c->gs, st);
}

// Forward of rows [r0, r1) of each sequence over a cache of seq_len rows;
// writes K/V of those rows into the cache and the final-normed hidden of the
// block rows [blk_start, blk_start + blk_len) to `hidden`.
fdllm_status forward_rows(fdllm_model* m, fdllm_cache* c, const int32_t* x, int batch, int seq_len,
                          int r0, int r1, int blk_start, int blk_len, void* hidden,
                          hipStream_t st) {
  const fdllm_model_config& cf = m->cfg;
  const int R = r1 - r0, M = batch * R;
  const int d = cf.d_model, D = cf.head_dim, qd = m->qd(), kvd = m->kvd();
  {
    ProfScope ps(&c->prof, st, "embed", (double)M * d * (m->es + 4.0));
    HIP_TRY(launch_embed(m->dt, x, seq_len, batch, r0, R, m->embed, d, c->h, c->ssq, cf.vocab,
                         m->layers[0].attn_norm, c->xs_a, st));
  }
  // Only the block rows' final hidden states are read (by the LM head), so
  // the last layer needs every row only for its q/k/v (its K and V go into
  // the cache); attention, O projection and FFN run on the block rows
  // alone. Done when those rows are one contiguous range (one sequence).
  const int off = blk_start - r0;
  const bool tail_only = batch == 1 && R > blk_len;
  for (int l = 0; l < cf.n_layers; ++l) {
    const Layer& L = m->layers[l];
    const bool tail = tail_only && l + 1 == cf.n_layers;
    const int Mt = tail ? blk_len : M;  // rows after the q/k/v projection
    float* const h_t = tail ? c->h + (size_t)off * d : c->h;
    GemmProblem g;
    g.dt = m->dt;
    g.M = M;
    g.K = d;
    g.eps = cf.norm_eps;
    // q, k, v (+RoPE, K/V into the cache)
    g.mode = kEpiQKV;
    g.x = c->xs_a;
    g.ldx = d;
    g.norm = true;
    g.ssq = c->ssq;
    g.ssq_tiles = d / 256;
    g.gain = L.attn_norm;
    g.w = L.qkv;
    g.N = qd + 2 * kvd;
    g.ep.rows_per_seq = R;
    g.ep.row0 = r0;
    g.ep.q_out = c->q;
    g.ep.k_cache = c->k[l];
    g.ep.vt_cache = c->vt[l];
    g.ep.ncap = c->ncap;
    g.ep.n_heads = cf.n_heads;
    g.ep.n_kv_heads = cf.n_kv_heads;
    g.ep.head_dim = D;
    g.ep.rope = m->rope;
    HIP_TRY(run_gemm(c, g, st));
    // attention over all seq_len cached rows
    AttnProblem a;
    a.dt = m->dt;
    a.qdt = kF32;
    a.q = tail ? (const void*)((const float*)c->q + (size_t)off * qd) : c->q;
    a.o = c->attn;
    a.xs_out = true;
    a.k = c->k[l];
    a.vt = c->vt[l];
    a.batch = batch;
    a.rows = tail ? blk_len : R;
    a.hq = cf.n_heads;
    a.hkv = cf.n_kv_heads;
    a.d = D;
    a.kv_len = seq_len;
    a.ncap = c->ncap;
    a.scale = 1.f / std::sqrt((float)D);
    a.splits = plan_attention_splits(batch, a.rows, cf.n_heads, seq_len);
    a.part = c->attn_part;
    a.tickets = c->attn_tickets;
    {
      ProfScope ps(&c->prof, st, "attention",
                   (double)batch * cf.n_kv_heads * seq_len * D * m->es * 2.0 + 2.0 * Mt * qd * 4.0,
                   4.0 * Mt * cf.n_heads * (double)seq_len * D);
      HIP_TRY(launch_attention(a, st));
    }
    // output projection + residual
    GemmProblem o = GemmProblem();
    o.dt = m->dt;
    o.mode = kEpiResid;
    o.x = c->attn;
    o.ldx = qd;
    o.w = L.wo;
    o.M = Mt;
    o.N = d;
    o.K = qd;
    o.ep.h = h_t;
    o.ep.ssq_out = c->ssq;
    o.ep.xs_next = (char*)c->xs_ffn;
    o.ep.gain_next = L.ffn_norm;
    HIP_TRY(run_gemm(c, o, st));
    // gate/up + SwiGLU
    GemmProblem gu = GemmProblem();
    gu.dt = m->dt;
    gu.mode = kEpiSwiGLU;
    gu.x = c->xs_ffn;
    gu.ldx = d;
    gu.norm = true;
    gu.ssq = c->ssq;
    gu.ssq_tiles = d / 256;
    gu.gain = L.ffn_norm;
    gu.eps = cf.norm_eps;
    gu.w = L.gateup;
    gu.M = Mt;
    gu.N = 2 * cf.ffn_dim;
    gu.K = d;
    gu.ep.act = c->act;
    HIP_TRY(run_gemm(c, gu, st));
    // down + residual
    GemmProblem dn = GemmProblem();
    dn.dt = m->dt;
    dn.mode = kEpiResid;
    dn.x = c->act;
    dn.ldx = cf.ffn_dim;
    dn.w = L.down;
    dn.M = Mt;
    dn.N = d;
    dn.K = cf.ffn_dim;
    dn.ep.h = h_t;
    dn.ep.ssq_out = c->ssq;
    if (l + 1 < cf.n_layers) {
      dn.ep.xs_next = (char*)c->xs_a;
      dn.ep.gain_next = m->layers[l + 1].attn_norm;
    }
    HIP_TRY(run_gemm(c, dn, st));
  }
  {
    ProfScope ps(&c->prof, st, "final_norm", (double)batch * blk_len * d * 8.0);
    // after a block-rows-only last layer, h's block rows start at off and
    // the sums of squares are laid out for blk_len rows
    if (tail_only)
      HIP_TRY(launch_final_norm(m->dt, c->h + (size_t)off * d, c->ssq, d, 1, blk_len, 0, blk_len,
                                m->final_norm, cf.norm_eps, hidden, st));
    else
      HIP_TRY(launch_final_norm(m->dt, c->h, c->ssq, d, batch, R, blk_start - r0, blk_len,
                                m->final_norm, cf.norm_eps, hidden, st));
  }
  return FDLLM_OK;
}

fdllm_status check_rows(const fdllm_cache* c, int batch, int seq_len, int blk_start, int blk_len) {
  if (batch < 1 || batch > c->batch) return fail(FDLLM_EINVAL, "batch %d outside [1, %d]", batch, c->batch);
  if (seq_len < 1 || seq_len > c->ncap || seq_len > c->model->cfg.max_seq_len)
    return fail(FDLLM_EINVAL, "seq_len %d exceeds the cache (%d) or model (%d)", seq_len, c->ncap,
                c->model->cfg.max_seq_len);
  if (blk_len < 1 || blk_len > kMaxBlock)
    return fail(FDLLM_EINVAL, "blk_len must be in [1, %d]", kMaxBlock);
  if (blk_start < 0 || blk_start + blk_len > seq_len)
    return fail(FDLLM_EINVAL, "block [%d, %d) outside the sequence", blk_start, blk_start + blk_len);
  return FDLLM_OK;
}

fdllm_status check_select(const fdllm_select_params* r, SelectRuleArgs* out) {
  if (!r) return fail(FDLLM_EINVAL, "selection parameters are NULL");
  if (!std::isfinite(r->tau)) return fail(FDLLM_EINVAL, "tau must be finite");
  if (!std::isfinite(r->factor) || r->factor < 0.f) return fail(FDLLM_EINVAL, "factor must be finite and >= 0");
  if (r->topk < 0) return fail(FDLLM_EINVAL, "topk must be >= 0");
  out->tau = r->tau;
  out->factor = r->factor;
  out->topk = r->topk;
  out->sampling = r->sampling != 0;
  out->seed = r->seed;
  return FDLLM_OK;
}

// Arguments of the logits-in unmask calls (shared by the workspace and the
// allocation-free entry points).
fdllm_status check_unmask_logits(const void* logits, int dtype, const int32_t* x,
                                 const uint8_t* masked, int batch, int seq_len, int blk_start,
                                 int blk_len, int vocab, const fdllm_select_params* rule, int step,
                                 int steps_per_block, SelectRuleArgs* ra) {
  if (!logits || !x || !masked) return fail(FDLLM_EINVAL, "NULL argument");
  if (dtype != FDLLM_F32 && dtype != FDLLM_BF16) return fail(FDLLM_EDTYPE, "dtype %d", dtype);
  if (batch < 1 || seq_len < 1 || blk_len < 1 || blk_len > kMaxBlock || blk_start < 0 ||
      blk_start + blk_len > seq_len)
    return fail(FDLLM_EINVAL, "bad block [%d, %d) in a sequence of %d", blk_start, blk_start + blk_len, seq_len);
  if (vocab < 8 || vocab % 8) return fail(FDLLM_ESHAPE, "vocab must be a positive multiple of 8");
  fdllm_status s = check_select(rule, ra);
  if (s) return s;
  if (steps_per_block < 1 || step < 0 || step >= steps_per_block)
    return fail(FDLLM_EINVAL, "need 0 <= step_in_block < steps_per_block");
  return FDLLM_OK;
}

fdllm_status unmask_fused(fdllm_model* m, fdllm_cache* c, const void* hidden, int32_t* x,
                          uint8_t* masked, int batch, int seq_len, int blk_start, int blk_len,
                          const SelectRuleArgs& rule, int step, int T, float* conf,
                          int32_t* argmax, int32_t* counts, float* logits, hipStream_t st) {
  GemmProblem g;
  g.dt = m->dt;
  g.mode = kEpiLMHead;
  g.x = hidden;
  g.ldx = m->cfg.d_model;
  g.w = m->lm;
  g.M = batch * blk_len;
  g.N = m->cfg.vocab;
  g.K = m->cfg.d_model;
  g.ep.logit_scale = m->cfg.logit_scale;
  g.ep.stats = c->lm_stats;
  g.ep.sstats = c->lm_sstats;
  g.ep.logits = logits;
  g.ep.final_ticket = c->lm_final_ticket;
  g.ep.x = x;
  g.ep.masked = masked;
  g.ep.batch = batch;
  g.ep.seq_len = seq_len;
  g.ep.blk_start = blk_start;
  g.ep.blk_len = blk_len;
  g.ep.step = step;
  g.ep.steps_per_block = T;
  g.ep.tau = rule.tau;
  g.ep.factor = rule.factor;
  g.ep.topk = rule.topk;
  g.ep.sampling = rule.sampling;
  g.ep.seed = rule.seed;
  g.ep.conf_out = conf;
  g.ep.argmax_out = argmax;
  g.ep.counts_out = counts;
  HIP_TRY(run_gemm(c, g, st));
  return FDLLM_OK;
}

}  // namespace

extern "C" {

const char* fdllm_version(void) { return "fdllm 0.1.0 (gfx950)"; }

const char* fdllm_last_error(void) { return g_err.c_str(); }

fdllm_status fdllm_model_packed_bytes(const fdllm_model_config* cfg, size_t* bytes) {
  fdllm_status s = check_config(cfg);
  if (s) return s;
  if (!bytes) return fail(FDLLM_EINVAL, "bytes is NULL");
  *bytes = carve_model(*cfg, nullptr, nullptr);
  return FDLLM_OK;
}

fdllm_status fdllm_model_create(const fdllm_model_config* cfg, const void* const* d_weights,
                                void* d_packed, size_t packed_bytes, void* stream,
                                fdllm_model** out) {
  fdllm_status s = check_config(cfg);
  if (s) return s;
  if (!d_weights || !d_packed || !out) return fail(FDLLM_EINVAL, "NULL argument");
  size_t need = carve_model(*cfg, nullptr, nullptr);
  if (packed_bytes < need) return fail(FDLLM_EINVAL, "packed buffer has %zu bytes, needs %zu", packed_bytes, need);
  if ((uintptr_t)d_packed % 256) return fail(FDLLM_EINVAL, "packed buffer must be 256-byte aligned");
  const int nw = 1 + 9 * cfg->n_layers + 2;
  for (int i = 0; i < nw; ++i)
    if (!d_weights[i]) return fail(FDLLM_EINVAL, "weight %d is NULL", i);
  s = check_device();
  if (s) return s;
  fdllm_model* m = new fdllm_model();
  m->cfg = *cfg;
  m->dt = cfg->dtype == FDLLM_BF16 ? kBF16 : kF32;
  m->es = dtype_bytes(m->dt);
  carve_model(*cfg, m, d_packed);
  hipStream_t st = (hipStream_t)stream;
  const int64_t d = cfg->d_model, qd = m->qd(), kvd = m->kvd(), F = cfg->ffn_dim, V = cfg->vocab;
  const size_t es = m->es;
  auto copy = [&](void* dst, const void* src, size_t bytes) {
    return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, st);
  };
  hipError_t e = copy(m->embed, d_weights[0], (size_t)V * d * es);
  for (int l = 0; l < cfg->n_layers && e == hipSuccess; ++l) {
    const void* const* w = d_weights + 1 + 9 * l;
    Layer& L = m->layers[l];
    if (e == hipSuccess) e = copy(L.attn_norm, w[0], d * es);
    if (e == hipSuccess) e = pack_matrix(m->dt, kPackQKV, w[1], w[2], w[3], qd, kvd, kvd, d, cfg->head_dim, L.qkv, st);
    if (e == hipSuccess) e = pack_matrix(m->dt, kPackPlain, w[4], nullptr, nullptr, d, 0, 0, qd, cfg->head_dim, L.wo, st);
    if (e == hipSuccess) e = copy(L.ffn_norm, w[5], d * es);
    if (e == hipSuccess) e = pack_matrix(m->dt, kPackGateUp, w[6], w[7], nullptr, F, 0, 0, d, cfg->head_dim, L.gateup, st);
    if (e == hipSuccess) e = pack_matrix(m->dt, kPackPlain, w[8], nullptr, nullptr, d, 0, 0, F, cfg->head_dim, L.down, st);
  }
  const void* const* tail = d_weights + 1 + 9 * cfg->n_layers;
  if (e == hipSuccess) e = copy(m->final_norm, tail[0], d * es);
  if (e == hipSuccess) e = pack_matrix(m->dt, kPackPlain, tail[1], nullptr, nullptr, V, 0, 0, d, cfg->head_dim, m->lm, st);
  // RoPE table: angle p * theta^(-2i/D) in double precision, stored as (cos, sin)
  const int half = cfg->head_dim / 2;
  m->rope_host.resize((size_t)cfg->max_seq_len * half);
  for (int p = 0; p < cfg->max_seq_len; ++p)
    for (int i = 0; i < half; ++i) {
      double ang = (double)p * std::pow((double)cfg->rope_theta, -2.0 * i / cfg->head_dim);
      m->rope_host[(size_t)p * half + i] = make_float2((float)std::cos(ang), (float)std::sin(ang));
    }
  if (e == hipSuccess)
    e = hipMemcpyAsync(m->rope, m->rope_host.data(), m->rope_host.size() * sizeof(float2),
                       hipMemcpyHostToDevice, st);
  if (e != hipSuccess) {
    delete m;
    return fail(FDLLM_EHIP, "model_create: %s", hipGetErrorString(e));
  }
  *out = m;
  return FDLLM_OK;
}

fdllm_status fdllm_model_destroy(fdllm_model* model) {
  delete model;
  return FDLLM_OK;
}

fdllm_status fdllm_cache_bytes(const fdllm_model* model, int32_t batch, int32_t max_seq,
                               size_t* bytes) {
  if (!model || !bytes) return fail(FDLLM_EINVAL, "NULL argument");
  if (batch < 1 || max_seq < 1 || max_seq > model->cfg.max_seq_len)
    return fail(FDLLM_EINVAL, "batch must be >= 1 and max_seq in [1, %d]", model->cfg.max_seq_len);
  *bytes = carve_cache(model, batch, max_seq, nullptr, nullptr);
  return FDLLM_OK;
}

fdllm_status fdllm_cache_create(const fdllm_model* model, int32_t batch, int32_t max_seq,
                                void* d_mem, size_t bytes, void* stream, fdllm_cache** out) {
  size_t need = 0;
  fdllm_status s = fdllm_cache_bytes(model, batch, max_seq, &need);
  if (s) return s;
  if (!d_mem || !out) return fail(FDLLM_EINVAL, "NULL argument");
  if (bytes < need) return fail(FDLLM_EINVAL, "cache buffer has %zu bytes, needs %zu", bytes, need);
  if ((uintptr_t)d_mem % 256) return fail(FDLLM_EINVAL, "cache buffer must be 256-byte aligned");
  fdllm_cache* c = new fdllm_cache();
  carve_cache(model, batch, max_seq, c, d_mem);
  hipError_t e = hipHostMalloc((void**)&c->host_counts, (size_t)batch * 2 * sizeof(int32_t), 0);
  if (e == hipSuccess) e = hipMemsetAsync(c->gs.tickets, 0, ticket_bytes(c), (hipStream_t)stream);
  if (e != hipSuccess) {
    if (c->host_counts) (void)hipHostFree(c->host_counts);
    delete c;
    return fail(FDLLM_EHIP, "cache_create: %s", hipGetErrorString(e));
  }
  *out = c;
  return FDLLM_OK;
}

fdllm_status fdllm_cache_destroy(fdllm_cache* cache) {
  if (cache) {
    if (cache->host_counts) (void)hipHostFree(cache->host_counts);
    delete cache;
  }
  return FDLLM_OK;
}

fdllm_status fdllm_cache_refresh(fdllm_model* model, fdllm_cache* cache, const int32_t* d_x,
                                 int32_t batch, int32_t seq_len, int32_t blk_start,
                                 int32_t blk_len, void* d_hidden_blk, void* stream) {
  if (!model || !cache || !d_x || !d_hidden_blk) return fail(FDLLM_EINVAL, "NULL argument");
  if ((uintptr_t)d_hidden_blk % 16) return fail(FDLLM_EINVAL, "d_hidden_blk must be 16-byte aligned");
  if (cache->model != model) return fail(FDLLM_EINVAL, "cache belongs to another model");
  fdllm_status s = check_rows(cache, batch, seq_len, blk_start, blk_len);
  if (s) return s;
  return forward_rows(model, cache, d_x, batch, seq_len, 0, seq_len, blk_start, blk_len,
                      d_hidden_blk, (hipStream_t)stream);
}

fdllm_status fdllm_block_forward(fdllm_model* model, fdllm_cache* cache, const int32_t* d_x,
                                 int32_t batch, int32_t seq_len, int32_t row_start,
                                 int32_t row_end, int32_t blk_start, int32_t blk_len,
                                 void* d_hidden_blk, void* stream) {
  if (!model || !cache || !d_x || !d_hidden_blk) return fail(FDLLM_EINVAL, "NULL argument");
  if ((uintptr_t)d_hidden_blk % 16) return fail(FDLLM_EINVAL, "d_hidden_blk must be 16-byte aligned");
  if (cache->model != model) return fail(FDLLM_EINVAL, "cache belongs to another model");
  fdllm_status s = check_rows(cache, batch, seq_len, blk_start, blk_len);
  if (s) return s;
  if (row_start != blk_start || row_end < blk_start + blk_len || row_end > seq_len)
    return fail(FDLLM_EINVAL, "rows [%d, %d) must start at the block and cover it", row_start, row_end);
  return forward_rows(model, cache, d_x, batch, seq_len, row_start, row_end, blk_start, blk_len,
                      d_hidden_blk, (hipStream_t)stream);
}

fdllm_status fdllm_block_attention_workspace(int32_t batch, int32_t q_rows, int32_t hq,
                                             int32_t head_dim, int32_t kv_len, size_t* bytes) {
  if (!bytes || batch < 1 || q_rows < 1 || hq < 1 || kv_len < 1)
    return fail(FDLLM_EINVAL, "bad attention shape");
  int s = plan_attention_splits(batch, q_rows, hq, kv_len);
  size_t b = (size_t)attention_tickets(batch, q_rows, hq) * 4;
  b = (size_t)round_up((int64_t)b, 256);
  if (s > 1) b += attention_part_floats(batch, q_rows, hq, head_dim, s) * 4;
  *bytes = b;
  return FDLLM_OK;
}

fdllm_status fdllm_block_attention(const void* d_q, const void* d_k, const void* d_v, void* d_o,
                                   float* d_lse, int32_t batch, int32_t q_rows, int32_t hq,
                                   int32_t hkv, int32_t head_dim, int32_t kv_len, int32_t dtype,
                                   float scale, void* d_workspace, size_t workspace_bytes,
                                   void* stream) {
  if (!d_q || !d_k || !d_v || !d_o) return fail(FDLLM_EINVAL, "NULL argument");
  if (dtype != FDLLM_F32 && dtype != FDLLM_BF16) return fail(FDLLM_EDTYPE, "dtype %d", dtype);
  if (batch < 1 || q_rows < 1 || hq < 1 || hkv < 1 || hq % hkv)
    return fail(FDLLM_ESHAPE, "bad head / row counts");
  if (head_dim != 64 && head_dim != 128) return fail(FDLLM_ESHAPE, "head_dim must be 64 or 128");
  if (kv_len < 1 || kv_len % 4) return fail(FDLLM_ESHAPE, "kv_len must be a positive multiple of 4");
  if (!std::isfinite(scale)) return fail(FDLLM_EINVAL, "scale must be finite");
  AttnProblem a;
  a.dt = dtype == FDLLM_BF16 ? kBF16 : kF32;
  a.qdt = a.dt;
  a.q = d_q;
  a.o = d_o;
  a.k = d_k;
  a.vt = d_v;
  a.batch = batch;
  a.rows = q_rows;
  a.hq = hq;
  a.hkv = hkv;
  a.d = head_dim;
  a.kv_len = kv_len;
  a.ncap = kv_len;
  a.scale = scale;
  a.splits = 1;
  a.lse = d_lse;
  if (d_workspace) {
    size_t need = 0;
    fdllm_block_attention_workspace(batch, q_rows, hq, head_dim, kv_len, &need);
    if (workspace_bytes < need) return fail(FDLLM_EINVAL, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    a.splits = plan_attention_splits(batch, q_rows, hq, kv_len);
    a.tickets = (int*)d_workspace;
    a.part = (float*)((char*)d_workspace +
                      round_up((int64_t)attention_tickets(batch, q_rows, hq) * 4, 256));
  }
  HIP_TRY(launch_attention(a, (hipStream_t)stream));
  return FDLLM_OK;
}

fdllm_status fdllm_tile_values(const void* d_v, void* d_vt, int32_t batch, int32_t hkv,
                               int32_t kv_len, int32_t head_dim, int32_t dtype, void* stream) {
  if (!d_v || !d_vt) return fail(FDLLM_EINVAL, "NULL argument");
  if (dtype != FDLLM_F32 && dtype != FDLLM_BF16) return fail(FDLLM_EDTYPE, "dtype %d", dtype);
  if (batch < 1 || hkv < 1 || kv_len < 1) return fail(FDLLM_ESHAPE, "bad batch / head / key counts");
  if (head_dim != 64 && head_dim != 128) return fail(FDLLM_ESHAPE, "head_dim must be 64 or 128");
  HIP_TRY(launch_tile_values(dtype == FDLLM_BF16 ? kBF16 : kF32, d_v, d_vt, batch, hkv, kv_len,
                             head_dim, (hipStream_t)stream));
  return FDLLM_OK;
}

fdllm_status fdllm_confidence_unmask(fdllm_model* model, fdllm_cache* cache,
                                     const void* d_hidden_blk, int32_t* d_x, uint8_t* d_masked,
                                     int32_t batch, int32_t seq_len, int32_t blk_start,
                                     int32_t blk_len, const fdllm_select_params* rule,
                                     int32_t step_in_block, int32_t steps_per_block, float* d_conf,
                                     int32_t* d_argmax, int32_t* d_counts, float* d_logits,
                                     void* stream) {
  if (!model || !cache || !d_hidden_blk || !d_x || !d_masked) return fail(FDLLM_EINVAL, "NULL argument");
  if ((uintptr_t)d_hidden_blk % 16) return fail(FDLLM_EINVAL, "d_hidden_blk must be 16-byte aligned");
  if (cache->model != model) return fail(FDLLM_EINVAL, "cache belongs to another model");
  fdllm_status s = check_rows(cache, batch, seq_len, blk_start, blk_len);
  if (s) return s;
  SelectRuleArgs ra;
  s = check_select(rule, &ra);
  if (s) return s;
  if (steps_per_block < 1 || step_in_block < 0 || step_in_block >= steps_per_block)
    return fail(FDLLM_EINVAL, "need 0 <= step_in_block < steps_per_block");
  if (batch * blk_len > kMaxBlock * 4)
    return fail(FDLLM_EINVAL, "batch * blk_len must be <= %d", kMaxBlock * 4);
  return unmask_fused(model, cache, d_hidden_blk, d_x, d_masked, batch, seq_len, blk_start,
                      blk_len, ra, step_in_block, steps_per_block, d_conf, d_argmax, d_counts,
                      d_logits, (hipStream_t)stream);
}

fdllm_status fdllm_unmask_logits_workspace(int32_t batch, int32_t blk_len, int32_t vocab,
                                           size_t* bytes) {
  if (!bytes || batch < 1 || blk_len < 1 || vocab < 1) return fail(FDLLM_EINVAL, "bad shape");
  *bytes = (size_t)batch * blk_len * unmask_chunks(vocab) * (sizeof(float4) + sizeof(float2));
  return FDLLM_OK;
}

fdllm_status fdllm_confidence_unmask_logits(const void* d_logits, int32_t dtype, int32_t* d_x,
                                            uint8_t* d_masked, int32_t batch, int32_t seq_len,
                                            int32_t blk_start, int32_t blk_len, int32_t vocab,
                                            const fdllm_select_params* rule, int32_t step_in_block,
                                            int32_t steps_per_block, float* d_conf,
                                            int32_t* d_argmax, int32_t* d_counts,
                                            void* d_workspace, size_t workspace_bytes,
                                            void* stream) {
  if (!d_workspace) return fail(FDLLM_EINVAL, "NULL argument");
  SelectRuleArgs ra;
  fdllm_status s = check_unmask_logits(d_logits, dtype, d_x, d_masked, batch, seq_len, blk_start,
                                       blk_len, vocab, rule, step_in_block, steps_per_block, &ra);
  if (s) return s;
  size_t need = 0;
  fdllm_unmask_logits_workspace(batch, blk_len, vocab, &need);
  if (workspace_bytes < need) return fail(FDLLM_EINVAL, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  float4* stats = (float4*)d_workspace;
  HIP_TRY(launch_unmask_logits(dtype == FDLLM_BF16 ? kBF16 : kF32, d_logits, d_x, d_masked, batch,
                               seq_len, blk_start, blk_len, vocab, ra, step_in_block,
                               steps_per_block, d_conf, d_argmax, d_counts, stats,
                               (hipStream_t)stream));
  return FDLLM_OK;
}

fdllm_status fdllm_workspace_bytes(const fdllm_model* model, int32_t batch, int32_t max_seq,
                                  size_t* bytes) {
  size_t total = 0;
  fdllm_status s = fdllm_cache_bytes(model, batch, max_seq, &total);
  if (s) return s;
  // the K/V blocks come first (from offset 0, each 256-byte aligned), the
  // working buffers after the last layer's V
  const fdllm_model_config& cf = model->cfg;
  const int64_t ncap = round_up(max_seq, 32);
  const size_t kv = (size_t)cf.n_layers * 2 *
                    round_up((int64_t)batch * cf.n_kv_heads * ncap * cf.head_dim * model->es, 256);
  *bytes = total - kv;
  return FDLLM_OK;
}

fdllm_status fdllm_stream_read_blocks(size_t bytes, int32_t* blocks) {
  if (!blocks || bytes % 16) return fail(FDLLM_EINVAL, "bytes must be a multiple of 16");
  *blocks = stream_read_blocks(bytes);
  return FDLLM_OK;
}

fdllm_status fdllm_stream_read(const void* d_buf, size_t bytes, float* d_out, void* stream) {
  if (!d_buf || !d_out) return fail(FDLLM_EINVAL, "NULL argument");
  if (bytes % 16) return fail(FDLLM_EINVAL, "bytes must be a multiple of 16");
  HIP_TRY(launch_stream_read(d_buf, bytes, d_out, (hipStream_t)stream));
  return FDLLM_OK;
}

fdllm_status fdllm_confidence_unmask_logits_noalloc(
    const void* d_logits, int32_t dtype, int32_t* d_x, uint8_t* d_masked, int32_t batch,
    int32_t seq_len, int32_t blk_start, int32_t blk_len, int32_t vocab,
    const fdllm_select_params* rule, int32_t step_in_block, int32_t steps_per_block, float* d_conf,
    int32_t* d_argmax, int32_t* d_counts, void* stream) {
  SelectRuleArgs ra;
  fdllm_status s = check_unmask_logits(d_logits, dtype, d_x, d_masked, batch, seq_len, blk_start,
                                       blk_len, vocab, rule, step_in_block, steps_per_block, &ra);
  if (s) return s;
  const int64_t entries = (int64_t)batch * blk_len * unmask_chunks(vocab);
  if (entries > kStaticUnmaskEntries)
    return fail(FDLLM_EINVAL,
                "batch * blk_len * ceil(vocab / 16384) = %lld exceeds the fixed scratch of %d entries",
                (long long)entries, kStaticUnmaskEntries);
  float4* stats = nullptr;
  HIP_TRY(unmask_static_scratch(&stats));
  HIP_TRY(launch_unmask_logits(dtype == FDLLM_BF16 ? kBF16 : kF32, d_logits, d_x, d_masked, batch,
                               seq_len, blk_start, blk_len, vocab, ra, step_in_block,
                               steps_per_block, d_conf, d_argmax, d_counts, stats,
                               (hipStream_t)stream));
  return FDLLM_OK;
}

fdllm_status fdllm_cache_kv(const fdllm_cache* cache, int32_t layer, void** d_k, void** d_v,
                            int32_t* ncap) {
  if (!cache || !d_k || !d_v || !ncap) return fail(FDLLM_EINVAL, "NULL argument");
  if (layer < 0 || layer >= cache->model->cfg.n_layers)
    return fail(FDLLM_EINVAL, "layer %d outside [0, %d)", layer, cache->model->cfg.n_layers);
  *d_k = cache->k[layer];
  *d_v = cache->vt[layer];
  *ncap = cache->ncap;
  return FDLLM_OK;
}

fdllm_status fdllm_kv_cosine(const void* d_k_a, const void* d_v_a, const void* d_k_b,
                             const void* d_v_b, int32_t batch, int32_t n_kv_heads, int32_t cap,
                             int32_t head_dim, int32_t row0, int32_t row1, int32_t dtype,
                             float* d_cos, void* stream) {
  if (!d_k_a || !d_v_a || !d_k_b || !d_v_b || !d_cos) return fail(FDLLM_EINVAL, "NULL argument");
  if (dtype != FDLLM_F32 && dtype != FDLLM_BF16) return fail(FDLLM_EDTYPE, "dtype %d", dtype);
  if (batch < 1 || n_kv_heads < 1 || head_dim < 1 || cap < 1)
    return fail(FDLLM_ESHAPE, "bad batch / head / capacity sizes");
  if (row0 < 0 || row1 < row0 || row1 > cap)
    return fail(FDLLM_EINVAL, "rows [%d, %d) outside [0, %d)", row0, row1, cap);
  HIP_TRY(launch_kv_cosine(dtype == FDLLM_BF16 ? kBF16 : kF32, d_k_a, d_v_a, d_k_b, d_v_b, batch,
                           n_kv_heads, cap, head_dim, row0, row1 - row0, d_cos,
                           (hipStream_t)stream));
  return FDLLM_OK;
}

fdllm_status fdllm_cache_profile_enable(fdllm_cache* cache, int32_t enable) {
  if (!cache) return fail(FDLLM_EINVAL, "cache is NULL");
  cache->prof.on = enable != 0;
  return FDLLM_OK;
}

fdllm_status fdllm_cache_profile_select(fdllm_cache* cache, const char* variant, int32_t stride) {
  if (!cache) return fail(FDLLM_EINVAL, "cache is NULL");
  if (stride < 1) return fail(FDLLM_EINVAL, "stride must be >= 1");
  cache->prof.only = variant ? variant : "";
  cache->prof.stride = stride;
  cache->prof.seen = 0;
  return FDLLM_OK;
}

fdllm_status fdllm_cache_profile_peaks(fdllm_cache* cache, double hbm_bytes_per_s,
                                      double flops_per_s) {
  if (!cache) return fail(FDLLM_EINVAL, "cache is NULL");
  if (!(hbm_bytes_per_s >= 0) || !(flops_per_s >= 0)) return fail(FDLLM_EINVAL, "peaks must be >= 0");
  cache->prof.peak_bw = hbm_bytes_per_s;
  cache->prof.peak_flops = flops_per_s;
  return FDLLM_OK;
}

fdllm_status fdllm_cache_profile_read(fdllm_cache* cache, char* buf, size_t len, int32_t reset) {
  if (!cache || (!buf && len)) return fail(FDLLM_EINVAL, "NULL argument");
  HIP_TRY(cache->prof.harvest());
  std::string out;
  char line[256];
  for (auto& kv : cache->prof.acc) {
    snprintf(line, sizeof line, "%s %ld %.6f %.0f %.0f %.6f\n", kv.first.c_str(), kv.second.launches,
             kv.second.ms, kv.second.bytes, kv.second.flops, kv.second.floor_ms);
    out += line;
  }
  if (reset) cache->prof.acc.clear();
  if (len) {
    size_t n = std::min(len - 1, out.size());
    memcpy(buf, out.data(), n);
    buf[n] = 0;
  }
  if (out.size() + 1 > len) return fail(FDLLM_EINVAL, "buffer too small (%zu bytes needed)", out.size() + 1);
  return FDLLM_OK;
}

fdllm_status fdllm_decode(fdllm_model* model, fdllm_cache* cache, int32_t* d_x, uint8_t* d_masked,
                          int32_t batch, int32_t prompt_len, const fdllm_decode_params* params,
                          fdllm_decode_stats* stats, void* stream) {
  if (!model || !cache || !d_x || !d_masked || !params) return fail(FDLLM_EINVAL, "NULL argument");
  if (cache->model != model) return fail(FDLLM_EINVAL, "cache belongs to another model");
  const fdllm_decode_params& P = *params;
  const int L = P.gen_length, B = P.block_size;
  if (L < 1 || B < 1 || L % B) return fail(FDLLM_EINVAL, "gen_length must be a positive multiple of block_size");
  if (B > kMaxBlock) return fail(FDLLM_EINVAL, "block_size must be <= %d", kMaxBlock);
  const int K = L / B;
  if (P.steps < 1 || P.steps % K) return fail(FDLLM_EINVAL, "steps must be a positive multiple of gen_length / block_size");
  const int T = P.steps / K;
  if (P.dual_cache && !P.use_cache) return fail(FDLLM_EINVAL, "dual cache requires use_cache");
  if (!std::isfinite(P.threshold)) return fail(FDLLM_EINVAL, "threshold must be finite");
  if (!std::isfinite(P.factor) || P.factor < 0.f) return fail(FDLLM_EINVAL, "factor must be finite and >= 0");
  if (P.refresh_interval < 0) return fail(FDLLM_EINVAL, "refresh_interval must be >= 0");
  SelectRuleArgs rule;
  {
    fdllm_select_params sp{P.threshold, P.factor, P.topk, P.sampling, P.seed};
    fdllm_status sr = check_select(&sp, &rule);
    if (sr) return sr;
  }
  if (prompt_len < 0) return fail(FDLLM_EINVAL, "prompt_len must be >= 0");
  const int N = prompt_len + L;
  fdllm_status s = check_rows(cache, batch, N, prompt_len, B);
  if (s) return s;
  if (batch * B > kMaxBlock * 4)
    return fail(FDLLM_EINVAL, "batch * block_size must be <= %d", kMaxBlock * 4);
  hipStream_t st = (hipStream_t)stream;
  // prompt ids must be real tokens
  if (prompt_len > 0) {
    std::vector<int32_t> hx((size_t)batch * N);
    HIP_TRY(hipMemcpyAsync(hx.data(), d_x, hx.size() * 4, hipMemcpyDeviceToHost, st));
    HIP_TRY(hipStreamSynchronize(st));
    for (int b = 0; b < batch; ++b)
      for (int i = 0; i < prompt_len; ++i) {
        int v = hx[(size_t)b * N + i];
        if (v < 0 || v >= model->cfg.vocab || v == model->cfg.mask_id)
          return fail(FDLLM_EINVAL, "prompt id %d at [%d][%d] is not a vocabulary token", v, b, i);
      }
  }
  fdllm_decode_stats local;
  fdllm_decode_stats* S = stats ? stats : &local;
  memset(S, 0, sizeof *S);
  for (int k = 0; k < K; ++k) {
    const int s0 = prompt_len + k * B;
    int t = 0;
    for (;;) {
      if (t == 0 || !P.use_cache || (P.refresh_interval > 0 && t % P.refresh_interval == 0)) {
        s = forward_rows(model, cache, d_x, batch, N, 0, N, s0, B, cache->hidden, st);
        if (P.use_cache || t == 0) S->refreshes++;
        else S->full_steps++;
      } else {
        const int r1 = P.dual_cache ? s0 + B : N;
        s = forward_rows(model, cache, d_x, batch, N, s0, r1, s0, B, cache->hidden, st);
        S->cached_steps++;
      }
      if (s) return s;
      s = unmask_fused(model, cache, cache->hidden, d_x, d_masked, batch, N, s0, B, rule, t, T,
                       nullptr, nullptr, cache->counts, nullptr, st);
      if (s) return s;
      HIP_TRY(hipMemcpyAsync(cache->host_counts, cache->counts, (size_t)batch * 2 * 4,
                             hipMemcpyDeviceToHost, st));
      HIP_TRY(hipStreamSynchronize(st));
      if (cache->prof.on) HIP_TRY(cache->prof.harvest());
      int left = 0, now = 0;
      for (int b = 0; b < batch; ++b) {
        now += cache->host_counts[2 * b];
        left += cache->host_counts[2 * b + 1];
      }
      S->committed += now;
      if (S->nfe < FDLLM_STATS_STEPS) S->commits_per_step[S->nfe] = now;
      S->nfe++;
      ++t;
      if (left == 0) break;
      if (t >= T) return fail(FDLLM_EBUDGET, "block %d still has %d masked positions after %d steps", k, left, T);
    }
    if (k < FDLLM_STATS_BLOCKS) S->steps_per_block[k] = t;
    S->max_steps_block = std::max(S->max_steps_block, t);
  }
  return FDLLM_OK;
}

}  // extern "C"

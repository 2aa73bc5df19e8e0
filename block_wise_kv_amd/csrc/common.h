// Device helpers shared by the fdllm HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fdllm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: workgroup i is dispatched to XCD i % 8

// ---- bf16 storage (uint16 bit patterns) -----------------------------------
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Round-to-nearest-even float -> bf16 (v_cvt_pk_bf16_f32 on gfx950; NaN stays NaN).
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// Two at once: a in the low half, b in the high half.
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}
// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi), for 8 values: the
// two bf16 terms a float32 operand enters a bf16 matrix product as.
__device__ __forceinline__ void split_bf16x8(const float* x, uint4& hi, uint4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h[j] = f2bf2(x[2 * j], x[2 * j + 1]);
    const float h0 = __uint_as_float(h[j] << 16), h1 = __uint_as_float(h[j] & 0xffff0000u);
    l[j] = f2bf2(x[2 * j] - h0, x[2 * j + 1] - h1);
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// ---- value cache layout ----------------------------------------------------
// V of one (sequence, kv head) is stored tile-major for the P V product:
// tile t of 32 keys is a contiguous [D][32] block at element t * D * 32, and
// within a row d, logical key k of the tile sits at column vtile_col(k), so
// that the 8 keys lane group g feeds to the MFMA (keys 4g..4g+3 and
// 16+4g..16+4g+3) are the contiguous columns 8g..8g+7.
__host__ __device__ __forceinline__ int vtile_col(int k) {
  return 8 * ((k & 15) >> 2) + 4 * (k >> 4) + (k & 3);
}
// element offset of (key, dim) in a [ceil(keys / 32)][D][32] block
__host__ __device__ __forceinline__ size_t vtile_off(int key, int d, int D) {
  return ((size_t)(key >> 5) * D + d) * 32 + vtile_col(key & 31);
}

// ---- split activation layout ----------------------------------------------
// A float32 activation matrix [rows][K] that only feeds an MFMA product is
// kept as that product's operand: 2 KB fragment slots, slot (m / 16, k / 32)
// at byte ((m / 16) * (K / 32) + k / 32) * 2048. Within a slot, lane
// l = m % 16 + 16 * ((k % 32) / 8) owns 16 bytes at l * 16 of the first KB
// and 16 bytes at 1024 + l * 16 of the second: for bf16 products the high
// and low bf16 terms (x = hi + lo) of the 8 values k - k % 8 .. + 7, for
// float32 products those values as float32, 0-3 then 4-7. A GEMM copies the
// slots of its tile straight into LDS.
__device__ __forceinline__ char* xs_lane(char* xs, int kslots, int m, int k) {
  return xs + ((size_t)(m >> 4) * kslots + (k >> 5)) * 2048 + ((m & 15) + 16 * ((k & 31) >> 3)) * 16;
}

// Element storage type tags.
struct BF16 {
  using store_t = uint16_t;
  static __device__ __forceinline__ float load(const uint16_t* p) { return bf2f(*p); }
  static __device__ __forceinline__ uint16_t from_f(float f) { return f2bf(f); }
  static __device__ __forceinline__ float to_f(uint16_t v) { return bf2f(v); }
};
struct F32 {
  using store_t = float;
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ float from_f(float f) { return f; }
  static __device__ __forceinline__ float to_f(float v) { return v; }
};

// Writes values k .. k+3 (k % 4 == 0) or k .. k+7 (k % 8 == 0) of row m in
// the split activation layout.
template <typename T> struct XSplit;
template <> struct XSplit<BF16> {
  static __device__ __forceinline__ void store4(char* xs, int kslots, int m, int k, float a, float b,
                                                float c, float d) {
    char* p = xs_lane(xs, kslots, m, k) + (k & 4) * 2;
    const uint32_t h0 = f2bf2(a, b), h1 = f2bf2(c, d);
    const uint32_t l0 = f2bf2(a - __uint_as_float(h0 << 16), b - __uint_as_float(h0 & 0xffff0000u));
    const uint32_t l1 = f2bf2(c - __uint_as_float(h1 << 16), d - __uint_as_float(h1 & 0xffff0000u));
    *(uint2*)p = make_uint2(h0, h1);
    *(uint2*)(p + 1024) = make_uint2(l0, l1);
  }
  static __device__ __forceinline__ void store8(char* xs, int kslots, int m, int k, const float* v) {
    char* p = xs_lane(xs, kslots, m, k);
    uint4 hi, lo;
    split_bf16x8(v, hi, lo);
    *(uint4*)p = hi;
    *(uint4*)(p + 1024) = lo;
  }
};
template <> struct XSplit<F32> {
  static __device__ __forceinline__ void store4(char* xs, int kslots, int m, int k, float a, float b,
                                                float c, float d) {
    *(float4*)(xs_lane(xs, kslots, m, k) + (k & 4) * 256) = make_float4(a, b, c, d);
  }
  static __device__ __forceinline__ void store8(char* xs, int kslots, int m, int k, const float* v) {
    char* p = xs_lane(xs, kslots, m, k);
    *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
    *(float4*)(p + 1024) = make_float4(v[4], v[5], v[6], v[7]);
  }
};

// ---- MFMA fragments --------------------------------------------------------
// A "fragment" feeds one 16x16 output tile over a 32-wide slice of the
// contraction index. Lane l holds 8 consecutive contraction elements
// 8*(l/16) .. 8*(l/16)+7 of row (A operand) or column (B operand) l%16.
// The accumulator tile holds C[4*(l/16) + i][l%16], i = 0..3.
// bf16: one v_mfma_f32_16x16x32_bf16. f32: eight v_mfma_f32_16x16x4_f32,
// MFMA j taking element j of every lane (the same lane->index map on both
// operands, so the sum covers all 32 contraction elements).
struct FragBF {
  uint4 v;  // 8 bf16
};
struct FragF32 {
  float4 lo, hi;  // 8 floats
};

template <typename T> struct Frag;
template <> struct Frag<BF16> { using type = FragBF; };
template <> struct Frag<F32> { using type = FragF32; };

__device__ __forceinline__ void mma(f32x4_t& acc, const FragBF& a, const FragBF& b) {
  bf16x8_t av = __builtin_bit_cast(bf16x8_t, a.v);
  bf16x8_t bv = __builtin_bit_cast(bf16x8_t, b.v);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
}

__device__ __forceinline__ void mma(f32x4_t& acc, const FragF32& a, const FragF32& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.x, b.lo.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.y, b.lo.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.z, b.lo.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.w, b.lo.w, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.x, b.hi.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.y, b.hi.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.z, b.hi.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.w, b.hi.w, acc, 0, 0, 0);
}

// Fragment element count and bytes per lane.
template <typename T> struct FragInfo;
template <> struct FragInfo<BF16> { static constexpr int kBytes = 16; };
template <> struct FragInfo<F32> { static constexpr int kBytes = 32; };

// Streaming (read-once) loads: non-temporal hint.
__device__ __forceinline__ uint4 ld_nt_u4(const void* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4_t*)p));
}
__device__ __forceinline__ float4 ld_nt_f4(const void* p) {
  return __builtin_bit_cast(float4, __builtin_nontemporal_load((const f32x4_t*)p));
}
__device__ __forceinline__ void load_frag(FragBF& f, const void* p) { f.v = ld_nt_u4(p); }
__device__ __forceinline__ void load_frag(FragF32& f, const void* p) {
  f.lo = ld_nt_f4(p);
  f.hi = ld_nt_f4((const float4*)p + 1);
}
__device__ __forceinline__ void load_frag_cached(FragBF& f, const void* p) { f.v = *(const uint4*)p; }
__device__ __forceinline__ void load_frag_cached(FragF32& f, const void* p) {
  f.lo = ((const float4*)p)[0];
  f.hi = ((const float4*)p)[1];
}

// ---- launch helpers ----------------------------------------------------------
// Maps the hardware block id to a work index so that consecutive work indices
// land on the same XCD (and so share its L2): blocks on XCD x take the x-th
// contiguous share of [0, nblocks).
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  int per = nblocks / kXcds, rem = nblocks % kXcds;
  int x = bid % kXcds, j = bid / kXcds;
  return x < rem ? x * (per + 1) + j : rem * (per + 1) + (x - rem) * per + j;
}

// Cross-workgroup hand-off of partial results. The L2 is per XCD and not
// coherent across XCDs within a kernel; agent-scope release/acquire fences
// would write back / invalidate the whole L2 of every XCD involved. Instead,
// partial results are written with agent-coherent stores (st_agent*: the
// line is written through to the device-coherent level) and read with
// agent-coherent loads (ld_agent*); a writer waits for its stores to be
// acknowledged (vmcnt 0) before taking the completion ticket. Each partial
// line has one writer workgroup, and the reader reads it only after the
// ticket shows that every writer finished.
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-byte agent-coherent accesses through a raw buffer resource (the sc1
// cache-policy bit, as the scalar agent-scope atomics above use). `base` must
// be 16-byte aligned and offsets below 2 GiB.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t agent_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}
constexpr int kSc1 = 16;  // buffer cache policy: sc1
__device__ __forceinline__ void st_agent4(__amdgpu_buffer_rsrc_t r, int byte_off, f32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, byte_off, 0, kSc1);
}
__device__ __forceinline__ f32x4_t ld_agent4(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kSc1));
}
// 8-byte variants (`base` 8-byte aligned)
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void st_agent2(__amdgpu_buffer_rsrc_t r, int byte_off, f32x2_t v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, v), r, byte_off, 0, kSc1);
}
__device__ __forceinline__ f32x2_t ld_agent2(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, kSc1));
}

// Completion ticket. Every workgroup of a group calls it once after writing
// its partial results with st_agent*; returns true in exactly one workgroup
// (the last to arrive), which may then read every partial of the group with
// ld_agent*. The ticket is reset for the next launch. Must be called by all
// threads of the block (contains __syncthreads).
__device__ __forceinline__ bool last_arrival(int* ticket, int group_size) {
  __shared__ int s_last;
  // vmcnt(0), expcnt/lgkmcnt unconstrained: this wave's stores are acknowledged
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  if (threadIdx.x == 0) {
    int prev = __hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int last = (prev == group_size - 1);
    if (last) __hip_atomic_store(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  return s_last != 0;
}

__device__ __forceinline__ float warp_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace fdllm

// Shared device helpers for the STILL kernels (gfx950, wave64).
//
// Matrix products use 16x16 output tiles on the MFMA units:
//   bf16: v_mfma_f32_16x16x32_bf16 (one instruction per 32-deep step)
//   f32 : v_mfma_f32_16x16x4f32    (eight instructions per 32-deep step)
// A "fragment" is what one lane contributes to one 16x16x32 step: 8 values.
// With lane = 16*g + r (r = lane & 15, g = lane >> 4):
//   A fragment (16 rows x 32 deep): row r, depth slots 8g .. 8g+7
//   B fragment (32 deep x 16 cols): col r, depth slots 8g .. 8g+7
//   accumulator (16 x 16, 4 floats): acc[i] = C[4g + i][r]
// Depth slots only need to mean the same index in A and B. When a B (or A)
// fragment is assembled from two accumulator tiles X0 (depth 0..15) and X1
// (depth 16..31), lane (r, g) holds depths {4g+i} and {16+4g+i}: slot s maps
// to depth perm(g, s) = s < 4 ? 4g + s : 16 + 4g + (s - 4). Operands paired
// with such fragments are laid out in LDS with the same permutation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace still {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define STILL_NEG_INF (-__builtin_huge_valf())

typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

template <typename T>
struct Frag;
template <>
struct Frag<bf16> {
  bf16x8 v;
};
template <>
struct Frag<f16> {
  f16x8 v;
};
template <>
struct Frag<float> {
  f32x4 lo, hi;
};

__device__ __forceinline__ void mma(f32x4& c, const Frag<bf16>& a, const Frag<bf16>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}

__device__ __forceinline__ void mma(f32x4& c, const Frag<f16>& a, const Frag<f16>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.v, c, 0, 0, 0);
}

__device__ __forceinline__ void mma(f32x4& c, const Frag<float>& a, const Frag<float>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[0], b.lo[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[1], b.lo[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[2], b.lo[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[3], b.lo[3], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[0], b.hi[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[1], b.hi[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[2], b.hi[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[3], b.hi[3], c, 0, 0, 0);
}

// 8 consecutive elements (16-byte aligned for bf16, 32-byte for f32).
__device__ __forceinline__ Frag<bf16> ld_frag(const bf16* p) {
  Frag<bf16> f;
  f.v = *reinterpret_cast<const bf16x8*>(p);
  return f;
}
__device__ __forceinline__ Frag<f16> ld_frag(const f16* p) {
  Frag<f16> f;
  f.v = *reinterpret_cast<const f16x8*>(p);
  return f;
}
__device__ __forceinline__ Frag<float> ld_frag(const float* p) {
  Frag<float> f;
  f.lo = *reinterpret_cast<const f32x4*>(p);
  f.hi = *reinterpret_cast<const f32x4*>(p + 4);
  return f;
}
// An LDS address the optimizer cannot see through (held in an SGPR).
// Accesses at constant offsets from it use the 16-bit offset field of the
// LDS instruction; without this, offsets from a known base above 64 KiB each
// take an address register of their own, which the compiler hoists out of
// loops.
// threadIdx.x through an empty asm: values derived from it are recomputed
// where they are used instead of being hoisted out of loops and kept live
__device__ __forceinline__ int opaque_tid() {
  int x = threadIdx.x;
  asm volatile("" : "+v"(x));
  return x;
}
typedef __attribute__((address_space(3))) char lds_char;
// The same through a VGPR, for code the compiler may place under divergent
// control flow.
template <typename X>
__device__ __forceinline__ X* lds_opaque_v(X* p) {
  unsigned a = (unsigned)(__UINTPTR_TYPE__)(lds_char*)(char*)p;
  asm volatile("" : "+v"(a));
  return (X*)(char*)(lds_char*)(__UINTPTR_TYPE__)a;
}
template <typename X>
__device__ __forceinline__ X* lds_opaque(X* p) {
  unsigned a = (unsigned)(__UINTPTR_TYPE__)(lds_char*)(char*)p;
  asm volatile("" : "+s"(a));
  return (X*)(char*)(lds_char*)(__UINTPTR_TYPE__)a;
}

// A 16-bit MFMA fragment read transposed from LDS (gfx950
// ds_read_b64_tr_b16): within each 16-lane group, lane i receives element
// i & 3 of the 8-byte chunks addressed by lanes (i >> 2) + 4k, k = 0..3.
// With lane c of group g addressing row R0 + 4g + (c >> 2), columns
// C0 + 4 (c & 3), lane (r, g) gets column C0 + r of rows R0 + 4g + k; a
// second read `step` elements further gives rows + 16: together the depth
// slots perm(g, 0..7) of a fragment whose depth runs along the rows.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
__device__ __forceinline__ Frag<f16> tr_frag(const f16* p, int step) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_char*)(char*)p);
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_char*)(char*)(p + step));
  Frag<f16> f;
  const f16x4_t a4 = __builtin_bit_cast(f16x4_t, a), b4 = __builtin_bit_cast(f16x4_t, b);
  f.v = f16x8{a4[0], a4[1], a4[2], a4[3], b4[0], b4[1], b4[2], b4[3]};
  return f;
}

// The same read for bf16 data (the transposing read moves 16-bit values,
// whatever their type).
__device__ __forceinline__ Frag<bf16> tr_frag_bf16(const bf16* p, int step) {
  const Frag<f16> f = tr_frag(reinterpret_cast<const f16*>(p), step);
  Frag<bf16> r;
  r.v = __builtin_bit_cast(bf16x8, f.v);
  return r;
}

// Buffer-resource loads: the lane-dependent part of an address is a 32-bit
// VGPR offset and the uniform part an SGPR offset, so unrolled loops over
// uniform offsets need no per-iteration 64-bit address registers. Reads at
// or past `bytes` return zero (raw buffer range check).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
template <typename T>
__device__ __forceinline__ Frag<T> ld_frag_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff);
// (POL: the cache policy bits of the load; CPOL_NT marks data read once,
// which the caches may evict first)
constexpr int CPOL_NT = 2;
template <typename T, int POL = 0>
__device__ __forceinline__ Frag<T> ld_frag_buf_p(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (sizeof(T) == 2) {
    Frag<T> f;
    f.v = __builtin_bit_cast(decltype(f.v), __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, POL));
    return f;
  } else {
    Frag<T> f;
    f.lo = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, POL));
    f.hi = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff + 16, POL));
    return f;
  }
}
template <>
__device__ __forceinline__ Frag<bf16> ld_frag_buf<bf16>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return ld_frag_buf_p<bf16>(r, voff, soff);
}
template <>
__device__ __forceinline__ Frag<float> ld_frag_buf<float>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return ld_frag_buf_p<float>(r, voff, soff);
}
__device__ __forceinline__ uint4 ld_u4_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return uint4{x[0], x[1], x[2], x[3]};
}

__device__ __forceinline__ void st_frag(bf16* p, const Frag<bf16>& f) {
  *reinterpret_cast<bf16x8*>(p) = f.v;
}
__device__ __forceinline__ void st_frag(f16* p, const Frag<f16>& f) {
  *reinterpret_cast<f16x8*>(p) = f.v;
}
__device__ __forceinline__ void st_frag(float* p, const Frag<float>& f) {
  *reinterpret_cast<f32x4*>(p) = f.lo;
  *reinterpret_cast<f32x4*>(p + 4) = f.hi;
}

template <typename T>
__device__ __forceinline__ Frag<T> zero_frag();
template <>
__device__ __forceinline__ Frag<bf16> zero_frag<bf16>() {
  Frag<bf16> f;
  for (int i = 0; i < 8; ++i) f.v[i] = (bf16)0.0f;
  return f;
}
template <>
__device__ __forceinline__ Frag<f16> zero_frag<f16>() {
  Frag<f16> f;
  for (int i = 0; i < 8; ++i) f.v[i] = (f16)0.0f;
  return f;
}
template <>
__device__ __forceinline__ Frag<float> zero_frag<float>() {
  Frag<float> f;
  f.lo = f32x4{0.f, 0.f, 0.f, 0.f};
  f.hi = f.lo;
  return f;
}

// Element-wise magnitude of a fragment (sign bits cleared).
__device__ __forceinline__ Frag<bf16> frag_abs(const Frag<bf16>& f) {
  Frag<bf16> r;
  r.v = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, f.v) & 0x7fff7fffu);
  return r;
}
__device__ __forceinline__ Frag<float> frag_abs(const Frag<float>& f) {
  Frag<float> r;
  r.lo = __builtin_bit_cast(f32x4, __builtin_bit_cast(u32x4, f.lo) & 0x7fffffffu);
  r.hi = __builtin_bit_cast(f32x4, __builtin_bit_cast(u32x4, f.hi) & 0x7fffffffu);
  return r;
}

// Fragment from two accumulator tiles (slots 0..3 from x0, 4..7 from x1).
template <typename T>
__device__ __forceinline__ Frag<T> frag_from(const f32x4& x0, const f32x4& x1);
template <>
__device__ __forceinline__ Frag<bf16> frag_from<bf16>(const f32x4& x0, const f32x4& x1) {
  Frag<bf16> f;
  f.v[0] = (bf16)x0[0]; f.v[1] = (bf16)x0[1]; f.v[2] = (bf16)x0[2]; f.v[3] = (bf16)x0[3];
  f.v[4] = (bf16)x1[0]; f.v[5] = (bf16)x1[1]; f.v[6] = (bf16)x1[2]; f.v[7] = (bf16)x1[3];
  return f;
}
template <>
__device__ __forceinline__ Frag<f16> frag_from<f16>(const f32x4& x0, const f32x4& x1) {
  Frag<f16> f;
  f.v[0] = (f16)x0[0]; f.v[1] = (f16)x0[1]; f.v[2] = (f16)x0[2]; f.v[3] = (f16)x0[3];
  f.v[4] = (f16)x1[0]; f.v[5] = (f16)x1[1]; f.v[6] = (f16)x1[2]; f.v[7] = (f16)x1[3];
  return f;
}
template <>
__device__ __forceinline__ Frag<float> frag_from<float>(const f32x4& x0, const f32x4& x1) {
  Frag<float> f;
  f.lo = x0;
  f.hi = x1;
  return f;
}

// Split fp32 values into three bf16 parts (hi + mid + lo carries ~24
// significant bits, the float32 value up to ~2^-27 relative); for f32 the
// "high" part is the value and the others are zero.
template <typename T>
__device__ __forceinline__ void split3_frag(const f32x4& x0, const f32x4& x1, Frag<T>& hi,
                                            Frag<T>& mid, Frag<T>& lo);
template <>
__device__ __forceinline__ void split3_frag<bf16>(const f32x4& x0, const f32x4& x1,
                                                  Frag<bf16>& hi, Frag<bf16>& mid,
                                                  Frag<bf16>& lo) {
  for (int i = 0; i < 8; ++i) {
    const float x = i < 4 ? x0[i] : x1[i - 4];
    const bf16 a = (bf16)x;
    const float r1 = x - (float)a;
    const bf16 b = (bf16)r1;
    hi.v[i] = a;
    mid.v[i] = b;
    lo.v[i] = (bf16)(r1 - (float)b);
  }
}
template <>
__device__ __forceinline__ void split3_frag<float>(const f32x4& x0, const f32x4& x1,
                                                   Frag<float>& hi, Frag<float>& mid,
                                                   Frag<float>& lo) {
  hi.lo = x0;
  hi.hi = x1;
  mid = zero_frag<float>();
  lo = mid;
}

// Split fp32 values into a high and a low bf16 part (hi + lo keeps ~16
// significant bits); for f32 the high part is the value and lo is zero.
template <typename T>
__device__ __forceinline__ void split2_frag(const f32x4& x0, const f32x4& x1, Frag<T>& hi,
                                            Frag<T>& lo);
template <>
__device__ __forceinline__ void split2_frag<bf16>(const f32x4& x0, const f32x4& x1,
                                                  Frag<bf16>& hi, Frag<bf16>& lo) {
  for (int i = 0; i < 8; ++i) {
    const float x = i < 4 ? x0[i] : x1[i - 4];
    const bf16 a = (bf16)x;
    hi.v[i] = a;
    lo.v[i] = (bf16)(x - (float)a);
  }
}
// fp16: the high part is x cut to 11 significant bits by clearing the low
// 13 mantissa bits (exact in fp16 over its normal range), the low part the
// exact remainder rounded to fp16 (~22 significant bits together); one
// mask, one subtraction and two packed conversions per pair of values.
template <>
__device__ __forceinline__ void split2_frag<f16>(const f32x4& x0, const f32x4& x1,
                                                 Frag<f16>& hi, Frag<f16>& lo) {
  for (int i = 0; i < 8; ++i) {
    const float x = i < 4 ? x0[i] : x1[i - 4];
    const float h = __uint_as_float(__float_as_uint(x) & 0xFFFFE000u);
    hi.v[i] = (f16)h;
    lo.v[i] = (f16)(x - h);
  }
}
template <>
__device__ __forceinline__ void split2_frag<float>(const f32x4& x0, const f32x4& x1,
                                                   Frag<float>& hi, Frag<float>& lo) {
  hi.lo = x0;
  hi.hi = x1;
  lo = zero_frag<float>();
}

// exp / log on float32 data use the accurate library routines; on bf16 data
// (rounded to 2^-9 anyway) the hardware approximations.
template <typename T>
__device__ __forceinline__ float exp_acc(float x) {
  if constexpr (sizeof(T) == 4) return expf(x);
  else return __expf(x);
}
template <typename T>
__device__ __forceinline__ float log_acc(float x) {
  if constexpr (sizeof(T) == 4) return logf(x);
  else return __logf(x);
}
// base-2 forms (v_exp_f32 / v_log_f32 are base 2)
constexpr float STILL_LOG2E = 1.4426950408889634f;
template <typename T>
__device__ __forceinline__ float exp2_acc(float x) {
  if constexpr (sizeof(T) == 4) return exp2f(x);
  else return __builtin_amdgcn_exp2f(x);
}
template <typename T>
__device__ __forceinline__ float log2_acc(float x) {
  if constexpr (sizeof(T) == 4) return log2f(x);
  else return __builtin_amdgcn_logf(x);
}
// 64-bit mask of the n lowest bits (n clamped to [0, 64])
__device__ __forceinline__ uint64_t low_bits(int n) {
  return n <= 0 ? 0ull : (n >= 64 ? ~0ull : ((1ull << n) - 1ull));
}
template <typename T>
__device__ __forceinline__ Frag<T> ones_frag();
template <>
__device__ __forceinline__ Frag<f16> ones_frag<f16>() {
  Frag<f16> f;
  for (int i = 0; i < 8; ++i) f.v[i] = (f16)1.0f;
  return f;
}
template <>
__device__ __forceinline__ Frag<float> ones_frag<float>() {
  Frag<float> f;
  f.lo = f32x4{1.f, 1.f, 1.f, 1.f};
  f.hi = f.lo;
  return f;
}

template <typename T>
__device__ __forceinline__ float frag_sumsq(const Frag<T>& f);
template <>
__device__ __forceinline__ float frag_sumsq<bf16>(const Frag<bf16>& f) {
  float s = 0.f;
  for (int i = 0; i < 8; ++i) {
    const float x = (float)f.v[i];
    s += x * x;
  }
  return s;
}
template <>
__device__ __forceinline__ float frag_sumsq<float>(const Frag<float>& f) {
  float s = 0.f;
  for (int i = 0; i < 4; ++i) s += f.lo[i] * f.lo[i] + f.hi[i] * f.hi[i];
  return s;
}

// The channel-wise sigmoid output gate [P4 "Synergizing Linear and Sparse
// Attention: A Deep Dive into Hybrid LLM Architectures", §4 Gating
// Mechanism]: sigmoid(g) = 1 / (1 + exp(-g)) (0 for g -> -inf, 1 for
// g -> +inf), the hardware exponential and reciprocal (~2 ulp).
__device__ __forceinline__ float sigmoid_gate(float g) {
  return __builtin_amdgcn_rcpf(1.f + __expf(-g));
}
// sigmoid gates of 4 consecutive elements at byte offset off of a buffer
// (zeros past its range give 1/2)
template <typename T>
__device__ __forceinline__ f32x4 sigmoid_gate4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  // (the loaded vector is cast whole: a bit cast of one element of it
  // keeps element 0 only)
  f32x4 g;
  if constexpr (sizeof(T) == 2) {
    typedef T t4 __attribute__((ext_vector_type(4)));
    const t4 x = __builtin_bit_cast(t4, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) g[i] = sigmoid_gate((float)x[i]);
  } else {
    const f32x4 x = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) g[i] = sigmoid_gate(x[i]);
  }
  return g;
}

// Paged kept pool (the decode state without its pool rows): page p of the
// caller's arena holds POOL_PAGE_ROWS key rows, then as many value rows, of
// D elements each; table[unit * width + i] is the physical page of the
// unit's logical page i (pool rows 16 i .. 16 i + 15).
constexpr int POOL_PAGE_ROWS = 16;
struct PoolPages {
  char* base;            // the arena, or null: the pool rows live in the state
  const int32_t* table;  // [units][width]
  int n_pages, width;
};
// Byte offset in the arena of pool row i of the unit (v = 0: key, 1: value;
// row_bytes = D * element size), or -1 where its page is not one of the
// arena's.
__device__ __forceinline__ long pool_page_off(const PoolPages& pg, int unit, int i, int v, int row_bytes) {
  const int p = pg.table[(size_t)unit * pg.width + i / POOL_PAGE_ROWS];
  if (p < 0 || p >= pg.n_pages) return -1;
  return ((long)p * 2 + v) * POOL_PAGE_ROWS * row_bytes + (long)(i % POOL_PAGE_ROWS) * row_bytes;
}

// acc + sum of squares of a bf16 fragment, by packed bf16 dot products
__device__ __forceinline__ float frag_dot2_sumsq(const Frag<bf16>& f, float acc) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2_t p = {f.v[2 * i], f.v[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(p, p, acc, false);
  }
  return acc;
}

__device__ __forceinline__ float frag_sum(const Frag<bf16>& f) {
  float s = 0.f;
  for (int i = 0; i < 8; ++i) s += (float)f.v[i];
  return s;
}
__device__ __forceinline__ float frag_sum(const Frag<f16>& f) {
  float s = 0.f;
  for (int i = 0; i < 8; ++i) s += (float)f.v[i];
  return s;
}
__device__ __forceinline__ float frag_sum(const Frag<float>& f) {
  return (f.lo[0] + f.lo[1]) + (f.lo[2] + f.lo[3]) + (f.hi[0] + f.hi[1]) + (f.hi[2] + f.hi[3]);
}

// Type of the operands whose range fits binary16 (softmax weights, values,
// NP-Map feature parts): fp16 next to bf16 data (3 more significand bits;
// bf16 -> fp16 is exact for values in fp16's normal range), float next to
// float data.
template <typename T>
struct HalfOf {
  typedef f16 type;
};
template <>
struct HalfOf<float> {
  typedef float type;
};

__device__ __forceinline__ float to_f32(f16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ f16 from_f32<f16>(float x) { return (f16)x; }

// Cross-lane exchange on the VALU: DPP within a row of 16 lanes and the
// gfx950 permlane swaps across rows, instead of LDS permutes. Every control
// used here is a full permutation within a row (quad_perm, row_mirror,
// row_half_mirror), so no source lane is out of range and bound_ctrl does
// not change the result; with it set the compiler folds the move into the
// consuming add (v_add_f32_dpp), one instruction per step instead of two.
template <int CTRL>
__device__ __forceinline__ float dppf(float x) {
  static_assert(CTRL == 0xB1 || CTRL == 0x4E || CTRL == 0x141 || CTRL == 0x140 || CTRL == 0x1B,
                "full in-row permutations only");
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
// value of lane ^ 16
__device__ __forceinline__ float xor16f(float x) {
  const auto q = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, x), false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 16) ? q[0] : q[1]);
}
// value of lane ^ 32
__device__ __forceinline__ float xor32f(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, x), false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? p[0] : p[1]);
}
// float64 forms, each 32-bit half moved on its own
template <int CTRL>
__device__ __forceinline__ double dppd(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const unsigned lo = (unsigned)__builtin_amdgcn_mov_dpp((int)(unsigned)u, CTRL, 0xF, 0xF, false);
  const unsigned hi = (unsigned)__builtin_amdgcn_mov_dpp((int)(unsigned)(u >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double xor16d(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const auto ql = __builtin_amdgcn_permlane16_swap((unsigned)u, (unsigned)u, false, false);
  const auto qh = __builtin_amdgcn_permlane16_swap((unsigned)(u >> 32), (unsigned)(u >> 32), false, false);
  const bool up = threadIdx.x & 16;
  return __builtin_bit_cast(double, ((uint64_t)(up ? qh[0] : qh[1]) << 32) | (up ? ql[0] : ql[1]));
}
__device__ __forceinline__ double xor32d(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const auto pl = __builtin_amdgcn_permlane32_swap((unsigned)u, (unsigned)u, false, false);
  const auto ph = __builtin_amdgcn_permlane32_swap((unsigned)(u >> 32), (unsigned)(u >> 32), false, false);
  const bool up = threadIdx.x & 32;
  return __builtin_bit_cast(double, ((uint64_t)(up ? ph[0] : ph[1]) << 32) | (up ? pl[0] : pl[1]));
}
// sum / max over the 64 lanes of a wave, every lane receiving the same value
__device__ __forceinline__ double wave_sum_d(double x) {
  x += dppd<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dppd<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dppd<0x141>(x);  // row_half_mirror
  x += dppd<0x140>(x);  // row_mirror
  x += xor16d(x);
  return x + xor32d(x);
}
__device__ __forceinline__ double wave_max_d(double x) {
  auto mx = [](double a, double b) { return b > a ? b : a; };
  x = mx(x, dppd<0xB1>(x));
  x = mx(x, dppd<0x4E>(x));
  x = mx(x, dppd<0x141>(x));
  x = mx(x, dppd<0x140>(x));
  x = mx(x, xor16d(x));
  return mx(x, xor32d(x));
}


// Routing metric: the score that ranks a chunk's tokens. The Self-Saliency
// Score, or an alternative of the STILL article's routing-metric ablation
// ("Ablation Studies"): the diagonal attention weight, the scaled self
// logit q.k, the key norm, evenly spaced offsets (uniform), or scores the
// caller supplies (random routing draws them outside the layer).
enum { ROUTE_SALIENCY = 0, ROUTE_DIAG, ROUTE_QK, ROUTE_KEYNORM, ROUTE_UNIFORM, ROUTE_EXTERNAL };

// Uniform routing: is offset r of a chunk of C one of floor(i C / lam),
// i < lam? The only candidate is i = ceil(r lam / C) (lam <= C: the range
// [r lam / C, (r + 1) lam / C) holds at most one integer).
__device__ __forceinline__ int uniform_mark(int r, int C, int lam) {
  if (lam <= 0) return 0;
  const int i = (r * lam + C - 1) / C;
  return (i < lam && (i * C) / lam == r) ? 1 : 0;
}

// Float64 dot product of two rows of D elements by one wave (products of
// bf16 / float32 values are exact in float64); every lane gets the sum.
template <typename T, int D>
__device__ __forceinline__ double row_dot_f64(const T* x, const T* y) {
  const int lane = threadIdx.x & 63;
  double s = 0.0;
#pragma unroll
  for (int i = lane; i < D; i += 64) s = fma((double)to_f32(x[i]), (double)to_f32(y[i]), s);
  return wave_sum_d(s);
}
// Sum / max over N consecutive aligned lanes (N = 1, 2, 4, 8, 16), every
// lane of the group receiving the result.
// Maximum without the quieting of signalling NaN inputs that fmaxf costs
// (an extra v_max per operand not known to be canonical, e.g. an MFMA
// result); a NaN operand gives NaN. For values that are never NaN.
__device__ __forceinline__ float fmax_nn(float a, float b) { return __builtin_elementwise_maximum(a, b); }

template <int N>
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (N >= 2) x += dppf<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x += dppf<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dppf<0x141>(x);  // row_half_mirror
  if constexpr (N >= 16) x += dppf<0x140>(x); // row_mirror
  return x;
}
template <int N>
__device__ __forceinline__ float row_max(float x) {
  if constexpr (N >= 2) x = fmax_nn(x, dppf<0xB1>(x));
  if constexpr (N >= 4) x = fmax_nn(x, dppf<0x4E>(x));
  if constexpr (N >= 8) x = fmax_nn(x, dppf<0x141>(x));
  if constexpr (N >= 16) x = fmax_nn(x, dppf<0x140>(x));
  return x;
}

// Sum / max over the four lanes sharing r (lanes r, r+16, r+32, r+48).
__device__ __forceinline__ float sum_over_g(float x) {
  x += xor16f(x);
  x += xor32f(x);
  return x;
}
__device__ __forceinline__ float max_over_g(float x) {
  x = fmax_nn(x, xor16f(x));
  x = fmax_nn(x, xor32f(x));
  return x;
}

// Position of key kk (0..63) of a 64-key block in a permuted LDS row, so that
// a 16-byte read at column 32*(kk/32) + 8g yields depth slots perm(g, 0..7).
__device__ __forceinline__ int perm_col(int kk) {
  const int k32 = kk & 31;
  return (kk & 32) + 8 * ((k32 & 15) >> 2) + ((k32 >> 4) << 2) + (k32 & 3);
}

// Chunks lying wholly at or before position cC - W, i.e. before the window
// of every query of chunk c.
__device__ __host__ __forceinline__ int full_chunks_before(int c, int W, int C) {
  const long x = (long)c * C - W + 1;
  return x >= 0 ? (int)(x / C) : 0;
}

// Kept-pool size when chunk c starts: lambda per decided chunk until the
// budget of m - W slots is full.
__device__ __host__ __forceinline__ int pool_count_at(int c, int lam, int cap_chunks) {
  if (lam <= 0) return 0;
  return (c < cap_chunks ? c : cap_chunks) * lam;
}

// ---- the kept pool as an 8-bit store: OCP E4M3 codes (sign, 4 exponent
// bits with bias 7, 3 mantissa bits; exponent field 0 holds the multiples of
// 2^-9 below 2^-6; 448 the largest finite value, code 0x7F a NaN) of x / 2^e
// and one scale exponent byte e + 127 per row, e the smallest integer with
// amax <= 448 * 2^e, at least -126 (0 for a zero row).

// Code of y: the nearest E4M3 value, ties to the even code, magnitudes from
// 448 up to 448. Works on the float's bit fields.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t bits = __float_as_uint(y), sign = (bits >> 24) & 0x80u;
  const float a = __uint_as_float(bits & 0x7FFFFFFFu);
  if (!(a < 448.f)) return sign | 0x7Eu;
  if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.f);  // exact scaling, ties to even
  const uint32_t ab = __float_as_uint(a);
  int e = (int)(ab >> 23) - 127;  // -6 .. 8
  uint32_t keep = (ab >> 20) & 7u;
  const uint32_t rem = ab & 0xFFFFFu;
  keep += (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) ? 1u : 0u;
  if (keep == 8u) { keep = 0u; ++e; }
  return sign | ((uint32_t)(e + 7) << 3) | keep;
}

// The scale exponent of a row whose largest magnitude is amax: with
// amax = 1.f * 2^E and 448 = 1.75 * 2^8, e = E - 8, plus one if f > 0.75;
// clamped to [-126, ..] (0 for a zero row).
__device__ __forceinline__ int e4m3_row_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  const uint32_t ab = __float_as_uint(amax);
  const int e = (int)(ab >> 23) - 127 - 8 + ((ab & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return e < -126 ? -126 : e;
}
// 2^k for k in [-126, 127] (a normal float32)
__device__ __forceinline__ float pow2_int(int k) { return __uint_as_float((uint32_t)(k + 127) << 23); }

// Largest value over NL consecutive lanes (NL a power of two dividing 64,
// the group aligned to NL): every lane of the group gets it.
template <int NL>
__device__ __forceinline__ float group_max(float m) {
#pragma unroll
  for (int o = 1; o < NL; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
  return m;
}

// Two E4M3 codes (bytes 0, 1 of c; with HI bytes 2, 3) times the power of
// two s, as two bf16 values packed in 32 bits (exact while the products are
// normal bf16 values).
template <bool HI = false>
__device__ __forceinline__ uint32_t e4m3x2_scaled_bf16x2(uint32_t c, float s) {
  typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, s, HI));
}

// A fragment loaded raw: with codes, its first 8 bytes are E4M3 codes, made
// 8 bf16 values times the power of two s; else it is returned as it is (Tag
// keeps this out of code paths a template discards).
template <typename T, typename Tag>
__device__ __forceinline__ Frag<T> e4m3x8_or_raw(Tag, bool codes, const Frag<T>& f, float s) {
  static_assert(sizeof(T) == 2 && Tag::value, "8-bit rows: 16-bit data");
  const u32x4 w = __builtin_bit_cast(u32x4, f.v);
  const u32x4 r = {e4m3x2_scaled_bf16x2<false>(w[0], s), e4m3x2_scaled_bf16x2<true>(w[0], s),
                   e4m3x2_scaled_bf16x2<false>(w[1], s), e4m3x2_scaled_bf16x2<true>(w[1], s)};
  Frag<T> g;
  g.v = __builtin_bit_cast(decltype(g.v), r);
  return codes ? g : f;
}

}  // namespace still

// Shared device helpers for the gfx950 kernels of the TTT-E2E prefill.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // raw bfloat16 storage
// raw IEEE half storage (a distinct type so that templates can tell it from bf16)
struct f16_t {
  uint16_t x;
};
typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));

#define DEVI __device__ __forceinline__

DEVI float to_f(float x) { return x; }
DEVI float to_f(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }
DEVI float to_f(f16_t x) { return (float)__builtin_bit_cast(_Float16, x.x); }

template <typename T> DEVI T from_f(float f);
template <> DEVI float from_f<float>(float f) { return f; }
// float -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
template <> DEVI bf16_t from_f<bf16_t>(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
// float -> half, round to nearest even.
template <> DEVI f16_t from_f<f16_t>(float f) { return f16_t{__builtin_bit_cast(uint16_t, (_Float16)f)}; }

// ---------------------------------------------------------------------------
// MFMA fragments.  A fragment is the 8 consecutive reduction-dim elements one
// lane feeds to a 16x16 tile product with a 32-long reduction:
//   lane l holds X[row = l % 16][k = 8 * (l / 16) + j], j = 0..7
// for both operands; the 16x16 fp32 result has lane l holding
//   D[row = 4 * (l / 16) + r][col = l % 16], r = 0..3.
// bf16 uses one v_mfma_f32_16x16x32_bf16; fp32 issues eight
// v_mfma_f32_16x16x4_f32, instruction j taking element j of every lane
// group, which sums the same 32 products in another order.
// f16 (v_mfma_f32_16x16x32_f16) has the same layout and rate as bf16.
template <typename T> struct Frag;
template <> struct Frag<bf16_t> { uint4 v; };
template <> struct Frag<f16_t> { uint4 v; };
template <> struct Frag<float> { float4 lo, hi; };

DEVI void mma(f32x4_v &acc, const Frag<bf16_t> &a, const Frag<bf16_t> &b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, a.v),
                                                __builtin_bit_cast(bf16x8_v, b.v), acc, 0, 0, 0);
}
DEVI void mma(f32x4_v &acc, const Frag<f16_t> &a, const Frag<f16_t> &b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_v, a.v), __builtin_bit_cast(f16x8_v, b.v),
                                               acc, 0, 0, 0);
}
DEVI void mma(f32x4_v &acc, const Frag<float> &a, const Frag<float> &b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.x, b.lo.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.y, b.lo.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.z, b.lo.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.w, b.lo.w, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.x, b.hi.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.y, b.hi.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.z, b.hi.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.w, b.hi.w, acc, 0, 0, 0);
}

// Load a fragment of 8 contiguous elements.
DEVI void load_frag(Frag<bf16_t> &f, const bf16_t *p) { f.v = *reinterpret_cast<const uint4 *>(p); }
DEVI void load_frag(Frag<f16_t> &f, const f16_t *p) { f.v = *reinterpret_cast<const uint4 *>(p); }
DEVI void load_frag(Frag<float> &f, const float *p) {
  f.lo = *reinterpret_cast<const float4 *>(p);
  f.hi = *reinterpret_cast<const float4 *>(p + 4);
}
// Fragment from two runs of 4 contiguous elements (p[0..3], q[0..3]).
DEVI void load_frag2(Frag<bf16_t> &f, const bf16_t *p, const bf16_t *q) {
  uint2 a = *reinterpret_cast<const uint2 *>(p);
  uint2 b = *reinterpret_cast<const uint2 *>(q);
  f.v = make_uint4(a.x, a.y, b.x, b.y);
}
DEVI void load_frag2(Frag<float> &f, const float *p, const float *q) {
  f.lo = *reinterpret_cast<const float4 *>(p);
  f.hi = *reinterpret_cast<const float4 *>(q);
}
DEVI void zero_frag(Frag<bf16_t> &f) { f.v = make_uint4(0, 0, 0, 0); }
DEVI void zero_frag(Frag<f16_t> &f) { f.v = make_uint4(0, 0, 0, 0); }
DEVI void zero_frag(Frag<float> &f) {
  f.lo = make_float4(0, 0, 0, 0);
  f.hi = f.lo;
}
typedef float f32x2_v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
// Two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
DEVI uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_v{a, b}, bf16x2_v));
}
typedef _Float16 f16x2_v __attribute__((ext_vector_type(2)));
// Two floats -> two halves (round to nearest even) in one v_cvt_pk_f16_f32.
DEVI uint32_t pack_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_v{a, b}, f16x2_v));
}
// Fragment from 8 floats (rounded to T).
DEVI void pack_frag(Frag<bf16_t> &f, const float *x) {
  f.v = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                   pack_bf16x2(x[6], x[7]));
}
DEVI void pack_frag(Frag<f16_t> &f, const float *x) {
  f.v = make_uint4(pack_f16x2(x[0], x[1]), pack_f16x2(x[2], x[3]), pack_f16x2(x[4], x[5]), pack_f16x2(x[6], x[7]));
}
DEVI void pack_frag(Frag<float> &f, const float *x) {
  f.lo = make_float4(x[0], x[1], x[2], x[3]);
  f.hi = make_float4(x[4], x[5], x[6], x[7]);
}

// Store 4 consecutive values (16 bytes fp32, 8 bytes bf16).
template <typename T> DEVI void store4(T *p, const float *v);
template <> DEVI void store4<float>(float *p, const float *v) {
  *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
template <> DEVI void store4<bf16_t>(bf16_t *p, const float *v) {
  *reinterpret_cast<uint2 *>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}
template <> DEVI void store4<f16_t>(f16_t *p, const float *v) {
  *reinterpret_cast<uint2 *>(p) = make_uint2(pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]));
}

// 16-byte vector of T (8 bf16 or 4 fp32).
template <typename T> struct Vec16 {
  static constexpr int N = 16 / sizeof(T);
};

// ---------------------------------------------------------------------------
// Wave-level reductions (64 lanes).
DEVI float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
DEVI float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
// Reduce across the four 16-lane groups (lanes l, l^16, l^32, l^48) with the
// gfx950 row-swap moves (VALU, no LDS traffic): permlane16_swap of a value
// with itself yields, in its two results, the value of lane l and of lane
// l^16; permlane32_swap likewise pairs lane l with l^32.
DEVI float xor16_pair_max(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
DEVI float group4_max(float v) {
  v = xor16_pair_max(v);
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// min over the four lanes l, l^16, l^32, l^48
DEVI int group4_min_int(int v) {
  v = min(v, __shfl_xor(v, 16));
  return min(v, __shfl_xor(v, 32));
}
DEVI float group4_sum(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
// 2^x with one v_exp_f32 (results below the normal range flush to zero,
// which softmax weights tolerate).
DEVI float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N> DEVI void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// Wait for this wave's LDS operations, then join the work-group barrier
// (unlike __syncthreads, no wait on outstanding global loads).
DEVI void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
}

typedef __attribute__((address_space(3))) void lds_void;
// Raw buffer descriptor word 3 for gfx9-family 32-bit data; offsets at or past
// the extent read as zero (BUF_OOB is such an offset for any real extent).
constexpr int BUF_RSRC_W3 = 0x00020000;
constexpr uint32_t BUF_OOB = 0x7FFFFF00u;

#define LOG2E_F 1.4426950408889634f
#define LN2_F 0.6931471805599453f

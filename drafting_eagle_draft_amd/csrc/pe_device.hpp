// pe_device.hpp -- device-side building blocks shared by the gfx950 kernels.
//
// Fragments.  Every matrix-core operand in this library is a 16-byte value
// per lane ("fragment"): 8 bf16 or 4 fp32.  A 16x16 output tile is produced
// from one fragment pair:
//   bf16: one v_mfma_f32_16x16x32_bf16; lane l supplies row (l % 16) and
//         k-slots 0..7 of lane group g = l / 16;
//   fp32: four v_mfma_f32_16x16x4_f32; op j takes slot j of every lane, so
//         lane group g, slot j stands for k = 4g + j.
// Because A and B use the same (lane group, slot) -> k assignment, any fixed
// mapping of the contraction index onto (g, slot) gives the same sum; the
// kernels choose the mapping that makes their loads contiguous.
// The 16x16 fp32 result sits in 4 registers per lane: lane l holds column
// (l % 16) and rows 4*(l/16) + r for r = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pe {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef uint16_t bf16_t;  // raw bf16 storage

// Elements of T per 16-byte fragment and per 64-lane tile row (k extent).
template <typename T> struct Frag;
template <> struct Frag<bf16_t> { static constexpr int E = 8; static constexpr int KTILE = 32; };
template <> struct Frag<float>  { static constexpr int E = 4; static constexpr int KTILE = 16; };

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(((unsigned)h) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Round to nearest even: gfx950 converts in hardware (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(unsigned, v);
}

// 2^x on the transcendental unit (no range fix-ups; results below the
// normal range flush to zero, which softmax weights tolerate).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T> struct Mma;

template <> struct Mma<bf16_t> {
  static __device__ __forceinline__ floatx4 run(u32x4 a, u32x4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  static __device__ __forceinline__ floatx4 run(u32x4 a, u32x4 b, floatx4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    return c;
  }
};

// Element offset of (row m, column k) in the fragment-tile layout of a
// matrix with KT k tiles per row group: 16-row groups, each a run of KT
// 1 KB fragments; lane (m % 16, (k % KTILE) / E) holds E consecutive k.
template <typename T>
__device__ __forceinline__ long frag_off(int m, int k, int KT) {
  constexpr int E = Frag<T>::E, KTILE = Frag<T>::KTILE;
  return ((long)((m >> 4) * KT + k / KTILE) * 64 + ((k % KTILE) / E) * 16 + (m & 15)) * E + (k % E);
}

// Key-column swizzle of an fp32 attention V tile staged transposed in LDS,
// Vt[d][key] (64 keys), for the row's 16-byte chunk cc = d / E: key bits
// 2..5 flip by cc & 15.  A wave's transposing stores then spread over the
// banks (without a swizzle they hit two bank offsets), and each 4-key group
// read by the matrix cores stays contiguous (bits 0..1 are kept).
__device__ __forceinline__ int vt_swizzle_b2(int cc) { return (cc & 15) << 2; }

// Workgroup barrier that waits for this wave's LDS operations only, so
// global loads already issued (prefetched tiles) stay in flight; the plain
// __syncthreads() also waits for every outstanding global access.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ u32x4 ldg16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}

// The same load marked non-temporal (nt), for data read once that should
// not displace lines other workgroups still use.
__device__ __forceinline__ u32x4 ldg16_nt(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

__device__ __forceinline__ void stg16(void *p, u32x4 v) {
  *reinterpret_cast<u32x4 *>(p) = v;
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// Sum or maximum of v over lane pairs (l, l ^ M), M 16 or 32, through the
// gfx950 lane-swap instructions (v_permlane16/32_swap: a register move, no
// LDS round trip).  With both operands v, each lane receives its own value
// and its partner's, in row order; the two operations commute, so both
// lanes of a pair get the same result as v op shfl_xor_f(v, M).
template <int M>
__device__ __forceinline__ void xor_pair(float v, float &a, float &b) {
  static_assert(M == 16 || M == 32, "lane-swap distance");
  const unsigned u = __float_as_uint(v);
  if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  }
}
template <int M>
__device__ __forceinline__ float xor_sum(float v) {
  float a, b;
  xor_pair<M>(v, a, b);
  return a + b;
}
template <int M>
__device__ __forceinline__ float xor_max(float v) {
  float a, b;
  xor_pair<M>(v, a, b);
  return fmaxf(a, b);
}

// Order-preserving map of a float onto uint32 (larger float -> larger code).
__device__ __forceinline__ unsigned ordered_bits(float v) {
  unsigned u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float unordered_bits(unsigned o) {
  unsigned u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

// Argmax key: the larger value wins, then the lower index.  -0.0 + 0.0 is
// +0.0 (round to nearest), so the two zeros, equal as values, get one key and
// a tie between them also goes to the lower index.
__device__ __forceinline__ unsigned long long argmax_key(float v, unsigned idx) {
  return ((unsigned long long)ordered_bits(v + 0.0f) << 32) | (unsigned long long)(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int mask) {
  unsigned lo = (unsigned)v, hi = (unsigned)(v >> 32);
  lo = __shfl_xor(lo, mask, 64);
  hi = __shfl_xor(hi, mask, 64);
  return ((unsigned long long)hi << 32) | lo;
}

// Row-major LDS tiles of bf16 keys/values with permuted chunks and their
// transposed reads (decode and training attention).
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ds_read_b64_tr_b16 from LDS byte address a: within each 16-lane group,
// result element j of lane i is element i % 4 of the 8 bytes addressed by
// lane 4j + i / 4.
__device__ __forceinline__ uint2 lds_tr8(unsigned a) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(size_t)a);
  return __builtin_bit_cast(uint2, v);
}

__device__ __forceinline__ u32x4 lds_b128(unsigned a) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4 *>((size_t)a);
}

// Chunk permutation of key row k (depends on k % 16 only): XOR of the
// row's chunk index; conflict-free K-operand reads (16 keys, one chunk) and
// transposed V reads (8 keys x 2 chunks per 32 lanes) in a 64-bank model.
template <int HD>
__device__ __forceinline__ int kv_sw(int k) {
  if constexpr (HD == 64) return (2 * ((k >> 1) & 3)) ^ ((k >> 3) & 1);
  else return (2 * (k & 7)) ^ ((k >> 3) & 1);
}

}  // namespace pe

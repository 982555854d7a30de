// Device helpers shared by the gfx950 kernels of the MoE verify step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mv {

typedef uint16_t bf16_t;  // bf16 storage: raw bit pattern
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

// Round a value to what storing it in T and reading it back gives.
template <typename T> __device__ __forceinline__ float round_to(float v) {
  return to_f32(from_f32<T>(v));
}

// Elements of T per 16-byte vector.
template <typename T> struct Vec { static constexpr int N = 16 / sizeof(T); };

// Unpack one 16-byte vector into fp32 values.
__device__ __forceinline__ void unpack(const uint4 &q, float *out, float) {
  out[0] = __uint_as_float(q.x); out[1] = __uint_as_float(q.y);
  out[2] = __uint_as_float(q.z); out[3] = __uint_as_float(q.w);
}
__device__ __forceinline__ void unpack(const uint4 &q, float *out, bf16_t) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Pack fp32 values (already exactly representable in T) into 16 bytes.
__device__ __forceinline__ uint4 pack(const float *v, float) {
  return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                    __float_as_uint(v[3]));
}
__device__ __forceinline__ uint4 pack(const float *v, bf16_t) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = static_cast<uint32_t>(f32_to_bf16(v[2 * i])) |
           (static_cast<uint32_t>(f32_to_bf16(v[2 * i + 1])) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Half of a 16-byte vector (8 bytes): 4 bf16 or 2 fp32 elements.
__device__ __forceinline__ void unpack8(const uint2 &q, float *out, float) {
  out[0] = __uint_as_float(q.x); out[1] = __uint_as_float(q.y);
}
__device__ __forceinline__ void unpack8(const uint2 &q, float *out, bf16_t) {
  out[0] = __uint_as_float(q.x << 16); out[1] = __uint_as_float(q.x & 0xffff0000u);
  out[2] = __uint_as_float(q.y << 16); out[3] = __uint_as_float(q.y & 0xffff0000u);
}
__device__ __forceinline__ uint2 pack8(const float *v, float) {
  return make_uint2(__float_as_uint(v[0]), __float_as_uint(v[1]));
}
__device__ __forceinline__ uint2 pack8(const float *v, bf16_t) {
  return make_uint2(static_cast<uint32_t>(f32_to_bf16(v[0])) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16),
                    static_cast<uint32_t>(f32_to_bf16(v[2])) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16));
}
__device__ __forceinline__ uint2 ld8(const void *p) { return *reinterpret_cast<const uint2 *>(p); }
__device__ __forceinline__ void st8(void *p, const uint2 &v) { *reinterpret_cast<uint2 *>(p) = v; }

// N consecutive fp32 values (N = 2 or 4) as one vector load or store.
template <int N> __device__ __forceinline__ void ld_f32(const float *p, float *o) {
  if constexpr (N == 4) {
    const float4 q = *reinterpret_cast<const float4 *>(p);
    o[0] = q.x; o[1] = q.y; o[2] = q.z; o[3] = q.w;
  } else {
    static_assert(N == 2, "2 or 4 values");
    const float2 q = *reinterpret_cast<const float2 *>(p);
    o[0] = q.x; o[1] = q.y;
  }
}
template <int N> __device__ __forceinline__ void st_f32(float *p, const float *v) {
  if constexpr (N == 4) *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
  else *reinterpret_cast<float2 *>(p) = make_float2(v[0], v[1]);
}

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
// 16 bytes of global memory through a global-space pointer: a global load
// even where the compiler cannot tell the pointer's space (arguments read
// from device memory), instead of a flat load, which counts on the LDS
// counter too and so holds up every LDS wait while it is in flight.  The
// load is of a vector type: a copy of uint4 would bind a flat reference.
__device__ __forceinline__ uint4 gld16(const void *p) {
  const u32x4_t v = *(const __attribute__((address_space(1))) u32x4_t *)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}
// Agent-scope relaxed atomics on global memory, through global-space
// pointers for the same reason as gld16.
template <typename V>
__device__ __forceinline__ V ld_agent(const V *p) {
  return __hip_atomic_load((const __attribute__((address_space(1))) V *)p, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
template <typename V>
__device__ __forceinline__ void st_agent(V *p, V v) {
  __hip_atomic_store((__attribute__((address_space(1))) V *)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename V>
__device__ __forceinline__ V add_agent(V *p, V v) {
  return __hip_atomic_fetch_add((__attribute__((address_space(1))) V *)p, v, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint4 ld16_stream(const void *p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st16(void *p, const uint4 &v) { *reinterpret_cast<uint4 *>(p) = v; }

// 16 bytes written earlier in the same launch by another block: four
// agent-scope loads, which no stale cache line can answer.
__device__ __forceinline__ uint4 ld16_agent(const void *p) {
  const uint32_t *q = static_cast<const uint32_t *>(p);
  return make_uint4(ld_agent(q), ld_agent(q + 1), ld_agent(q + 2), ld_agent(q + 3));
}
// 16 bytes that other blocks of the same launch read: write-through stores.
__device__ __forceinline__ void st16_through(void *p, const uint4 &v) {
  uint32_t *q = static_cast<uint32_t *>(p);
  st_agent(q, v.x);
  st_agent(q + 1, v.y);
  st_agent(q + 2, v.z);
  st_agent(q + 3, v.w);
}

// One 16x16 MFMA accumulation over the K-window that one 16-byte vector per
// lane covers: 32 bf16 (one v_mfma_f32_16x16x32_bf16) or 16 fp32 (four
// v_mfma_f32_16x16x4_f32).  Lane l supplies row (l % 16) of A and column
// (l % 16) of B, at the same K positions, so the window's K order is the same
// for both operands.  D: lane l holds column l % 16, rows 4*(l/16) + 0..3.
__device__ __forceinline__ void mfma16(f32x4_t &acc, const uint4 &a, const uint4 &b, bf16_t) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma16(f32x4_t &acc, const uint4 &a, const uint4 &b, float) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

// One 32x32x16 bf16 MFMA (v_mfma_f32_32x32x16_bf16): lane l supplies row
// (l % 32) of A and column (l % 32) of B, K elements 8*(l/32) .. +7 of the
// 16-element window; D: lane l holds column l % 32, element q at row
// 8*(q/4) + 4*(l/32) + q%4.
typedef float f32x16_t __attribute__((ext_vector_type(16)));
__device__ __forceinline__ void mfma32(f32x16_t &acc, const uint4 &a, const uint4 &b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), o);
  uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), o);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Order-preserving map of fp32 to uint32 (larger float -> larger key);
// -0 is folded onto +0 so that the two compare equal.
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// (value, index) packed so that the unsigned max is the largest value and,
// among equal values, the lowest index.
__device__ __forceinline__ uint64_t argmax_key(float v, uint32_t idx) {
  return (static_cast<uint64_t>(ordered_bits(v)) << 32) | static_cast<uint32_t>(~idx);
}
__device__ __forceinline__ uint32_t key_index(uint64_t key) {
  return ~static_cast<uint32_t>(key);
}

}  // namespace mv

// Device-side helpers shared by the kernels: wavefront primitives for CDNA4's
// 64-lane waves, element conversions, and 16-byte vector accesses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ffnwb {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// Same vector with only 4-byte alignment: gfx950 global_load/store_dwordx4 need dword
// alignment only, so rows with a 4-byte-aligned stride still move in 16-byte accesses.
typedef u32x4 u32x4_a4 __attribute__((aligned(4)));

__device__ __forceinline__ uint32_t lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// Number of set bits of `m` at lanes below the calling lane.
__device__ __forceinline__ uint32_t count_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

__device__ __forceinline__ uint64_t wave_ballot(bool p) { return __ballot(p); }

// Sum of one value per lane over the calling wave; every lane receives it.
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
#pragma unroll
  for (int d = kWave / 2; d > 0; d >>= 1) x += __shfl_xor(x, d);
  return x;
}

template <typename T>
__device__ __forceinline__ T uniform(T v) {
  return static_cast<T>(__builtin_amdgcn_readfirstlane(static_cast<int>(v)));
}

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Orders this wave's LDS accesses across lanes (cheap: no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------- element conversions
__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// float -> bfloat16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float f16_to_f32(uint32_t h16) {
  _Float16 h = __builtin_bit_cast(_Float16, static_cast<uint16_t>(h16));
  return static_cast<float>(h);
}

__device__ __forceinline__ uint32_t f32_to_f16_rne(float f) {
  _Float16 h = static_cast<_Float16>(f);  // v_cvt_f16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

// Element type tags used as template parameters.
struct TF16 { static constexpr int kBytes = 2; };
struct TBF16 { static constexpr int kBytes = 2; };
struct TF32 { static constexpr int kBytes = 4; };

template <class T> __device__ __forceinline__ float load_elem(const void* p, int64_t i);
template <> __device__ __forceinline__ float load_elem<TF16>(const void* p, int64_t i) {
  return f16_to_f32(static_cast<const uint16_t*>(p)[i]);
}
template <> __device__ __forceinline__ float load_elem<TBF16>(const void* p, int64_t i) {
  return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}
template <> __device__ __forceinline__ float load_elem<TF32>(const void* p, int64_t i) {
  return static_cast<const float*>(p)[i];
}

template <class T> __device__ __forceinline__ void store_elem(void* p, int64_t i, float v);
template <> __device__ __forceinline__ void store_elem<TF16>(void* p, int64_t i, float v) {
  static_cast<uint16_t*>(p)[i] = static_cast<uint16_t>(f32_to_f16_rne(v));
}
template <> __device__ __forceinline__ void store_elem<TBF16>(void* p, int64_t i, float v) {
  static_cast<uint16_t*>(p)[i] = static_cast<uint16_t>(f32_to_bf16_rne(v));
}
template <> __device__ __forceinline__ void store_elem<TF32>(void* p, int64_t i, float v) {
  static_cast<float*>(p)[i] = v;
}

// Widen the elements held in one 16-byte chunk to floats (8 for 16-bit types, 4 for FP32).
template <class T> struct Chunk;
template <> struct Chunk<TF16> {
  static constexpr int kElems = 8;
  __device__ static void widen(const u32x4& v, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[2 * i] = f16_to_f32(v[i] & 0xffffu); f[2 * i + 1] = f16_to_f32(v[i] >> 16); }
  }
  __device__ static u32x4 narrow(const float (&f)[8]) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = f32_to_f16_rne(f[2 * i]) | (f32_to_f16_rne(f[2 * i + 1]) << 16);
    return v;
  }
};
template <> struct Chunk<TBF16> {
  static constexpr int kElems = 8;
  __device__ static void widen(const u32x4& v, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[2 * i] = __uint_as_float(v[i] << 16); f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u); }
  }
  __device__ static u32x4 narrow(const float (&f)[8]) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = f32_to_bf16_rne(f[2 * i]) | (f32_to_bf16_rne(f[2 * i + 1]) << 16);
    return v;
  }
};
template <> struct Chunk<TF32> {
  static constexpr int kElems = 4;
  __device__ static void widen(const u32x4& v, float (&f)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
  __device__ static u32x4 narrow(const float (&f)[4]) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
    return v;
  }
};

}  // namespace ffnwb

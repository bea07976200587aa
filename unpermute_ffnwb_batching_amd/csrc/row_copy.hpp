// Row moves by one wavefront, shared by the kernels that copy whole token rows.
#pragma once

#include "device_common.hpp"

namespace ffnwb {

// Row copies by one wavefront.  VEC = 16: every address 16-byte aligned; VEC = 4: 4-byte
// aligned (16-byte accesses at dword alignment plus a dword tail); VEC = 1: bytes.  A row
// moves in pieces of kPiece 16-byte accesses per lane (16 KiB per wave); the loads of a
// piece are all issued before its first store.
constexpr int kPiece = 16;

template <int VEC> struct RowVec { typedef u32x4 type; };
template <> struct RowVec<4> { typedef u32x4_a4 type; };

template <int VEC>
struct RowPiece {
  typedef typename RowVec<VEC>::type V;
  V v[kPiece];
  __device__ __forceinline__ void load(const uint8_t* __restrict__ src, int64_t n16, int64_t b, uint32_t lane) {
    const V* s4 = reinterpret_cast<const V*>(src);
#pragma unroll
    for (int u = 0; u < kPiece; ++u) {
      const int64_t i = b + u * kWave + lane;
      if (i < n16) v[u] = __builtin_nontemporal_load(s4 + i);  // streamed once: do not keep in cache
    }
  }
  // the same with ordinary loads, for a row several wavefronts read at once (the later
  // reads hit in L2)
  __device__ __forceinline__ void load_cached(const uint8_t* __restrict__ src, int64_t n16, int64_t b,
                                              uint32_t lane) {
    const V* s4 = reinterpret_cast<const V*>(src);
#pragma unroll
    for (int u = 0; u < kPiece; ++u) {
      const int64_t i = b + u * kWave + lane;
      if (i < n16) v[u] = s4[i];
    }
  }
  __device__ __forceinline__ void store(uint8_t* __restrict__ dst, int64_t n16, int64_t b, uint32_t lane) const {
    V* d4 = reinterpret_cast<V*>(dst);
#pragma unroll
    for (int u = 0; u < kPiece; ++u) {
      const int64_t i = b + u * kWave + lane;
      if (i < n16) __builtin_nontemporal_store(v[u], d4 + i);
    }
  }
  // the same with ordinary stores
  __device__ __forceinline__ void store_cached(uint8_t* __restrict__ dst, int64_t n16, int64_t b,
                                               uint32_t lane) const {
    V* d4 = reinterpret_cast<V*>(dst);
#pragma unroll
    for (int u = 0; u < kPiece; ++u) {
      const int64_t i = b + u * kWave + lane;
      if (i < n16) d4[i] = v[u];
    }
  }
};

// Copies bytes [from, bytes) of a row (the part not moved by an earlier piece).
template <int VEC>
__device__ __forceinline__ void copy_row_rest(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                              int64_t bytes, int64_t from16, uint32_t lane) {
  if (VEC == 1) {
    for (int64_t i = lane; i < bytes; i += kWave) dst[i] = src[i];
    return;
  }
  const int64_t n16 = bytes >> 4;
  for (int64_t b = from16; b < n16; b += kWave * kPiece) {
    RowPiece<VEC> piece;
    piece.load(src, n16, b, lane);
    piece.store(dst, n16, b, lane);
  }
  if (VEC == 4) {
    const int64_t tail = (bytes & 15) >> 2;
    if (lane < tail) {
      reinterpret_cast<uint32_t*>(dst + n16 * 16)[lane] = reinterpret_cast<const uint32_t*>(src + n16 * 16)[lane];
    }
  }
}

template <int VEC>
__device__ __forceinline__ void copy_row(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t bytes,
                                         uint32_t lane) {
  copy_row_rest<VEC>(src, dst, bytes, 0, lane);
}

}  // namespace ffnwb

// Routing-map tiles shared by the probs compaction and the forward permute: tiles of
// kMaskRows token rows; a work item is kMaskGroupRows consecutive rows x W consecutive
// columns (W = 4 when the columns come in aligned groups of 4, else 1), read as one
// W-byte load per row.  mask_tile_count_kernel writes hist[tile*E + e], the non-zero
// entries of column e in the tile.
#pragma once

#include "device_common.hpp"

namespace ffnwb {

constexpr int kMaskRows = 256;
constexpr int kMaskGroupRows = 16;
constexpr int kMaskGroups = kMaskRows / kMaskGroupRows;
constexpr int kMaskLdsHist = 16384;    // histogram words a compaction workgroup holds
constexpr int kMaskFusedMaxExperts = 1024;

template <int W>
__device__ __forceinline__ uint32_t load_map_unit(const uint8_t* p) {
  if (W == 4) return *reinterpret_cast<const uint32_t*>(p);
  return *p;
}

// Loads the map units of one work item (rows clamped to the map) and counts its
// non-zero entries per column.
template <int W>
__device__ __forceinline__ void mask_item_counts(const uint8_t* __restrict__ map, int64_t T, int32_t E, int64_t r0,
                                                 int c, uint32_t (&x)[kMaskGroupRows], uint32_t (&cnt)[W]) {
#pragma unroll
  for (int r = 0; r < kMaskGroupRows; ++r) x[r] = load_map_unit<W>(map + min(r0 + r, T - 1) * E + c * W);
#pragma unroll
  for (int w = 0; w < W; ++w) cnt[w] = 0u;
#pragma unroll
  for (int r = 0; r < kMaskGroupRows; ++r) {
#pragma unroll
    for (int w = 0; w < W; ++w) cnt[w] += (r0 + r < T && ((x[r] >> (8 * w)) & 0xffu) != 0) ? 1u : 0u;
  }
}

template <int W>
__global__ __launch_bounds__(256) void mask_tile_count_kernel(const uint8_t* __restrict__ map, int64_t T, int32_t E,
                                                              uint32_t* __restrict__ hist) {
  extern __shared__ uint32_t colc[];  // [E]
  for (int e = threadIdx.x; e < E; e += blockDim.x) colc[e] = 0u;
  __syncthreads();
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kMaskRows;
  const int cu = E / W;
  for (int it = threadIdx.x; it < kMaskGroups * cu; it += blockDim.x) {
    const int g = it / cu;
    const int c = it - g * cu;
    uint32_t x[kMaskGroupRows], cnt[W];
    mask_item_counts<W>(map, T, E, t0 + g * kMaskGroupRows, c, x, cnt);
#pragma unroll
    for (int w = 0; w < W; ++w)
      if (cnt[w] != 0) atomicAdd(&colc[c * W + w], cnt[w]);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[static_cast<int64_t>(blockIdx.x) * E + e] = colc[e];
}

}  // namespace ffnwb

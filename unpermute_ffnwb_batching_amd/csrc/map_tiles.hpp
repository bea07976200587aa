// Routing-map tiles shared by the probs compaction and the forward permute: tiles of
// kMaskRows token rows; a work item is kMaskGroupRows consecutive rows x W consecutive
// columns (W = 4 when the columns come in aligned groups of 4, else 1), read as one
// W-byte load per row.  mask_tile_count_kernel writes hist[tile*E + e], the non-zero
// entries of column e in the tile.  Its workgroups split each tile by column ranges of
// kMaskRangeUnits work-item columns, one item per thread, so that a map of a few MB is
// read by several times more compute units than there are tiles.
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

// Maps whose tile histogram does not fit one workgroup's LDS: tiles of kMaskTile tokens,
// thread e of a tile's workgroup walks column e of the tile, so within a column the
// tile's entries are in token order and their rank is a running count.
constexpr int kMaskTile = 32;

// hist[tile*E + e] = number of non-zero map entries of column e in the tile.
[[maybe_unused]] static __global__ __launch_bounds__(256) void mask_count_kernel(const uint8_t* __restrict__ map,
                                                                                 int64_t T, int32_t E,
                                                                                 uint32_t* __restrict__ hist) {
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kMaskTile;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    uint8_t m[kMaskTile];
#pragma unroll
    for (int i = 0; i < kMaskTile; ++i) m[i] = map[(t0 + i < T ? t0 + i : T - 1) * E + e];  // clamped: no branch
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < kMaskTile; ++i) c += (t0 + i < T && m[i] != 0) ? 1u : 0u;
    hist[static_cast<int64_t>(blockIdx.x) * E + e] = c;
  }
}

constexpr int kMaskRangeUnits = 8;                                // work-item columns per range
constexpr int kMaskSplitThreads = kMaskGroups * kMaskRangeUnits;   // 128: one item per thread

// Column ranges of a map with E columns read W at a time.
__host__ __device__ inline int mask_ranges(int32_t E, int W) {
  return (E / W + kMaskRangeUnits - 1) / kMaskRangeUnits;
}

// Grid (tiles, mask_ranges(E, W)) of kMaskSplitThreads threads.  Thread i takes row group
// i / kMaskRangeUnits and work-item column i % kMaskRangeUnits of its range.  With
// range_tot given, range_tot[tile * ranges + r] = the range's non-zero entries in the tile.
template <int W>
__global__ __launch_bounds__(kMaskSplitThreads) void mask_tile_count_kernel(const uint8_t* __restrict__ map,
                                                                            int64_t T, int32_t E,
                                                                            uint32_t* __restrict__ hist,
                                                                            uint32_t* __restrict__ range_tot) {
  __shared__ uint32_t colc[kMaskRangeUnits * W];
  const int tid = threadIdx.x;
  const int u0 = blockIdx.y * kMaskRangeUnits;
  const int nu = min(kMaskRangeUnits, E / W - u0);
  const int ncols = nu * W;
  const int g = tid / kMaskRangeUnits, u = tid % kMaskRangeUnits;
  const bool act = u < nu;
  uint32_t x[kMaskGroupRows], cnt[W];
  mask_item_counts<W>(map, T, E, static_cast<int64_t>(blockIdx.x) * kMaskRows + g * kMaskGroupRows,
                      u0 + (act ? u : 0), x, cnt);
  if (tid < ncols) colc[tid] = 0u;
  __syncthreads();
  if (act) {
#pragma unroll
    for (int w = 0; w < W; ++w)
      if (cnt[w] != 0) atomicAdd(&colc[u * W + w], cnt[w]);
  }
  __syncthreads();
  if (tid < kWave) {  // ncols <= 32: one wave writes the range
    const uint32_t v = tid < ncols ? colc[tid] : 0u;
    if (tid < ncols) hist[static_cast<int64_t>(blockIdx.x) * E + u0 * W + tid] = v;
    if (range_tot != nullptr) {
      const uint32_t sum = wave_sum(v);
      if (tid == 0) range_tot[static_cast<int64_t>(blockIdx.x) * gridDim.y + blockIdx.y] = sum;
    }
  }
}

}  // namespace ffnwb

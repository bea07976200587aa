// Forward MoE token permute with routing map on gfx950.  The MoeTokenUnpermuteWithRoutingMap
// article names this step in "Operator positioning" (tokens regrouped by expert so that each
// expert reads its tokens contiguously; sortedIndices for the way back); its outputs are the
// arrangement the unpermute's formulas ("Function description and formulas", branches 1-4)
// invert.
//
// Three launches:
//   1. mask_tile_count_kernel: per tile of kMaskRows tokens, the non-zero entries of every
//      expert column (map_tiles.hpp);
//   2. permute_order_kernel: one workgroup per tile copies the whole tile histogram to LDS,
//      derives the column totals, the column starts and its own tile prefix, and gives
//      every non-zero entry (t, e) of its tile a place:
//        non-padded  row r = start[e] + (entries of column e in earlier tiles) + (entries
//                    of column e in earlier rows of this tile); source_of[r] = t;
//        padded      position j of the entry within expert e's capacity block;
//                    sorted_indices[e*C + j] = t while j < C, and the capacity row
//                    e*C + j (or -1) of every (t, e) in a [T][E] table.
//      Non-padded, a token's rows rise with its expert (rows are expert-major), so its
//      slots are its entries in ascending expert order: each row of the tile is walked
//      once more, and slot k takes the row of the k-th entry, whose offset inside the tile
//      was kept in LDS (one byte per row and expert);
//   3. permute_scatter_kernel reads each token row once and writes it to every row its
//      list names (non-padded: its topK slots; padded: its row of the table), and fills the
//      rows no list names (non-padded: zero rows past the non-zero entries and rows of
//      experts beyond a token's topK; padded: zero rows of unused capacity).  Reading the
//      token row once per output row instead (one wavefront per output row) read each
//      padded token row once per expert it is routed to: 121.7 us for the row moves at
//      E=64, C=512, T=8192, H=5120 FP16 with 4 experts per token, against 77-84 us in
//      token order.
// Maps with more than kPermuteMaxExperts experts, or whose tile histogram does not fit
// one workgroup's LDS, take four launches instead: mask_count_kernel (32-token tiles),
// the histogram scan, permute_table_kernel (the row, or capacity row, of every (t, e) in
// a [T][E] table), and permute_scatter_kernel reading its lists from that table, which
// then also writes the non-padded sorted_indices.
#include <stdio.h>

#include "internal.hpp"
#include "map_tiles.hpp"
#include "row_copy.hpp"
#include "sort_engine.hpp"

namespace ffnwb {

constexpr int kPermuteThreads = 1024;
constexpr int kPermuteMaxExperts = 256;

// LDS bytes of permute_order_kernel.
inline size_t permute_order_lds_bytes(int ntiles, int E, bool padded) {
  const size_t words = static_cast<size_t>(ntiles) * E + static_cast<size_t>(kMaskGroups) * E + 2 * static_cast<size_t>(E);
  return words * sizeof(uint32_t) + (padded ? 0 : static_cast<size_t>(kMaskRows) * E);
}

// Places the non-zero entries of NR consecutive rows (rows rbase .. rbase+NR-1 of group g)
// of one work item, in row order, from the running offsets off[w] of its W columns.
// Padded, every (row, column) of the item also gets its capacity row in dest ([T][E],
// -1 where the entry is zero or past the capacity).
template <int W, bool PADDED, int NR>
__device__ __forceinline__ void permute_place_rows(const uint32_t (&xr)[NR], int rbase, int g, int c, int64_t t0,
                                                   int64_t T, int32_t E, const uint32_t* base, uint32_t (&off)[W],
                                                   int64_t N, int64_t C, int32_t* __restrict__ source_of,
                                                   int32_t* __restrict__ sorted_indices, uint8_t* inoff,
                                                   int32_t* __restrict__ dest) {
  const int64_t r0 = t0 + g * kMaskGroupRows + rbase;
  uint32_t bs[W];
#pragma unroll
  for (int w = 0; w < W; ++w) bs[w] = base[c * W + w];  // read once, outside the per-entry branches
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    if (PADDED) {
      int32_t dv[W];
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const bool nz = r0 + r < T && ((xr[r] >> (8 * w)) & 0xffu) != 0;
        const int e = c * W + w;
        const uint32_t place = bs[w] + off[w];
        const bool kept = nz && place < static_cast<uint64_t>(C);
        dv[w] = kept ? static_cast<int32_t>(e * C + place) : -1;
        if (kept) sorted_indices[e * C + place] = static_cast<int32_t>(r0 + r);
        off[w] += nz ? 1u : 0u;
      }
      if (r0 + r < T) {
        int32_t* drow = dest + (r0 + r) * E + c * W;
        if (W == 4) *reinterpret_cast<int4*>(drow) = make_int4(dv[0], dv[W > 1 ? 1 : 0], dv[W > 2 ? 2 : 0], dv[W - 1]);
        else drow[0] = dv[0];
      }
      continue;
    }
#pragma unroll
    for (int w = 0; w < W; ++w) {
      if (r0 + r < T && ((xr[r] >> (8 * w)) & 0xffu) != 0) {
        const int e = c * W + w;
        const uint32_t place = bs[w] + off[w];
        if (place < static_cast<uint64_t>(N)) source_of[place] = static_cast<int32_t>(r0 + r);
        inoff[(g * kMaskGroupRows + rbase + r) * E + e] = static_cast<uint8_t>(off[w]);
        ++off[w];
      }
    }
  }
}

template <int W, bool PADDED>
__global__ __launch_bounds__(kPermuteThreads) void permute_order_kernel(const uint8_t* __restrict__ map, int64_t T,
                                                                        int32_t E, int ntiles,
                                                                        const uint32_t* __restrict__ hist,
                                                                        int64_t N, int32_t K, int64_t C,
                                                                        int32_t* __restrict__ source_of,
                                                                        int32_t* __restrict__ sorted_indices,
                                                                        int32_t* __restrict__ dest) {
  constexpr int NT = kPermuteThreads;
  extern __shared__ uint32_t lds[];
  uint32_t* h = lds;                     // [ntiles][E] tile histogram
  uint32_t* gc = h + ntiles * E;         // [kMaskGroups][E] group counts -> offsets in the tile
  uint32_t* tot = gc + kMaskGroups * E;  // [E] column totals
  uint32_t* base = tot + E;              // [E] first place of column e's entries of this tile
  uint8_t* inoff = reinterpret_cast<uint8_t*>(base + E);  // [kMaskRows][E] (non-padded)
  __shared__ uint32_t wsum[NT / kWave + 1];
  const int tid = threadIdx.x;
  const int tile = blockIdx.x;
  const int64_t t0 = static_cast<int64_t>(tile) * kMaskRows;
  const int cu = E / W;
  const int items = kMaskGroups * cu;
  const int hw = ntiles * E;
  // 1. the histogram to LDS (16 loads in flight per thread, clamped) and this tile's
  //    per-group counts
  for (int i0 = 0; i0 < hw; i0 += NT * 16) {
    uint32_t v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = hist[min(i0 + u * NT + tid, hw - 1)];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (i0 + u * NT + tid < hw) h[i0 + u * NT + tid] = v[u];
  }
  for (int it = tid; it < items; it += NT) {
    const int g = it / cu;
    const int c = it - g * cu;
    uint32_t x[kMaskGroupRows], cnt[W];
    mask_item_counts<W>(map, T, E, t0 + g * kMaskGroupRows, c, x, cnt);
#pragma unroll
    for (int w = 0; w < W; ++w) gc[g * E + c * W + w] = cnt[w];
  }
  __syncthreads();
  // 2. column totals and this tile's prefix; thread i owns the columns [i*per, (i+1)*per)
  const int per = (E + NT - 1) / NT;
  const int lo = min(E, tid * per);
  const int hi = min(E, lo + per);
  uint32_t mine = 0;
  for (int e = lo; e < hi; ++e) {
    uint32_t t_all = 0, t_pre = 0;
    for (int t = 0; t < ntiles; ++t) {
      const uint32_t v = h[t * E + e];
      t_pre += (t < tile) ? v : 0u;
      t_all += v;
    }
    tot[e] = t_all;
    base[e] = t_pre;
    mine += t_all;
  }
  uint32_t filled;
  uint32_t start = block_exscan<NT>(mine, wsum, filled);  // first row of column lo (non-padded)
  for (int e = lo; e < hi; ++e) {
    if (!PADDED) base[e] += start;
    start += tot[e];
    uint32_t run = 0;
    for (int g = 0; g < kMaskGroups; ++g) {
      const uint32_t c = gc[g * E + e];
      gc[g * E + e] = run;
      run += c;
    }
  }
  __syncthreads();
  // 3. a place for every entry of the tile, rows in order within each item; when the
  //    workgroup has twice as many threads as items, two adjacent lanes share an item (8
  //    rows each, the second starting after the first's counts)
  if (2 * items <= NT) {
    constexpr int kHalf = kMaskGroupRows / 2;
    const int it = tid >> 1, hf = tid & 1;
    const bool act = it < items;
    const int g = act ? it / cu : 0;
    const int c = act ? it - g * cu : 0;
    const int64_t r0 = t0 + g * kMaskGroupRows + hf * kHalf;
    uint32_t x[kHalf], cnt[W];
#pragma unroll
    for (int r = 0; r < kHalf; ++r) x[r] = load_map_unit<W>(map + min(r0 + r, T - 1) * E + c * W);  // clamped
#pragma unroll
    for (int w = 0; w < W; ++w) {
      cnt[w] = 0u;
#pragma unroll
      for (int r = 0; r < kHalf; ++r) cnt[w] += (r0 + r < T && ((x[r] >> (8 * w)) & 0xffu) != 0) ? 1u : 0u;
    }
    uint32_t off[W];
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const uint32_t first_half = static_cast<uint32_t>(__shfl_xor(static_cast<int>(cnt[w]), 1));
      off[w] = (act ? gc[g * E + c * W + w] : 0u) + (hf ? first_half : 0u);
    }
    if (act)
      permute_place_rows<W, PADDED, kHalf>(x, hf * kHalf, g, c, t0, T, E, base, off, N, C, source_of, sorted_indices,
                                           inoff, dest);
  } else {
    for (int it = tid; it < items; it += NT) {
      const int g = it / cu;
      const int c = it - g * cu;
      uint32_t x[kMaskGroupRows], cnt[W];
      mask_item_counts<W>(map, T, E, t0 + g * kMaskGroupRows, c, x, cnt);
      uint32_t off[W];
#pragma unroll
      for (int w = 0; w < W; ++w) off[w] = gc[g * E + c * W + w];
      permute_place_rows<W, PADDED, kMaskGroupRows>(x, 0, g, c, t0, T, E, base, off, N, C, source_of,
                                                    sorted_indices, inoff, dest);
    }
  }
  if (PADDED) {
    // 4. unused capacity: -1 (every workgroup takes a share of the E*C places)
    const int64_t all = static_cast<int64_t>(E) * C;
    for (int64_t i = static_cast<int64_t>(tile) * NT + tid; i < all; i += static_cast<int64_t>(gridDim.x) * NT) {
      const int32_t e = static_cast<int32_t>(i / C);
      if (i - static_cast<int64_t>(e) * C >= static_cast<int64_t>(tot[e])) sorted_indices[i] = -1;
    }
    return;
  }
  __syncthreads();
  // 4. the slots of each token of the tile: its entries in ascending expert order.  A
  //    token's map row is spread over lanes (one map unit each) and each entry's slot k
  //    comes from ballots: the non-zero entries of lower lanes plus the lane's earlier
  //    ones.  (One thread per token walking its row serially took half the kernel.)
  {
    const uint32_t lane = lane_id();
    const int wv = tid / kWave;
    constexpr int NW = NT / kWave;
    if (cu <= 32) {
      // two tokens per wave iteration: lanes [0, 32) and [32, 64); every map load of the
      // wave's tokens is issued before the first is used
      constexpr int kIters = kMaskRows / (2 * NW);
      const int sub = static_cast<int>(lane >> 5);
      const int ul = static_cast<int>(lane & 31u);
      const uint64_t half = sub ? 0xFFFFFFFF00000000ull : 0x00000000FFFFFFFFull;
      uint32_t xs[kIters];
#pragma unroll
      for (int i = 0; i < kIters; ++i) {
        const int64_t t = min(t0 + (wv * kIters + i) * 2 + sub, T - 1);
        xs[i] = load_map_unit<W>(map + t * E + min(ul, cu - 1) * W);  // clamped
      }
#pragma unroll
      for (int i = 0; i < kIters; ++i) {
        const int rr = (wv * kIters + i) * 2 + sub;
        const int64_t t = t0 + rr;
        const bool uok = t < T && ul < cu;
        uint32_t f[W], below = 0, total = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) {
          f[w] = (uok && ((xs[i] >> (8 * w)) & 0xffu) != 0) ? 1u : 0u;
          const uint64_t m = wave_ballot(f[w] != 0) & half;
          below += count_below(m);
          total += static_cast<uint32_t>(__popcll(m));
        }
        // the lane's row places, read outside the per-entry branches (a lane's W experts
        // are adjacent: one read of base, one of the in-tile offsets)
        const int ue = min(ul, cu - 1) * W;
        uint32_t rp[W];
#pragma unroll
        for (int w = 0; w < W; ++w) rp[w] = base[ue + w] + inoff[rr * E + ue + w];
        uint32_t k = below;
#pragma unroll
        for (int w = 0; w < W; ++w) {
          if (f[w]) {
            const uint32_t r = rp[w];
            if (k < static_cast<uint32_t>(K)) {
              sorted_indices[t * K + k] = (r < static_cast<uint64_t>(N)) ? static_cast<int32_t>(r) : -1;
            } else if (r < static_cast<uint64_t>(N)) {
              source_of[r] = -static_cast<int32_t>(t) - 2;  // a row no slot lists (token beyond topK)
            }
            ++k;
          }
        }
        if (t < T)
          for (int q = static_cast<int>(total) + ul; q < K; q += 32) sorted_indices[t * K + q] = -1;
      }
    } else {
      // one token per wave iteration, its map units 64 at a time
      for (int rr = wv; rr < kMaskRows; rr += NW) {
        const int64_t t = t0 + rr;
        if (t >= T) break;  // uniform
        uint32_t k0 = 0;
        for (int c0 = 0; c0 < cu; c0 += kWave) {
          const int u = c0 + static_cast<int>(lane);
          const uint32_t x = load_map_unit<W>(map + t * E + min(u, cu - 1) * W);  // clamped
          uint32_t f[W], below = 0, total = 0;
#pragma unroll
          for (int w = 0; w < W; ++w) {
            f[w] = (u < cu && ((x >> (8 * w)) & 0xffu) != 0) ? 1u : 0u;
            const uint64_t m = wave_ballot(f[w] != 0);
            below += count_below(m);
            total += static_cast<uint32_t>(__popcll(m));
          }
          const int ue = min(u, cu - 1) * W;
          uint32_t rp[W];
#pragma unroll
          for (int w = 0; w < W; ++w) rp[w] = base[ue + w] + inoff[rr * E + ue + w];
          uint32_t k = k0 + below;
#pragma unroll
          for (int w = 0; w < W; ++w) {
            if (f[w]) {
              const uint32_t r = rp[w];
              if (k < static_cast<uint32_t>(K)) {
                sorted_indices[t * K + k] = (r < static_cast<uint64_t>(N)) ? static_cast<int32_t>(r) : -1;
              } else if (r < static_cast<uint64_t>(N)) {
                source_of[r] = -static_cast<int32_t>(t) - 2;
              }
              ++k;
            }
          }
          k0 += total;
        }
        for (int q = static_cast<int>(k0 + lane); q < K; q += kWave) sorted_indices[t * K + q] = -1;
      }
    }
  }
  // 5. rows past the non-zero entries have no source
  for (int64_t r = static_cast<int64_t>(tile) * NT + tid; r < N; r += static_cast<int64_t>(gridDim.x) * NT)
    if (r >= filled) source_of[r] = -1;
}

// Fallback order (see the file comment), after mask_count_kernel and the histogram scan
// over 32-token tiles: thread e of a tile's workgroup walks column e of the tile in token
// order, so a running count from the tile's base gives each entry its place among the
// column's entries:
//   non-padded  row start[e] + (entries of column e in earlier tiles) + running count;
//   padded      place j = (entries in earlier tiles) + running count: capacity row
//               e*C + j while j < C, with sorted_indices[e*C + j] = t.
// table[t*E + e] = that row (non-padded rows may lie past N: dropped later), or -1 for a
// zero entry or a padded entry past the capacity.  Padded, every workgroup also takes a
// share of the unused capacity: sorted_indices = -1.
template <bool PADDED>
__global__ __launch_bounds__(256) void permute_table_kernel(const uint8_t* __restrict__ map, int64_t T, int32_t E,
                                                            Placement pl, int64_t C, int32_t* __restrict__ table,
                                                            int32_t* __restrict__ sorted_indices) {
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kMaskTile;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    uint32_t off = pl.tile_base(blockIdx.x, static_cast<uint32_t>(e));
    const uint32_t first = pl.start[e];
    uint8_t m[kMaskTile];
#pragma unroll
    for (int i = 0; i < kMaskTile; ++i) m[i] = map[min(t0 + i, T - 1) * E + e];  // clamped: no branch
#pragma unroll
    for (int i = 0; i < kMaskTile; ++i) {
      const int64_t t = t0 + i;
      if (t >= T) break;
      int32_t v = -1;
      if (m[i] != 0) {
        if (PADDED) {
          if (off < static_cast<uint64_t>(C)) {
            v = static_cast<int32_t>(e * C + off);
            sorted_indices[e * C + off] = static_cast<int32_t>(t);
          }
        } else {
          v = static_cast<int32_t>(first + off);
        }
        ++off;
      }
      table[t * E + e] = v;
    }
  }
  if (PADDED) {
    const int64_t all = static_cast<int64_t>(E) * C;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < all;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
      const int64_t e = i / C;
      if (i - e * C >= static_cast<int64_t>(pl.start[e + 1] - pl.start[e])) sorted_indices[i] = -1;
    }
  }
}

// Writes zeros over one row (one wavefront).
template <int VEC>
__device__ __forceinline__ void zero_row(uint8_t* __restrict__ dst, int64_t row_bytes, uint32_t lane) {
  if (VEC == 1) {
    for (int64_t i = lane; i < row_bytes; i += kWave) dst[i] = 0;
    return;
  }
  typedef typename RowVec<VEC>::type V;
  V* d4 = reinterpret_cast<V*>(dst);
  const int64_t n16 = row_bytes >> 4;
  const V z = {0u, 0u, 0u, 0u};
  for (int64_t i = lane; i < n16; i += kWave) __builtin_nontemporal_store(z, d4 + i);
  if (VEC == 4) {
    const int64_t tail = (row_bytes & 15) >> 2;
    if (lane < tail) reinterpret_cast<uint32_t*>(dst + n16 * 16)[lane] = 0u;
  }
}

// Row moves.  Workgroups below token_blocks: S wavefronts per token (consecutive global
// wavefront numbers) read its list (lists[t*K .. t*K+K), -1 = none; K = topK non-padded,
// E padded or from the [T][E] table) 64 entries at a time; wavefront `sub` gathers the
// listed rows in [0, N) whose list index is sub (mod S) into a per-wave LDS list, then
// loads each 16 KiB piece of the token's row once and stores it to every row of its
// list, with ordinary stores: this kernel writes several times what it reads, and for
// such write-heavy traffic ordinary stores measured faster than non-temporal ones (243
// vs 250 us at T=16384, topK=8, H=4096 BF16).  Non-padded, 4 wavefronts per token with
// ordinary loads (the token's row is read from HBM once and from L2 by the others)
// measured 225 us against 243 us for one; padded (4 rows per token, 10 KiB each) one
// wavefront with non-temporal loads stays fastest (86 against 91 us).  With topk > 0
// the list is the non-padded table, and wavefront 0 of the token also writes its
// slots: sorted_out[t*topk + k] = the row of its k-th listed entry (-1 past N, and for k
// past its entries).
// The rest: one wavefront per 64 output rows handles the rows no list names:
// source_of[r] = -1 (zeros) or -(t+2) (token t), or, without source_of, zeros for the
// rows from *filled (the number of non-zero entries) up to N.
constexpr int kDestCap = 256;  // listed rows a wavefront gathers before it copies

template <int VEC, bool CACHED>
__device__ __forceinline__ void copy_to_rows(const uint8_t* __restrict__ src, int64_t row_bytes,
                                             const int32_t* rows, uint32_t nd, uint8_t* __restrict__ out,
                                             uint32_t lane) {
  if (VEC == 1) {
    for (uint32_t j = 0; j < nd; ++j) copy_row<1>(src, out + static_cast<int64_t>(rows[j]) * row_bytes, row_bytes, lane);
    return;
  }
  const int64_t n16 = row_bytes >> 4;
  for (int64_t b = 0; b < n16; b += kWave * kPiece) {
    RowPiece<VEC> piece;
    if (CACHED) piece.load_cached(src, n16, b, lane);
    else piece.load(src, n16, b, lane);
    for (uint32_t j = 0; j < nd; ++j) piece.store_cached(out + static_cast<int64_t>(rows[j]) * row_bytes, n16, b, lane);
  }
  if (VEC == 4) {
    const int64_t tail = (row_bytes & 15) >> 2;
    uint32_t v = 0;
    if (lane < tail) v = reinterpret_cast<const uint32_t*>(src + n16 * 16)[lane];
    for (uint32_t j = 0; j < nd; ++j)
      if (lane < tail) reinterpret_cast<uint32_t*>(out + static_cast<int64_t>(rows[j]) * row_bytes + n16 * 16)[lane] = v;
  }
}

template <int VEC, int S, bool CACHED>
__global__ __launch_bounds__(256) void permute_scatter_kernel(const uint8_t* __restrict__ tokens, int64_t stride,
                                                              int64_t row_bytes,
                                                              const int32_t* __restrict__ lists, int64_t T,
                                                              int32_t K, int32_t topk,
                                                              int32_t* __restrict__ sorted_out,
                                                              const int32_t* __restrict__ source_of,
                                                              const uint32_t* __restrict__ filled, int64_t N,
                                                              uint8_t* __restrict__ out, unsigned token_blocks) {
  __shared__ int32_t dests[4][kDestCap];
  const uint32_t lane = lane_id();
  const int wv = uniform(static_cast<int>(threadIdx.x) / kWave);
  if (blockIdx.x < token_blocks) {
    const int64_t gw = static_cast<int64_t>(blockIdx.x) * 4 + wv;
    const int64_t t = gw / S;
    const int sub = static_cast<int>(gw % S);
    if (t >= T) return;
    const uint8_t* src = tokens + t * stride;
    int32_t* dl = dests[wv];
    uint32_t nd = 0, k0 = 0;
    for (int c0 = 0; c0 < K; c0 += kWave) {
      const int32_t d = (c0 + static_cast<int>(lane) < K) ? lists[t * K + c0 + lane] : -1;
      if (topk > 0) {
        const uint64_t nz = wave_ballot(d != -1);
        const uint32_t k = k0 + count_below(nz);
        if (sub == 0 && d != -1 && k < static_cast<uint32_t>(topk))
          sorted_out[t * topk + k] = (d >= 0 && d < N) ? d : -1;
        k0 += static_cast<uint32_t>(__popcll(nz));
      }
      const bool ok = d >= 0 && d < N && (S == 1 || (c0 + static_cast<int>(lane)) % S == sub);
      const uint64_t m = wave_ballot(ok);
      if (ok) dl[nd + count_below(m)] = d;
      nd += static_cast<uint32_t>(__popcll(m));
      if (nd > kDestCap - kWave) {  // the next chunk might not fit: copy now
        wave_lds_sync();
        copy_to_rows<VEC, CACHED>(src, row_bytes, dl, nd, out, lane);
        wave_lds_sync();
        nd = 0;
      }
    }
    if (topk > 0 && sub == 0)
      for (uint32_t q = k0 + lane; q < static_cast<uint32_t>(topk); q += kWave) sorted_out[t * topk + q] = -1;
    if (nd > 0) {
      wave_lds_sync();
      copy_to_rows<VEC, CACHED>(src, row_bytes, dl, nd, out, lane);
    }
    return;
  }
  const int64_t r0 = (static_cast<int64_t>(blockIdx.x - token_blocks) * 4 + wv) * kWave;
  const int64_t r = r0 + lane;
  int32_t v = 0;
  if (source_of != nullptr) v = (r < N) ? source_of[r] : 0;
  else v = (r < N && r >= static_cast<int64_t>(*filled)) ? -1 : 0;
  uint64_t m = wave_ballot(r < N && v < 0);
  while (m != 0) {
    const int l = static_cast<int>(__builtin_ctzll(m));
    m &= m - 1;
    const int32_t vl = __builtin_amdgcn_readlane(v, l);
    uint8_t* dst = out + (r0 + l) * row_bytes;
    if (vl == -1) zero_row<VEC>(dst, row_bytes, lane);
    else copy_row<VEC>(tokens + static_cast<int64_t>(-vl - 2) * stride, dst, row_bytes, lane);
  }
}

static int element_bytes(int dtype) {
  switch (dtype) {
    case FFNWB_DT_FP16: case FFNWB_DT_BF16: return 2;
    case FFNWB_DT_INT8: return 1;
    case FFNWB_DT_FP32: return 4;
    default: return 0;
  }
}

int plan_permute(const moe_permute_desc* d, PermutePlan* p) {
  if (d == nullptr || p == nullptr) return FFNWB_ERR_PARAM_NULLPTR;
  if (d->tokens == nullptr || d->routing_map == nullptr || d->permuted_tokens == nullptr ||
      d->sorted_indices == nullptr)
    return FFNWB_ERR_PARAM_NULLPTR;
  const int elt = element_bytes(d->dtype);
  if (elt == 0) return FFNWB_ERR_PARAM_INVALID;
  if (d->padded_mode != 0 && d->padded_mode != 1) return FFNWB_ERR_PARAM_INVALID;
  const int64_t T = d->num_tokens, H = d->hidden, E = d->num_experts, N = d->num_out_rows;
  if (T < 1 || H < 1 || E < 1 || E > kMaxExperts || N < 0 || d->capacity < 0) return FFNWB_ERR_PARAM_INVALID;
  const int64_t lim = (int64_t{1} << 31) - 1;
  if (T > lim / E || N > lim || H > (int64_t{1} << 30)) return FFNWB_ERR_PARAM_INVALID;
  const int64_t ntiles = (T + kMaskRows - 1) / kMaskRows;
  // the one-launch order holds the tile histogram and a byte per (row, expert) of a tile in LDS
  p->table = E > kPermuteMaxExperts || ntiles * E > kMaskLdsHist;
  p->padded = d->padded_mode == 1;
  if (p->padded) {
    if (N != E * d->capacity) return FFNWB_ERR_PARAM_INVALID;
    p->K = 0;
  } else {
    if (N % T != 0) return FFNWB_ERR_PARAM_INVALID;
    p->K = N / T;
  }
  p->row_bytes = H * elt;
  p->stride = d->token_row_stride ? d->token_row_stride : p->row_bytes;
  if (p->stride < p->row_bytes) return FFNWB_ERR_PARAM_INVALID;
  if (static_cast<double>(T) * p->stride > 9.0e18 || static_cast<double>(N) * p->row_bytes > 9.0e18)
    return FFNWB_ERR_PARAM_INVALID;
  p->T = T;
  p->E = E;
  p->N = N;
  p->ntiles = ntiles;
  Carve c;
  if (p->table) {
    const int64_t nt32 = (T + kMaskTile - 1) / kMaskTile;
    c.take<uint32_t>(static_cast<size_t>(nt32 * E));       // 32-token tile histogram -> offsets
    c.take<uint32_t>(static_cast<size_t>(E) + 1);          // column starts
    c.take<int32_t>(static_cast<size_t>(T * E));           // (capacity) row of every entry
  } else {
    c.take<uint32_t>(static_cast<size_t>(ntiles * E));       // tile histogram
    if (!p->padded) c.take<int32_t>(static_cast<size_t>(N));  // source token of every row
    else c.take<int32_t>(static_cast<size_t>(T * E));         // capacity row of every entry
  }
  p->ws_bytes = c.off;
  return FFNWB_OK;
}

// S wavefronts per token (4 with ordinary loads for the non-padded slot lists, else 1
// with non-temporal loads); the row pass follows the token blocks.
template <int S, bool CACHED, typename... Args>
static bool launch_scatter(int vec, int64_t T, int64_t N, hipStream_t s, void* evb, void* eve, Args... args) {
  const unsigned tb = static_cast<unsigned>((T * S + 3) / 4);
  const unsigned rb = static_cast<unsigned>((N + 4 * kWave - 1) / (4 * kWave));
  const dim3 grid(tb + rb);
  if (vec == 16) return launch_bound(permute_scatter_kernel<16, S, CACHED>, grid, dim3(256), 0, s, evb, eve, args..., tb);
  if (vec == 4) return launch_bound(permute_scatter_kernel<4, S, CACHED>, grid, dim3(256), 0, s, evb, eve, args..., tb);
  return launch_bound(permute_scatter_kernel<1, S, CACHED>, grid, dim3(256), 0, s, evb, eve, args..., tb);
}

int launch_permute(const moe_permute_desc* d, const PermutePlan& p, void* ws, hipStream_t s) {
  if (p.N == 0) return FFNWB_OK;
  Carve c;
  c.base = static_cast<char*>(ws);
  const uint8_t* map = d->routing_map;
  const int32_t E = static_cast<int32_t>(p.E);
  const int vec = vec_class(reinterpret_cast<uintptr_t>(d->tokens), reinterpret_cast<uintptr_t>(d->permuted_tokens),
                            p.stride, p.row_bytes, p.row_bytes);
  const uint8_t* tok = static_cast<const uint8_t*>(d->tokens);
  uint8_t* out = static_cast<uint8_t*>(d->permuted_tokens);
  // the optional hooks are bound to the row-copy launch
  void* evb = d->ev_copy_begin;
  void* eve = d->ev_copy_end;
  if (p.table) {
    const int nt32 = static_cast<int>((p.T + kMaskTile - 1) / kMaskTile);
    uint32_t* hist = c.take<uint32_t>(static_cast<size_t>(nt32) * E);
    uint32_t* start = c.take<uint32_t>(static_cast<size_t>(E) + 1);
    int32_t* table = c.take<int32_t>(static_cast<size_t>(p.T * p.E));
    const int th = static_cast<int>(E >= 256 ? 256 : (E + 63) / 64 * 64);
    hipLaunchKernelGGL(mask_count_kernel, dim3(nt32), dim3(th), 0, s, map, p.T, E, hist);
    ScanTail none{nullptr, 0, nullptr, nullptr, nullptr};
    const size_t lds = scan_lds_bytes(E);
    allow_large_lds(reinterpret_cast<const void*>(&scan_hist_kernel), lds);
    hipLaunchKernelGGL(scan_hist_kernel, dim3(1), dim3(kScanThreads), lds, s, hist, static_cast<int>(E), nt32, start,
                       static_cast<uint32_t*>(nullptr), none);
    const Placement pl{nullptr, hist, start, static_cast<int>(E), 0};
    if (p.padded)
      hipLaunchKernelGGL(permute_table_kernel<true>, dim3(nt32), dim3(th), 0, s, map, p.T, E, pl, d->capacity, table,
                         d->sorted_indices);
    else
      hipLaunchKernelGGL(permute_table_kernel<false>, dim3(nt32), dim3(th), 0, s, map, p.T, E, pl, d->capacity, table,
                         d->sorted_indices);
    if (hipGetLastError() != hipSuccess) return FFNWB_ERR_RUNTIME;
    // padded: rows whose sorted_indices entry is -1 are zero; non-padded: rows from the
    // number of non-zero entries (start[E]) on
    const bool ok = launch_scatter<1, false>(vec, p.T, p.N, s, evb, eve, tok, p.stride, p.row_bytes,
                                   static_cast<const int32_t*>(table), p.T, E,
                                   static_cast<int32_t>(p.padded ? 0 : p.K), d->sorted_indices,
                                   static_cast<const int32_t*>(p.padded ? d->sorted_indices : nullptr),
                                   static_cast<const uint32_t*>(start + E), p.N, out);
    if (!ok) return FFNWB_ERR_RUNTIME;
    return hipGetLastError() == hipSuccess ? FFNWB_OK : FFNWB_ERR_RUNTIME;
  }
  uint32_t* hist = c.take<uint32_t>(static_cast<size_t>(p.ntiles * p.E));
  int32_t* source_of = p.padded ? d->sorted_indices : c.take<int32_t>(static_cast<size_t>(p.N));
  int32_t* dest = p.padded ? c.take<int32_t>(static_cast<size_t>(p.T * p.E)) : nullptr;
  const int nt = static_cast<int>(p.ntiles);
  const bool wide = E % 4 == 0 && reinterpret_cast<uintptr_t>(map) % 4 == 0;
  const size_t lds = permute_order_lds_bytes(nt, E, p.padded);
  auto go = [&](auto wtag, auto ptag) {
    constexpr int W = decltype(wtag)::value;
    constexpr bool PADDED = decltype(ptag)::value;
    allow_large_lds(reinterpret_cast<const void*>(&permute_order_kernel<W, PADDED>), lds);
    hipLaunchKernelGGL(mask_tile_count_kernel<W>, dim3(nt, mask_ranges(E, W)), dim3(kMaskSplitThreads), 0, s, map,
                       p.T, E, hist, static_cast<uint32_t*>(nullptr));
    hipLaunchKernelGGL((permute_order_kernel<W, PADDED>), dim3(nt), dim3(kPermuteThreads), lds, s, map, p.T, E, nt,
                       hist, p.N, static_cast<int32_t>(p.K), d->capacity, source_of, d->sorted_indices, dest);
  };
  if (wide) {
    if (p.padded) go(std::integral_constant<int, 4>(), std::true_type());
    else go(std::integral_constant<int, 4>(), std::false_type());
  } else {
    if (p.padded) go(std::integral_constant<int, 1>(), std::true_type());
    else go(std::integral_constant<int, 1>(), std::false_type());
  }
  if (hipGetLastError() != hipSuccess) return FFNWB_ERR_RUNTIME;
  // token rows to their rows: non-padded through the topK slots (rows past them through
  // source_of), padded through the [T][E] table (zero rows are sorted_indices' -1 entries)
  const int32_t K = static_cast<int32_t>(p.padded ? p.E : p.K);
  const int32_t* lists = p.padded ? dest : d->sorted_indices;
  const int32_t* src_of = source_of;
  int32_t* no_slots = nullptr;
  const uint32_t* no_filled = nullptr;
  const bool ok =
      p.padded ? launch_scatter<1, false>(vec, p.T, p.N, s, evb, eve, tok, p.stride, p.row_bytes, lists, p.T, K,
                                          int32_t{0}, no_slots, src_of, no_filled, p.N, out)
               : launch_scatter<4, true>(vec, p.T, p.N, s, evb, eve, tok, p.stride, p.row_bytes, lists, p.T, K,
                                         int32_t{0}, no_slots, src_of, no_filled, p.N, out);
  if (!ok) return FFNWB_ERR_RUNTIME;
  return hipGetLastError() == hipSuccess ? FFNWB_OK : FFNWB_ERR_RUNTIME;
}

}  // namespace ffnwb

// MoE token unpermute with routing map on gfx950 (MoeTokenUnpermuteWithRoutingMap article,
// "Function description and formulas", branches 1-4; "Kernel implementation").
//
// Non-padded mode (branches 2 and 4):
//   [probs]  probs compaction: the non-zero routing-map entries in expert-major order
//            -> permute_probs, zero-padded.  Two launches over 256-token tiles split by
//            column ranges (count, then compact), or for large maps a counting sort
//            (count, scan, scatter);
//   reduce:  one workgroup per token gathers its topK slots' permuted rows and sums
//            x * w in FP32 (slot order), one RNE store;
//   [aux]    out_index / permute_token_id: stable sort of the slots by sortedIndices+1
//            (LSD passes when the row count exceeds one pass's bucket budget), on the
//            caller's stream, or on the caller's auxiliary stream when the descriptor
//            names one: forked when the compaction's first kernel completes, submitted
//            after the reduce and joined after it.
// Padded mode (branches 1 and 3):
//   invert:  stable counting sort of the capacity entries by token id (rank, scan,
//            scatter -> out_index, permute_token_id, permute_probs, per-token segments);
//   reduce:  one workgroup per token sums its segment's rows in ascending row order.
// No atomics anywhere, so every output is deterministic.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <type_traits>

#include "internal.hpp"
#include "map_tiles.hpp"
#include "range_order.hpp"
#include "reduce_kernels.hpp"
#include "sort_engine.hpp"

namespace ffnwb {

// Probs compaction (non-padded with probs): permute_probs lists probs[t, e] for the
// non-zero routing-map entries in expert-major order, i.e. a stable counting sort of
// the entries t*E + e by e.  For large maps: mask_count_kernel (map_tiles.hpp), the
// histogram scan, then mask_scatter_kernel.

// permute_probs[start[e] + (tile's base for e) + running count] = probs[t, e]; entries
// at positions >= N are dropped; positions from start[E] (the number of non-zero
// entries) up to N get 0.  `pl` is the scanned histogram (its packed field is unused).
template <typename P>
__global__ __launch_bounds__(256) void mask_scatter_kernel(const uint8_t* __restrict__ map,
                                                           const P* __restrict__ probs, int64_t T, int32_t E,
                                                           Placement pl, P* __restrict__ pp, int64_t N) {
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kMaskTile;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    uint32_t pos = pl.start[e] + pl.tile_base(blockIdx.x, static_cast<uint32_t>(e));
    // map bytes and probs of the whole tile column are loaded first (clamped rows, no
    // branch), so the loads are in flight together; probs reads are coalesced across e
    uint8_t m[kMaskTile];
    P v[kMaskTile];
#pragma unroll
    for (int i = 0; i < kMaskTile; ++i) {
      const int64_t row = (t0 + i < T ? t0 + i : T - 1) * E + e;
      m[i] = map[row];
      v[i] = probs[row];
    }
#pragma unroll
    for (int i = 0; i < kMaskTile; ++i) {
      if (t0 + i < T && m[i] != 0) {
        if (pos < N) pp[pos] = v[i];
        ++pos;
      }
    }
  }
  const uint32_t filled = pl.start[E];
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < N;
       g += static_cast<int64_t>(gridDim.x) * blockDim.x)
    if (g >= filled) pp[g] = P(0);
}

// Probs compaction in two launches, for maps whose tile histogram is small (at most
// kMaskLdsHist words).  Tiles of kMaskRows token rows; a work item is kMaskGroupRows
// consecutive rows x W consecutive columns (W = 4 when the columns come in aligned groups
// of 4, else 1), read as one W-byte map load and one W-element probs load per row.  Both
// launches run on the grid (tiles, column ranges of kMaskRangeUnits work-item columns).
//   mask_tile_count_kernel  hist[tile*E + e] = non-zero entries of column e in the tile,
//                           range_tot[tile*ranges + r] = those of range r;
//   mask_compact_kernel     workgroup (tile, r): its first column starts after the
//                           entries of all lower ranges (their range totals over all
//                           tiles), each further column after the lower columns of the
//                           range (their totals over all tiles); the column's counts in
//                           earlier tiles give the start of the tile's run in each
//                           column; the items stage their entries in LDS (row order within
//                           each column, no branch per entry), and the runs are copied out
//                           with consecutive stores.
// No scan launch: every workgroup reads the histogram words of its own columns only.
template <int W, typename P>
struct ProbUnit {
  P v[W];
  __device__ __forceinline__ void load(const P* p) {
    if (W == 4 && sizeof(P) == 4) {
      const uint4 q = *reinterpret_cast<const uint4*>(p);
      v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    } else if (W == 4) {
      const uint2 q = *reinterpret_cast<const uint2*>(p);
      v[0] = static_cast<P>(q.x & 0xffffu); v[1] = static_cast<P>(q.x >> 16);
      v[2] = static_cast<P>(q.y & 0xffffu); v[3] = static_cast<P>(q.y >> 16);
    } else {
#pragma unroll
      for (int w = 0; w < W; ++w) v[w] = p[w];
    }
  }
};

// One work item's map units and probs, loaded before they are needed.
template <int W, typename P>
struct MaskItem {
  uint32_t x[kMaskGroupRows];
  ProbUnit<W, P> pv[kMaskGroupRows];
  __device__ __forceinline__ void load(const uint8_t* __restrict__ map, const P* __restrict__ probs, int64_t T,
                                       int32_t E, int64_t r0, int c) {
#pragma unroll
    for (int r = 0; r < kMaskGroupRows; ++r) {
      const int64_t row = min(r0 + r, T - 1);  // clamped: unconditional loads
      x[r] = load_map_unit<W>(map + row * E + c * W);
      pv[r].load(probs + row * E + c * W);
    }
  }
  __device__ __forceinline__ void count(int64_t T, int64_t r0, uint32_t (&cnt)[W]) const {
#pragma unroll
    for (int w = 0; w < W; ++w) cnt[w] = 0u;
#pragma unroll
    for (int r = 0; r < kMaskGroupRows; ++r) {
#pragma unroll
      for (int w = 0; w < W; ++w) cnt[w] += (r0 + r < T && ((x[r] >> (8 * w)) & 0xffu) != 0) ? 1u : 0u;
    }
  }
  // stages every entry of the item in LDS without a branch: a non-zero entry of column w
  // goes to slot sp[w] (then the next one) with its output position gp[w] (then the next
  // one), any other entry to the lane's trash slot
  __device__ __forceinline__ void stage(int64_t T, int64_t r0, uint32_t (&sp)[W], uint32_t (&gp)[W],
                                        uint2* __restrict__ st, uint32_t trash) const {
#pragma unroll
    for (int r = 0; r < kMaskGroupRows; ++r) {
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const bool nz = (r0 + r < T) & (((x[r] >> (8 * w)) & 0xffu) != 0);
        st[nz ? sp[w] : trash] = make_uint2(static_cast<uint32_t>(pv[r].v[w]), gp[w]);
        sp[w] += nz ? 1u : 0u;
        gp[w] += nz ? 1u : 0u;
      }
    }
  }
};

template <int W, typename P>
__global__ __launch_bounds__(kMaskSplitThreads) void mask_compact_kernel(const uint8_t* __restrict__ map,
                                                                         const P* __restrict__ probs, int64_t T,
                                                                         int32_t E, int ntiles,
                                                                         const uint32_t* __restrict__ hist,
                                                                         const uint32_t* __restrict__ range_tot,
                                                                         P* __restrict__ pp, int64_t N) {
  constexpr int NT = kMaskSplitThreads;
  constexpr int NW = NT / kWave;
  constexpr int MC = kMaskRangeUnits * W;  // columns of a full range
  constexpr int kHistBatch = 16;           // histogram words per thread per load round
  constexpr int kRangeBatch = 4;           // range totals per thread per load round
  __shared__ uint32_t gc[kMaskGroups * MC];  // [group][column] item counts -> offsets in the tile's column run
  __shared__ uint32_t part[2 * NT];          // column partials: all tiles | earlier tiles
  __shared__ uint32_t rsum[2 * NW];          // per-wave range totals: all | lower ranges
  __shared__ uint32_t cst[MC], coff[MC];    // per column: output start, staging offset
  __shared__ uint32_t staged;                // entries of the workgroup
  __shared__ uint2 stage[kMaskRows * MC + kWave];  // (value, output position): column runs back to back; trash
  const int tid = threadIdx.x;
  const int lane = static_cast<int>(lane_id());
  const int tile = blockIdx.x;
  const int r = blockIdx.y;
  const int R = gridDim.y;
  const int u0 = r * kMaskRangeUnits;
  const int nu = min(kMaskRangeUnits, E / W - u0);
  const int ncols = nu * W;
  const int e0 = u0 * W;
  const int g = tid / kMaskRangeUnits, u = tid % kMaskRangeUnits;
  const bool act = u < nu;
  const int64_t r0 = static_cast<int64_t>(tile) * kMaskRows + g * kMaskGroupRows;
  // 1. the global loads of the first round all at once: the item's map units and probs,
  //    the thread's histogram words (column c, tiles q, q + ppc, ...), its range totals
  MaskItem<W, P> item;
  item.load(map, probs, T, E, r0, u0 + (act ? u : 0));
  int ppc = 1;  // threads per column: a power of two, ppc * ncols <= NT
  while (ppc * 2 * ncols <= NT) ppc *= 2;
  const int c = tid % ncols, q = tid / ncols;
  const int nrt = ntiles * R;
  uint32_t call = 0, cpre = 0, rall = 0, rlow = 0;
  for (int i = 0;; ++i) {
    const int t0 = q + i * ppc * kHistBatch;
    const int j0 = tid + i * NT * kRangeBatch;
    const bool more_h = q < ppc && t0 < ntiles;
    const bool more_r = j0 < nrt;
    if (!(more_h || more_r)) break;
    uint32_t hv[kHistBatch], rv[kRangeBatch];
#pragma unroll
    for (int k = 0; k < kHistBatch; ++k)
      hv[k] = hist[static_cast<int64_t>(min(t0 + k * ppc, ntiles - 1)) * E + e0 + c];
#pragma unroll
    for (int k = 0; k < kRangeBatch; ++k) rv[k] = range_tot[min(j0 + k * NT, nrt - 1)];
#pragma unroll
    for (int k = 0; k < kHistBatch; ++k) {
      const int t = t0 + k * ppc;
      call += (q < ppc && t < ntiles) ? hv[k] : 0u;
      cpre += (q < ppc && t < tile) ? hv[k] : 0u;
    }
#pragma unroll
    for (int k = 0; k < kRangeBatch; ++k) {
      const int j = j0 + k * NT;
      rall += j < nrt ? rv[k] : 0u;
      rlow += (j < nrt && j % R < r) ? rv[k] : 0u;
    }
  }
  uint32_t cnt[W];
  item.count(T, r0, cnt);
  if (act) {
#pragma unroll
    for (int w = 0; w < W; ++w) gc[g * MC + u * W + w] = cnt[w];
  }
  part[tid] = call;  // zero for q >= ppc
  part[NT + tid] = cpre;
  rall = wave_sum(rall);
  rlow = wave_sum(rlow);
  if (lane == 0) {
    rsum[tid / kWave] = rall;
    rsum[NW + tid / kWave] = rlow;
  }
  // 2. column sums: a tree over the ppc partials of each column
  for (int h = ppc / 2; h >= 1; h /= 2) {
    __syncthreads();
    if (q < h) {
      part[q * ncols + c] += part[(q + h) * ncols + c];
      part[NT + q * ncols + c] += part[NT + (q + h) * ncols + c];
    }
  }
  __syncthreads();
  uint32_t filled = 0, low = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    filled += rsum[w];
    low += rsum[NW + w];
  }
  // 3. wave 0, one lane per column: the column's output start and, over the row groups,
  //    each item's offset in the column's run; the runs are staged back to back
  if (tid < kWave) {
    const uint32_t tot = tid < ncols ? part[tid] : 0u;
    uint32_t n = 0;
    if (tid < ncols) {
      for (int gg = 0; gg < kMaskGroups; ++gg) {
        const uint32_t v = gc[gg * MC + tid];
        gc[gg * MC + tid] = n;
        n += v;
      }
    }
    const uint32_t incl_tot = wave_inclusive_scan(tot, lane);
    const uint32_t incl_n = wave_inclusive_scan(n, lane);
    if (tid < ncols) {
      cst[tid] = low + incl_tot - tot + part[NT + tid];
      coff[tid] = incl_n - n;
    }
    if (tid == kWave - 1) staged = incl_n;
  }
  __syncthreads();
  // 4. stage the item's entries, rows in order, then copy the staged entries out: the
  //    column runs are consecutive positions, so neighbouring lanes store neighbours
  if (act) {
    uint32_t sp[W], gp[W];
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const uint32_t o = gc[g * MC + u * W + w];
      sp[w] = coff[u * W + w] + o;
      gp[w] = cst[u * W + w] + o;
    }
    item.stage(T, r0, sp, gp, stage, kMaskRows * MC + lane);
  }
  __syncthreads();
  constexpr int kOut = 4;  // staged entries per thread per round, read together
  const uint32_t M = staged;
  for (uint32_t f0 = tid; f0 < M; f0 += kOut * NT) {
    uint2 e[kOut];
#pragma unroll
    for (int k = 0; k < kOut; ++k) e[k] = stage[min(f0 + k * NT, M - 1)];
#pragma unroll
    for (int k = 0; k < kOut; ++k)
      if (f0 + k * NT < M && e[k].y < N) pp[e[k].y] = static_cast<P>(e[k].x);
  }
  // 5. positions from the number of non-zero entries up to N get 0
  const int64_t nwg = static_cast<int64_t>(ntiles) * R;
  const int64_t b = static_cast<int64_t>(tile) * R + r;
  for (int64_t gi = b * NT + tid; gi < N; gi += nwg * NT)
    if (gi >= filled) pp[gi] = P(0);
}

// Words of the compaction's second workspace region: the column starts of the
// three-launch path, or the range totals of the two-launch path (at most
// tiles * mask_ranges(E, 1) of them, W = 1 giving the most ranges).
static size_t mask_aux_words(int64_t E, int nt) {
  const size_t ranges = static_cast<size_t>(mask_ranges(static_cast<int32_t>(E), 1));
  return std::max(static_cast<size_t>(E) + 1, ranges * static_cast<size_t>(nt));
}

// Padded inversion, single pass: out_index / permute_token_id at the sorted position, and
// the capacity entry's prob permute_probs[j] = probs[sI[j], j / C] (0 for invalid tokens).
template <typename P>
__global__ __launch_bounds__(256) void padded_scatter_kernel(const int32_t* __restrict__ sI, int32_t T,
                                                             Placement pl, int64_t n,
                                                             int32_t* __restrict__ out_index,
                                                             int32_t* __restrict__ token_out,
                                                             const P* __restrict__ probs, int64_t E, int64_t C,
                                                             P* __restrict__ pp) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j >= n) return;
  const int32_t v = sI[j];
  uint32_t pos, dig;
  if (pl.position(j, pos, dig)) {
    out_index[pos] = static_cast<int32_t>(j);
    if (token_out != nullptr) token_out[pos] = v;
  }
  if (pp != nullptr) pp[j] = (v >= 0 && v < T) ? probs[static_cast<int64_t>(v) * E + j / C] : P(0);
}

// Padded inversion in one launch: the range-partitioned order of the capacity entries by
// token (invalid ids share the last key T).  Workgroup b owns the keys [lo, lo + kr): it
// writes seg[t], the first sorted position of token t, for its keys, and out_index /
// permute_token_id at the sorted positions of its entries; the workgroup that owns key T
// also writes seg[T + 1] = n.  Every workgroup also gathers permute_probs for its share of
// the entries, its first ids loaded in the count pass's load round.
template <typename P>
__global__ __launch_bounds__(kRoThreads) void padded_order_kernel(const int32_t* __restrict__ sI, int32_t T,
                                                                  int64_t n, uint32_t kr, int nbits,
                                                                  int32_t* __restrict__ order,
                                                                  int32_t* __restrict__ token_out,
                                                                  uint32_t* __restrict__ seg,
                                                                  const P* __restrict__ probs, int64_t E, int64_t C,
                                                                  P* __restrict__ pp) {
  extern __shared__ uint32_t lds_words[];  // range-order layout (ro_lds_words)
  __shared__ uint32_t wsum[2 * kRoWaves + 2];
  const uint32_t nkeys = static_cast<uint32_t>(T) + 1u;
  const uint32_t lo = blockIdx.x * kr;
  const uint32_t krr = min(kr, nkeys - lo);
  uint32_t* cnt = ro_counters(lds_words);
  for (int i = threadIdx.x; i < kRoWaves * static_cast<int>(krr); i += kRoThreads) cnt[i] = 0u;
  __syncthreads();
  // permute_probs for this workgroup's share of the entries: the first id is loaded with
  // the count pass's keys and its prob after the pass, so the gather adds one load round
  const int64_t share = (n + gridDim.x - 1) / gridDim.x;
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * share + threadIdx.x;
  const int64_t j1 = min(n, static_cast<int64_t>(blockIdx.x) * share + share);
  const int32_t v0 = sI[min(j0, n - 1)];
  const int w = uniform(static_cast<int>(threadIdx.x) / kWave);
  uint32_t b, e;
  ro_slice(static_cast<uint32_t>(n), w, b, e);
  const RoKeysPadded ks{sI, T, static_cast<uint32_t>(n)};
  const RoWave wv = ro_wave(lds_words, w, krr);
  uint32_t len;
  // 8 blocks of loads at once: a whole 2048-entry slice in one round
  const uint32_t below = ro_count<8>(ks, b, e, lo, krr, wv, len, [](uint32_t, uint32_t, bool, bool) {});
  if (pp != nullptr) {
    for (int64_t j = j0; j < j1; j += kRoThreads) {
      const int32_t v = j == j0 ? v0 : sI[j];
      pp[j] = (v >= 0 && v < T) ? probs[static_cast<int64_t>(v) * E + j / C] : P(0);
    }
  }
  uint32_t kcount, end;
  const uint32_t first = ro_middle(cnt, krr, below, wsum, kcount, end);
  if (threadIdx.x < krr) seg[lo + threadIdx.x] = first;
  if (threadIdx.x == 0 && lo + krr == nkeys) seg[nkeys] = end;
  ro_place(ks, b, e, lo, krr, nbits, wv, len, [&](uint32_t j, uint32_t key, uint32_t pos) {
    order[pos] = static_cast<int32_t>(j);
    // the raw id equals the key except in the invalid bucket: no load on the common path
    if (token_out != nullptr) token_out[pos] = key < static_cast<uint32_t>(T) ? static_cast<int32_t>(key) : sI[j];
  });
}

template <typename P>
__global__ __launch_bounds__(256) void padded_probs_kernel(const int32_t* __restrict__ sI, int32_t T, int64_t n,
                                                           const P* __restrict__ probs, int64_t E, int64_t C,
                                                           P* __restrict__ pp) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j >= n) return;
  const int32_t v = sI[j];
  pp[j] = (v >= 0 && v < T) ? probs[static_cast<int64_t>(v) * E + j / C] : P(0);
}

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ------------------------------------------------------------------ host side

static unsigned grid_for(int64_t n, int threads) { return static_cast<unsigned>((n + threads - 1) / threads); }

template <class KS>
static void launch_rank(const SortPass& p, KS ks, uint32_t* packed, uint32_t* hist, uint32_t* tile_err,
                        hipStream_t s) {
  if (p.nt == 0) return;
  const size_t lds = rank_lds_bytes(p.nb);
  allow_large_lds(reinterpret_cast<const void*>(p.R == 4 ? &sort_rank_kernel<4, KS> : &sort_rank_kernel<16, KS>), lds);
  if (p.R == 4)
    hipLaunchKernelGGL((sort_rank_kernel<4, KS>), dim3(p.nt), dim3(kRankThreads), lds, s, ks, p.n, p.shift, p.nbits,
                       p.nb, packed, hist, tile_err);
  else
    hipLaunchKernelGGL((sort_rank_kernel<16, KS>), dim3(p.nt), dim3(kRankThreads), lds, s, ks, p.n, p.shift,
                       p.nbits, p.nb, packed, hist, tile_err);
}

// Scans a histogram of nb digits x nt tiles and returns where its elements go.
static Placement launch_scan(int nb, int nt, int tile_shift, const uint32_t* packed, uint32_t* hist, uint32_t* start,
                             hipStream_t s) {
  ScanTail none{nullptr, 0, nullptr, nullptr, nullptr};
  const size_t lds = scan_lds_bytes(nb);
  allow_large_lds(reinterpret_cast<const void*>(&scan_hist_kernel), lds);
  hipLaunchKernelGGL(scan_hist_kernel, dim3(1), dim3(kScanThreads), lds, s, hist, nb, nt, start,
                     static_cast<uint32_t*>(nullptr), none);
  return Placement{packed, hist, start, nb, tile_shift};
}

struct SortBufs {
  uint32_t* packed;
  uint32_t* hist;
  uint32_t* start;  // nb + 1 entries of the widest pass
  uint32_t* kA; uint32_t* vA; uint32_t* kB; uint32_t* vB;
};

static void carve_sort_bufs(Carve& c, const SortPlan& sp, int64_t n, SortBufs* b) {
  b->packed = c.take<uint32_t>(n);
  b->hist = c.take<uint32_t>(sp.hist_words);
  b->start = c.take<uint32_t>(static_cast<size_t>(sp.max_nb) + 1);
  if (sp.npasses > 1) {
    b->kA = c.take<uint32_t>(n); b->vA = c.take<uint32_t>(n);
    b->kB = c.take<uint32_t>(n); b->vB = c.take<uint32_t>(n);
  }
}

// Runs every pass but the scatter of the last one; returns the keys/values of the last
// pass's input (nullptr for a single pass, whose input is the key source itself) and the
// last pass's placement.
template <class KS>
static Placement run_passes_but_last_scatter(const SortPlan& sp, KS ks0, const SortBufs& b, const uint32_t** keys_in,
                                             const uint32_t** vals_in, hipStream_t s) {
  const uint32_t* kin = nullptr;
  const uint32_t* vin = nullptr;
  uint32_t* kout = b.kA;
  uint32_t* vout = b.vA;
  Placement pl{};
  for (int i = 0; i < sp.npasses; ++i) {
    const SortPass& p = sp.pass[i];
    if (i == 0) launch_rank(p, ks0, b.packed, b.hist, nullptr, s);
    else launch_rank(p, KeyArray{kin}, b.packed, b.hist, nullptr, s);
    pl = launch_scan(p.nb, p.nt, p.tile_shift, b.packed, b.hist, b.start, s);
    if (i == sp.npasses - 1) break;
    const unsigned g = grid_for(p.n, 256);
    if (i == 0)
      hipLaunchKernelGGL((lsd_scatter_kernel<KS, true, 0>), dim3(g), dim3(256), 0, s, ks0, vin, pl, p.n, kout, vout,
                         static_cast<int32_t*>(nullptr), static_cast<int32_t*>(nullptr),
                         static_cast<const int32_t*>(nullptr), 0);
    else
      hipLaunchKernelGGL((lsd_scatter_kernel<KeyArray, false, 0>), dim3(g), dim3(256), 0, s, KeyArray{kin}, vin, pl,
                         p.n, kout, vout, static_cast<int32_t*>(nullptr), static_cast<int32_t*>(nullptr),
                         static_cast<const int32_t*>(nullptr), 0);
    kin = kout;
    vin = vout;
    kout = (kout == b.kA) ? b.kB : b.kA;
    vout = (vout == b.vA) ? b.vB : b.vA;
  }
  *keys_in = kin;
  *vals_in = vin;
  return pl;
}

// The caller's auxiliary stream for the non-padded out_index / permute_token_id sort, with
// the two events that fork it from and join it back to the caller's stream.  The library
// keeps no stream or event of its own: without an auxiliary stream the sort runs on the
// caller's stream, in order with the rest of the call.
struct AuxFork {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr;
  hipEvent_t join = nullptr;
};

static AuxFork aux_fork_of(const moe_unpermute_desc* d, hipStream_t caller) {
  AuxFork f;
  if (d->aux_stream == nullptr || static_cast<hipStream_t>(d->aux_stream) == caller) return f;
  f.stream = static_cast<hipStream_t>(d->aux_stream);
  f.fork = static_cast<hipEvent_t>(d->aux_fork_event);
  f.join = static_cast<hipEvent_t>(d->aux_join_event);
  return f;
}

int plan_unpermute(const moe_unpermute_desc* d, UnpermutePlan* p) {
  if (d == nullptr || p == nullptr) return FFNWB_ERR_PARAM_NULLPTR;
  if (d->permuted_tokens == nullptr || d->sorted_indices == nullptr || d->unpermuted_tokens == nullptr)
    return FFNWB_ERR_PARAM_NULLPTR;
  if (d->dtype != FFNWB_DT_FP16 && d->dtype != FFNWB_DT_BF16 && d->dtype != FFNWB_DT_FP32)
    return FFNWB_ERR_PARAM_INVALID;
  const bool has_probs = d->probs != nullptr;
  if ((d->routing_map != nullptr) != has_probs) return FFNWB_ERR_PARAM_INVALID;
  if (has_probs && !(d->probs_dtype == d->dtype || (d->dtype == FFNWB_DT_BF16 && d->probs_dtype == FFNWB_DT_FP32)))
    return FFNWB_ERR_PARAM_INVALID;
  if (d->padded_mode != 0 && d->padded_mode != 1) return FFNWB_ERR_PARAM_INVALID;
  if (d->weight_index != 0 && d->weight_index != 1) return FFNWB_ERR_PARAM_INVALID;
  if ((d->skip_zero_weight != 0 && d->skip_zero_weight != 1) || d->reserved0 != 0) return FFNWB_ERR_PARAM_INVALID;
  if (d->aux_stream != nullptr && (d->aux_fork_event == nullptr || d->aux_join_event == nullptr))
    return FFNWB_ERR_PARAM_NULLPTR;
  if (d->hidden <= 0 || d->num_tokens < 0 || d->num_indices < 0 || d->num_rows < 0) return FFNWB_ERR_PARAM_INVALID;
  if (d->num_rows != d->num_indices) return FFNWB_ERR_PARAM_INVALID;
  const int64_t lim = (int64_t{1} << 31) - 2;
  if (d->num_indices > lim || d->num_tokens > lim || d->hidden > (int64_t{1} << 30)) return FFNWB_ERR_PARAM_INVALID;
  if (has_probs && (d->num_experts <= 0 || d->num_experts > kMaxExperts)) return FFNWB_ERR_INNER_NULLPTR;
  if (has_probs && d->num_tokens * d->num_experts > lim) return FFNWB_ERR_PARAM_INVALID;

  p->T = d->num_tokens;
  p->H = d->hidden;
  p->N = d->num_indices;
  p->rows = d->num_rows;
  p->E = has_probs ? d->num_experts : 0;
  p->has_probs = has_probs;
  p->padded = d->padded_mode != 0;
  p->elt = d->dtype == FFNWB_DT_FP32 ? 4 : 2;
  p->pelt = has_probs ? (d->probs_dtype == FFNWB_DT_FP32 ? 4 : 2) : 0;
  if (static_cast<double>(p->T) * p->H * p->elt > 9.0e18 || static_cast<double>(p->rows) * p->H * p->elt > 9.0e18)
    return FFNWB_ERR_PARAM_INVALID;

  Carve c;
  if (!p->padded) {
    if (p->T == 0) {
      if (p->N != 0) return FFNWB_ERR_PARAM_INVALID;
      p->K = 0;
    } else {
      if (p->N % p->T != 0) return FFNWB_ERR_PARAM_INVALID;
      p->K = p->N / p->T;
    }
    if (p->K > 512) return FFNWB_ERR_INNER_NULLPTR;
    if (has_probs) {
      const int64_t fused_tiles = (p->T + kMaskRows - 1) / kMaskRows;
      p->mask_fused = p->E <= kMaskFusedMaxExperts && fused_tiles * p->E <= kMaskLdsHist;
      p->mask_tiles = p->mask_fused ? fused_tiles : (p->T + kMaskTile - 1) / kMaskTile;
      const int nt = static_cast<int>(p->mask_tiles);
      c.take<uint32_t>(static_cast<size_t>(p->E) * nt);                 // histogram
      c.take<uint32_t>(mask_aux_words(p->E, nt));                        // column starts or range totals
      if (d->permute_probs == nullptr) c.take<uint8_t>(static_cast<size_t>(p->N) * p->pelt);
    }
    p->need_aux = d->out_index != nullptr || d->permute_token_id != nullptr;
    if (p->need_aux && p->N > 0) {
      p->sort = make_sort_plan(p->N, static_cast<uint64_t>(p->rows) + 1);
      SortBufs b{};
      carve_sort_bufs(c, p->sort, p->N, &b);
    }
  } else {
    if (has_probs) {
      if (p->N % p->E != 0) return FFNWB_ERR_PARAM_INVALID;
      p->C = p->N / p->E;
    }
    if (log_enabled()) {
      if (has_probs && p->C > p->T)
        log_warn("moe_unpermute: padded mode with capacity %lld > tokens %lld", (long long)p->C, (long long)p->T);
      if (has_probs && p->T > 0 && p->N / p->T > p->E)
        log_warn("moe_unpermute: padded mode with topK %lld > experts %lld", (long long)(p->N / p->T),
                 (long long)p->E);
    }
    p->range_order = ro_fits(p->N, static_cast<uint64_t>(p->T) + 1);
    if (!p->range_order) {
      p->sort = make_sort_plan(p->N, static_cast<uint64_t>(p->T) + 1);
      SortBufs b{};
      carve_sort_bufs(c, p->sort, p->N, &b);               // sort buffers
    }
    c.take<uint32_t>(static_cast<size_t>(p->T) + 2);       // token segments
    if (d->out_index == nullptr) c.take<int32_t>(p->N);    // sorted order for the reduce
    if (has_probs && d->permute_probs == nullptr) c.take<uint8_t>(static_cast<size_t>(p->N) * p->pelt);
    if (p->sort.npasses > 1) c.take<uint32_t>(p->N);       // sorted keys
  }
  p->ws_bytes = c.off;
  return FFNWB_OK;
}

// Reduce launch shape: `cpt` 16-byte chunks per thread (0 = element-wise kernel).
struct ReduceShape {
  int cpt = 1;
  int threads = 64;
};

static ReduceShape reduce_shape(bool vec, int64_t H, int elt) {
  ReduceShape r;
  const int64_t work = vec ? (H * elt / 16) : H;
  if (!vec) {
    r.cpt = 0;
  } else if (work <= 1024) {
    r.cpt = 1;
  } else if (work <= 2048) {
    r.cpt = 2;
  } else {
    r.cpt = 4;
  }
  const int64_t per = r.cpt > 0 ? (work + r.cpt - 1) / r.cpt : work;
  int64_t th = (per + 63) / 64 * 64;
  if (th > 1024) th = 1024;
  if (th < 64) th = 64;
  r.threads = static_cast<int>(th);
  return r;
}

// The optional hooks ev_begin / ev_end are bound to the reduce launch; with no launch
// (T = 0) they are recorded back to back.
template <class TT, class TW, int MODE>
static bool launch_reduce_t(const ReduceArgs& ra, const ReduceShape& sh, int64_t T, hipStream_t s, void* evb,
                            void* eve) {
  if (T == 0) return record_event(evb, s) && record_event(eve, s);
  const dim3 grid(static_cast<unsigned>(T)), block(sh.threads);
  switch (sh.cpt) {
    case 0: return launch_bound(unpermute_reduce_elem_kernel<TT, TW, MODE>, grid, block, 0, s, evb, eve, ra);
    case 1: return launch_bound(unpermute_reduce_kernel<TT, TW, MODE, 1>, grid, block, 0, s, evb, eve, ra);
    case 2: return launch_bound(unpermute_reduce_kernel<TT, TW, MODE, 2>, grid, block, 0, s, evb, eve, ra);
    default: return launch_bound(unpermute_reduce_kernel<TT, TW, MODE, 4>, grid, block, 0, s, evb, eve, ra);
  }
}

template <class TT, class TW>
static bool launch_reduce_w(const ReduceArgs& ra, int mode, const ReduceShape& sh, int64_t T, hipStream_t s,
                            void* evb, void* eve) {
  switch (mode) {
    case kNonPad: return launch_reduce_t<TT, TW, kNonPad>(ra, sh, T, s, evb, eve);
    case kNonPadW2: return launch_reduce_t<TT, TW, kNonPadW2>(ra, sh, T, s, evb, eve);
    case kNonPadW1: return launch_reduce_t<TT, TW, kNonPadW1>(ra, sh, T, s, evb, eve);
    case kPad: return launch_reduce_t<TT, TW, kPad>(ra, sh, T, s, evb, eve);
    default: return launch_reduce_t<TT, TW, kPadW>(ra, sh, T, s, evb, eve);
  }
}

static bool launch_reduce(const ReduceArgs& ra, int dtype, int pdtype, int mode, const ReduceShape& sh, int64_t T,
                          hipStream_t s, void* evb, void* eve) {
  if (dtype == FFNWB_DT_FP16) return launch_reduce_w<TF16, TF16>(ra, mode, sh, T, s, evb, eve);
  if (dtype == FFNWB_DT_FP32) return launch_reduce_w<TF32, TF32>(ra, mode, sh, T, s, evb, eve);
  if (pdtype == FFNWB_DT_FP32) return launch_reduce_w<TBF16, TF32>(ra, mode, sh, T, s, evb, eve);
  return launch_reduce_w<TBF16, TBF16>(ra, mode, sh, T, s, evb, eve);
}

int launch_unpermute(const moe_unpermute_desc* d, const UnpermutePlan& p, void* ws, hipStream_t s) {
  Carve c;
  c.base = static_cast<char*>(ws);
  const int32_t* sI = d->sorted_indices;
  void* pprobs = d->permute_probs;
  const bool vec = ((p.H * p.elt) % 16 == 0) &&
                   ((reinterpret_cast<uintptr_t>(d->permuted_tokens) | reinterpret_cast<uintptr_t>(d->unpermuted_tokens)) % 16 == 0);
  const ReduceShape shape = reduce_shape(vec, p.H, p.elt);

  ReduceArgs ra{};
  ra.x = static_cast<const uint8_t*>(d->permuted_tokens);
  ra.rows = p.rows;
  ra.H = p.H;
  ra.T = p.T;
  ra.out = static_cast<uint8_t*>(d->unpermuted_tokens);
  ra.skip_zero = d->skip_zero_weight;

  if (!p.padded) {
    // workspace regions, in the order plan_unpermute sized them
    const int nt = static_cast<int>(p.mask_tiles);
    uint32_t* mhist = nullptr;
    uint32_t* cstart = nullptr;
    if (p.has_probs) {
      mhist = c.take<uint32_t>(static_cast<size_t>(p.E) * nt);
      cstart = c.take<uint32_t>(mask_aux_words(p.E, nt));  // three-launch path: column starts; else range totals
      if (pprobs == nullptr) pprobs = c.take<uint8_t>(static_cast<size_t>(p.N) * p.pelt);
    }
    SortBufs b{};
    const bool aux = p.need_aux && p.N > 0;
    if (aux) carve_sort_bufs(c, p.sort, p.N, &b);
    // The auxiliary order (out_index / permute_token_id) runs on the caller's auxiliary
    // stream when one is given, else on the caller's stream.
    AuxFork side_f;
    AuxFork* side = nullptr;
    if (aux) {
      side_f = aux_fork_of(d, s);
      if (side_f.stream != nullptr) side = &side_f;
    }
    const bool fused = p.has_probs && nt > 0 && p.mask_fused;
    const uint8_t* map = d->routing_map;
    const int32_t E = static_cast<int32_t>(p.E);
    const bool wide = fused && p.E % 4 == 0 && reinterpret_cast<uintptr_t>(map) % 4 == 0 &&
                      reinterpret_cast<uintptr_t>(d->probs) % (4 * p.pelt) == 0;
    // 1. the first kernel on the caller's stream: the compaction's count kernel, whose
    //    completion (all earlier work on the stream done) is the fork point; without it a
    //    fork event is recorded.  The auxiliary order is submitted after the reduce (it
    //    reads only sortedIndices and writes only its own outputs and workspace): on an
    //    idle GPU the caller's kernels are dispatched first, and the auxiliary stream's
    //    wait usually finds its fork point already passed (an isolated call 260 -> 228 us
    //    on the non-padded workload).
    bool forked = false;
    if (fused) {
      void* fork_ev = side != nullptr ? static_cast<void*>(side->fork) : nullptr;
      const int W = wide ? 4 : 1;
      const dim3 grid(static_cast<unsigned>(nt), static_cast<unsigned>(mask_ranges(E, W)));
      const bool ok = wide ? launch_bound(mask_tile_count_kernel<4>, grid, dim3(kMaskSplitThreads), 0, s, nullptr,
                                          fork_ev, map, p.T, E, mhist, cstart)
                           : launch_bound(mask_tile_count_kernel<1>, grid, dim3(kMaskSplitThreads), 0, s, nullptr,
                                          fork_ev, map, p.T, E, mhist, cstart);
      if (!ok) return FFNWB_ERR_RUNTIME;
      forked = fork_ev != nullptr;
    } else if (side != nullptr) {
      forked = hipEventRecord(side->fork, s) == hipSuccess;
    }
    // 2. the rest of the probs compaction, then the gather-reduce, on the caller's stream
    if (fused) {
      auto go = [&](auto wtag, auto ptag) {
        constexpr int W = decltype(wtag)::value;
        using P = decltype(ptag);
        const dim3 grid(static_cast<unsigned>(nt), static_cast<unsigned>(mask_ranges(E, W)));
        hipLaunchKernelGGL((mask_compact_kernel<W, P>), grid, dim3(kMaskSplitThreads), 0, s, map,
                           static_cast<const P*>(d->probs), p.T, E, nt, mhist, cstart, static_cast<P*>(pprobs), p.N);
      };
      if (wide) {
        if (p.pelt == 4) go(std::integral_constant<int, 4>(), uint32_t());
        else go(std::integral_constant<int, 4>(), uint16_t());
      } else {
        if (p.pelt == 4) go(std::integral_constant<int, 1>(), uint32_t());
        else go(std::integral_constant<int, 1>(), uint16_t());
      }
    } else if (p.has_probs && nt > 0) {
      const int th = static_cast<int>(p.E >= 256 ? 256 : (p.E + 63) / 64 * 64);
      hipLaunchKernelGGL(mask_count_kernel, dim3(nt), dim3(th), 0, s, d->routing_map, p.T,
                         static_cast<int32_t>(p.E), mhist);
      const Placement mpl = launch_scan(static_cast<int>(p.E), nt, 0, nullptr, mhist, cstart, s);
      if (p.pelt == 4)
        hipLaunchKernelGGL(mask_scatter_kernel<uint32_t>, dim3(nt), dim3(th), 0, s, d->routing_map,
                           static_cast<const uint32_t*>(d->probs), p.T, static_cast<int32_t>(p.E), mpl,
                           static_cast<uint32_t*>(pprobs), p.N);
      else
        hipLaunchKernelGGL(mask_scatter_kernel<uint16_t>, dim3(nt), dim3(th), 0, s, d->routing_map,
                           static_cast<const uint16_t*>(d->probs), p.T, static_cast<int32_t>(p.E), mpl,
                           static_cast<uint16_t*>(pprobs), p.N);
    }
    ra.sI = sI;
    ra.K = static_cast<int32_t>(p.K);
    ra.w = pprobs;
    const int mode = !p.has_probs ? kNonPad : (d->weight_index == 1 ? kNonPadW1 : kNonPadW2);
    if (!launch_reduce(ra, d->dtype, d->probs_dtype, mode, shape, p.T, s, d->ev_reduce_begin, d->ev_reduce_end))
      return FFNWB_ERR_RUNTIME;
    // 3. the auxiliary order, then the join
    if (aux) {
      hipStream_t as = s;
      if (side != nullptr) {
        if (!forked || hipStreamWaitEvent(side->stream, side->fork, 0) != hipSuccess) return FFNWB_ERR_RUNTIME;
        as = side->stream;
      }
      KeyNonPadded ks{sI, static_cast<int32_t>(p.rows)};
      const uint32_t *kin, *vin;
      const Placement pl = run_passes_but_last_scatter(p.sort, ks, b, &kin, &vin, as);
      const unsigned g = grid_for(p.N, 256);
      if (p.sort.npasses == 1)
        hipLaunchKernelGGL((lsd_scatter_kernel<KeyNonPadded, true, 1>), dim3(g), dim3(256), 0, as, ks,
                           static_cast<const uint32_t*>(nullptr), pl, p.N, static_cast<uint32_t*>(nullptr),
                           static_cast<uint32_t*>(nullptr), d->out_index, d->permute_token_id, sI,
                           static_cast<int32_t>(p.K));
      else
        hipLaunchKernelGGL((lsd_scatter_kernel<KeyArray, false, 1>), dim3(g), dim3(256), 0, as, KeyArray{kin}, vin,
                           pl, p.N, static_cast<uint32_t*>(nullptr), static_cast<uint32_t*>(nullptr), d->out_index,
                           d->permute_token_id, sI, static_cast<int32_t>(p.K));
      if (side != nullptr && hipEventRecord(side->join, side->stream) != hipSuccess) return FFNWB_ERR_RUNTIME;
    }
    if (side != nullptr && hipStreamWaitEvent(s, side->join, 0) != hipSuccess) return FFNWB_ERR_RUNTIME;
  } else {
    SortBufs b{};
    if (!p.range_order) carve_sort_bufs(c, p.sort, p.N, &b);
    uint32_t* seg = c.take<uint32_t>(static_cast<size_t>(p.T) + 2);
    int32_t* order = d->out_index ? d->out_index : c.take<int32_t>(p.N);
    if (p.has_probs && pprobs == nullptr) pprobs = c.take<uint8_t>(static_cast<size_t>(p.N) * p.pelt);
    if (!p.has_probs) pprobs = nullptr;  // nothing to gather without probs
    uint32_t* skeys = (p.sort.npasses > 1) ? c.take<uint32_t>(p.N) : nullptr;
    KeyPadded ks{sI, static_cast<int32_t>(p.T)};
    const unsigned g = grid_for(p.N, 256);
    if (p.N == 0) {
      hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for(p.T + 2, 256)), dim3(256), 0, s, seg, p.T + 2, 0u);
    } else if (p.range_order) {
      const RoPlan rp = ro_plan(static_cast<uint64_t>(p.T) + 1, kRoGroups);
      const size_t lds = ro_lds_words(rp.kr) * sizeof(uint32_t);
      if (p.pelt == 4) {
        allow_large_lds(reinterpret_cast<const void*>(&padded_order_kernel<uint32_t>), lds);
        hipLaunchKernelGGL(padded_order_kernel<uint32_t>, dim3(rp.grid), dim3(kRoThreads), lds, s, sI,
                           static_cast<int32_t>(p.T), p.N, rp.kr, rp.nbits, order, d->permute_token_id, seg,
                           static_cast<const uint32_t*>(d->probs), p.E, p.C, static_cast<uint32_t*>(pprobs));
      } else {
        allow_large_lds(reinterpret_cast<const void*>(&padded_order_kernel<uint16_t>), lds);
        hipLaunchKernelGGL(padded_order_kernel<uint16_t>, dim3(rp.grid), dim3(kRoThreads), lds, s, sI,
                           static_cast<int32_t>(p.T), p.N, rp.kr, rp.nbits, order, d->permute_token_id, seg,
                           static_cast<const uint16_t*>(d->probs), p.E, p.C, static_cast<uint16_t*>(pprobs));
      }
    } else if (p.sort.npasses == 1) {
      const SortPass& ps = p.sort.pass[0];
      launch_rank(ps, ks, b.packed, b.hist, nullptr, s);
      // digit starts = token segments
      const Placement pl = launch_scan(ps.nb, ps.nt, ps.tile_shift, b.packed, b.hist, seg, s);
      if (p.pelt == 4)
        hipLaunchKernelGGL(padded_scatter_kernel<uint32_t>, dim3(g), dim3(256), 0, s, sI, static_cast<int32_t>(p.T),
                           pl, p.N, order, d->permute_token_id, static_cast<const uint32_t*>(d->probs), p.E, p.C,
                           static_cast<uint32_t*>(pprobs));
      else
        hipLaunchKernelGGL(padded_scatter_kernel<uint16_t>, dim3(g), dim3(256), 0, s, sI, static_cast<int32_t>(p.T),
                           pl, p.N, order, d->permute_token_id, static_cast<const uint16_t*>(d->probs), p.E, p.C,
                           static_cast<uint16_t*>(pprobs));
    } else {
      const uint32_t *kin, *vin;
      const Placement pl = run_passes_but_last_scatter(p.sort, ks, b, &kin, &vin, s);
      hipLaunchKernelGGL((lsd_scatter_kernel<KeyArray, false, 2>), dim3(g), dim3(256), 0, s, KeyArray{kin}, vin, pl,
                         p.N, skeys, static_cast<uint32_t*>(nullptr), order, d->permute_token_id, sI, 0);
      hipLaunchKernelGGL(segment_bounds_kernel, dim3(grid_for(p.N + 1, 256)), dim3(256), 0, s, skeys, p.N,
                         static_cast<uint32_t>(p.T) + 1u, seg);
      if (p.has_probs) {
        if (p.pelt == 4)
          hipLaunchKernelGGL(padded_probs_kernel<uint32_t>, dim3(g), dim3(256), 0, s, sI, static_cast<int32_t>(p.T),
                             p.N, static_cast<const uint32_t*>(d->probs), p.E, p.C, static_cast<uint32_t*>(pprobs));
        else
          hipLaunchKernelGGL(padded_probs_kernel<uint16_t>, dim3(g), dim3(256), 0, s, sI, static_cast<int32_t>(p.T),
                             p.N, static_cast<const uint16_t*>(d->probs), p.E, p.C, static_cast<uint16_t*>(pprobs));
      }
    }
    ra.seg = seg;
    ra.order = order;
    ra.w = pprobs;
    const int mode = p.has_probs ? kPadW : kPad;
    if (!launch_reduce(ra, d->dtype, d->probs_dtype, mode, shape, p.T, s, d->ev_reduce_begin, d->ev_reduce_end))
      return FFNWB_ERR_RUNTIME;
  }
  return hipGetLastError() == hipSuccess ? FFNWB_OK : FFNWB_ERR_RUNTIME;
}

}  // namespace ffnwb

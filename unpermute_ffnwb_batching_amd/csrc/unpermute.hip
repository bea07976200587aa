// MoE token unpermute with routing map on gfx950 (MoeTokenUnpermuteWithRoutingMap article,
// "Function description and formulas", branches 1-4; "Kernel implementation").
//
// Non-padded mode (branches 2 and 4):
//   [probs]  probs compaction: stable counting sort of the non-zero routing-map entries
//            j = t*E + e by expert e (rank, scan, scatter) -> permute_probs, zero-padded;
//   reduce:  one workgroup per token gathers its topK slots' permuted rows and sums
//            x * w in FP32 (slot order), one RNE store;
//   [aux]    out_index / permute_token_id: stable sort of the slots by sortedIndices+1
//            (LSD passes when the row count exceeds one pass's bucket budget).
// Padded mode (branches 1 and 3):
//   invert:  stable counting sort of the capacity entries by token id (rank, scan,
//            scatter -> out_index, permute_token_id, permute_probs, per-token segments);
//   reduce:  one workgroup per token sums its segment's rows in ascending row order.
// No atomics anywhere, so every output is deterministic.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <type_traits>

#include "internal.hpp"
#include "sort_engine.hpp"

namespace ffnwb {

enum ReduceMode { kNonPad = 0, kNonPadW2 = 1, kNonPadW1 = 2, kPad = 3, kPadW = 4 };

struct ReduceArgs {
  const uint8_t* x;
  int64_t rows, H, T;
  const int32_t* sI;     // non-padded: slot -> permuted row
  int32_t K;
  const uint32_t* seg;   // padded: token segments of the sorted order
  const int32_t* order;  // padded: sorted position -> permuted row (out_index)
  const void* w;         // permute_probs (weights), probs element type
  uint8_t* out;
};

// One workgroup per token; each thread owns CPT 16-byte chunks of the hidden dimension
// (or single elements when rows are not 16-byte multiples).  Every wave fetches the
// token's entry list itself, one entry per lane with a single coalesced load, and marks
// the valid ones with a ballot; it then walks the valid entries in ascending order, 8 at
// a time, broadcasting each row index with readlane so that the 8 x CPT row loads of a
// batch are all in flight before the first one is used.  The weight of each entry is
// gathered per lane before the row loads and read back with readlane after them.
template <class TT, class TW, int MODE, int CPT>
__global__ __launch_bounds__(1024) void unpermute_reduce_kernel(ReduceArgs a) {
  constexpr bool kPadded = MODE >= kPad;
  constexpr bool kHasW = (MODE == kNonPadW2) || (MODE == kNonPadW1) || (MODE == kPadW);
  constexpr int VE = Chunk<TT>::kElems;
  constexpr int B = 8;
  const int64_t t = blockIdx.x;
  const uint32_t lane = lane_id();
  int64_t ebase, nent;
  if (kPadded) {
    ebase = uniform64(static_cast<int64_t>(a.seg[t]));
    nent = uniform64(static_cast<int64_t>(a.seg[t + 1])) - ebase;
  } else {
    ebase = t * a.K;
    nent = a.K;
  }
  const int64_t chunks = a.H * TT::kBytes / 16;
  const u32x4* __restrict__ x4 = reinterpret_cast<const u32x4*>(a.x);
  u32x4* __restrict__ o4 = reinterpret_cast<u32x4*>(a.out);
  for (int64_t c0 = 0; c0 < chunks; c0 += static_cast<int64_t>(CPT) * blockDim.x) {
    int64_t cidx[CPT];
    bool cok[CPT];
    float acc[CPT][VE];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      cidx[i] = c0 + threadIdx.x + static_cast<int64_t>(i) * blockDim.x;
      cok[i] = cidx[i] < chunks;
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[i][e] = 0.0f;
    }
    for (int64_t g = 0; g < nent; g += kWave) {
      const int64_t k = g + lane;
      int32_t r = 0;
      bool ok = false;
      if (k < nent) {
        const int32_t idx = kPadded ? a.order[ebase + k] : a.sI[ebase + k];
        ok = kPadded || (idx >= 0 && idx < a.rows);
        r = idx;
      }
      float wl = 1.0f;
      if (kHasW && ok) wl = load_elem<TW>(a.w, MODE == kNonPadW1 ? ebase + k : static_cast<int64_t>(r));
      uint64_t vm = wave_ballot(ok);
      while (vm != 0) {
        int32_t rr[B];
        int lsel[B];
        int nb = 0;
#pragma unroll
        for (int u = 0; u < B; ++u) {
          rr[u] = 0;
          lsel[u] = 0;
          if (vm != 0) {
            const int l = static_cast<int>(__builtin_ctzll(vm));
            vm &= vm - 1;
            lsel[u] = l;
            rr[u] = __builtin_amdgcn_readlane(r, l);
            nb = u + 1;
          }
        }
        u32x4 xv[B][CPT];
#pragma unroll
        for (int u = 0; u < B; ++u) {
          if (u < nb) {
#pragma unroll
            for (int i = 0; i < CPT; ++i)
              if (cok[i]) xv[u][i] = __builtin_nontemporal_load(x4 + static_cast<int64_t>(rr[u]) * chunks + cidx[i]);
          }
        }
#pragma unroll
        for (int u = 0; u < B; ++u) {
          if (u < nb) {
            const float w = kHasW ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), lsel[u])) : 1.0f;
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
              if (!cok[i]) continue;
              float f[VE];
              Chunk<TT>::widen(xv[u][i], f);
#pragma unroll
              for (int e = 0; e < VE; ++e) acc[i][e] = kHasW ? acc[i][e] + f[e] * w : acc[i][e] + f[e];
            }
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      if (cok[i]) o4[t * chunks + cidx[i]] = Chunk<TT>::narrow(acc[i]);
  }
}

// Element-wise variant for rows that are not a multiple of 16 bytes (or misaligned).
template <class TT, class TW, int MODE>
__global__ __launch_bounds__(1024) void unpermute_reduce_elem_kernel(ReduceArgs a) {
  constexpr bool kPadded = MODE >= kPad;
  constexpr bool kHasW = (MODE == kNonPadW2) || (MODE == kNonPadW1) || (MODE == kPadW);
  const int64_t t = blockIdx.x;
  int64_t ebase, nent;
  if (kPadded) {
    ebase = uniform64(static_cast<int64_t>(a.seg[t]));
    nent = uniform64(static_cast<int64_t>(a.seg[t + 1])) - ebase;
  } else {
    ebase = t * a.K;
    nent = a.K;
  }
  for (int64_t h = threadIdx.x; h < a.H; h += blockDim.x) {
    float acc = 0.0f;
    for (int64_t k = 0; k < nent; ++k) {
      const int64_t idx = kPadded ? a.order[ebase + k] : a.sI[ebase + k];
      if (!kPadded && !(idx >= 0 && idx < a.rows)) continue;
      const float f = load_elem<TT>(a.x, idx * a.H + h);
      if (kHasW) {
        const float w = load_elem<TW>(a.w, MODE == kNonPadW1 ? ebase + k : idx);
        acc = acc + f * w;
      } else {
        acc = acc + f;
      }
    }
    store_elem<TT>(a.out, t * a.H + h, acc);
  }
}

// Probs compaction (non-padded with probs): permute_probs lists probs[t, e] for the
// non-zero routing-map entries in expert-major order, i.e. a stable counting sort of
// the entries t*E + e by e.  The map is cut into tiles of kMaskTile tokens; thread e of
// a tile's workgroup walks column e of the tile, so within a column the tile's entries
// are already in token order and their rank is a running count.
constexpr int kMaskTile = 32;

// hist[tile*E + e] = number of non-zero map entries of column e in the tile.
__global__ __launch_bounds__(256) void mask_count_kernel(const uint8_t* __restrict__ map, int64_t T, int32_t E,
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

// permute_probs[start[e] + off[tile*E + e] + running count] = probs[t, e]; entries at
// positions >= N are dropped; positions from start[E] (the number of non-zero entries)
// up to N get 0.
template <typename P>
__global__ __launch_bounds__(256) void mask_scatter_kernel(const uint8_t* __restrict__ map,
                                                           const P* __restrict__ probs, int64_t T, int32_t E,
                                                           const uint32_t* __restrict__ off,
                                                           const uint32_t* __restrict__ start,
                                                           P* __restrict__ pp, int64_t N) {
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kMaskTile;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    uint32_t pos = start[e] + off[static_cast<int64_t>(blockIdx.x) * E + e];
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
  const uint32_t filled = start[E];
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < N;
       g += static_cast<int64_t>(gridDim.x) * blockDim.x)
    if (g >= filled) pp[g] = P(0);
}

// Padded inversion, single pass: out_index / permute_token_id at the sorted position, and
// the capacity entry's prob permute_probs[j] = probs[sI[j], j / C] (0 for invalid tokens).
template <typename P>
__global__ __launch_bounds__(256) void padded_scatter_kernel(const int32_t* __restrict__ sI, int32_t T,
                                                             const uint32_t* __restrict__ packed,
                                                             const uint32_t* __restrict__ off,
                                                             const uint32_t* __restrict__ start, int nb,
                                                             int tile_shift, int64_t n,
                                                             int32_t* __restrict__ out_index,
                                                             int32_t* __restrict__ token_out,
                                                             const P* __restrict__ probs, int64_t E, int64_t C,
                                                             P* __restrict__ pp) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j >= n) return;
  const int32_t v = sI[j];
  uint32_t pos, dig;
  if (placed_position(packed, off, start, nb, tile_shift, j, pos, dig)) {
    out_index[pos] = static_cast<int32_t>(j);
    if (token_out != nullptr) token_out[pos] = v;
  }
  if (pp != nullptr) pp[j] = (v >= 0 && v < T) ? probs[static_cast<int64_t>(v) * E + j / C] : P(0);
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
                       p.nb, packed, hist, p.nt, tile_err);
  else
    hipLaunchKernelGGL((sort_rank_kernel<16, KS>), dim3(p.nt), dim3(kRankThreads), lds, s, ks, p.n, p.shift,
                       p.nbits, p.nb, packed, hist, p.nt, tile_err);
}

static void launch_scan(const SortPass& p, uint32_t* hist, uint32_t* start, uint32_t* total, hipStream_t s) {
  ScanTail none{nullptr, 0, nullptr, nullptr, nullptr};
  const size_t lds = scan_lds_bytes(p.nb);
  allow_large_lds(reinterpret_cast<const void*>(&scan_hist_kernel), lds);
  hipLaunchKernelGGL(scan_hist_kernel, dim3(1), dim3(kScanThreads), lds, s, hist, p.nb, p.nt, start, total, none);
}

struct SortBufs {
  uint32_t* packed;
  uint32_t* hist;
  uint32_t* start;  // nb + 1 entries of the widest pass
  uint32_t* kA; uint32_t* vA; uint32_t* kB; uint32_t* vB;
};

// Runs every pass but the scatter of the last one; returns the keys/values of the last
// pass's input (nullptr for a single pass, whose input is the key source itself).
template <class KS>
static void run_passes_but_last_scatter(const SortPlan& sp, KS ks0, const SortBufs& b, const uint32_t** keys_in,
                                        const uint32_t** vals_in, hipStream_t s) {
  const uint32_t* kin = nullptr;
  const uint32_t* vin = nullptr;
  uint32_t* kout = b.kA;
  uint32_t* vout = b.vA;
  for (int i = 0; i < sp.npasses; ++i) {
    const SortPass& p = sp.pass[i];
    if (i == 0) launch_rank(p, ks0, b.packed, b.hist, nullptr, s);
    else launch_rank(p, KeyArray{kin}, b.packed, b.hist, nullptr, s);
    launch_scan(p, b.hist, b.start, nullptr, s);
    if (i == sp.npasses - 1) break;
    const unsigned g = grid_for(p.n, 256);
    if (i == 0)
      hipLaunchKernelGGL((lsd_scatter_kernel<KS, true, 0>), dim3(g), dim3(256), 0, s, ks0, vin, b.packed, b.hist,
                         b.start, p.nb, p.tile_shift, p.n, kout, vout, static_cast<int32_t*>(nullptr),
                         static_cast<int32_t*>(nullptr), static_cast<const int32_t*>(nullptr), 0);
    else
      hipLaunchKernelGGL((lsd_scatter_kernel<KeyArray, false, 0>), dim3(g), dim3(256), 0, s, KeyArray{kin}, vin,
                         b.packed, b.hist, b.start, p.nb, p.tile_shift, p.n, kout, vout, static_cast<int32_t*>(nullptr),
                         static_cast<int32_t*>(nullptr), static_cast<const int32_t*>(nullptr), 0);
    kin = kout;
    vin = vout;
    kout = (kout == b.kA) ? b.kB : b.kA;
    vout = (vout == b.vA) ? b.vB : b.vA;
  }
  *keys_in = kin;
  *vals_in = vin;
}

// A library-owned stream per device on which the non-padded auxiliary sort runs, forked
// from and joined back to the caller's stream with events, so that it overlaps the probs
// compaction and the gather-reduce (it depends only on sortedIndices).  Created on first
// use at the default priority; the mutex keeps each fork's record/wait pair together.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr;
  hipEvent_t join = nullptr;
  bool failed = false;
};
constexpr int kMaxDevices = 64;
static std::mutex g_side_mu;
static SideStream g_side[kMaxDevices];

static SideStream* side_stream_for(hipStream_t caller) {
  int dev = 0;
  if (caller != nullptr) dev = hipGetStreamDeviceId(caller);
  else if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  SideStream& ss = g_side[dev];
  if (ss.stream == nullptr && !ss.failed) {
    int cur = 0;
    (void)hipGetDevice(&cur);
    const bool switch_dev = cur != dev;
    if (switch_dev) (void)hipSetDevice(dev);
    if (hipStreamCreateWithFlags(&ss.stream, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess) {
      ss.failed = true;
      ss.stream = nullptr;
    }
    if (switch_dev) (void)hipSetDevice(cur);
  }
  return ss.failed ? nullptr : &ss;
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
      p->mask_tiles = (p->T + kMaskTile - 1) / kMaskTile;
      c.take<uint32_t>(static_cast<size_t>(p->E) * p->mask_tiles);           // histogram
      c.take<uint32_t>(static_cast<size_t>(p->E) + 1);                        // column starts
      if (d->permute_probs == nullptr) c.take<uint8_t>(static_cast<size_t>(p->N) * p->pelt);
    }
    p->need_aux = d->out_index != nullptr || d->permute_token_id != nullptr;
    if (p->need_aux && p->N > 0) {
      p->sort = make_sort_plan(p->N, static_cast<uint64_t>(p->rows) + 1);
      c.take<uint32_t>(p->N);
      c.take<uint32_t>(p->sort.hist_words);
      c.take<uint32_t>(static_cast<size_t>(p->sort.max_nb) + 1);
      if (p->sort.npasses > 1)
        for (int i = 0; i < 4; ++i) c.take<uint32_t>(p->N);
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
    p->sort = make_sort_plan(p->N, static_cast<uint64_t>(p->T) + 1);
    c.take<uint32_t>(p->N);                                // packed
    c.take<uint32_t>(p->sort.hist_words);                  // histogram
    c.take<uint32_t>(static_cast<size_t>(p->sort.max_nb) + 1);  // digit starts of a pass
    c.take<uint32_t>(static_cast<size_t>(p->T) + 2);       // token segments
    if (d->out_index == nullptr) c.take<int32_t>(p->N);    // sorted order for the reduce
    if (has_probs && d->permute_probs == nullptr) c.take<uint8_t>(static_cast<size_t>(p->N) * p->pelt);
    if (p->sort.npasses > 1)
      for (int i = 0; i < 5; ++i) c.take<uint32_t>(p->N);
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

template <class TT, class TW, int MODE>
static void launch_reduce_t(const ReduceArgs& ra, const ReduceShape& sh, int64_t T, hipStream_t s) {
  if (T == 0) return;
  const dim3 grid(static_cast<unsigned>(T)), block(sh.threads);
  switch (sh.cpt) {
    case 0: hipLaunchKernelGGL((unpermute_reduce_elem_kernel<TT, TW, MODE>), grid, block, 0, s, ra); break;
    case 1: hipLaunchKernelGGL((unpermute_reduce_kernel<TT, TW, MODE, 1>), grid, block, 0, s, ra); break;
    case 2: hipLaunchKernelGGL((unpermute_reduce_kernel<TT, TW, MODE, 2>), grid, block, 0, s, ra); break;
    default: hipLaunchKernelGGL((unpermute_reduce_kernel<TT, TW, MODE, 4>), grid, block, 0, s, ra); break;
  }
}

template <class TT, class TW>
static void launch_reduce_w(const ReduceArgs& ra, int mode, const ReduceShape& sh, int64_t T, hipStream_t s) {
  switch (mode) {
    case kNonPad: launch_reduce_t<TT, TW, kNonPad>(ra, sh, T, s); break;
    case kNonPadW2: launch_reduce_t<TT, TW, kNonPadW2>(ra, sh, T, s); break;
    case kNonPadW1: launch_reduce_t<TT, TW, kNonPadW1>(ra, sh, T, s); break;
    case kPad: launch_reduce_t<TT, TW, kPad>(ra, sh, T, s); break;
    default: launch_reduce_t<TT, TW, kPadW>(ra, sh, T, s); break;
  }
}

static void launch_reduce(const ReduceArgs& ra, int dtype, int pdtype, int mode, const ReduceShape& sh, int64_t T,
                          hipStream_t s) {
  if (dtype == FFNWB_DT_FP16) launch_reduce_w<TF16, TF16>(ra, mode, sh, T, s);
  else if (dtype == FFNWB_DT_FP32) launch_reduce_w<TF32, TF32>(ra, mode, sh, T, s);
  else if (pdtype == FFNWB_DT_FP32) launch_reduce_w<TBF16, TF32>(ra, mode, sh, T, s);
  else launch_reduce_w<TBF16, TBF16>(ra, mode, sh, T, s);
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

  if (!p.padded) {
    // workspace regions, in the order plan_unpermute sized them
    const int nt = static_cast<int>(p.mask_tiles);
    uint32_t* mhist = nullptr;
    uint32_t* cstart = nullptr;
    if (p.has_probs) {
      mhist = c.take<uint32_t>(static_cast<size_t>(p.E) * nt);
      cstart = c.take<uint32_t>(static_cast<size_t>(p.E) + 1);
      if (pprobs == nullptr) pprobs = c.take<uint8_t>(static_cast<size_t>(p.N) * p.pelt);
    }
    SortBufs b{};
    const bool aux = p.need_aux && p.N > 0;
    if (aux) {
      b.packed = c.take<uint32_t>(p.N);
      b.hist = c.take<uint32_t>(p.sort.hist_words);
      b.start = c.take<uint32_t>(static_cast<size_t>(p.sort.max_nb) + 1);
      if (p.sort.npasses > 1) {
        b.kA = c.take<uint32_t>(p.N); b.vA = c.take<uint32_t>(p.N);
        b.kB = c.take<uint32_t>(p.N); b.vB = c.take<uint32_t>(p.N);
      }
    }
    // auxiliary order (out_index / permute_token_id) on the side stream
    SideStream* side = nullptr;
    if (aux) {
      std::lock_guard<std::mutex> lock(g_side_mu);
      side = side_stream_for(s);
      hipStream_t as = s;
      if (side != nullptr && hipEventRecord(side->fork, s) == hipSuccess &&
          hipStreamWaitEvent(side->stream, side->fork, 0) == hipSuccess) {
        as = side->stream;
      } else {
        side = nullptr;
      }
      KeyNonPadded ks{sI, static_cast<int32_t>(p.rows)};
      const uint32_t *kin, *vin;
      run_passes_but_last_scatter(p.sort, ks, b, &kin, &vin, as);
      const SortPass& last = p.sort.pass[p.sort.npasses - 1];
      const unsigned g = grid_for(p.N, 256);
      if (p.sort.npasses == 1)
        hipLaunchKernelGGL((lsd_scatter_kernel<KeyNonPadded, true, 1>), dim3(g), dim3(256), 0, as, ks,
                           static_cast<const uint32_t*>(nullptr), b.packed, b.hist, b.start, last.nb,
                           last.tile_shift, p.N,
                           static_cast<uint32_t*>(nullptr), static_cast<uint32_t*>(nullptr), d->out_index,
                           d->permute_token_id, sI, static_cast<int32_t>(p.K));
      else
        hipLaunchKernelGGL((lsd_scatter_kernel<KeyArray, false, 1>), dim3(g), dim3(256), 0, as, KeyArray{kin}, vin,
                           b.packed, b.hist, b.start, last.nb, last.tile_shift, p.N,
                           static_cast<uint32_t*>(nullptr),
                           static_cast<uint32_t*>(nullptr), d->out_index, d->permute_token_id, sI,
                           static_cast<int32_t>(p.K));
      if (side != nullptr && hipEventRecord(side->join, side->stream) != hipSuccess) return FFNWB_ERR_RUNTIME;
    }
    // probs compaction, then the gather-reduce, on the caller's stream
    if (p.has_probs && nt > 0) {
      const int th = static_cast<int>(p.E >= 256 ? 256 : (p.E + 63) / 64 * 64);
      hipLaunchKernelGGL(mask_count_kernel, dim3(nt), dim3(th), 0, s, d->routing_map, p.T,
                         static_cast<int32_t>(p.E), mhist);
      SortPass mp;
      mp.nb = static_cast<int>(p.E);
      mp.nt = nt;
      launch_scan(mp, mhist, cstart, nullptr, s);
      if (p.pelt == 4)
        hipLaunchKernelGGL(mask_scatter_kernel<uint32_t>, dim3(nt), dim3(th), 0, s, d->routing_map,
                           static_cast<const uint32_t*>(d->probs), p.T, static_cast<int32_t>(p.E), mhist, cstart,
                           static_cast<uint32_t*>(pprobs), p.N);
      else
        hipLaunchKernelGGL(mask_scatter_kernel<uint16_t>, dim3(nt), dim3(th), 0, s, d->routing_map,
                           static_cast<const uint16_t*>(d->probs), p.T, static_cast<int32_t>(p.E), mhist, cstart,
                           static_cast<uint16_t*>(pprobs), p.N);
    }
    ra.sI = sI;
    ra.K = static_cast<int32_t>(p.K);
    ra.w = pprobs;
    const int mode = !p.has_probs ? kNonPad : (d->weight_index == 1 ? kNonPadW1 : kNonPadW2);
    if (!record_event(d->ev_reduce_begin, s)) return FFNWB_ERR_RUNTIME;
    launch_reduce(ra, d->dtype, d->probs_dtype, mode, shape, p.T, s);
    if (!record_event(d->ev_reduce_end, s)) return FFNWB_ERR_RUNTIME;
    if (side != nullptr && hipStreamWaitEvent(s, side->join, 0) != hipSuccess) return FFNWB_ERR_RUNTIME;
  } else {
    SortBufs b{};
    b.packed = c.take<uint32_t>(p.N);
    b.hist = c.take<uint32_t>(p.sort.hist_words);
    b.start = c.take<uint32_t>(static_cast<size_t>(p.sort.max_nb) + 1);
    uint32_t* seg = c.take<uint32_t>(static_cast<size_t>(p.T) + 2);
    int32_t* order = d->out_index ? d->out_index : c.take<int32_t>(p.N);
    if (p.has_probs && pprobs == nullptr) pprobs = c.take<uint8_t>(static_cast<size_t>(p.N) * p.pelt);
    if (!p.has_probs) pprobs = nullptr;  // nothing to gather without probs
    uint32_t* skeys = nullptr;
    if (p.sort.npasses > 1) {
      b.kA = c.take<uint32_t>(p.N); b.vA = c.take<uint32_t>(p.N);
      b.kB = c.take<uint32_t>(p.N); b.vB = c.take<uint32_t>(p.N);
      skeys = c.take<uint32_t>(p.N);
    }
    KeyPadded ks{sI, static_cast<int32_t>(p.T)};
    const unsigned g = grid_for(p.N, 256);
    if (p.N == 0) {
      hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for(p.T + 2, 256)), dim3(256), 0, s, seg, p.T + 2, 0u);
    } else if (p.sort.npasses == 1) {
      const SortPass& ps = p.sort.pass[0];
      launch_rank(ps, ks, b.packed, b.hist, nullptr, s);
      launch_scan(ps, b.hist, seg, nullptr, s);  // digit starts = token segments
      if (p.pelt == 4)
        hipLaunchKernelGGL(padded_scatter_kernel<uint32_t>, dim3(g), dim3(256), 0, s, sI, static_cast<int32_t>(p.T),
                           b.packed, b.hist, seg, ps.nb, ps.tile_shift, p.N, order, d->permute_token_id,
                           static_cast<const uint32_t*>(d->probs), p.E, p.C, static_cast<uint32_t*>(pprobs));
      else
        hipLaunchKernelGGL(padded_scatter_kernel<uint16_t>, dim3(g), dim3(256), 0, s, sI, static_cast<int32_t>(p.T),
                           b.packed, b.hist, seg, ps.nb, ps.tile_shift, p.N, order, d->permute_token_id,
                           static_cast<const uint16_t*>(d->probs), p.E, p.C, static_cast<uint16_t*>(pprobs));
    } else {
      const uint32_t *kin, *vin;
      run_passes_but_last_scatter(p.sort, ks, b, &kin, &vin, s);
      const SortPass& last = p.sort.pass[p.sort.npasses - 1];
      hipLaunchKernelGGL((lsd_scatter_kernel<KeyArray, false, 2>), dim3(g), dim3(256), 0, s, KeyArray{kin}, vin,
                         b.packed, b.hist, b.start, last.nb, last.tile_shift, p.N, skeys,
                         static_cast<uint32_t*>(nullptr),
                         order, d->permute_token_id, sI, 0);
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
    if (!record_event(d->ev_reduce_begin, s)) return FFNWB_ERR_RUNTIME;
    launch_reduce(ra, d->dtype, d->probs_dtype, mode, shape, p.T, s);
    if (!record_event(d->ev_reduce_end, s)) return FFNWB_ERR_RUNTIME;
  }
  return hipGetLastError() == hipSuccess ? FFNWB_OK : FFNWB_ERR_RUNTIME;
}

}  // namespace ffnwb

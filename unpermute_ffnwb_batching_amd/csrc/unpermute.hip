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

// One workgroup per token.  Each thread owns 16-byte chunks of the hidden dimension
// (VEC) or single elements; the token's (row, weight) entries are uniform across the
// workgroup and are fetched 8 at a time so that 8 row loads are in flight per thread.
template <class TT, class TW, int MODE, bool VEC>
__global__ __launch_bounds__(1024) void unpermute_reduce_kernel(ReduceArgs a) {
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
  constexpr int B = 8;
  if (VEC) {
    constexpr int VE = Chunk<TT>::kElems;
    const int64_t chunks = a.H * TT::kBytes / 16;
    const u32x4* __restrict__ x4 = reinterpret_cast<const u32x4*>(a.x);
    u32x4* __restrict__ o4 = reinterpret_cast<u32x4*>(a.out);
    for (int64_t c = threadIdx.x; c < chunks; c += blockDim.x) {
      float acc[VE];
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[e] = 0.0f;
      for (int64_t k0 = 0; k0 < nent; k0 += B) {
        int64_t r[B];
        float w[B];
        bool ok[B];
#pragma unroll
        for (int u = 0; u < B; ++u) {
          const int64_t k = k0 + u;
          ok[u] = k < nent;
          r[u] = 0;
          w[u] = 1.0f;
          if (ok[u]) {
            const int64_t idx = kPadded ? a.order[ebase + k] : a.sI[ebase + k];
            if (!kPadded) ok[u] = idx >= 0 && idx < a.rows;
            r[u] = idx;
            if (ok[u] && kHasW) w[u] = load_elem<TW>(a.w, MODE == kNonPadW1 ? ebase + k : idx);
          }
        }
        u32x4 xv[B];
#pragma unroll
        for (int u = 0; u < B; ++u)
          if (ok[u]) xv[u] = x4[r[u] * chunks + c];
#pragma unroll
        for (int u = 0; u < B; ++u) {
          if (!ok[u]) continue;
          float f[VE];
          Chunk<TT>::widen(xv[u], f);
#pragma unroll
          for (int e = 0; e < VE; ++e) acc[e] = kHasW ? acc[e] + f[e] * w[u] : acc[e] + f[e];
        }
      }
      o4[t * chunks + c] = Chunk<TT>::narrow(acc);
    }
  } else {
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
}

// Probs compaction scatter: permute_probs[pos(j)] = probs[j] for placed entries, then
// zero from the number of placed entries up to N (entries beyond N are dropped).
template <typename P>
__global__ __launch_bounds__(256) void mask_scatter_kernel(const uint32_t* __restrict__ packed,
                                                           const uint32_t* __restrict__ off, int nt, int tile_shift,
                                                           int64_t n, const P* __restrict__ probs,
                                                           P* __restrict__ pp, int64_t N,
                                                           const uint32_t* __restrict__ total) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j < n) {
    uint32_t pos, dig;
    if (placed_position(packed, off, nt, tile_shift, j, pos, dig) && pos < N) pp[pos] = probs[j];
  }
  if (j < N && j >= static_cast<int64_t>(*total)) pp[j] = P(0);
}

// Padded inversion, single pass: out_index / permute_token_id at the sorted position, and
// the capacity entry's prob permute_probs[j] = probs[sI[j], j / C] (0 for invalid tokens).
template <typename P>
__global__ __launch_bounds__(256) void padded_scatter_kernel(const int32_t* __restrict__ sI, int32_t T,
                                                             const uint32_t* __restrict__ packed,
                                                             const uint32_t* __restrict__ off, int nt,
                                                             int tile_shift, int64_t n,
                                                             int32_t* __restrict__ out_index,
                                                             int32_t* __restrict__ token_out,
                                                             const P* __restrict__ probs, int64_t E, int64_t C,
                                                             P* __restrict__ pp) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j >= n) return;
  const int32_t v = sI[j];
  uint32_t pos, dig;
  if (placed_position(packed, off, nt, tile_shift, j, pos, dig)) {
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

static void launch_scan(const SortPass& p, uint32_t* hist, uint32_t* total, uint32_t* bucket_start, hipStream_t s) {
  ScanTail none{nullptr, 0, nullptr, nullptr, nullptr};
  hipLaunchKernelGGL(scan_hist_kernel, dim3(1), dim3(kScanThreads), 0, s, hist,
                     static_cast<int64_t>(p.nb) * p.nt, total, bucket_start, p.nb, p.nt, none);
}

struct SortBufs {
  uint32_t* packed;
  uint32_t* hist;
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
    launch_scan(p, b.hist, nullptr, nullptr, s);
    if (i == sp.npasses - 1) break;
    const unsigned g = grid_for(p.n, 256);
    if (i == 0)
      hipLaunchKernelGGL((lsd_scatter_kernel<KS, true, 0>), dim3(g), dim3(256), 0, s, ks0, vin, b.packed, b.hist,
                         p.nt, p.tile_shift, p.n, kout, vout, static_cast<int32_t*>(nullptr),
                         static_cast<int32_t*>(nullptr), static_cast<const int32_t*>(nullptr), 0);
    else
      hipLaunchKernelGGL((lsd_scatter_kernel<KeyArray, false, 0>), dim3(g), dim3(256), 0, s, KeyArray{kin}, vin,
                         b.packed, b.hist, p.nt, p.tile_shift, p.n, kout, vout, static_cast<int32_t*>(nullptr),
                         static_cast<int32_t*>(nullptr), static_cast<const int32_t*>(nullptr), 0);
    kin = kout;
    vin = vout;
    kout = (kout == b.kA) ? b.kB : b.kA;
    vout = (vout == b.vA) ? b.vB : b.vA;
  }
  *keys_in = kin;
  *vals_in = vin;
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
      const int64_t n0 = p->T * p->E;
      p->mask_pass = make_pass(n0, static_cast<int>(p->E), bits_for(static_cast<uint64_t>(p->E - 1)), 0);
      c.take<uint32_t>(n0);                                                   // packed
      c.take<uint32_t>(static_cast<size_t>(p->E) * p->mask_pass.nt);          // histogram
      c.take<uint32_t>(1);                                                    // compacted count
      if (d->permute_probs == nullptr) c.take<uint8_t>(static_cast<size_t>(p->N) * p->pelt);
    }
    p->need_aux = d->out_index != nullptr || d->permute_token_id != nullptr;
    if (p->need_aux && p->N > 0) {
      p->sort = make_sort_plan(p->N, static_cast<uint64_t>(p->rows) + 1);
      c.take<uint32_t>(p->N);
      c.take<uint32_t>(p->sort.hist_words);
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
    c.take<uint32_t>(static_cast<size_t>(p->T) + 2);       // token segments
    if (d->out_index == nullptr) c.take<int32_t>(p->N);    // sorted order for the reduce
    if (has_probs && d->permute_probs == nullptr) c.take<uint8_t>(static_cast<size_t>(p->N) * p->pelt);
    if (p->sort.npasses > 1)
      for (int i = 0; i < 5; ++i) c.take<uint32_t>(p->N);
  }
  p->ws_bytes = c.off;
  return FFNWB_OK;
}

template <class TT, class TW, int MODE>
static void launch_reduce_t(const ReduceArgs& ra, bool vec, int64_t T, int threads, hipStream_t s) {
  if (T == 0) return;
  if (vec)
    hipLaunchKernelGGL((unpermute_reduce_kernel<TT, TW, MODE, true>), dim3(static_cast<unsigned>(T)), dim3(threads),
                       0, s, ra);
  else
    hipLaunchKernelGGL((unpermute_reduce_kernel<TT, TW, MODE, false>), dim3(static_cast<unsigned>(T)),
                       dim3(threads), 0, s, ra);
}

template <class TT, class TW>
static void launch_reduce_w(const ReduceArgs& ra, int mode, bool vec, int64_t T, int threads, hipStream_t s) {
  switch (mode) {
    case kNonPad: launch_reduce_t<TT, TW, kNonPad>(ra, vec, T, threads, s); break;
    case kNonPadW2: launch_reduce_t<TT, TW, kNonPadW2>(ra, vec, T, threads, s); break;
    case kNonPadW1: launch_reduce_t<TT, TW, kNonPadW1>(ra, vec, T, threads, s); break;
    case kPad: launch_reduce_t<TT, TW, kPad>(ra, vec, T, threads, s); break;
    default: launch_reduce_t<TT, TW, kPadW>(ra, vec, T, threads, s); break;
  }
}

static void launch_reduce(const ReduceArgs& ra, int dtype, int pdtype, int mode, bool vec, int64_t T, int threads,
                          hipStream_t s) {
  if (dtype == FFNWB_DT_FP16) launch_reduce_w<TF16, TF16>(ra, mode, vec, T, threads, s);
  else if (dtype == FFNWB_DT_FP32) launch_reduce_w<TF32, TF32>(ra, mode, vec, T, threads, s);
  else if (pdtype == FFNWB_DT_FP32) launch_reduce_w<TBF16, TF32>(ra, mode, vec, T, threads, s);
  else launch_reduce_w<TBF16, TBF16>(ra, mode, vec, T, threads, s);
}

template <typename P>
static void launch_mask_scatter(const UnpermutePlan& p, const uint32_t* packed, const uint32_t* hist,
                                const void* probs, void* pp, const uint32_t* total, hipStream_t s) {
  const int64_t n0 = p.T * p.E;
  const int64_t g = n0 > p.N ? n0 : p.N;
  if (g == 0) return;
  hipLaunchKernelGGL(mask_scatter_kernel<P>, dim3(grid_for(g, 256)), dim3(256), 0, s, packed, hist, p.mask_pass.nt,
                     p.mask_pass.tile_shift, n0, static_cast<const P*>(probs), static_cast<P*>(pp), p.N, total);
}

int launch_unpermute(const moe_unpermute_desc* d, const UnpermutePlan& p, void* ws, hipStream_t s) {
  Carve c;
  c.base = static_cast<char*>(ws);
  const int32_t* sI = d->sorted_indices;
  void* pprobs = d->permute_probs;
  const bool vec = ((p.H * p.elt) % 16 == 0) &&
                   ((reinterpret_cast<uintptr_t>(d->permuted_tokens) | reinterpret_cast<uintptr_t>(d->unpermuted_tokens)) % 16 == 0);
  const int64_t work = vec ? (p.H * p.elt / 16) : p.H;
  int threads = static_cast<int>(((work < 1024 ? work : 1024) + 63) / 64 * 64);
  if (threads < 64) threads = 64;

  ReduceArgs ra{};
  ra.x = static_cast<const uint8_t*>(d->permuted_tokens);
  ra.rows = p.rows;
  ra.H = p.H;
  ra.T = p.T;
  ra.out = static_cast<uint8_t*>(d->unpermuted_tokens);

  if (!p.padded) {
    if (p.has_probs) {
      const int64_t n0 = p.T * p.E;
      uint32_t* packed = c.take<uint32_t>(n0);
      uint32_t* hist = c.take<uint32_t>(static_cast<size_t>(p.E) * p.mask_pass.nt);
      uint32_t* total = c.take<uint32_t>(1);
      if (pprobs == nullptr) pprobs = c.take<uint8_t>(static_cast<size_t>(p.N) * p.pelt);
      if (n0 > 0) {
        launch_rank(p.mask_pass, KeyRoutingMap{d->routing_map, static_cast<int32_t>(p.E)}, packed, hist, nullptr, s);
        launch_scan(p.mask_pass, hist, total, nullptr, s);
      } else {
        hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(256), 0, s, total, int64_t{1}, 0u);
      }
      if (p.pelt == 4) launch_mask_scatter<uint32_t>(p, packed, hist, d->probs, pprobs, total, s);
      else launch_mask_scatter<uint16_t>(p, packed, hist, d->probs, pprobs, total, s);
    }
    ra.sI = sI;
    ra.K = static_cast<int32_t>(p.K);
    ra.w = pprobs;
    const int mode = !p.has_probs ? kNonPad : (d->weight_index == 1 ? kNonPadW1 : kNonPadW2);
    if (!record_event(d->ev_reduce_begin, s)) return FFNWB_ERR_RUNTIME;
    launch_reduce(ra, d->dtype, d->probs_dtype, mode, vec, p.T, threads, s);
    if (!record_event(d->ev_reduce_end, s)) return FFNWB_ERR_RUNTIME;
    if (p.need_aux && p.N > 0) {
      SortBufs b{};
      b.packed = c.take<uint32_t>(p.N);
      b.hist = c.take<uint32_t>(p.sort.hist_words);
      if (p.sort.npasses > 1) {
        b.kA = c.take<uint32_t>(p.N); b.vA = c.take<uint32_t>(p.N);
        b.kB = c.take<uint32_t>(p.N); b.vB = c.take<uint32_t>(p.N);
      }
      KeyNonPadded ks{sI, static_cast<int32_t>(p.rows)};
      const uint32_t *kin, *vin;
      run_passes_but_last_scatter(p.sort, ks, b, &kin, &vin, s);
      const SortPass& last = p.sort.pass[p.sort.npasses - 1];
      const unsigned g = grid_for(p.N, 256);
      if (p.sort.npasses == 1)
        hipLaunchKernelGGL((lsd_scatter_kernel<KeyNonPadded, true, 1>), dim3(g), dim3(256), 0, s, ks,
                           static_cast<const uint32_t*>(nullptr), b.packed, b.hist, last.nt, last.tile_shift, p.N,
                           static_cast<uint32_t*>(nullptr), static_cast<uint32_t*>(nullptr), d->out_index,
                           d->permute_token_id, sI, static_cast<int32_t>(p.K));
      else
        hipLaunchKernelGGL((lsd_scatter_kernel<KeyArray, false, 1>), dim3(g), dim3(256), 0, s, KeyArray{kin}, vin,
                           b.packed, b.hist, last.nt, last.tile_shift, p.N, static_cast<uint32_t*>(nullptr),
                           static_cast<uint32_t*>(nullptr), d->out_index, d->permute_token_id, sI,
                           static_cast<int32_t>(p.K));
    }
  } else {
    SortBufs b{};
    b.packed = c.take<uint32_t>(p.N);
    b.hist = c.take<uint32_t>(p.sort.hist_words);
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
      launch_scan(ps, b.hist, nullptr, seg, s);
      if (p.pelt == 4)
        hipLaunchKernelGGL(padded_scatter_kernel<uint32_t>, dim3(g), dim3(256), 0, s, sI, static_cast<int32_t>(p.T),
                           b.packed, b.hist, ps.nt, ps.tile_shift, p.N, order, d->permute_token_id,
                           static_cast<const uint32_t*>(d->probs), p.E, p.C, static_cast<uint32_t*>(pprobs));
      else
        hipLaunchKernelGGL(padded_scatter_kernel<uint16_t>, dim3(g), dim3(256), 0, s, sI, static_cast<int32_t>(p.T),
                           b.packed, b.hist, ps.nt, ps.tile_shift, p.N, order, d->permute_token_id,
                           static_cast<const uint16_t*>(d->probs), p.E, p.C, static_cast<uint16_t*>(pprobs));
    } else {
      const uint32_t *kin, *vin;
      run_passes_but_last_scatter(p.sort, ks, b, &kin, &vin, s);
      const SortPass& last = p.sort.pass[p.sort.npasses - 1];
      hipLaunchKernelGGL((lsd_scatter_kernel<KeyArray, false, 2>), dim3(g), dim3(256), 0, s, KeyArray{kin}, vin,
                         b.packed, b.hist, last.nt, last.tile_shift, p.N, skeys, static_cast<uint32_t*>(nullptr),
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
    launch_reduce(ra, d->dtype, d->probs_dtype, mode, vec, p.T, threads, s);
    if (!record_event(d->ev_reduce_end, s)) return FFNWB_ERR_RUNTIME;
  }
  return hipGetLastError() == hipSuccess ? FFNWB_OK : FFNWB_ERR_RUNTIME;
}

}  // namespace ffnwb

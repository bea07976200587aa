// Stable counting sort on CDNA4, used by every ordering step of the library:
//   - batching: slots keyed by (layer, expert)              (one pass, <= 8192 buckets)
//   - unpermute, padded: capacity entries keyed by token     (one pass while T+1 <= 20480)
//   - unpermute, non-padded: the auxiliary out_index ordering keyed by sortedIndices
//     (LSD passes when the key range is large)
//
// A pass over n elements splits them into tiles of 256*R consecutive elements, one
// 256-thread workgroup (4 waves) per tile.  Wave w owns the contiguous sub-range
// [w*64R, (w+1)*64R) of its tile and walks it in R rounds of 64 lanes.  In each round
// the lanes holding the same digit are found with one ballot per digit bit (no
// serialisation over distinct digits); the lowest such lane adds the group size to the
// wave's private LDS counter of that digit, and every lane's rank is the counter's old
// value plus the number of equal-digit lanes below it.  After a barrier, a per-digit
// prefix over the 4 waves turns the per-wave counters into per-wave bases and gives the
// tile's digit histogram, written tile-major (hist[tile*nb + digit], coalesced).
// One workgroup then turns each digit's column into a prefix over tiles (in place) and
// scans the digit totals into start[digit]; element j's output position is
// start[digit] + hist[tile*nb + digit] + rank: ties keep input order.
#pragma once

#include "device_common.hpp"

namespace ffnwb {

constexpr int kRankWaves = 4;
constexpr int kRankThreads = kRankWaves * kWave;  // 256
constexpr uint32_t kNoRank = 0xffffffffu;          // packed value of elements not placed
constexpr int kScanThreads = 1024;

// Per-element packed result of a ranking pass: digit in the high 16 bits, rank in tile low 16.
__device__ __forceinline__ uint32_t pack_rank(uint32_t digit, uint32_t rank) { return (digit << 16) | rank; }

// LDS words needed by the ranking kernels for `nb` buckets (u16 counters, 4 waves).
__host__ __device__ inline int rank_lds_stride(int nb) { return (nb + 1) & ~1; }
__host__ __device__ inline size_t rank_lds_bytes(int nb) {
  return static_cast<size_t>(kRankWaves) * rank_lds_stride(nb) * sizeof(uint16_t);
}

__device__ __forceinline__ void lds_zero_words(uint32_t* p, int words) {
  for (int i = threadIdx.x; i < words; i += blockDim.x) p[i] = 0u;
}

// Ranks R rounds of this wave's elements.  `wh` is the wave's private u16 counter array.
template <int R>
__device__ __forceinline__ void rank_rounds(const uint32_t (&dig)[R], const bool (&val)[R], int nbits,
                                            uint16_t* wh, uint32_t (&rank)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    uint64_t peers = wave_ballot(val[r]);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (dig[r] >> b) & 1u;
      const uint64_t m = wave_ballot(bit);
      peers &= bit ? m : ~m;
    }
    uint32_t base = 0;
    if (val[r]) base = wh[dig[r]];
    const uint32_t below = count_below(peers);
    if (val[r] && below == 0) wh[dig[r]] = static_cast<uint16_t>(base + static_cast<uint32_t>(__popcll(peers)));
    rank[r] = base + below;
    wave_lds_sync();
  }
}

// Inclusive scan of one value per lane across the calling wave.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

// K independent exclusive scans over a workgroup of NT threads, whose results are laid
// end to end: the K sequences are concatenated in order (sequence 0 first), so v[k] of
// thread i becomes the sum of all sequences before k plus sequence k's values of
// threads before i.  `lds` holds K * NT/64 + 1 words; total = sum of everything.
template <int NT, int K>
__device__ __forceinline__ void block_exscan_multi(uint32_t (&v)[K], uint32_t* lds, uint32_t& total) {
  constexpr int NW = NT / kWave;
  static_assert(K * NW <= kWave, "wave totals must fit one wave");
  const int lane = static_cast<int>(lane_id());
  const int w = threadIdx.x / kWave;
  uint32_t x[K];
#pragma unroll
  for (int k = 0; k < K; ++k) x[k] = wave_inclusive_scan(v[k], lane);
  if (lane == kWave - 1) {
#pragma unroll
    for (int k = 0; k < K; ++k) lds[k * NW + w] = x[k];
  }
  __syncthreads();
  if (w == 0) {
    const uint32_t y = lane < K * NW ? lds[lane] : 0u;
    const uint32_t inc = wave_inclusive_scan(y, lane);
    if (lane < K * NW) lds[lane] = inc - y;
    if (lane == kWave - 1) lds[K * NW] = inc;
  }
  __syncthreads();
  total = lds[K * NW];
#pragma unroll
  for (int k = 0; k < K; ++k) v[k] = lds[k * NW + w] + x[k] - v[k];
  __syncthreads();
}

// Exclusive scan over a workgroup of NT threads.  `lds` holds NT/64 + 1 words.
template <int NT>
__device__ __forceinline__ uint32_t block_exscan(uint32_t v, uint32_t* lds, uint32_t& total) {
  uint32_t a[1] = {v};
  block_exscan_multi<NT, 1>(a, lds, total);
  return a[0];
}

// ------------------------------------------------------------------ key sources
// Each returns the element's key and whether it takes part in the sort; `err` flags
// elements dropped because of an out-of-range id (batching only).  Callers pass an
// in-range index (clamped), and the sources load unconditionally, so that the loads of
// all rounds of a tile are in flight together instead of one round at a time.

// Padded unpermute: key = token id, entries outside [0, T) share the last bucket T.
struct KeyPadded {
  const int32_t* sI; int32_t T;
  __device__ uint32_t key(int64_t j, bool& valid, bool& err) const {
    const int32_t v = sI[j];
    valid = true; err = false;
    return (v >= 0 && v < T) ? static_cast<uint32_t>(v) : static_cast<uint32_t>(T);
  }
};

// Non-padded auxiliary order: key = sortedIndices + 1, invalid slots (outside [0, rows)) -> 0.
struct KeyNonPadded {
  const int32_t* sI; int32_t rows;
  __device__ uint32_t key(int64_t j, bool& valid, bool& err) const {
    const int32_t v = sI[j];
    valid = true; err = false;
    return (v >= 0 && v < rows) ? static_cast<uint32_t>(v) + 1u : 0u;
  }
};

// Later LSD passes: keys already materialised.
struct KeyArray {
  const uint32_t* keys;
  __device__ uint32_t key(int64_t j, bool& valid, bool& err) const { valid = true; err = false; return keys[j]; }
};

// ------------------------------------------------------------------ ranking pass
// packed[j] = pack_rank(digit, rank within tile) or kNoRank; hist_g[tile*nb + d] = count.
// tile_err[tile] = number of elements with err set (if tile_err != nullptr).
template <int R, class KS>
__global__ __launch_bounds__(kRankThreads) void sort_rank_kernel(KS ks, int64_t n, int shift, int nbits, int nb,
                                                                 uint32_t* __restrict__ packed,
                                                                 uint32_t* __restrict__ hist_g,
                                                                 uint32_t* __restrict__ tile_err) {
  extern __shared__ uint32_t lds_words[];
  __shared__ uint32_t err_w[kRankWaves];
  uint16_t* hist = reinterpret_cast<uint16_t*>(lds_words);
  const int nbp = rank_lds_stride(nb);
  lds_zero_words(lds_words, kRankWaves * nbp / 2);
  __syncthreads();

  const int w = uniform(static_cast<int>(threadIdx.x) / kWave);
  const uint32_t lane = lane_id();
  const int64_t base = static_cast<int64_t>(blockIdx.x) * (kRankThreads * R) + static_cast<int64_t>(w) * (kWave * R);
  const uint32_t dmask = (nbits >= 32) ? ~0u : ((1u << nbits) - 1u);
  uint32_t dig[R], rank[R];
  bool val[R], bad[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t j = base + r * kWave + lane;
    const bool in = j < n;
    bool v = false, e = false;
    const uint32_t key = ks.key(in ? j : n - 1, v, e);
    dig[r] = (key >> shift) & dmask;
    val[r] = v && in;
    bad[r] = e && in;
  }
  // the ballots come after every round's loads: a ballot between rounds keeps the next
  // round's loads from being issued before it
  uint32_t nerr = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) nerr += static_cast<uint32_t>(__popcll(wave_ballot(bad[r])));
  rank_rounds<R>(dig, val, nbits, hist + w * nbp, rank);
  if (lane == 0) err_w[w] = nerr;
  __syncthreads();
  for (int k = threadIdx.x; k < nb; k += kRankThreads) {
    uint32_t run = 0;
#pragma unroll
    for (int ww = 0; ww < kRankWaves; ++ww) {
      const uint32_t c = hist[ww * nbp + k];
      hist[ww * nbp + k] = static_cast<uint16_t>(run);
      run += c;
    }
    hist_g[static_cast<int64_t>(blockIdx.x) * nb + k] = run;
  }
  if (tile_err != nullptr && threadIdx.x == 0)
    tile_err[blockIdx.x] = err_w[0] + err_w[1] + err_w[2] + err_w[3];
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t j = base + r * kWave + lane;
    if (j < n) packed[j] = val[r] ? pack_rank(dig[r], rank[r] + hist[w * nbp + dig[r]]) : kNoRank;
  }
}

// ------------------------------------------------------------------ scan of the histogram
// One 1024-thread workgroup turns the tile-major histogram into per-digit prefixes over
// tiles, in place (h[t*nb + k] = elements of digit k in tiles before t), and writes
// start[k] = elements with a smaller digit (start[nb] = total).  Digit k's column is
// walked by consecutive threads for consecutive k (coalesced); when there are fewer
// digits than threads, each column is split into G tile segments walked in parallel and
// joined through LDS; when there are more, each thread walks several columns with their
// loads interleaved.  Column totals are kept in LDS and scanned in digit order.
// Optional tail for batching: compact group_list rows {k, count_k} for count_k > 0 then
// {0,0}, actual_token_num and err_count = sum of tile_err[0..nt).
struct ScanTail {
  int64_t* group_list;    // nullptr = no batching tail
  int64_t group_rows;
  int64_t* actual_token_num;
  int32_t* err_count;     // may be nullptr
  const uint32_t* tile_err;
};

constexpr int kScanMaxBuckets = 20480;  // digit totals in LDS: 80 KiB

// Sums (or, with `write`, overwrites with running prefixes starting at `base`) the cells
// h[t*nb + k] for t in [t0, t1), B loads in flight at a time (clamped, no branch).
template <int B = 16>  // wider batches measured slower: one CU's memory pipeline is the limit
__device__ __forceinline__ uint32_t walk_column(uint32_t* __restrict__ h, int nb, int k, int t0, int t1,
                                                bool write, uint32_t base) {
  uint32_t run = base;
  for (int t = t0; t < t1; t += B) {
    uint32_t c[B];
#pragma unroll
    for (int u = 0; u < B; ++u) c[u] = h[static_cast<int64_t>(min(t + u, t1 - 1)) * nb + k];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      if (t + u < t1) {
        if (write) h[static_cast<int64_t>(t + u) * nb + k] = run;
        run += c[u];
      }
    }
  }
  return run;
}

[[maybe_unused]] static __global__ __launch_bounds__(kScanThreads) void scan_hist_kernel(uint32_t* __restrict__ h, int nb, int nt,
                                                                        uint32_t* __restrict__ start,
                                                                        uint32_t* __restrict__ total_out,
                                                                        ScanTail tail) {
  extern __shared__ uint32_t tot[];  // [nb] digit totals, then [G][KW] segment sums
  __shared__ uint32_t wsum[kScanThreads / kWave + 1];
  const int tid = threadIdx.x;
  if (nb * 2 <= kScanThreads && nt >= 256) {
    // few digits, long columns: G segments per column
    const int KW = (nb + kWave - 1) / kWave * kWave;
    const int G = kScanThreads / KW;
    const int kk = tid % KW, g = tid / KW;
    const int S = (nt + G - 1) / G;
    const int t0 = min(nt, g * S), t1 = min(nt, t0 + S);
    uint32_t* seg = tot + nb;
    const bool act = g < G && kk < nb;
    const uint32_t sum = act ? walk_column(h, nb, kk, t0, t1, false, 0) : 0u;
    if (g < G) seg[g * KW + kk] = sum;
    __syncthreads();
    if (act) {
      uint32_t base = 0;
      for (int gg = 0; gg < g; ++gg) base += seg[gg * KW + kk];
      walk_column(h, nb, kk, t0, t1, true, base);
      if (g == G - 1) tot[kk] = base + sum;
    }
  } else {
    // thread walks columns k = tid, tid + 1024, ...; up to 4 columns interleaved when short
    const int per = (nt <= 8) ? 4 : 1;
    for (int k0 = tid; k0 < nb; k0 += kScanThreads * per) {
      if (per == 4 && nt <= 8) {
        uint32_t c[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k = min(k0 + i * kScanThreads, nb - 1);
#pragma unroll
          for (int u = 0; u < 8; ++u) c[i][u] = h[static_cast<int64_t>(min(u, nt - 1)) * nb + k];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k = k0 + i * kScanThreads;
          if (k >= nb) continue;
          uint32_t run = 0;
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            if (u < nt) {
              h[static_cast<int64_t>(u) * nb + k] = run;
              run += c[i][u];
            }
          }
          tot[k] = run;
        }
      } else {
        tot[k0] = walk_column(h, nb, k0, 0, nt, true, 0);
      }
    }
  }
  __syncthreads();
  // exclusive scan of tot[0..nb): thread i owns the contiguous run [i*per, (i+1)*per)
  const int per = (nb + kScanThreads - 1) / kScanThreads;
  const int lo = min(nb, tid * per);
  const int hi = min(nb, lo + per);
  uint32_t sum = 0;
  for (int k = lo; k < hi; ++k) sum += tot[k];
  uint32_t total;
  uint32_t pre = block_exscan<kScanThreads>(sum, wsum, total);
  for (int k = lo; k < hi; ++k) {
    start[k] = pre;
    pre += tot[k];
  }
  if (tid == 0) {
    start[nb] = total;
    if (total_out != nullptr) *total_out = total;
  }
  if (tail.group_list == nullptr) return;
  __syncthreads();
  uint32_t carry = 0;
  for (int k0 = 0; k0 < nb; k0 += kScanThreads) {
    const int k = k0 + tid;
    const uint32_t cnt = (k < nb) ? tot[k] : 0u;
    uint32_t present;
    const uint32_t slot = carry + block_exscan<kScanThreads>(cnt > 0 ? 1u : 0u, wsum, present);
    if (cnt > 0) {
      tail.group_list[2 * static_cast<int64_t>(slot)] = k;
      tail.group_list[2 * static_cast<int64_t>(slot) + 1] = cnt;
    }
    carry += present;
  }
  for (int64_t gi = carry + tid; gi < tail.group_rows; gi += kScanThreads) {
    tail.group_list[2 * gi] = 0;
    tail.group_list[2 * gi + 1] = 0;
  }
  uint32_t e = 0;
  for (int t = tid; t < nt; t += kScanThreads) e += tail.tile_err[t];
  uint32_t etot;
  (void)block_exscan<kScanThreads>(e, wsum, etot);
  if (tid == 0) {
    *tail.actual_token_num = static_cast<int64_t>(total);
    if (tail.err_count != nullptr) *tail.err_count = static_cast<int32_t>(etot);
  }
}

// Dynamic LDS of scan_hist_kernel for nb digits.
__host__ __device__ inline size_t scan_lds_bytes(int nb) {
  return (static_cast<size_t>(nb) + kScanThreads) * sizeof(uint32_t);
}

// Output bases of a scanned ranking pass (see scan_hist_kernel).
struct Placement {
  const uint32_t* packed;  // per element: digit << 16 | rank in tile, or kNoRank
  const uint32_t* off;     // [nt * nb] per-digit prefixes over tiles
  const uint32_t* start;   // [nb + 1] digit starts
  int nb;
  int tile_shift;          // tile of element j = j >> tile_shift

  // first position of `digit` in `tile`, minus start[digit]
  __device__ __forceinline__ uint32_t tile_base(int64_t tile, uint32_t digit) const { return off[tile * nb + digit]; }
  // output position of element j (false if not placed)
  __device__ __forceinline__ bool position(int64_t j, uint32_t& pos, uint32_t& digit) const {
    const uint32_t p = packed[j];
    if (p == kNoRank) return false;
    digit = p >> 16;
    pos = start[digit] + tile_base(j >> tile_shift, digit) + (p & 0xffffu);
    return true;
  }
};

// ------------------------------------------------------------------ LSD scatter passes
// FINAL = 0: intermediate pass -> keys_out / vals_out.
// FINAL = 1: last pass of the non-padded auxiliary order -> out_index = val, token = val / K.
// FINAL = 2: last pass of the padded inversion -> out_index = val, token = sI[val], keys_out.
template <class KS, bool FIRST, int FINAL>
__global__ __launch_bounds__(256) void lsd_scatter_kernel(KS ks, const uint32_t* __restrict__ vals_in, Placement pl,
                                                          int64_t n, uint32_t* __restrict__ keys_out,
                                                          uint32_t* __restrict__ vals_out,
                                                          int32_t* __restrict__ out_index,
                                                          int32_t* __restrict__ token_out,
                                                          const int32_t* __restrict__ sI, int32_t K) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j >= n) return;
  uint32_t pos, digit;
  if (!pl.position(j, pos, digit)) return;
  bool v, e;
  const uint32_t key = ks.key(j, v, e);
  const uint32_t val = FIRST ? static_cast<uint32_t>(j) : vals_in[j];
  if (FINAL == 0) {
    keys_out[pos] = key;
    vals_out[pos] = val;
  } else if (FINAL == 1) {
    if (out_index != nullptr) out_index[pos] = static_cast<int32_t>(val);
    if (token_out != nullptr) token_out[pos] = static_cast<int32_t>(val / static_cast<uint32_t>(K));
  } else {
    out_index[pos] = static_cast<int32_t>(val);
    if (token_out != nullptr) token_out[pos] = sI[val];
    if (keys_out != nullptr) keys_out[pos] = key;
  }
}

// seg[k] = first sorted position whose key is >= k, for k in [0, nkeys]; seg[nkeys] = n
// when every key is < nkeys.  Each seg entry is written by exactly one thread.
[[maybe_unused]] static __global__ __launch_bounds__(256) void segment_bounds_kernel(const uint32_t* __restrict__ skeys, int64_t n,
                                                             uint32_t nkeys, uint32_t* __restrict__ seg) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j > n) return;
  const int64_t prev = (j == 0) ? -1 : static_cast<int64_t>(skeys[j - 1]);
  const int64_t cur = (j == n) ? static_cast<int64_t>(nkeys) : static_cast<int64_t>(skeys[j]);
  for (int64_t k = prev + 1; k <= cur && k <= static_cast<int64_t>(nkeys); ++k) seg[k] = static_cast<uint32_t>(j);
}

}  // namespace ffnwb

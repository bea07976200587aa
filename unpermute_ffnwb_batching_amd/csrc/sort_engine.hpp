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
// One workgroup then turns every digit's column of that matrix into an exclusive prefix
// over tiles (in place) and scans the digit totals into start[digit].  Element j's output
// position is start[digit] + hist[tile*nb + digit] + rank: ties keep input order.
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

// Exclusive scan over a workgroup of NT threads.  `lds` holds NT/64 + 1 words.
template <int NT>
__device__ __forceinline__ uint32_t block_exscan(uint32_t v, uint32_t* lds, uint32_t& total) {
  constexpr int NW = NT / kWave;
  const int lane = static_cast<int>(lane_id());
  const int w = threadIdx.x / kWave;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == kWave - 1) lds[w] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t run = 0;
    for (int i = 0; i < NW; ++i) { const uint32_t t = lds[i]; lds[i] = run; run += t; }
    lds[NW] = run;
  }
  __syncthreads();
  total = lds[NW];
  const uint32_t r = lds[w] + x - v;
  __syncthreads();
  return r;
}

// ------------------------------------------------------------------ key sources
// Each returns the element's key and whether it takes part in the sort; `err` flags
// elements dropped because of an out-of-range id (batching only).

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
                                                                 uint32_t* __restrict__ hist_g, int nt,
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
  bool val[R];
  uint32_t nerr = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t j = base + r * kWave + lane;
    bool v = false, e = false;
    uint32_t key = 0;
    if (j < n) key = ks.key(j, v, e);
    dig[r] = (key >> shift) & dmask;
    val[r] = v;
    nerr += static_cast<uint32_t>(__popcll(wave_ballot(e)));
  }
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
// One 1024-thread workgroup.  Phase 1: thread k walks digit k's column of the tile-major
// histogram (coalesced across threads), replacing each count by the number of elements
// with that digit in earlier tiles, and keeps the digit's total in LDS.  Phase 2: an
// exclusive scan of the totals gives start[k] (start[nb] = n placed).  Optional tail for
// batching: compact group_list rows {k, count_k} for count_k > 0 then {0,0},
// actual_token_num and err_count = sum of tile_err[0..nt).
struct ScanTail {
  int64_t* group_list;    // nullptr = no batching tail
  int64_t group_rows;
  int64_t* actual_token_num;
  int32_t* err_count;     // may be nullptr
  const uint32_t* tile_err;
};

constexpr int kScanMaxBuckets = 20480;  // LDS holds every digit total (80 KiB)

static __global__ __launch_bounds__(kScanThreads) void scan_hist_kernel(uint32_t* __restrict__ h, int nb, int nt,
                                                                        uint32_t* __restrict__ start,
                                                                        uint32_t* __restrict__ total_out,
                                                                        ScanTail tail) {
  extern __shared__ uint32_t tot[];  // [nb]
  __shared__ uint32_t wsum[kScanThreads / kWave + 1];
  for (int k = threadIdx.x; k < nb; k += kScanThreads) {
    uint32_t run = 0;
    int t = 0;
    for (; t + 8 <= nt; t += 8) {
      uint32_t c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = h[static_cast<int64_t>(t + u) * nb + k];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        h[static_cast<int64_t>(t + u) * nb + k] = run;
        run += c[u];
      }
    }
    for (; t < nt; ++t) {
      const uint32_t c = h[static_cast<int64_t>(t) * nb + k];
      h[static_cast<int64_t>(t) * nb + k] = run;
      run += c;
    }
    tot[k] = run;
  }
  __syncthreads();
  // exclusive scan of tot[0..nb): thread i owns the contiguous run [i*per, (i+1)*per)
  const int per = (nb + kScanThreads - 1) / kScanThreads;
  const int lo = min(nb, static_cast<int>(threadIdx.x) * per);
  const int hi = min(nb, lo + per);
  uint32_t sum = 0;
  for (int k = lo; k < hi; ++k) sum += tot[k];
  uint32_t total;
  uint32_t pre = block_exscan<kScanThreads>(sum, wsum, total);
  for (int k = lo; k < hi; ++k) {
    start[k] = pre;
    pre += tot[k];
  }
  if (threadIdx.x == 0) {
    start[nb] = total;
    if (total_out != nullptr) *total_out = total;
  }
  if (tail.group_list == nullptr) return;
  __syncthreads();
  uint32_t carry = 0;
  for (int k0 = 0; k0 < nb; k0 += kScanThreads) {
    const int k = k0 + threadIdx.x;
    const uint32_t cnt = (k < nb) ? tot[k] : 0u;
    uint32_t present;
    const uint32_t slot = carry + block_exscan<kScanThreads>(cnt > 0 ? 1u : 0u, wsum, present);
    if (cnt > 0) {
      tail.group_list[2 * static_cast<int64_t>(slot)] = k;
      tail.group_list[2 * static_cast<int64_t>(slot) + 1] = cnt;
    }
    carry += present;
  }
  for (int64_t g = carry + threadIdx.x; g < tail.group_rows; g += kScanThreads) {
    tail.group_list[2 * g] = 0;
    tail.group_list[2 * g + 1] = 0;
  }
  uint32_t e = 0;
  for (int t = threadIdx.x; t < nt; t += kScanThreads) e += tail.tile_err[t];
  uint32_t etot;
  (void)block_exscan<kScanThreads>(e, wsum, etot);
  if (threadIdx.x == 0) {
    *tail.actual_token_num = static_cast<int64_t>(total);
    if (tail.err_count != nullptr) *tail.err_count = static_cast<int32_t>(etot);
  }
}

// Output position of element j after a ranking pass and the scan (false if not placed).
__device__ __forceinline__ bool placed_position(const uint32_t* __restrict__ packed, const uint32_t* __restrict__ off,
                                                const uint32_t* __restrict__ start, int nb, int tile_shift,
                                                int64_t j, uint32_t& pos, uint32_t& digit) {
  const uint32_t p = packed[j];
  if (p == kNoRank) return false;
  digit = p >> 16;
  pos = start[digit] + off[(j >> tile_shift) * nb + digit] + (p & 0xffffu);
  return true;
}

// ------------------------------------------------------------------ LSD scatter passes
// FINAL = 0: intermediate pass -> keys_out / vals_out.
// FINAL = 1: last pass of the non-padded auxiliary order -> out_index = val, token = val / K.
// FINAL = 2: last pass of the padded inversion -> out_index = val, token = sI[val], keys_out.
template <class KS, bool FIRST, int FINAL>
__global__ __launch_bounds__(256) void lsd_scatter_kernel(KS ks, const uint32_t* __restrict__ vals_in,
                                                          const uint32_t* __restrict__ packed,
                                                          const uint32_t* __restrict__ off,
                                                          const uint32_t* __restrict__ start, int nb, int tile_shift,
                                                          int64_t n, uint32_t* __restrict__ keys_out,
                                                          uint32_t* __restrict__ vals_out,
                                                          int32_t* __restrict__ out_index,
                                                          int32_t* __restrict__ token_out,
                                                          const int32_t* __restrict__ sI, int32_t K) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j >= n) return;
  uint32_t pos, digit;
  if (!placed_position(packed, off, start, nb, tile_shift, j, pos, digit)) return;
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
static __global__ __launch_bounds__(256) void segment_bounds_kernel(const uint32_t* __restrict__ skeys, int64_t n,
                                                             uint32_t nkeys, uint32_t* __restrict__ seg) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j > n) return;
  const int64_t prev = (j == 0) ? -1 : static_cast<int64_t>(skeys[j - 1]);
  const int64_t cur = (j == n) ? static_cast<int64_t>(nkeys) : static_cast<int64_t>(skeys[j]);
  for (int64_t k = prev + 1; k <= cur && k <= static_cast<int64_t>(nkeys); ++k) seg[k] = static_cast<uint32_t>(j);
}

}  // namespace ffnwb

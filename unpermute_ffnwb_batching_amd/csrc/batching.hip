// FFN-worker batching on gfx950 (aclnnFfnWorkerBatching API page, "Function description"
// steps 2-4 and the calculation formula).
//
// Three launches in the general case:
//   1. sort_rank_kernel<KeyBatching>: per slot key (masked / bad ids -> not placed), stable
//      in-tile rank, per-tile key histogram (bucket-major), per-tile count of bad ids;
//   2. scan_hist_kernel: exclusive scan of the histogram -> first output row of every
//      (key, tile) run; its tail writes group_list, actual_token_num and err_count;
//   3. batching_gather_kernel: one wavefront per slot copies the slot's H-element row to
//      its output row with 16-byte accesses and writes the per-row IDs and scale.
// Small problems (one tile, small rows) run all three steps in one workgroup.
#include <stdio.h>

#include "internal.hpp"
#include "range_order.hpp"
#include "row_copy.hpp"
#include "sort_engine.hpp"

namespace ffnwb {

constexpr int64_t kBatchingRangeMaxSlots = 8192;

struct BatchArgs {
  int64_t Y, chunk;
  int32_t per_layer, L, layer_num;
  int32_t has_mask, use_layers;  // whether mask / layer_ids hold data (the pointers are always readable)
  const int32_t* expert_ids;
  const uint8_t* mask;       // never null: stands in with expert_ids' bytes when there is no mask
  const int32_t* layer_ids;  // never null: stands in with expert_ids when layers are not used
  const int32_t* session_ids;
  const int32_t* micro_batch_ids;
  const uint8_t* token_data;
  int64_t stride;
  const uint8_t* scale_base;  // INT8 only
  int64_t scale_stride;
  uint8_t* y;
  int64_t row_bytes;
  int32_t* session_out;
  int32_t* mb_out;
  int32_t* token_ids;
  int32_t* offsets;
  float* dyn_scale;           // nullptr unless INT8
  const uint64_t* chunk_src;  // context mode: address of each chunk's first row, else nullptr
};

// A device address as a pointer into global memory: made in the global address space,
// so that the compiler keeps global (not flat) loads for everything derived from it.
typedef const __attribute__((address_space(1))) uint8_t* GlobalBytes;
__device__ __forceinline__ const uint8_t* global_bytes(uint64_t addr) {
  return (const uint8_t*)((GlobalBytes)addr);
}

// Source row of slot s: token_data + s * stride, or in context mode entry s % chunk of
// chunk s / chunk, whose rows start at chunk_src[chunk] (the branch is uniform).
__device__ __forceinline__ const uint8_t* slot_row(const BatchArgs& a, int64_t s) {
  if (a.chunk_src == nullptr) return a.token_data + s * a.stride;
  const uint32_t chunk = static_cast<uint32_t>(a.chunk);
  const uint32_t c = static_cast<uint32_t>(s) / chunk;
  const uint32_t j = static_cast<uint32_t>(s) - c * chunk;
  return global_bytes(a.chunk_src[c]) + static_cast<int64_t>(j) * a.stride;
}

// INT8 dynamic scale of slot s; in context mode packed after the row's H bytes.
__device__ __forceinline__ const uint8_t* slot_scale(const BatchArgs& a, int64_t s) {
  if (a.chunk_src == nullptr) return a.scale_base + s * a.scale_stride;
  return slot_row(a, s) + a.row_bytes;
}

// Slot key: layer * experts_per_layer + expert id; masked slots do not take part, and
// unmasked slots with an out-of-range expert or layer id are dropped and counted.
// Every input is loaded unconditionally and the tests combine with bitwise operators: a
// load behind a test of its pointer, or a short-circuit test, compiles to a branch, and
// the wait at its end serialised the rounds of a tile (8 rounds: 11 us instead of ~3).
struct KeyBatching {
  BatchArgs a;
  __device__ uint32_t key(int64_t s, bool& valid, bool& err) const {
    const uint32_t c = static_cast<uint32_t>(s) / static_cast<uint32_t>(a.chunk);
    const uint8_t m0 = a.mask[s];
    const int32_t l0 = a.layer_ids[c];
    const int32_t e = a.expert_ids[s];
    const bool live = !a.has_mask | (m0 == 0);
    const int32_t layer = a.use_layers ? l0 : 0;
    const bool ok = (e >= 0) & (e < a.per_layer) & (layer >= 0) & (layer < a.L);
    valid = live & ok;
    err = live & !ok;
    return valid ? static_cast<uint32_t>(layer * a.per_layer + e) : 0u;
  }
};

// The slot keys of 4 consecutive slots j0..j0+3 (j0 a multiple of 4) for the
// range-partitioned order: one 16-byte load of expert ids and one 4-byte load of mask
// bytes where aligned, and at most two layer lookups (4 consecutive slots cross at most
// one chunk boundary when chunks hold at least 4 slots).  Same keys as KeyBatching.
struct RoKeysBatching {
  BatchArgs a;
  __device__ __forceinline__ void key4(uint32_t j0, uint32_t (&k)[kRoVec], bool (&v)[kRoVec],
                                       bool (&er)[kRoVec]) const {
    const uint32_t Y = static_cast<uint32_t>(a.Y);
    const bool full = j0 + kRoVec <= Y;
    int32_t ex[kRoVec];
    if (full && (reinterpret_cast<uintptr_t>(a.expert_ids) & 15) == 0) {
      const int4 q = *reinterpret_cast<const int4*>(a.expert_ids + j0);
      ex[0] = q.x; ex[1] = q.y; ex[2] = q.z; ex[3] = q.w;
    } else {
#pragma unroll
      for (int i = 0; i < kRoVec; ++i) ex[i] = a.expert_ids[min(j0 + i, Y - 1)];
    }
    uint32_t m[kRoVec];
    if (full && (reinterpret_cast<uintptr_t>(a.mask) & 3) == 0) {
      const uint32_t q = *reinterpret_cast<const uint32_t*>(a.mask + j0);
#pragma unroll
      for (int i = 0; i < kRoVec; ++i) m[i] = a.has_mask ? (q >> (8 * i)) & 0xffu : 0u;
    } else {
#pragma unroll
      for (int i = 0; i < kRoVec; ++i) m[i] = a.has_mask ? a.mask[min(j0 + i, Y - 1)] : 0u;
    }
    int32_t layer[kRoVec];
    {
      const uint32_t chunk = static_cast<uint32_t>(a.chunk);
      if (chunk >= kRoVec) {
        const uint32_t jc = min(j0, Y - 1);
        const uint32_t c0 = jc / chunk;
        const uint32_t last = Y / chunk - 1u;  // last chunk
        const uint32_t next = (c0 + 1u) * chunk;  // first slot of chunk c0 + 1 (<= Y < 2^31)
        const int32_t l0 = a.layer_ids[c0];
        const int32_t l1 = a.layer_ids[min(c0 + 1u, last)];
#pragma unroll
        for (int i = 0; i < kRoVec; ++i) layer[i] = (j0 + i < next) ? l0 : l1;
      } else {
#pragma unroll
        for (int i = 0; i < kRoVec; ++i) layer[i] = a.layer_ids[min(j0 + i, Y - 1) / chunk];
      }
    }
#pragma unroll
    for (int i = 0; i < kRoVec; ++i) {
      const int32_t li = a.use_layers ? layer[i] : 0;
      const bool ok = (ex[i] >= 0) & (ex[i] < a.per_layer) & (li >= 0) & (li < a.L);
      v[i] = (m[i] == 0) & ok;
      er[i] = (m[i] == 0) & !ok;
      k[i] = v[i] ? static_cast<uint32_t>(li * a.per_layer + ex[i]) : 0u;
    }
  }
};

__device__ __forceinline__ float load_scale(const uint8_t* p) {
  const uint32_t v = static_cast<uint32_t>(p[0]) | (static_cast<uint32_t>(p[1]) << 8) |
                     (static_cast<uint32_t>(p[2]) << 16) | (static_cast<uint32_t>(p[3]) << 24);
  return __uint_as_float(v);
}

__device__ __forceinline__ void write_row_ids(const BatchArgs& a, int64_t s, uint32_t pos, uint32_t first) {
  const uint32_t c = static_cast<uint32_t>(s) / static_cast<uint32_t>(a.chunk);
  a.token_ids[pos] = static_cast<int32_t>(s);
  a.offsets[pos] = static_cast<int32_t>(pos - first);
  a.session_out[pos] = a.session_ids ? a.session_ids[c] : static_cast<int32_t>(c);
  a.mb_out[pos] = a.micro_batch_ids ? a.micro_batch_ids[c] : 0;
  if (a.dyn_scale != nullptr) a.dyn_scale[pos] = load_scale(slot_scale(a, s));
}

// One wavefront per source slot (4 slots per workgroup).  The slot's output row is
// start[key] + (its tile's base for key) + rank; its group's first row is start[key].
// The first piece of the source row is loaded before that lookup, so the lookup's
// latency hides under the row loads.
template <int VEC>
__global__ __launch_bounds__(256) void batching_gather_kernel(BatchArgs a, Placement pl) {
  const int64_t s = static_cast<int64_t>(blockIdx.x) * 4 + uniform(static_cast<int>(threadIdx.x) / kWave);
  if (s >= a.Y) return;
  const uint32_t p = uniform(pl.packed[s]);
  if (p == kNoRank) return;
  const uint32_t lane = lane_id();
  const uint8_t* src = slot_row(a, s);
  const int64_t n16 = a.row_bytes >> 4;
  RowPiece<VEC> first;
  if (VEC != 1) first.load(src, n16, 0, lane);
  const uint32_t key = p >> 16;
  const uint32_t gstart = uniform(pl.start[key]);
  const uint32_t pos = gstart + uniform(pl.tile_base(s >> pl.tile_shift, key)) + (p & 0xffffu);
  uint8_t* dst = a.y + static_cast<int64_t>(pos) * a.row_bytes;
  if (VEC != 1) {
    first.store(dst, n16, 0, lane);
    copy_row_rest<VEC>(src, dst, a.row_bytes, kWave * kPiece, lane);
  } else {
    copy_row_rest<VEC>(src, dst, a.row_bytes, 0, lane);
  }
  if (lane == 0) write_row_ids(a, s, pos, gstart);
}

// Slot order in one launch (range-partitioned, see range_order.hpp).  Workgroup b owns
// the keys [lo, lo + kr): for its slots it writes the output row pos_of[s] and the row
// IDs (token id, offset in the group, session, micro-batch; the per-chunk ids are staged
// in LDS so that placing a slot issues stores only), and for its non-empty keys their
// group_list rows.  A key's group_list row is the number of
// non-empty keys below it, which every workgroup finds from a presence array of the keys
// below lo (filled with relaxed stores of 1: no read-modify-write).  Workgroup 0 also
// marks the slots that are not placed, zero-fills group_list after the non-empty rows and
// writes err_count; the workgroup owning the last key writes actual_token_num.
// LDS: the range-order layout (ro_lds_words(kr)), then presence [nb] | first row of each
// owned key [kr] | session and micro-batch id of each chunk [2][A].
__global__ __launch_bounds__(kRoThreads) void batching_order_kernel(BatchArgs a, uint32_t nb, uint32_t kr, int nbits,
                                                                    uint32_t* __restrict__ pos_of,
                                                                    int64_t* __restrict__ group_list,
                                                                    int64_t group_rows,
                                                                    int64_t* __restrict__ actual,
                                                                    int32_t* __restrict__ err_count) {
  extern __shared__ uint32_t lds_words[];
  __shared__ uint32_t wsum[3 * kRoWaves + 4];  // block scans of up to 3 sequences
  __shared__ uint32_t bcast[2];
  const uint32_t lo = blockIdx.x * kr;
  const uint32_t krr = min(kr, nb - lo);
  uint32_t* cnt = ro_counters(lds_words);
  uint32_t* pres = cnt + kRoWaves * kr;
  uint32_t* kfirst = pres + nb;
  int32_t* ses = reinterpret_cast<int32_t*>(kfirst + kr);
  const uint32_t nchunks = static_cast<uint32_t>(a.Y / a.chunk);
  int32_t* mbs = ses + nchunks;
  const bool g0 = blockIdx.x == 0;
  const uint32_t plim = g0 ? nb : lo;  // presence is tracked for keys < plim
  for (int i = threadIdx.x; i < kRoWaves * static_cast<int>(krr); i += kRoThreads) cnt[i] = 0u;
  for (uint32_t i = threadIdx.x; i < plim; i += kRoThreads) pres[i] = 0u;
  // per-chunk ids (A <= 1024 chunks: one per thread), loaded now, stored to LDS after pass 1
  const uint32_t cid = threadIdx.x;
  int32_t ses_v = static_cast<int32_t>(cid), mbs_v = 0;
  if (cid < nchunks) {
    if (a.session_ids != nullptr) ses_v = a.session_ids[cid];
    if (a.micro_batch_ids != nullptr) mbs_v = a.micro_batch_ids[cid];
  }
  __syncthreads();
  const int w = uniform(static_cast<int>(threadIdx.x) / kWave);
  uint32_t b, e;
  ro_slice(static_cast<uint32_t>(a.Y), w, b, e);
  const RoKeysBatching ks{a};
  const RoWave wv = ro_wave(lds_words, w, krr);
  uint32_t nerr = 0;
  uint32_t len;
  const uint32_t below = ro_count(ks, b, e, lo, krr, wv, len, [&](uint32_t s, uint32_t key, bool v, bool er) {
    if (v && key < plim) __hip_atomic_store(&pres[key], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (g0) {
      if (!v) pos_of[s] = kNoRank;
      nerr += er ? 1u : 0u;
    }
  });
  uint32_t kcount, end;
  const uint32_t first = ro_middle(cnt, krr, below, wsum, kcount, end);
  const uint32_t k = threadIdx.x;
  if (k < krr) kfirst[k] = first;
  if (cid < nchunks) {
    ses[cid] = ses_v;
    mbs[cid] = mbs_v;
  }
  // one scan of three sequences: [non-empty owned keys | present keys below plim | bad ids];
  // thread 0's results give the first two totals
  uint32_t pcount = 0;
  for (uint32_t i = k; i < plim; i += kRoThreads) pcount += pres[i];
  const bool nonempty = k < krr && kcount > 0;
  uint32_t v[3] = {nonempty ? 1u : 0u, pcount, nerr};
  uint32_t all;
  block_exscan_multi<kRoThreads, 3>(v, wsum, all);
  if (k == 0) {
    bcast[0] = v[1];  // non-empty owned keys
    bcast[1] = v[2];  // ... plus present keys below plim
  }
  __syncthreads();  // bcast; kfirst and the chunk ids for pass 2
  const uint32_t ptotal = bcast[1] - bcast[0];  // workgroup 0: all non-empty keys
  const uint32_t row = (g0 ? 0u : ptotal) + v[0];
  if (nonempty) {
    group_list[2 * static_cast<int64_t>(row)] = lo + k;
    group_list[2 * static_cast<int64_t>(row) + 1] = kcount;
  }
  if (g0) {
    for (int64_t r = static_cast<int64_t>(ptotal) + k; r < group_rows; r += kRoThreads) {
      group_list[2 * r] = 0;
      group_list[2 * r + 1] = 0;
    }
    if (k == 0 && err_count != nullptr) *err_count = static_cast<int32_t>(all - bcast[1]);
  }
  if (k == 0 && lo + krr == nb) *actual = static_cast<int64_t>(end);
  const uint32_t chunk = static_cast<uint32_t>(a.chunk);
  ro_place(ks, b, e, lo, krr, nbits, wv, len, [&](uint32_t s, uint32_t key, uint32_t pos) {
    const uint32_t c = s / chunk;
    pos_of[s] = pos;
    a.token_ids[pos] = static_cast<int32_t>(s);
    a.offsets[pos] = static_cast<int32_t>(pos - kfirst[key - lo]);
    a.session_out[pos] = ses[c];
    a.mb_out[pos] = mbs[c];
  });
}

// Slot order in one 1024-thread workgroup, for Y <= 8192 slots and nb <= 2048 keys.
// Wave w owns the R*64 consecutive slots from w*R*64; every load of a slot (key inputs,
// its chunk's session and micro-batch ids) is issued in one batch before any use.  The
// ballot ranking gives each slot's rank among equal keys of its wave (per-wave u16
// counters in LDS), a prefix over the 16 waves and a scan over the keys give each
// key's first row and group_list.  The workgroup writes, coalesced, the output row of
// every slot and its group's first row; the row copy that follows writes the row IDs
// (from one CU, scattered ID stores took 17 us for 4608 slots).
// LDS: u16 counters [16][nbp] | u16 totals of each group of 4 waves [4][nbp] | first row
// of each key [nb].
constexpr int kWgThreads = 1024;
constexpr int kWgWaves = kWgThreads / kWave;
constexpr int64_t kWgMaxSlots = 8192;
constexpr int kWgMaxKeys = 2048;

template <int R>
__global__ __launch_bounds__(kWgThreads) void batching_wg_order_kernel(BatchArgs a, int nbits, int nb,
                                                                      uint32_t* __restrict__ pos_of,
                                                                      uint32_t* __restrict__ first_of,
                                                                      int64_t* __restrict__ group_list,
                                                                      int64_t group_rows, int64_t* __restrict__ actual,
                                                                      int32_t* __restrict__ err_count) {
  extern __shared__ uint32_t lds_words[];
  __shared__ uint32_t wsum[2][2 * kWgWaves + 1];  // ping-pong: a scan's totals are read after it
  __shared__ uint32_t err_w[kWgWaves];
  const int nbp = rank_lds_stride(nb);
  uint16_t* hist = reinterpret_cast<uint16_t*>(lds_words);
  uint16_t* gsum = hist + kWgWaves * nbp;
  uint32_t* start = lds_words + (kWgWaves + 4) * nbp / 2;
  lds_zero_words(lds_words, kWgWaves * nbp / 2);
  __syncthreads();

  const KeyBatching ks{a};
  const int w = uniform(static_cast<int>(threadIdx.x) / kWave);
  const uint32_t lane = lane_id();
  uint32_t dig[R], rank[R];
  bool val[R], bad[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t s = static_cast<int64_t>(w) * (kWave * R) + r * kWave + lane;
    const bool in = s < a.Y;
    bool v = false, e = false;
    dig[r] = ks.key(in ? s : a.Y - 1, v, e);
    val[r] = v && in;
    bad[r] = e && in;
  }
  // ballots after every round's loads: a ballot between rounds keeps the next round's
  // loads from being issued before it
  uint32_t nerr = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) nerr += static_cast<uint32_t>(__popcll(wave_ballot(bad[r])));
  rank_rounds<R>(dig, val, nbits, hist + w * nbp, rank);
  if (lane == 0) err_w[w] = nerr;
  __syncthreads();
  // per key: each wave's base among the key's slots, and the key's total, in two levels
  // (4 groups of 4 waves, then the groups) so that no thread walks all 16 waves
  // (counters are read into registers before anything is written back: with the row
  // pitch nbp a runtime value, the compiler cannot reorder a read-modify-write sequence)
  const int kq = threadIdx.x & 255, grp = threadIdx.x >> 8;
  constexpr int kPasses = kWgMaxKeys / 256;
  uint32_t pre[kPasses][4];
#pragma unroll
  for (int m = 0; m < kPasses; ++m) {
    const int k = kq + m * 256;
    if (k < nb) {
      uint32_t c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] = hist[(4 * grp + i) * nbp + k];
      uint32_t run = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pre[m][i] = run;
        run += c[i];
      }
      gsum[grp * nbp + k] = static_cast<uint16_t>(run);
    }
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < kPasses; ++m) {
    const int k = kq + m * 256;
    if (k < nb) {
      uint32_t g[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) g[i] = gsum[i * nbp + k];
      uint32_t base = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) base += i < grp ? g[i] : 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) hist[(4 * grp + i) * nbp + k] = static_cast<uint16_t>(pre[m][i] + base);
      if (grp == 3) start[k] = base + g[3];
    }
  }
  __syncthreads();
  // start[k] <- first output row of key k; group_list in the same sweep (one scan of
  // [counts | presence]: the presence prefix is offset by the counts' total)
  uint32_t carry = 0, gcarry = 0;
  for (int k0 = 0, it = 0; k0 < nb; k0 += kWgThreads, it ^= 1) {
    const int k = k0 + threadIdx.x;
    const uint32_t cnt = (k < nb) ? start[k] : 0u;
    uint32_t v[2] = {cnt, cnt > 0 ? 1u : 0u};
    uint32_t all;
    block_exscan_multi<kWgThreads, 2>(v, wsum[it], all);
    const uint32_t tot = wsum[it][kWgWaves];  // sequence 1 starts after all counts
    if (k < nb) start[k] = carry + v[0];
    if (cnt > 0) {
      const int64_t slot = gcarry + v[1] - tot;
      group_list[2 * slot] = k;
      group_list[2 * slot + 1] = cnt;
    }
    carry += tot;
    gcarry += all - tot;
  }
  for (int64_t g = gcarry + threadIdx.x; g < group_rows; g += kWgThreads) {
    group_list[2 * g] = 0;
    group_list[2 * g + 1] = 0;
  }
  if (threadIdx.x == 0) {
    *actual = static_cast<int64_t>(carry);
    if (err_count != nullptr) {
      uint32_t e = 0;
      for (int ww = 0; ww < kWgWaves; ++ww) e += err_w[ww];
      *err_count = static_cast<int32_t>(e);
    }
  }
  __syncthreads();  // start[] complete
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t s = static_cast<int64_t>(w) * (kWave * R) + r * kWave + lane;
    if (s >= a.Y) continue;
    const uint32_t first = start[dig[r]];
    pos_of[s] = val[r] ? first + hist[w * nbp + dig[r]] + rank[r] : kNoRank;
    first_of[s] = first;
  }
}

// Row copy after batching_order_kernel: one wavefront per slot; the INT8 scale moves
// with its row.
// With first_of (after batching_wg_order_kernel), lane 0 also writes the row IDs.
template <int VEC>
__global__ __launch_bounds__(256) void batching_copy_kernel(BatchArgs a, const uint32_t* __restrict__ pos_of,
                                                            const uint32_t* __restrict__ first_of) {
  const int64_t s = static_cast<int64_t>(blockIdx.x) * 4 + uniform(static_cast<int>(threadIdx.x) / kWave);
  if (s >= a.Y) return;
  const uint32_t pos = uniform(pos_of[s]);
  if (pos == kNoRank) return;
  const uint32_t lane = lane_id();
  copy_row<VEC>(slot_row(a, s), a.y + static_cast<int64_t>(pos) * a.row_bytes, a.row_bytes, lane);
  if (lane == 0) {
    if (first_of != nullptr) write_row_ids(a, s, pos, first_of[s]);  // also moves the scale
    else if (a.dyn_scale != nullptr) a.dyn_scale[pos] = load_scale(slot_scale(a, s));
  }
}

// Copy unit of the one-workgroup path: 16, 4 or 1 bytes.
template <int VEC> struct SmallUnit { typedef u32x4 type; };
template <> struct SmallUnit<4> { typedef uint32_t type; };
template <> struct SmallUnit<1> { typedef uint8_t type; };
constexpr int kSmallUnits = 8;

// All steps in one 256-thread workgroup, for Y <= 1024 slots and <= 4096 keys.
// LDS: u16 counters [4][nbp] | u32 key starts [nb + 1] | u32 output row of each slot [1024].
template <int VEC>
__global__ __launch_bounds__(256) void batching_small_kernel(BatchArgs a, int nbits, int nb, int64_t* group_list,
                                                             int64_t group_rows, int64_t* actual,
                                                             int32_t* err_count) {
  constexpr int R = 4;
  extern __shared__ uint32_t lds_words[];
  __shared__ uint32_t wsum[kRankThreads / kWave + 1];  // block_exscan scratch
  __shared__ uint32_t err_w[kRankWaves];
  const int nbp = rank_lds_stride(nb);
  uint16_t* hist = reinterpret_cast<uint16_t*>(lds_words);
  uint32_t* start = lds_words + kRankWaves * nbp / 2;
  uint32_t* pos_of = start + nb + 1;
  lds_zero_words(lds_words, kRankWaves * nbp / 2);
  __syncthreads();

  KeyBatching ks{a};
  const int w = uniform(static_cast<int>(threadIdx.x) / kWave);
  const uint32_t lane = lane_id();
  uint32_t dig[R], rank[R];
  bool val[R], bad[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t s = static_cast<int64_t>(w) * (kWave * R) + r * kWave + lane;
    const bool in = s < a.Y;
    bool v = false, e = false;
    dig[r] = ks.key(in ? s : a.Y - 1, v, e);
    val[r] = v && in;
    bad[r] = e && in;
  }
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
    start[k] = run;
  }
  __syncthreads();
  // start[k] <- first output row of key k; group_list in the same sweep.
  uint32_t carry = 0, gcarry = 0;
  for (int k0 = 0; k0 < nb; k0 += kRankThreads) {
    const int k = k0 + threadIdx.x;
    const uint32_t cnt = (k < nb) ? start[k] : 0u;
    uint32_t tot, present;
    const uint32_t ex = block_exscan<kRankThreads>(cnt, wsum, tot);
    const uint32_t slot = gcarry + block_exscan<kRankThreads>(cnt > 0 ? 1u : 0u, wsum, present);
    if (k < nb) start[k] = carry + ex;
    if (cnt > 0) {
      group_list[2 * static_cast<int64_t>(slot)] = k;
      group_list[2 * static_cast<int64_t>(slot) + 1] = cnt;
    }
    carry += tot;
    gcarry += present;
  }
  for (int64_t g = gcarry + threadIdx.x; g < group_rows; g += kRankThreads) {
    group_list[2 * g] = 0;
    group_list[2 * g + 1] = 0;
  }
  if (threadIdx.x == 0) {
    *actual = static_cast<int64_t>(carry);
    if (err_count != nullptr) *err_count = static_cast<int32_t>(err_w[0] + err_w[1] + err_w[2] + err_w[3]);
  }
  __syncthreads();
  // each thread places its own slots and writes their row IDs
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t s = static_cast<int64_t>(w) * (kWave * R) + r * kWave + lane;
    if (s >= a.Y) continue;
    const uint32_t first = start[dig[r]];
    const uint32_t pos = first + hist[w * nbp + dig[r]] + rank[r];
    pos_of[s] = val[r] ? pos : kNoRank;
    if (val[r]) write_row_ids(a, s, pos, first);
  }
  __syncthreads();
  // the rows as one flat run of VEC-byte units over all threads (Y * row_bytes <= 4 MiB),
  // kSmallUnits loads in flight per thread: one memory round trip for a small problem
  // instead of one per row and wavefront
  typedef typename SmallUnit<VEC>::type U;
  const uint32_t nu = static_cast<uint32_t>(a.row_bytes / VEC);
  const uint32_t total = static_cast<uint32_t>(a.Y) * nu;
  for (uint32_t u0 = threadIdx.x; u0 < total; u0 += kRankThreads * kSmallUnits) {
    U v[kSmallUnits];
    uint32_t dst[kSmallUnits];
#pragma unroll
    for (int k = 0; k < kSmallUnits; ++k) {
      const uint32_t u = u0 + k * kRankThreads;
      const uint32_t sl = min(u, total - 1) / nu;
      const uint32_t part = min(u, total - 1) - sl * nu;
      const uint32_t pos = pos_of[sl];
      const bool placed = u < total && pos != kNoRank;
      dst[k] = placed ? pos * nu + part : 0xffffffffu;
      // an unplaced slot's row is never read (from a rejected ScheduleContext its address
      // is 0): its load takes the output's first unit instead, so every load stays
      // unconditional and in bounds
      const U* src = placed ? reinterpret_cast<const U*>(slot_row(a, sl)) + part : reinterpret_cast<const U*>(a.y);
      v[k] = *src;
    }
#pragma unroll
    for (int k = 0; k < kSmallUnits; ++k)
      if (dst[k] != 0xffffffffu) reinterpret_cast<U*>(a.y)[dst[k]] = v[k];
  }
}

// Placement by tiles after sort_rank_kernel<KeyBatching>, for at most kPlaceMaxTiles
// tiles; it replaces the one-workgroup histogram scan.  Workgroup t reads the whole
// tile-major histogram (nt x nb words, in L2) and sums each key's column over all tiles
// and over the tiles before t.  An exclusive scan of the sums gives each key's first
// output row, so every workgroup places its own tile's slots without waiting for another:
// inv[row] = slot.  Every workgroup writes the first rows (kstart) and group_list rows
// of its share of the keys; workgroup 0 writes actual_token_num and err_count.  The row copy that follows walks the output rows
// (random reads, sequential writes, which measured faster than walking the slots) and
// writes the row IDs, in row order.
// LDS: key sums -> first rows [nb] | sums before the tile [nb].
constexpr int kPlaceMaxTiles = 64;

template <int B>  // histogram loads in flight per thread: B >= nt walks a column in one round
__global__ __launch_bounds__(kWgThreads) void batching_place_kernel(BatchArgs a, const uint32_t* __restrict__ packed,
                                                                    const uint32_t* __restrict__ hist_g,
                                                                    const uint32_t* __restrict__ tile_err, int nb,
                                                                    int nt, int tile_shift,
                                                                    uint32_t* __restrict__ inv,
                                                                    uint32_t* __restrict__ kstart,
                                                                    int64_t* __restrict__ group_list,
                                                                    int64_t group_rows,
                                                                    int64_t* __restrict__ actual,
                                                                    int32_t* __restrict__ err_count) {
  extern __shared__ uint32_t lds_words[];
  __shared__ uint32_t wsum[2][2 * kWgWaves + 1];  // ping-pong: a scan's totals are read after it
  uint32_t* cnt = lds_words;
  uint32_t* bef = cnt + nb;
  const int t = blockIdx.x;
  const uint32_t Y = static_cast<uint32_t>(a.Y);
  const uint32_t tile = 1u << tile_shift;
  const uint32_t j0 = static_cast<uint32_t>(t) << tile_shift;
  // the tile's packed ranks (at most 4 per thread), loaded before the histogram is walked
  uint32_t pk[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t j = j0 + r * kWgThreads + threadIdx.x;
    pk[r] = (r * kWgThreads < static_cast<int>(tile) && j < Y) ? packed[j] : kNoRank;
  }
  // 1. per key: the sum over all tiles and over the tiles before t
  for (int k = threadIdx.x; k < nb; k += kWgThreads) {
    uint32_t all = 0, before = 0;
    for (int u0 = 0; u0 < nt; u0 += B) {
      uint32_t c[B];
#pragma unroll
      for (int u = 0; u < B; ++u) c[u] = hist_g[static_cast<int64_t>(min(u0 + u, nt - 1)) * nb + k];
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const int tu = u0 + u;
        all += tu < nt ? c[u] : 0u;
        before += tu < t ? c[u] : 0u;
      }
    }
    cnt[k] = all;
    bef[k] = before;
  }
  __syncthreads();
  // 2. cnt[k] <- first output row of key k (one scan of [sums | presence]: the presence
  //    prefix is offset by the sums' total).  Every workgroup holds the whole scan, so
  //    each writes the key starts and group_list rows of its own share of the keys
  const bool g0 = t == 0;
  const int share = (nb + nt - 1) / nt;
  const int klo = t * share, khi = min(nb, klo + share);
  uint32_t carry = 0, gcarry = 0;
  for (int k0 = 0, it = 0; k0 < nb; k0 += kWgThreads, it ^= 1) {
    const int kk = k0 + threadIdx.x;
    const uint32_t c = (kk < nb) ? cnt[kk] : 0u;
    uint32_t v[2] = {c, c > 0 ? 1u : 0u};
    uint32_t all;
    block_exscan_multi<kWgThreads, 2>(v, wsum[it], all);
    const uint32_t tot = wsum[it][kWgWaves];  // sequence 1 starts after all sums
    const bool mine = kk >= klo && kk < khi;
    if (kk < nb) cnt[kk] = carry + v[0];
    if (mine) kstart[kk] = carry + v[0];
    if (mine && c > 0) {
      const int64_t slot = gcarry + v[1] - tot;
      group_list[2 * slot] = kk;
      group_list[2 * slot + 1] = c;
    }
    carry += tot;
    gcarry += all - tot;
  }
  // the {0, 0} rows after the present keys, split over the workgroups
  {
    const int64_t zrows = group_rows - gcarry;
    const int64_t zshare = (zrows + nt - 1) / nt;
    const int64_t zlo = gcarry + t * zshare, zhi = min(group_rows, zlo + zshare);
    for (int64_t g = zlo + threadIdx.x; g < zhi; g += kWgThreads) {
      group_list[2 * g] = 0;
      group_list[2 * g + 1] = 0;
    }
  }
  if (g0) {
    uint32_t e = 0;
    for (int u = threadIdx.x; u < nt; u += kWgThreads) e += tile_err[u];
    e = wave_sum(e);
    if (threadIdx.x == 0) {
      *actual = static_cast<int64_t>(carry);
      if (err_count != nullptr) *err_count = static_cast<int32_t>(e);  // nt <= 64: wave 0 holds them all
    }
  }
  __syncthreads();  // first rows complete
  // 3. place the tile's slots
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t p = pk[r];
    if (p == kNoRank) continue;
    const uint32_t d = p >> 16;
    inv[cnt[d] + bef[d] + (p & 0xffffu)] = j0 + r * kWgThreads + threadIdx.x;
  }
}

// Row copy after batching_place_kernel: one wavefront per output row below
// actual_token_num, reading the row of slot inv[row].  Lane 0 writes the row IDs (the
// slot's key from its packed rank, and the key's first row, are looked up while the row
// loads are in flight); the INT8 scale moves with its row.
template <int VEC>
__global__ __launch_bounds__(256) void batching_copy_out_kernel(BatchArgs a, const uint32_t* __restrict__ inv,
                                                                const uint32_t* __restrict__ packed,
                                                                const uint32_t* __restrict__ kstart,
                                                                const int64_t* __restrict__ actual) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 4 + uniform(static_cast<int>(threadIdx.x) / kWave);
  if (i >= uniform64(*actual)) return;
  const uint32_t s = uniform(inv[i]);
  const uint32_t lane = lane_id();
  const uint32_t pk = packed[s];  // used after the row loads are issued
  const uint8_t* src = slot_row(a, s);
  uint8_t* dst = a.y + i * a.row_bytes;
  const int64_t n16 = a.row_bytes >> 4;
  RowPiece<VEC> first;
  if (VEC != 1) first.load(src, n16, 0, lane);
  const uint32_t c = s / static_cast<uint32_t>(a.chunk);
  const uint32_t gstart = kstart[pk >> 16];
  const int32_t ses = a.session_ids ? a.session_ids[c] : static_cast<int32_t>(c);
  const int32_t mb = a.micro_batch_ids ? a.micro_batch_ids[c] : 0;
  if (lane == 0) {
    a.token_ids[i] = static_cast<int32_t>(s);
    a.offsets[i] = static_cast<int32_t>(static_cast<uint32_t>(i) - gstart);
    a.session_out[i] = ses;
    a.mb_out[i] = mb;
    if (a.dyn_scale != nullptr) a.dyn_scale[i] = load_scale(slot_scale(a, s));
  }
  if (VEC != 1) {
    first.store(dst, n16, 0, lane);
    copy_row_rest<VEC>(src, dst, a.row_bytes, kWave * kPiece, lane);
  } else {
    copy_row_rest<VEC>(src, dst, a.row_bytes, 0, lane);
  }
}

// ------------------------------------------------------------------ host side

SortPass make_pass(int64_t n, int nb, int nbits, int shift) {
  SortPass p;
  p.n = n;
  p.nb = nb;
  p.nbits = nbits;
  p.shift = shift;
  const int64_t tiles4 = (n + 1023) / 1024;
  p.R = (static_cast<int64_t>(nb) * tiles4 <= 65536) ? 4 : 16;
  const int64_t tile = 256 * p.R;
  p.nt = static_cast<int>((n + tile - 1) / tile);
  p.tile_shift = (p.R == 4) ? 10 : 12;
  return p;
}

SortPlan make_sort_plan(int64_t n, uint64_t nkeys) {
  SortPlan sp;
  if (nkeys <= 1) nkeys = 1;
  const int B = bits_for(nkeys - 1);
  if (nkeys <= static_cast<uint64_t>(kMaxSinglePassBuckets)) {
    sp.npasses = 1;
    sp.pass[0] = make_pass(n, static_cast<int>(nkeys), B, 0);
  } else {
    int P = (B + 12) / 13;
    if (P < 2) P = 2;
    const int D = (B + P - 1) / P;
    sp.npasses = P;
    for (int i = 0; i < P; ++i) {
      const int shift = i * D;
      const int bits = (shift + D <= B) ? D : (B - shift);
      const uint64_t top = ((nkeys - 1) >> shift);
      const int nb = (i == P - 1) ? static_cast<int>(top + 1) : (1 << bits);
      sp.pass[i] = make_pass(n, nb, bits, shift);
    }
  }
  for (int i = 0; i < sp.npasses; ++i) {
    const int64_t w = static_cast<int64_t>(sp.pass[i].nb) * sp.pass[i].nt;
    if (w > sp.hist_words) sp.hist_words = w;
    if (sp.pass[i].nb > sp.max_nb) sp.max_nb = sp.pass[i].nb;
  }
  return sp;
}


int plan_batching(const ffnwb_batching_desc* d, BatchingPlan* p, bool from_context) {
  if (d == nullptr || p == nullptr) return FFNWB_ERR_PARAM_NULLPTR;
  if (!from_context && (d->token_data == nullptr || d->expert_ids == nullptr)) return FFNWB_ERR_PARAM_NULLPTR;
  if (d->y == nullptr || d->session_ids_out == nullptr ||
      d->micro_batch_ids_out == nullptr || d->token_ids == nullptr || d->expert_offsets == nullptr ||
      d->group_list == nullptr || d->actual_token_num == nullptr)
    return FFNWB_ERR_PARAM_NULLPTR;
  if (d->token_dtype != FFNWB_DT_FP16 && d->token_dtype != FFNWB_DT_BF16 && d->token_dtype != FFNWB_DT_INT8)
    return FFNWB_ERR_PARAM_INVALID;
  const bool int8 = d->token_dtype == FFNWB_DT_INT8;
  if (int8 && d->dynamic_scale == nullptr) return FFNWB_ERR_PARAM_NULLPTR;
  if (d->need_schedule != 0) return FFNWB_ERR_PARAM_INVALID;
  if (d->expert_num <= 0 || d->expert_num > kMaxExperts) return FFNWB_ERR_PARAM_INVALID;
  if (d->A <= 0 || d->A > 1024 || d->BS <= 0 || d->K1 <= 0 || d->K1 > 64 || d->H <= 0)
    return FFNWB_ERR_PARAM_INVALID;
  if (d->layer_num < 0 || d->layer_num > d->expert_num) return FFNWB_ERR_PARAM_INVALID;
  const int64_t L = d->layer_num > 1 ? d->layer_num : 1;
  if (d->expert_num % L != 0) return FFNWB_ERR_PARAM_INVALID;
  if (d->BS > (int64_t{1} << 31) / (d->A * d->K1)) return FFNWB_ERR_PARAM_INVALID;
  const int64_t Y = d->A * d->BS * d->K1;
  if (Y >= (int64_t{1} << 31)) return FFNWB_ERR_PARAM_INVALID;
  if (d->H > (int64_t{1} << 40)) return FFNWB_ERR_PARAM_INVALID;
  const int64_t row = d->H * (int8 ? 1 : 2);
  const bool packed_scale = int8 && d->token_scale == nullptr;
  const int64_t min_stride = row + (packed_scale ? 4 : 0);
  const int64_t stride = d->token_row_stride ? d->token_row_stride : min_stride;
  if (stride < min_stride) return FFNWB_ERR_PARAM_INVALID;
  if (int8 && !packed_scale && d->scale_stride < 0) return FFNWB_ERR_PARAM_INVALID;
  // output rows are addressed with 32-bit row numbers times the row size
  if (static_cast<double>(Y) * static_cast<double>(stride) > 9.0e18) return FFNWB_ERR_PARAM_INVALID;

  p->Y = Y;
  p->row_bytes = row;
  p->stride = stride;
  if (int8) {
    if (packed_scale) {
      p->scale_base = from_context ? nullptr : static_cast<const uint8_t*>(d->token_data) + row;
      p->scale_stride = stride;
    } else {
      p->scale_base = reinterpret_cast<const uint8_t*>(d->token_scale);
      p->scale_stride = d->scale_stride ? d->scale_stride : 4;
    }
  }
  const int nb = static_cast<int>(d->expert_num);
  p->pass = make_pass(Y, nb, bits_for(static_cast<uint64_t>(nb - 1)), 0);
  const uintptr_t base = from_context ? 0 : reinterpret_cast<uintptr_t>(d->token_data);
  p->vec = vec_class(base, reinterpret_cast<uintptr_t>(d->y), stride, row, row);
  p->small = (p->pass.nt == 1) && p->pass.R == 4 && nb <= 4096 && Y * row <= (int64_t{1} << 22);
  // the slot key reads three inputs, so the one-launch order pays off only for moderate
  // slot counts (measured crossover with the rank / scan / gather path: ~8K slots)
  p->wg_order = !p->small && Y <= kWgMaxSlots && nb <= kWgMaxKeys;
  p->range_order = !p->small && !p->wg_order && ro_fits(Y, static_cast<uint64_t>(nb), kBatchingRangeMaxSlots);
  p->place = !p->small && !p->wg_order && !p->range_order && p->pass.nt <= kPlaceMaxTiles;
  if (p->small) {
    p->ws_bytes = 0;
  } else if (p->wg_order || p->range_order) {
    Carve c;
    c.take<uint32_t>(Y);                                              // output row of every slot
    if (p->wg_order) c.take<uint32_t>(Y);                             // ... and its group's first row
    p->ws_bytes = c.off;
  } else {
    Carve c;
    c.take<uint32_t>(Y);                                              // packed digit / rank
    c.take<uint32_t>(static_cast<size_t>(nb) * p->pass.nt);           // histogram -> offsets
    c.take<uint32_t>(static_cast<size_t>(nb) + 1);                    // key starts
    c.take<uint32_t>(p->pass.nt);                                     // per-tile bad-id counts
    if (p->place) c.take<uint32_t>(Y);                                // slot of every output row
    p->ws_bytes = c.off;
  }
  return FFNWB_OK;
}

template <class F>
static hipError_t launch_vec(int vec, F&& f) {
  if (vec == 16) f(std::integral_constant<int, 16>());
  else if (vec == 4) f(std::integral_constant<int, 4>());
  else f(std::integral_constant<int, 1>());
  return hipGetLastError();
}

int launch_batching(const ffnwb_batching_desc* d, const BatchingPlan& p, void* ws, hipStream_t s,
                    const uint64_t* chunk_src) {
  BatchArgs a{};
  a.Y = p.Y;
  a.chunk = d->BS * d->K1;
  a.L = static_cast<int32_t>(d->layer_num > 1 ? d->layer_num : 1);
  a.per_layer = static_cast<int32_t>(d->expert_num / a.L);
  a.layer_num = static_cast<int32_t>(d->layer_num);
  a.expert_ids = d->expert_ids;
  a.has_mask = d->mask != nullptr;
  a.use_layers = d->layer_ids != nullptr && d->layer_num >= 1;
  // absent inputs point at expert_ids (Y readable words, and A <= Y): loads stay unconditional
  a.mask = a.has_mask ? d->mask : reinterpret_cast<const uint8_t*>(d->expert_ids);
  a.layer_ids = a.use_layers ? d->layer_ids : d->expert_ids;
  a.session_ids = d->session_ids;
  a.micro_batch_ids = d->micro_batch_ids;
  a.token_data = static_cast<const uint8_t*>(d->token_data);
  a.stride = p.stride;
  a.scale_base = p.scale_base;
  a.scale_stride = p.scale_stride;
  a.y = static_cast<uint8_t*>(d->y);
  a.row_bytes = p.row_bytes;
  a.session_out = d->session_ids_out;
  a.mb_out = d->micro_batch_ids_out;
  a.token_ids = d->token_ids;
  a.offsets = d->expert_offsets;
  a.dyn_scale = (d->token_dtype == FFNWB_DT_INT8) ? d->dynamic_scale : nullptr;
  a.chunk_src = chunk_src;
  const int nb = p.pass.nb;
  hipError_t err = hipSuccess;

  if (p.small) {
    const size_t lds = rank_lds_bytes(nb) + (static_cast<size_t>(nb) + 1 + 1024) * sizeof(uint32_t);
    bool launched = false;
    err = launch_vec(p.vec, [&](auto v) {
      launched = launch_bound(batching_small_kernel<decltype(v)::value>, dim3(1), dim3(kRankThreads), lds, s,
                              d->ev_gather_begin, d->ev_gather_end, a, p.pass.nbits, nb, d->group_list,
                              d->expert_num, d->actual_token_num, d->err_count);
    });
    if (!launched) return FFNWB_ERR_RUNTIME;
    return err == hipSuccess ? FFNWB_OK : FFNWB_ERR_RUNTIME;
  }

  Carve c;
  c.base = static_cast<char*>(ws);
  if (p.wg_order) {
    uint32_t* pos_of = c.take<uint32_t>(p.Y);
    uint32_t* first_of = c.take<uint32_t>(p.Y);
    const size_t lds = static_cast<size_t>(kWgWaves + 4) * rank_lds_stride(nb) * sizeof(uint16_t) +
                       static_cast<size_t>(nb) * sizeof(uint32_t);
    // as few rounds per wave as the slots need (the ranking's time grows with them)
    const int rounds = static_cast<int>((p.Y + kWgThreads - 1) / kWgThreads);
    auto go = [&](auto rc) {
      constexpr int R = decltype(rc)::value;
      allow_large_lds(reinterpret_cast<const void*>(&batching_wg_order_kernel<R>), lds);
      hipLaunchKernelGGL(batching_wg_order_kernel<R>, dim3(1), dim3(kWgThreads), lds, s, a, p.pass.nbits, nb, pos_of,
                         first_of, d->group_list, d->expert_num, d->actual_token_num, d->err_count);
    };
    switch (rounds) {
      case 1: go(std::integral_constant<int, 1>()); break;
      case 2: go(std::integral_constant<int, 2>()); break;
      case 3: go(std::integral_constant<int, 3>()); break;
      case 4: go(std::integral_constant<int, 4>()); break;
      case 5: go(std::integral_constant<int, 5>()); break;
      case 6: go(std::integral_constant<int, 6>()); break;
      case 7: go(std::integral_constant<int, 7>()); break;
      default: go(std::integral_constant<int, 8>()); break;
    }
    if ((err = hipGetLastError()) != hipSuccess) return FFNWB_ERR_RUNTIME;
    const unsigned blocks = static_cast<unsigned>((p.Y + 3) / 4);
    bool launched = false;
    err = launch_vec(p.vec, [&](auto v) {
      launched = launch_bound(batching_copy_kernel<decltype(v)::value>, dim3(blocks), dim3(256), 0, s,
                              d->ev_gather_begin, d->ev_gather_end, a, static_cast<const uint32_t*>(pos_of),
                              static_cast<const uint32_t*>(first_of));
    });
    if (!launched) return FFNWB_ERR_RUNTIME;
    return err == hipSuccess ? FFNWB_OK : FFNWB_ERR_RUNTIME;
  }
  if (p.range_order) {
    uint32_t* pos_of = c.take<uint32_t>(p.Y);
    const RoPlan rp = ro_plan(static_cast<uint64_t>(nb), kRoGroups);
    const size_t lds = (ro_lds_words(rp.kr) + nb + rp.kr + 2 * static_cast<size_t>(d->A)) * sizeof(uint32_t);
    allow_large_lds(reinterpret_cast<const void*>(&batching_order_kernel), lds);
    hipLaunchKernelGGL(batching_order_kernel, dim3(rp.grid), dim3(kRoThreads), lds, s, a, static_cast<uint32_t>(nb),
                       rp.kr, rp.nbits, pos_of, d->group_list, d->expert_num, d->actual_token_num, d->err_count);
    if ((err = hipGetLastError()) != hipSuccess) return FFNWB_ERR_RUNTIME;
    const unsigned blocks = static_cast<unsigned>((p.Y + 3) / 4);
    bool launched = false;
    err = launch_vec(p.vec, [&](auto v) {
      launched = launch_bound(batching_copy_kernel<decltype(v)::value>, dim3(blocks), dim3(256), 0, s,
                              d->ev_gather_begin, d->ev_gather_end, a, static_cast<const uint32_t*>(pos_of),
                              static_cast<const uint32_t*>(nullptr));
    });
    if (!launched) return FFNWB_ERR_RUNTIME;
    return err == hipSuccess ? FFNWB_OK : FFNWB_ERR_RUNTIME;
  }
  uint32_t* packed = c.take<uint32_t>(p.Y);
  uint32_t* hist = c.take<uint32_t>(static_cast<size_t>(nb) * p.pass.nt);
  uint32_t* kstart = c.take<uint32_t>(static_cast<size_t>(nb) + 1);
  uint32_t* tile_err = c.take<uint32_t>(p.pass.nt);

  KeyBatching ks{a};
  const size_t lds = rank_lds_bytes(nb);
  allow_large_lds(reinterpret_cast<const void*>(p.pass.R == 4 ? &sort_rank_kernel<4, KeyBatching>
                                                               : &sort_rank_kernel<16, KeyBatching>), lds);
  if (p.pass.R == 4)
    hipLaunchKernelGGL((sort_rank_kernel<4, KeyBatching>), dim3(p.pass.nt), dim3(kRankThreads), lds, s, ks, p.Y, 0,
                       p.pass.nbits, nb, packed, hist, tile_err);
  else
    hipLaunchKernelGGL((sort_rank_kernel<16, KeyBatching>), dim3(p.pass.nt), dim3(kRankThreads), lds, s, ks, p.Y, 0,
                       p.pass.nbits, nb, packed, hist, tile_err);
  if ((err = hipGetLastError()) != hipSuccess) return FFNWB_ERR_RUNTIME;

  if (p.place) {
    uint32_t* inv = c.take<uint32_t>(p.Y);
    const size_t plds = 2 * static_cast<size_t>(nb) * sizeof(uint32_t);
    auto place = [&](auto bc) {
      constexpr int B = decltype(bc)::value;
      allow_large_lds(reinterpret_cast<const void*>(&batching_place_kernel<B>), plds);
      hipLaunchKernelGGL(batching_place_kernel<B>, dim3(p.pass.nt), dim3(kWgThreads), plds, s, a,
                         static_cast<const uint32_t*>(packed), static_cast<const uint32_t*>(hist),
                         static_cast<const uint32_t*>(tile_err), nb, p.pass.nt, p.pass.tile_shift, inv, kstart,
                         d->group_list, d->expert_num, d->actual_token_num, d->err_count);
    };
    // as many histogram loads in flight as there are tiles (clamped duplicates cost
    // L2-to-CU bandwidth: 64 loads for 36 tiles measured 9-11 us, 40 loads 7.3 us)
    const int nt = p.pass.nt;
    if (nt <= 8) place(std::integral_constant<int, 8>());
    else if (nt <= 16) place(std::integral_constant<int, 16>());
    else if (nt <= 24) place(std::integral_constant<int, 24>());
    else if (nt <= 32) place(std::integral_constant<int, 32>());
    else if (nt <= 40) place(std::integral_constant<int, 40>());
    else if (nt <= 48) place(std::integral_constant<int, 48>());
    else place(std::integral_constant<int, 64>());
    if ((err = hipGetLastError()) != hipSuccess) return FFNWB_ERR_RUNTIME;
    const unsigned blocks = static_cast<unsigned>((p.Y + 3) / 4);
    bool launched = false;
    err = launch_vec(p.vec, [&](auto v) {
      launched = launch_bound(batching_copy_out_kernel<decltype(v)::value>, dim3(blocks), dim3(256), 0, s,
                              d->ev_gather_begin, d->ev_gather_end, a, static_cast<const uint32_t*>(inv),
                              static_cast<const uint32_t*>(packed), static_cast<const uint32_t*>(kstart),
                              static_cast<const int64_t*>(d->actual_token_num));
    });
    if (!launched) return FFNWB_ERR_RUNTIME;
    return err == hipSuccess ? FFNWB_OK : FFNWB_ERR_RUNTIME;
  }

  ScanTail tail{d->group_list, d->expert_num, d->actual_token_num, d->err_count, tile_err};
  const size_t scan_lds = scan_lds_bytes(nb);
  allow_large_lds(reinterpret_cast<const void*>(&scan_hist_kernel), scan_lds);
  hipLaunchKernelGGL(scan_hist_kernel, dim3(1), dim3(kScanThreads), scan_lds, s, hist, nb, p.pass.nt, kstart,
                     static_cast<uint32_t*>(nullptr), tail);
  if ((err = hipGetLastError()) != hipSuccess) return FFNWB_ERR_RUNTIME;

  const Placement pl{packed, hist, kstart, nb, p.pass.tile_shift};
  const unsigned blocks = static_cast<unsigned>((p.Y + 3) / 4);
  bool launched = false;
  err = launch_vec(p.vec, [&](auto v) {
    launched = launch_bound(batching_gather_kernel<decltype(v)::value>, dim3(blocks), dim3(256), 0, s,
                            d->ev_gather_begin, d->ev_gather_end, a, pl);
  });
  if (!launched) return FFNWB_ERR_RUNTIME;
  return err == hipSuccess ? FFNWB_OK : FFNWB_ERR_RUNTIME;
}

}  // namespace ffnwb

// Range-partitioned stable counting sort: a whole ordering in one launch, for element
// counts up to a few hundred thousand.
//
// Workgroup b owns the keys [lo, lo + kr) and reads every element once.  It never needs
// another workgroup's counts: the number of elements that sort before its keys is
// counted directly, so no histogram, scan or second launch is involved.  Wave w of a
// workgroup owns the contiguous slice [w*per, (w+1)*per) of the elements.
//   pass 1  each lane counts the elements whose key is below lo; each wave counts its
//           slice's elements of every owned key (LDS atomics: the counts do not depend
//           on the order of the additions) and appends them, in element order, to a
//           wave-private list (position = owned elements of lower lanes, from 4
//           ballots, plus those earlier in the lane);
//   middle  per owned key, prefixes over the waves; one exclusive scan over
//           [below counts of all lanes | owned key totals] gives the first output
//           position of every owned key;
//   pass 2  each wave ranks its list, 64 entries a round: the lanes with equal keys are
//           matched with one ballot per key bit, and each lane's position is the wave's
//           running counter of its key plus the number of equal lanes below it.  A wave
//           whose list overflowed reads its slice again instead, with the same ranking.
// Ties keep input order: slices in wave order, entries in order, lanes in order.
// Keys are read 4 consecutive elements per lane (16-byte loads).
#pragma once

#include "sort_engine.hpp"

namespace ffnwb {

constexpr int kRoWaves = 16;
constexpr int kRoThreads = kRoWaves * kWave;  // 1024
constexpr int kRoMaxKeys = kRoThreads;        // owned keys per workgroup: one per thread in the middle step
constexpr int kRoVec = 4;                     // consecutive elements per lane per block (one 16-byte load)
constexpr int kRoBlock = kWave * kRoVec;      // elements per wave per block
constexpr int kRoUnroll = 4;                  // blocks whose loads are issued together
constexpr int64_t kRoMaxElems = int64_t{1} << 18;  // above this, the multi-launch sort is cheaper
constexpr unsigned kRoGroups = 128;                 // workgroups aimed at (each reads every element)
constexpr uint32_t kRoOut = 0xffffffffu;            // transposed digit of an element not owned

// Whether an ordering of n elements over nkeys keys takes the range-partitioned path:
// at most max_elems elements (every workgroup reads all of them, so the launch's time
// grows with n while the multi-launch sort's grows far more slowly), and at most
// 2 * kRoGroups workgroups of kRoMaxKeys keys.
__host__ __device__ inline bool ro_fits(int64_t n, uint64_t nkeys, int64_t max_elems = kRoMaxElems) {
  return n <= max_elems && max_elems <= kRoMaxElems && nkeys <= static_cast<uint64_t>(kRoMaxKeys) * 2 * kRoGroups;
}

// Slice [b, e) of wave w: whole blocks, the last slices possibly short or empty.  Element
// indices are 32-bit: n <= kRoMaxElems.
__device__ __forceinline__ void ro_slice(uint32_t n, int w, uint32_t& b, uint32_t& e) {
  const uint32_t per = ((n + kRoWaves - 1) / kRoWaves + kRoBlock - 1) / kRoBlock * kRoBlock;
  b = min(n, static_cast<uint32_t>(w) * per);
  e = min(n, b + per);
}

// Key sources give the keys of 4 consecutive elements j0..j0+3 (j0 a multiple of 4):
//   key4(j0, key, valid, err)
// loading every element in range of the array (a clamped index past its end), with
// one 16-byte load where the array is 16-byte aligned.

// Padded unpermute: key = token id, ids outside [0, T) share the last key T.
struct RoKeysPadded {
  const int32_t* sI;
  int32_t T;
  uint32_t n;
  __device__ __forceinline__ void key4(uint32_t j0, uint32_t (&k)[kRoVec], bool (&v)[kRoVec],
                                       bool (&er)[kRoVec]) const {
    int32_t x[kRoVec];
    if (j0 + kRoVec <= n && (reinterpret_cast<uintptr_t>(sI) & 15) == 0) {
      const int4 q = *reinterpret_cast<const int4*>(sI + j0);
      x[0] = q.x; x[1] = q.y; x[2] = q.z; x[3] = q.w;
    } else {
#pragma unroll
      for (int i = 0; i < kRoVec; ++i) x[i] = sI[min(j0 + i, n - 1)];
    }
#pragma unroll
    for (int i = 0; i < kRoVec; ++i) {
      k[i] = (x[i] >= 0 && x[i] < T) ? static_cast<uint32_t>(x[i]) : static_cast<uint32_t>(T);
      v[i] = true;
      er[i] = false;
    }
  }
};

// Per-wave LDS views of a range-order workgroup.
constexpr int kRoListCap = 768;  // owned elements a wave keeps for pass 2
constexpr int kRoKeyBits = 10;   // list entry = (element << kRoKeyBits) | (key - lo); kRoMaxKeys = 1 << 10
static_assert(kRoMaxKeys <= (1 << kRoKeyBits), "owned key index must fit a list entry");
static_assert(kRoMaxElems <= (int64_t{1} << (32 - kRoKeyBits)), "element index must fit a list entry");

struct RoWave {
  uint32_t* cnt;   // [kr] owned-key counters, then running positions
  uint32_t* list;  // [kRoListCap] owned elements in element order
  uint32_t* tbuf;  // [kRoBlock] transpose buffer of the overflow path
};

// LDS layout: transpose buffers [kRoWaves][kRoBlock] | lists [kRoWaves][kRoListCap] |
// counters [kRoWaves][kr]; `extra` words follow for the kernel's own use.
__host__ __device__ inline size_t ro_lds_words(uint32_t kr) {
  return static_cast<size_t>(kRoWaves) * (kRoBlock + kRoListCap + kr);
}
__device__ __forceinline__ RoWave ro_wave(uint32_t* lds, int w, uint32_t kr) {
  RoWave v;
  v.tbuf = lds + w * kRoBlock;
  v.list = lds + kRoWaves * kRoBlock + w * kRoListCap;
  v.cnt = lds + kRoWaves * (kRoBlock + kRoListCap) + w * kr;
  return v;
}
__device__ __forceinline__ uint32_t* ro_counters(uint32_t* lds) { return lds + kRoWaves * (kRoBlock + kRoListCap); }

// Pass 1 over this wave's slice.  Returns the lane's count of elements with key < lo;
// `len` = the wave's number of owned elements (uniform).  seen(j, key, valid, err) is
// called for every element of the slice (j < e).
// U blocks of loads are issued together (the default kRoUnroll, or a whole slice's
// worth where registers allow).
template <int U = kRoUnroll, class KS, class Seen>
__device__ __forceinline__ uint32_t ro_count(const KS& ks, uint32_t b, uint32_t e, uint32_t lo, uint32_t kr,
                                             const RoWave& wv, uint32_t& len, Seen seen) {
  const uint32_t lane = lane_id();
  uint32_t below = 0;
  uint32_t n_own = 0;
  for (uint32_t j0 = b; j0 < e; j0 += U * kRoBlock) {
    uint32_t key[U][kRoVec];
    bool v[U][kRoVec], er[U][kRoVec];
#pragma unroll
    for (int u = 0; u < U; ++u) ks.key4(j0 + u * kRoBlock + lane * kRoVec, key[u], v[u], er[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t jl = j0 + u * kRoBlock + lane * kRoVec;
      bool own[kRoVec];
#pragma unroll
      for (int i = 0; i < kRoVec; ++i) {
        const bool in = jl + i < e;
        const bool ok = in && v[u][i];
        below += (ok && key[u][i] < lo) ? 1u : 0u;
        own[i] = ok && (key[u][i] - lo) < kr;  // unsigned: keys below lo wrap above kr
        if (in) seen(jl + i, key[u][i], v[u][i], er[u][i]);
      }
      uint64_t bal[kRoVec];
#pragma unroll
      for (int i = 0; i < kRoVec; ++i) bal[i] = wave_ballot(own[i]);
      if ((bal[0] | bal[1] | bal[2] | bal[3]) == 0) continue;  // uniform
      uint32_t at = n_own;
#pragma unroll
      for (int i = 0; i < kRoVec; ++i) at += count_below(bal[i]);
#pragma unroll
      for (int i = 0; i < kRoVec; ++i) {
        if (bal[i] == 0) continue;  // uniform: most sub-elements own nothing in the wave
        if (own[i]) {
          const uint32_t d = key[u][i] - lo;
          atomicAdd(&wv.cnt[d], 1u);
          if (at < static_cast<uint32_t>(kRoListCap)) wv.list[at] = ((jl + i) << kRoKeyBits) | d;
        }
        at += own[i] ? 1u : 0u;
      }
#pragma unroll
      for (int i = 0; i < kRoVec; ++i) n_own += static_cast<uint32_t>(__popcll(bal[i]));
    }
  }
  len = n_own;
  return below;
}

// Middle step, called by every thread after pass 1 (`cnt` = the counter region, laid
// out [wave][kr]).  Turns cnt[w*kr + k] into the running position of key lo+k for wave
// w and returns, for thread k < kr, the first position of key lo+k; key_count = its
// element count (thread k), end = the position after the owned keys.  `wsum` holds
// 2 * kRoWaves + 1 words; it is free again when this returns (the last barrier of the
// scan follows every read of it).
__device__ __forceinline__ uint32_t ro_middle(uint32_t* cnt, uint32_t kr, uint32_t below, uint32_t* wsum,
                                              uint32_t& key_count, uint32_t& end) {
  __syncthreads();
  const uint32_t k = threadIdx.x;
  // all 16 counters are read before any is written back: with kr unknown at compile
  // time, a read-modify-write per wave could not be reordered and cost 16 serial LDS
  // round trips per key, twice
  uint32_t pre[kRoWaves];
  uint32_t tot = 0;
  if (k < kr) {
    uint32_t c[kRoWaves];
#pragma unroll
    for (int w = 0; w < kRoWaves; ++w) c[w] = cnt[w * kr + k];
#pragma unroll
    for (int w = 0; w < kRoWaves; ++w) {
      pre[w] = tot;
      tot += c[w];
    }
  }
  // sequence 0: lanes' below counts, sequence 1: key totals -> v[1] = first position of key k
  uint32_t v[2] = {below, tot};
  block_exscan_multi<kRoThreads, 2>(v, wsum, end);
  if (k < kr) {
#pragma unroll
    for (int w = 0; w < kRoWaves; ++w) cnt[w * kr + k] = pre[w] + v[1];
  }
  __syncthreads();
  key_count = tot;
  return v[1];
}

// Ranks one round of owned elements: `in` lanes hold digit d (key - lo) of element j.
template <class Emit>
__device__ __forceinline__ void ro_rank_round(bool in, uint32_t d, uint32_t j, uint32_t lo, int nbits, uint32_t* run,
                                              Emit& emit) {
  uint64_t peers = wave_ballot(in);
  if (peers == 0) return;  // uniform
  for (int bb = 0; bb < nbits; ++bb) {
    const bool bit = (d >> bb) & 1u;
    const uint64_t m = wave_ballot(bit);
    peers &= bit ? m : ~m;
  }
  uint32_t base = 0;
  if (in) base = run[d];
  const uint32_t nb_below = count_below(peers);
  if (in && nb_below == 0) run[d] = base + static_cast<uint32_t>(__popcll(peers));
  if (in) emit(j, lo + d, base + nb_below);
  wave_lds_sync();
}

// Pass 2 of this wave: emit(j, key, pos) for every owned element, in element order.
template <class KS, class Emit>
__device__ __forceinline__ void ro_place(const KS& ks, uint32_t b, uint32_t e, uint32_t lo, uint32_t kr, int nbits,
                                         const RoWave& wv, uint32_t len, Emit emit) {
  const uint32_t lane = lane_id();
  if (len <= static_cast<uint32_t>(kRoListCap)) {
    for (uint32_t r0 = 0; r0 < len; r0 += kWave) {
      const uint32_t idx = r0 + lane;
      const bool in = idx < len;
      const uint32_t ent = wv.list[in ? idx : 0];
      ro_rank_round(in, ent & ((1u << kRoKeyBits) - 1u), ent >> kRoKeyBits, lo, nbits, wv.cnt, emit);
    }
    return;
  }
  // overflow: read the slice again; a block's digits are transposed through tbuf so that
  // sub-round r holds elements r*64 + lane of the block (element order)
  for (uint32_t j0 = b; j0 < e; j0 += kRoUnroll * kRoBlock) {
    uint32_t key[kRoUnroll][kRoVec];
    bool v[kRoUnroll][kRoVec], er[kRoUnroll][kRoVec];
#pragma unroll
    for (int u = 0; u < kRoUnroll; ++u) ks.key4(j0 + u * kRoBlock + lane * kRoVec, key[u], v[u], er[u]);
#pragma unroll
    for (int u = 0; u < kRoUnroll; ++u) {
      const uint32_t jb = j0 + u * kRoBlock;
      uint32_t dg[kRoVec];
      bool any = false;
#pragma unroll
      for (int i = 0; i < kRoVec; ++i) {
        const bool in = v[u][i] && jb + lane * kRoVec + i < e && (key[u][i] - lo) < kr;
        dg[i] = in ? key[u][i] - lo : kRoOut;
        any = any || in;
      }
      if (wave_ballot(any) == 0) continue;  // uniform
#pragma unroll
      for (int i = 0; i < kRoVec; ++i) wv.tbuf[lane * kRoVec + i] = dg[i];
      wave_lds_sync();
#pragma unroll
      for (int r = 0; r < kRoVec; ++r) {
        const uint32_t d = wv.tbuf[r * kWave + lane];
        ro_rank_round(d != kRoOut, d, jb + r * kWave + lane, lo, nbits, wv.cnt, emit);
      }
    }
  }
}

// Host: owned keys per workgroup and grid for nkeys keys, aiming at `groups` workgroups.
struct RoPlan {
  uint32_t kr = 1;
  int nbits = 0;
  unsigned grid = 1;
};

inline RoPlan ro_plan(uint64_t nkeys, unsigned groups) {
  RoPlan r;
  if (nkeys == 0) nkeys = 1;
  uint64_t kr = (nkeys + groups - 1) / groups;
  if (kr < 1) kr = 1;
  if (kr > static_cast<uint64_t>(kRoMaxKeys)) kr = kRoMaxKeys;
  r.kr = static_cast<uint32_t>(kr);
  int bits = 0;
  while ((uint64_t{1} << bits) < kr) ++bits;
  r.nbits = bits;
  r.grid = static_cast<unsigned>((nkeys + kr - 1) / kr);
  return r;
}


}  // namespace ffnwb

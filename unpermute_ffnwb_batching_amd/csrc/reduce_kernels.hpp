// Token-wise gather-reduce of the MoE token unpermute (MoeTokenUnpermuteWithRoutingMap
// article, "Function description and formulas", branches 1-4): out[t] = sum over the
// token's entries of permuted row x weight, accumulated in FP32 in entry order and
// rounded once to the token dtype.  Kept in its own header so that measurements taken
// of this kernel can name the exact source they were taken on.
#pragma once

#include "device_common.hpp"

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
  int32_t skip_zero;     // with weights: leave out terms of weight 0 (their rows are not read)
};

// One workgroup per token; each thread owns CPT 16-byte chunks of the hidden dimension
// (or single elements when rows are not 16-byte multiples).  Every wave fetches the
// token's entry list itself, one entry per lane with a single coalesced load, and marks
// the valid ones with a ballot; it then walks the valid entries in ascending order, 8 at
// a time, broadcasting each row index with readlane so that the 8 x CPT row loads of a
// batch are all in flight before the first one is used.  The weight of each entry is
// gathered per lane before the row loads and read back with readlane after them.  Row
// loads and the output stores are non-temporal: every byte is touched once.
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
      if (kHasW && a.skip_zero != 0) ok = ok && wl != 0.0f;  // uniform switch
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
    // the output row is written once and not read again here: streaming stores
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      if (cok[i]) __builtin_nontemporal_store(Chunk<TT>::narrow(acc[i]), o4 + t * chunks + cidx[i]);
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
      if (kHasW) {
        const float w = load_elem<TW>(a.w, MODE == kNonPadW1 ? ebase + k : idx);
        if (a.skip_zero != 0 && w == 0.0f) continue;
        acc = acc + load_elem<TT>(a.x, idx * a.H + h) * w;
      } else {
        acc = acc + load_elem<TT>(a.x, idx * a.H + h);
      }
    }
    store_elem<TT>(a.out, t * a.H + h, acc);
  }
}

}  // namespace ffnwb

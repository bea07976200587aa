// Host-side plans and launchers shared by the API layer and the kernel files.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ffnwb.h"

namespace ffnwb {

// gfx950 lets one workgroup address all 160 KiB of a CU's LDS.
constexpr size_t kMaxLdsBytes = 160 * 1024;
// A single counting-sort pass holds 4 waves x nb u16 counters in LDS.
constexpr int kMaxSinglePassBuckets = 20480;
constexpr int kMaxExperts = 8192;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline int bits_for(uint64_t max_value) {  // bits needed to represent values <= max_value
  int b = 0;
  while (b < 64 && (max_value >> b) != 0) ++b;
  return b;
}

// Workspace carve-out helper: records offsets while sizing, hands out pointers while launching.
struct Carve {
  size_t off = 0;
  char* base = nullptr;
  template <class T>
  T* take(size_t count) {
    const size_t o = off;
    off = align_up(off + count * sizeof(T), 256);
    return base ? reinterpret_cast<T*>(base + o) : nullptr;
  }
};

// One stable counting-sort pass over n elements with nb buckets.
struct SortPass {
  int64_t n = 0;
  int nb = 0;        // buckets of this pass
  int nbits = 0;     // digit width (ballot rounds)
  int shift = 0;     // digit = (key >> shift) & ((1 << nbits) - 1)
  int R = 4;         // rounds per wave: tile = 256 * R elements
  int nt = 0;        // tiles
  int tile_shift = 0;
};

SortPass make_pass(int64_t n, int nb, int nbits, int shift);

// A full stable sort of n keys in [0, nkeys): one pass when nkeys fits in LDS, else LSD passes.
struct SortPlan {
  int npasses = 0;
  SortPass pass[4];
  int64_t hist_words = 0;  // largest nb * nt over the passes
  int max_nb = 0;          // largest nb over the passes
};

SortPlan make_sort_plan(int64_t n, uint64_t nkeys);

struct BatchingPlan {
  int64_t Y = 0;
  int64_t row_bytes = 0;
  int64_t stride = 0;
  const uint8_t* scale_base = nullptr;
  int64_t scale_stride = 0;
  bool small = false;  // single fused workgroup
  bool place = false;        // rank, then placement by tiles (no scan launch), then a copy in output order
  bool wg_order = false;     // slot order in one 1024-thread workgroup, then a row copy
  bool range_order = false;  // slot order in one range-partitioned launch, then a row copy
  SortPass pass;
  int vec = 16;        // row copy width class: 16, 4 or 1
  size_t ws_bytes = 0;
};

// from_context: the rows and per-slot inputs come from the ScheduleContext decode, so
// their pointers are not checked here and the row base counts as 16-byte aligned (the
// decode verifies that on the device before any row is read).
int plan_batching(const ffnwb_batching_desc* d, BatchingPlan* p, bool from_context = false);
// chunk_src (context mode): device array of the address of each chunk's first row; the
// rows of a chunk follow each other `stride` bytes apart.  NULL: rows from d->token_data.
int launch_batching(const ffnwb_batching_desc* d, const BatchingPlan& p, void* ws, hipStream_t s,
                    const uint64_t* chunk_src = nullptr);

struct BatchingCtxPlan {
  BatchingPlan flat;    // the batching of the decoded slots
  size_t flat_ws = 0;   // its part of the workspace (first)
  size_t ws_bytes = 0;  // plus the decoded per-slot and per-chunk arrays
};

int plan_batching_ctx(const ffnwb_batching_ctx_desc* d, BatchingCtxPlan* p);
int launch_batching_ctx(const ffnwb_batching_ctx_desc* d, const BatchingCtxPlan& p, void* ws, hipStream_t s);

struct UnpermutePlan {
  int64_t T = 0, H = 0, N = 0, E = 0, rows = 0, K = 0, C = 0;
  bool has_probs = false;
  bool padded = false;
  int elt = 0, pelt = 0;
  bool need_aux = false;     // out_index / permute_token_id requested (non-padded)
  int64_t mask_tiles = 0;    // non-padded probs compaction: token tiles
  bool mask_fused = false;   // probs compaction in two launches (tile histogram fits LDS)
  bool range_order = false;  // padded inversion in one range-partitioned launch
  SortPlan sort;             // padded inversion, or non-padded auxiliary order
  size_t ws_bytes = 0;
};

int plan_unpermute(const moe_unpermute_desc* d, UnpermutePlan* p);
int launch_unpermute(const moe_unpermute_desc* d, const UnpermutePlan& p, void* ws, hipStream_t s);

struct PermutePlan {
  int64_t T = 0, E = 0, N = 0, K = 0, ntiles = 0;
  int64_t row_bytes = 0, stride = 0;
  bool padded = false;
  bool table = false;  // four-launch order through a [T][E] table (many experts or tiles)
  size_t ws_bytes = 0;
};

int plan_permute(const moe_permute_desc* d, PermutePlan* p);
int launch_permute(const moe_permute_desc* d, const PermutePlan& p, void* ws, hipStream_t s);

int plan_update_expert(const moe_update_expert_desc* d);
int launch_update_expert(const moe_update_expert_desc* d, hipStream_t s);

// Widest row-copy access (16, 4 or 1 bytes) that two base addresses, two strides and the
// row size all allow.
inline int vec_class(uintptr_t a, uintptr_t b, int64_t s1, int64_t s2, int64_t bytes) {
  const uint64_t m = static_cast<uint64_t>(a | b | static_cast<uint64_t>(s1) | static_cast<uint64_t>(s2) |
                                           static_cast<uint64_t>(bytes));
  if ((m & 15) == 0) return 16;
  if ((m & 3) == 0) return 4;
  return 1;
}

bool log_enabled();

// Records an optional timing event (a hipEvent_t passed as void*) on stream s.
inline bool record_event(void* ev, hipStream_t s) {
  return ev == nullptr || hipEventRecord(static_cast<hipEvent_t>(ev), s) == hipSuccess;
}

// Whether work enqueued on s is being captured into a graph (then events must be
// recorded: a captured launch keeps no events bound to it).
inline bool stream_capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &st) == hipSuccess && st != hipStreamCaptureStatusNone;
}

// Launches `kernel` on s with optional events bound to this launch: `begin` takes the
// kernel's start and `end` its completion, from the kernel's own dispatch.  A bound event
// puts no packet of its own on the stream (a recorded timing event costs several
// microseconds of stream time and its span includes them).  A lone `begin` is recorded
// on s before the launch (a lone `end` is still bound); under graph capture both are
// recorded around the launch.  Returns false when the launch or a record fails.
template <typename K, typename... Args>
inline bool launch_bound(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, void* begin, void* end,
                         Args... args) {
  if ((begin != nullptr || end != nullptr) && stream_capturing(s)) {
    if (!record_event(begin, s)) return false;
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
    if (hipGetLastError() != hipSuccess) return false;
    return record_event(end, s);
  }
  if (begin != nullptr && end != nullptr) {
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, static_cast<hipEvent_t>(begin), static_cast<hipEvent_t>(end), 0,
                          args...);
  } else {
    if (!record_event(begin, s)) return false;
    if (end != nullptr) {
      hipExtLaunchKernelGGL(kernel, grid, block, lds, s, nullptr, static_cast<hipEvent_t>(end), 0, args...);
    } else {
      hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
    }
  }
  return hipGetLastError() == hipSuccess;
}
void log_warn(const char* fmt, ...);

// Allows a kernel to be launched with more than 64 KiB of dynamic LDS (gfx950: up to 160 KiB).
inline void allow_large_lds(const void* kernel, size_t bytes) {
  if (bytes > 32768) (void)hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
}

}  // namespace ffnwb

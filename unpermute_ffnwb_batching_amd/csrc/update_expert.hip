// MoeUpdateExpert on gfx950 (its README page: "Function description", the parameter
// table, "Constraints").
//
// Every tensor may be strided (the parameter table allows non-contiguous tensors): a row
// stride per 2-D tensor, an element stride for the threshold and the active mask.
// At most BS * K = 512 * 16 = 8192 slots: one 1024-thread workgroup takes all of them,
// 8 per thread.  Its cost is three dependent load rounds (ids and scales; the table
// counts; the chosen instance ids), so every thread issues each round for all its slots
// before it uses any result.  The error count is a block sum written by one thread: no
// atomics, no clearing launch.
#include "device_common.hpp"
#include "internal.hpp"

namespace ffnwb {

constexpr int kUeThreads = 1024;
constexpr int kUePerThread = 8;   // 1024 * 8 = the largest BS * K
constexpr int kUeMaxBs = 512, kUeMaxK = 16, kUeMaxExperts = 1024, kUeMaxWorld = 768;

struct UeArgs {
  int32_t n, K, E, F;          // n = BS * K
  int32_t rank, mode;
  // strides in elements: rows of ids / table / scales / outputs, entries of thr / active
  int64_t ids_s, tab_s, sc_s, thr_s, act_s, oid_s, om_s;
  const void* ids;
  const int32_t* table;
  const void* scales;
  const float* thr;
  const uint8_t* active;
  void* out_ids;
  uint8_t* out_mask;
  int32_t* err_count;
};

struct TNone {};

template <class S> __device__ __forceinline__ float load_scale_elem(const void* p, int32_t i) {
  return load_elem<S>(p, i);
}

// Every load is unconditional, at a clamped index, with the result selected after it:
// a guarded load compiles to a branch and a wait per slot, which serialises the rounds.
template <typename IdT, class S, bool kActive>
__global__ __launch_bounds__(kUeThreads) void update_expert_kernel(UeArgs a) {
  constexpr bool kScales = !__is_same(S, TNone);
  __shared__ uint32_t wave_err[kUeThreads / kWave];
  const IdT* ids = static_cast<const IdT*>(a.ids);
  int64_t v[kUePerThread];
  float sc[kUePerThread], th[kUePerThread];
  uint8_t act[kUePerThread];
  // round 1: the slot's logical expert (and scale, threshold, token activity)
#pragma unroll
  for (int r = 0; r < kUePerThread; ++r) {
    const int32_t ic = min(static_cast<int32_t>(threadIdx.x) + r * kUeThreads, a.n - 1);
    const int64_t t = ic / a.K, k = ic - t * a.K;
    v[r] = static_cast<int64_t>(ids[t * a.ids_s + k]);
    if constexpr (kScales) {
      sc[r] = load_scale_elem<S>(a.scales, static_cast<int32_t>(t * a.sc_s + k));
      th[r] = a.thr[k * a.thr_s];
      act[r] = kActive ? a.active[t * a.act_s] : 1;
    }
  }
  // round 2: the expert's replica count (row 0 stands in for an id out of range)
  int32_t row[kUePerThread], cnt[kUePerThread];
#pragma unroll
  for (int r = 0; r < kUePerThread; ++r) {
    row[r] = (v[r] >= 0 && v[r] < a.E) ? static_cast<int32_t>(v[r]) : 0;
    cnt[r] = a.table[static_cast<int64_t>(row[r]) * a.tab_s];
  }
  // round 3: the chosen replica's instance id
  int32_t inst[kUePerThread];
  bool ok[kUePerThread];
#pragma unroll
  for (int r = 0; r < kUePerThread; ++r) {
    const int32_t i = threadIdx.x + r * kUeThreads;
    ok[r] = v[r] >= 0 && v[r] < a.E && cnt[r] >= 1 && cnt[r] <= a.F - 1;
    const int32_t c = ok[r] ? cnt[r] : 1;
    const int32_t pick = (a.mode == 0 ? a.rank : i / a.K) % c;   // < c <= F - 1
    inst[r] = a.table[static_cast<int64_t>(row[r]) * a.tab_s + 1 + pick];
  }
  uint32_t nerr = 0;
#pragma unroll
  for (int r = 0; r < kUePerThread; ++r) {
    const int32_t i = threadIdx.x + r * kUeThreads;
    if (i >= a.n) continue;
    const int64_t t = i / a.K, k = i - t * a.K;
    static_cast<IdT*>(a.out_ids)[t * a.oid_s + k] = static_cast<IdT>(ok[r] ? inst[r] : -1);
    if constexpr (kScales) a.out_mask[t * a.om_s + k] = (ok[r] && act[r] != 0 && !(sc[r] < th[r])) ? 1 : 0;
    nerr += ok[r] ? 0u : 1u;
  }
  // block sum of the error counts
  for (int off = kWave / 2; off > 0; off >>= 1) nerr += __shfl_xor(nerr, off);
  if (lane_id() == 0) wave_err[threadIdx.x / kWave] = nerr;
  __syncthreads();
  if (threadIdx.x == 0 && a.err_count != nullptr) {
    uint32_t tot = 0;
    for (int w = 0; w < kUeThreads / kWave; ++w) tot += wave_err[w];
    *a.err_count = static_cast<int32_t>(tot);
  }
}

// ------------------------------------------------------------------ host side

int plan_update_expert(const moe_update_expert_desc* d) {
  if (d == nullptr) return FFNWB_ERR_PARAM_NULLPTR;
  if (d->expert_ids == nullptr || d->eplb_table == nullptr || d->balanced_expert_ids == nullptr)
    return FFNWB_ERR_PARAM_NULLPTR;
  const bool scales = d->expert_scales != nullptr;
  if (scales != (d->pruning_threshold != nullptr)) return FFNWB_ERR_PARAM_INVALID;
  if (!scales && d->active_mask != nullptr) return FFNWB_ERR_PARAM_INVALID;
  if (scales && d->balanced_active_mask == nullptr) return FFNWB_ERR_PARAM_NULLPTR;
  if (d->reserved0 != 0) return FFNWB_ERR_PARAM_INVALID;
  if (d->id_dtype != FFNWB_DT_INT32 && d->id_dtype != FFNWB_DT_INT64) return FFNWB_ERR_PARAM_INVALID;
  if (scales && d->scale_dtype != FFNWB_DT_FP16 && d->scale_dtype != FFNWB_DT_BF16 &&
      d->scale_dtype != FFNWB_DT_FP32)
    return FFNWB_ERR_PARAM_INVALID;
  if (d->bs <= 0 || d->bs > kUeMaxBs || d->k <= 0 || d->k > kUeMaxK) return FFNWB_ERR_PARAM_INVALID;
  if (d->moe_expert_num <= 0 || d->moe_expert_num > kUeMaxExperts || d->k > d->moe_expert_num)
    return FFNWB_ERR_PARAM_INVALID;
  if (d->balance_mode != 0 && d->balance_mode != 1) return FFNWB_ERR_PARAM_INVALID;
  const int64_t wmin = d->balance_mode == 0 ? 2 : 1;
  if (d->world_size < wmin || d->world_size > kUeMaxWorld) return FFNWB_ERR_PARAM_INVALID;
  if (d->balance_mode == 0 && (d->local_rank_id < 0 || d->local_rank_id >= d->world_size))
    return FFNWB_ERR_PARAM_INVALID;
  if (d->table_cols < 2 || d->table_cols > d->world_size + 1) return FFNWB_ERR_PARAM_INVALID;
  // strides: 0 = dense; a row stride is at least its row, an element stride at least 1;
  // every element address must fit the kernels' 32-bit scale index (BS * stride < 2^31)
  const int64_t row_strides[5] = {d->expert_ids_stride, d->expert_scales_stride, d->out_ids_stride,
                                  d->out_mask_stride, d->eplb_table_stride};
  for (int i = 0; i < 5; ++i) {
    const int64_t st = row_strides[i], need = i == 4 ? d->table_cols : d->k;
    if (st != 0 && (st < need || st > (int64_t{1} << 20))) return FFNWB_ERR_PARAM_INVALID;
  }
  if (d->threshold_stride < 0 || d->threshold_stride > (int64_t{1} << 20) || d->active_mask_stride < 0 ||
      d->active_mask_stride > (int64_t{1} << 20))
    return FFNWB_ERR_PARAM_INVALID;
  return FFNWB_OK;
}

template <typename IdT, bool kActive>
static void launch_scales(const UeArgs& a, int scale_dtype, bool scales, hipStream_t s) {
  const dim3 g(1), b(kUeThreads);
  if (!scales) hipLaunchKernelGGL((update_expert_kernel<IdT, TNone, false>), g, b, 0, s, a);
  else if (scale_dtype == FFNWB_DT_FP16) hipLaunchKernelGGL((update_expert_kernel<IdT, TF16, kActive>), g, b, 0, s, a);
  else if (scale_dtype == FFNWB_DT_BF16) hipLaunchKernelGGL((update_expert_kernel<IdT, TBF16, kActive>), g, b, 0, s, a);
  else hipLaunchKernelGGL((update_expert_kernel<IdT, TF32, kActive>), g, b, 0, s, a);
}

template <typename IdT>
static void launch_ids(const UeArgs& a, int scale_dtype, bool scales, hipStream_t s) {
  if (a.active != nullptr) launch_scales<IdT, true>(a, scale_dtype, scales, s);
  else launch_scales<IdT, false>(a, scale_dtype, scales, s);
}

int launch_update_expert(const moe_update_expert_desc* d, hipStream_t s) {
  UeArgs a{};
  a.n = static_cast<int32_t>(d->bs * d->k);
  a.K = static_cast<int32_t>(d->k);
  a.E = static_cast<int32_t>(d->moe_expert_num);
  a.F = static_cast<int32_t>(d->table_cols);
  a.rank = static_cast<int32_t>(d->balance_mode == 0 ? d->local_rank_id : 0);
  a.mode = d->balance_mode;
  a.ids = d->expert_ids;
  a.table = d->eplb_table;
  a.scales = d->expert_scales;
  a.thr = d->pruning_threshold;
  a.active = d->active_mask;
  a.out_ids = d->balanced_expert_ids;
  a.out_mask = d->balanced_active_mask;
  a.err_count = d->err_count;
  a.ids_s = d->expert_ids_stride ? d->expert_ids_stride : d->k;
  a.tab_s = d->eplb_table_stride ? d->eplb_table_stride : d->table_cols;
  a.sc_s = d->expert_scales_stride ? d->expert_scales_stride : d->k;
  a.thr_s = d->threshold_stride ? d->threshold_stride : 1;
  a.act_s = d->active_mask_stride ? d->active_mask_stride : 1;
  a.oid_s = d->out_ids_stride ? d->out_ids_stride : d->k;
  a.om_s = d->out_mask_stride ? d->out_mask_stride : d->k;
  const bool scales = d->expert_scales != nullptr;
  if (d->id_dtype == FFNWB_DT_INT32) launch_ids<int32_t>(a, d->scale_dtype, scales, s);
  else launch_ids<int64_t>(a, d->scale_dtype, scales, s);
  return hipGetLastError() == hipSuccess ? FFNWB_OK : FFNWB_ERR_RUNTIME;
}

}  // namespace ffnwb

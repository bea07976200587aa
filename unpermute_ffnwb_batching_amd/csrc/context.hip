// ScheduleContext front-end of FFN-worker batching (aclnnFfnWorkerBatching API page:
// "Function description" step 1; the scheduleContext, needSchedule and maxOutShape rows of
// the parameter table; the usage example's packed ScheduleContext and FfnDataDesc).
//
// One decode launch reads the 1024-byte context on the device, checks it against the
// call, and turns the chosen chunks of the attention->FFN data area into the inputs of
// the flat batching: the expert id and mask of every slot, and the layer id, micro-batch
// id and first-row address of every chunk.  The flat batching then runs on those, its row
// copies reading each chunk's rows in place in token_data (no staging copy).
#include <string.h>

#include "device_common.hpp"
#include "internal.hpp"

namespace ffnwb {

constexpr int kCtxThreads = 256;
constexpr int kCtxFfnArea = 384;     // byte offset of FfnArea in the packed context
constexpr uint32_t kCtxMaxMicroBatches = 64;

struct CtxDecodeArgs {
  const uint8_t* ctx;
  int64_t A, BS, K1, n;      // n = BS * K1 slots per chunk
  int64_t expert_num;        // over all layers
  int64_t L;                 // max(layer_num, 1)
  int64_t stride;            // bytes from one token_data row to the next
  int32_t need_schedule;
  int32_t* expert_ids;       // [A * n]
  uint8_t* mask;             // [A * n]
  int32_t* layer_ids;        // [A]
  int32_t* micro_batch_ids;  // [A]
  uint64_t* chunk_src;       // [A]
  int32_t* status;           // [1]
};

// The context's checks, from words every thread reads alike.  Sizes are compared by
// division so that no product can overflow (A*M*n < 2^63 since A*n < 2^31 and M < 2^32).
__device__ __forceinline__ uint32_t ctx_check(const CtxDecodeArgs& a, uint32_t M, uint64_t info, uint64_t info_size,
                                              uint64_t data, uint64_t data_size, uint64_t polling) {
  const uint32_t* common = reinterpret_cast<const uint32_t*>(a.ctx);
  uint32_t st = 0;
  if (common[0] != static_cast<uint64_t>(a.A) || common[2] != static_cast<uint64_t>(a.BS) ||
      common[3] != static_cast<uint64_t>(a.K1) ||
      static_cast<uint64_t>(common[4]) * static_cast<uint64_t>(a.L) != static_cast<uint64_t>(a.expert_num))
    st |= FFNWB_CTX_SHAPE;
  if (M < 1 || M > kCtxMaxMicroBatches || polling >= M) st |= FFNWB_CTX_POLLING;
  if (info == 0 || data == 0 || (info & 3) != 0 || (data & 15) != 0) st |= FFNWB_CTX_POINTER;
  const uint64_t chunks = static_cast<uint64_t>(a.A) * M;
  const uint64_t desc_bytes = 8 + 4 * static_cast<uint64_t>(a.n);
  if (info_size / desc_bytes < chunks || data_size / static_cast<uint64_t>(a.stride) < chunks * a.n)
    st |= FFNWB_CTX_BUFFER;
  return st;
}

// One workgroup per session s; its threads decode the entries j of session s's chunk at the
// polling index.  Thread 0 reads the chunk's flag once (an acquire load, when
// need_schedule is 1), then the chunk's layer id, which it writes out itself; it hands the
// decision to the workgroup through LDS: every slot of the chunk takes that one decision, so a flag that a producer sets
// while the decode runs gives a chunk that is batched whole or not at all, never a part
// of it.  The other threads read the chunk's expert ids after the workgroup barrier, so
// after the acquire.
__global__ __launch_bounds__(kCtxThreads) void ctx_decode_kernel(CtxDecodeArgs a) {
  __shared__ int32_t s_ready;
  const uint32_t M = reinterpret_cast<const uint32_t*>(a.ctx)[1];
  const uint64_t* ffn = reinterpret_cast<const uint64_t*>(a.ctx + kCtxFfnArea);
  const uint64_t info = ffn[0], info_size = ffn[1], data = ffn[2], data_size = ffn[3], polling = ffn[4];
  const uint32_t st = ctx_check(a, M, info, info_size, data, data_size, polling);
  const int64_t s = blockIdx.x;
  const uint64_t c = static_cast<uint64_t>(s) * M + polling;  // chunk number in the data area
  const int32_t* desc = reinterpret_cast<const int32_t*>(info + c * (8 + 4 * static_cast<uint64_t>(a.n)));
  if (threadIdx.x == 0) {
    int32_t ready = 0, layer = 0;
    if (st == 0) {
      // the flag is written by the sender: the acquire orders this chunk's reads after it
      ready = a.need_schedule == 0 ||
              __hip_atomic_load(const_cast<int32_t*>(desc), __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_SYSTEM) == 1;
      if (ready) layer = desc[1];
    }
    s_ready = ready;
    if (s == 0) *a.status = static_cast<int32_t>(st);
    a.layer_ids[s] = layer;
    a.micro_batch_ids[s] = st == 0 ? static_cast<int32_t>(polling) : 0;
    a.chunk_src[s] = st == 0 ? data + c * static_cast<uint64_t>(a.n) * static_cast<uint64_t>(a.stride) : 0;
  }
  __syncthreads();
  const bool ready = s_ready != 0;
  for (int64_t j = threadIdx.x; j < a.n; j += kCtxThreads) {
    const int64_t g = s * a.n + j;
    a.expert_ids[g] = ready ? desc[2 + j] : 0;
    a.mask[g] = ready ? 0 : 1;
  }
}

// ------------------------------------------------------------------ host side

static void flat_desc(const ffnwb_batching_ctx_desc* d, ffnwb_batching_desc* f) {
  memset(f, 0, sizeof(*f));
  f->A = d->A;
  f->BS = d->BS;
  f->K1 = d->K1;
  f->H = d->H;
  f->expert_num = d->expert_num;
  f->layer_num = d->layer_num;
  f->token_dtype = d->token_dtype;
  f->need_schedule = 0;      // the decode has done the scan
  f->token_row_stride = 0;   // rows back to back; INT8 rows carry their scale
  f->y = d->y;
  f->session_ids_out = d->session_ids_out;
  f->micro_batch_ids_out = d->micro_batch_ids_out;
  f->token_ids = d->token_ids;
  f->expert_offsets = d->expert_offsets;
  f->dynamic_scale = d->dynamic_scale;
  f->group_list = d->group_list;
  f->actual_token_num = d->actual_token_num;
  f->err_count = d->err_count;
  f->ev_gather_begin = d->ev_gather_begin;
  f->ev_gather_end = d->ev_gather_end;
}

struct CtxArrays {
  int32_t* expert_ids;
  uint8_t* mask;
  int32_t* layer_ids;
  int32_t* micro_batch_ids;
  uint64_t* chunk_src;
};

static CtxArrays carve_ctx(Carve& c, int64_t Y, int64_t A) {
  CtxArrays r;
  r.expert_ids = c.take<int32_t>(Y);
  r.mask = c.take<uint8_t>(Y);
  r.layer_ids = c.take<int32_t>(A);
  r.micro_batch_ids = c.take<int32_t>(A);
  r.chunk_src = c.take<uint64_t>(A);
  return r;
}

int plan_batching_ctx(const ffnwb_batching_ctx_desc* d, BatchingCtxPlan* p) {
  if (d == nullptr || p == nullptr) return FFNWB_ERR_PARAM_NULLPTR;
  if (d->schedule_context == nullptr || d->ctx_status == nullptr) return FFNWB_ERR_PARAM_NULLPTR;
  if (d->need_schedule != 0 && d->need_schedule != 1) return FFNWB_ERR_PARAM_INVALID;
  if ((reinterpret_cast<uintptr_t>(d->schedule_context) & 7) != 0) return FFNWB_ERR_PARAM_INVALID;
  ffnwb_batching_desc f;
  flat_desc(d, &f);
  const int st = plan_batching(&f, &p->flat, true);
  if (st != FFNWB_OK) return st;
  Carve c;
  c.off = align_up(p->flat.ws_bytes, 256);
  p->flat_ws = c.off;
  (void)carve_ctx(c, p->flat.Y, d->A);
  p->ws_bytes = c.off;
  return FFNWB_OK;
}

int launch_batching_ctx(const ffnwb_batching_ctx_desc* d, const BatchingCtxPlan& p, void* ws, hipStream_t s) {
  Carve c;
  c.base = static_cast<char*>(ws);
  c.off = p.flat_ws;
  const CtxArrays arr = carve_ctx(c, p.flat.Y, d->A);

  CtxDecodeArgs a{};
  a.ctx = static_cast<const uint8_t*>(d->schedule_context);
  a.A = d->A;
  a.BS = d->BS;
  a.K1 = d->K1;
  a.n = d->BS * d->K1;
  a.expert_num = d->expert_num;
  a.L = d->layer_num > 1 ? d->layer_num : 1;
  a.stride = p.flat.stride;
  a.need_schedule = d->need_schedule;
  a.expert_ids = arr.expert_ids;
  a.mask = arr.mask;
  a.layer_ids = arr.layer_ids;
  a.micro_batch_ids = arr.micro_batch_ids;
  a.chunk_src = arr.chunk_src;
  a.status = d->ctx_status;
  hipLaunchKernelGGL(ctx_decode_kernel, dim3(static_cast<unsigned>(d->A)), dim3(kCtxThreads), 0, s, a);
  if (hipGetLastError() != hipSuccess) return FFNWB_ERR_RUNTIME;

  ffnwb_batching_desc f;
  flat_desc(d, &f);
  f.expert_ids = arr.expert_ids;
  f.mask = arr.mask;
  f.layer_ids = arr.layer_ids;
  f.micro_batch_ids = arr.micro_batch_ids;
  return launch_batching(&f, p.flat, ws, s, arr.chunk_src);
}

}  // namespace ffnwb

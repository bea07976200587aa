/*
 * ffnwb.h -- C ABI of the MI355X (gfx950) MoE token-reordering library.
 *
 * Two operations, each with the two-phase shape of the pages' aclnn interface
 * (a host-only workspace query that also validates every argument, then an
 * asynchronous launch on a caller stream):
 *
 *   ffnwb_batching  -- FFN-worker batching.  Defined by the aclnnFfnWorkerBatching
 *                      API page ("Function description" steps 2-4, the
 *                      calculation formula, the parameter and output tables,
 *                      "Constraints").
 *   moe_unpermute   -- MoE token unpermute with routing map.  Defined by the
 *                      article "MoeTokenUnpermuteWithRoutingMap 算子全解析",
 *                      section "Function description and formulas" (four
 *                      branches: padded x has-probs), "Parameters",
 *                      "Supplementary notes", "Constraints", "Return values
 *                      and error codes".
 *   ffnwb_batching_ctx -- the same batching, fed the way the API page's own interface
 *                      feeds it: a 1024-byte ScheduleContext whose FfnArea points at
 *                      the attention->FFN data area ("Function description" step 1,
 *                      the scheduleContext / needSchedule rows of the parameter table,
 *                      the usage example's packed struct definitions).
 *   moe_update_expert -- logical -> physical expert instances through a placement
 *                      table, with threshold pruning (MoeUpdateExpert README:
 *                      "Function description", the parameter table, "Constraints").
 *   moe_permute     -- the forward permute the same article names in "Operator
 *                      positioning"; its outputs are the arrangement the
 *                      unpermute's formulas invert (see its section below).
 *
 * Conventions shared by every entry point
 *   - All array pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronises; it only enqueues kernels on
 *     `stream` (a hipStream_t; NULL = the legacy default stream) and returns.
 *   - The caller allocates the workspace (device memory of the size the query
 *     returned, 256-byte aligned; FFNWB_ERR_WORKSPACE otherwise) and keeps it alive
 *     until the work on `stream` has finished.  Its contents on entry do not matter.
 *   - Inputs are read-only.  Inputs and outputs must not overlap.
 *   - Calls are stateless: the library holds no stream, event, buffer or lock of its
 *     own, so calls may run concurrently on different streams with distinct
 *     workspaces and outputs, and never wait on each other.  (moe_unpermute may
 *     also use an auxiliary stream and two events that the caller passes in.)  The
 *     one exception is moe_unpermute_noalloc, whose workspace is a device array the
 *     library holds on each GPU.
 *   - Every result is deterministic (bit-identical across runs).
 *   - Data errors inside arrays never fault: out-of-range ids / indices are
 *     treated as masked (batching) or skipped (unpermute), as documented below.
 *
 * Status codes: FFNWB_OK, or one of the values below.  Validation happens in
 * full before anything is enqueued, so an error return leaves every output
 * untouched.
 */
#ifndef FFNWB_H
#define FFNWB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FFNWB_ABI_VERSION 6

/* Status codes.  The first three take the aclnn values both pages list. */
#define FFNWB_OK                 0
#define FFNWB_ERR_PARAM_NULLPTR  161001 /* a required pointer is NULL */
#define FFNWB_ERR_PARAM_INVALID  161002 /* a type, shape or range is outside the supported set */
#define FFNWB_ERR_INNER_NULLPTR  561103 /* unpermute: topK > 512, or probs has an unsupported shape */
#define FFNWB_ERR_WORKSPACE      1      /* workspace NULL, smaller than the query returned, or not 256-byte aligned */
#define FFNWB_ERR_RUNTIME        2      /* the HIP runtime refused a launch or a device query */
#define FFNWB_ERR_SCRATCH        3      /* moe_unpermute_noalloc: the call needs more than
                                           FFNWB_NOALLOC_SCRATCH_BYTES of workspace */

/* Element types. 0..2 are the batching page's tokenDtype values. */
#define FFNWB_DT_FP16 0
#define FFNWB_DT_BF16 1
#define FFNWB_DT_INT8 2 /* batching: INT8 data with an FP32 dynamic scale per row; permute: 1-byte elements */
#define FFNWB_DT_FP32 3 /* unpermute and permute */
#define FFNWB_DT_INT32 4 /* moe_update_expert ids */
#define FFNWB_DT_INT64 5 /* moe_update_expert ids */

/* ------------------------------------------------------------------------------------------
 * FFN-worker batching (aclnnFfnWorkerBatching API page).
 *
 * Y = A * BS * K1 slots; slot s belongs to chunk a = s / (BS*K1) (one
 * (session, micro-batch) block of the attention->FFN data area).  Slot s is
 * valid when it is not masked, its expert id lies in [0, expert_num/L) and its
 * chunk's layer id lies in [0, L), L = max(layer_num, 1).  Its sort key is
 * layer * (expert_num / L) + expert_id.  Valid slots are emitted in ascending
 * key order, ties in ascending slot order (stable), as output rows
 * i = 0 .. actual_token_num-1:
 *   y[i]               = token row of slot g_i (H elements, bit copy)
 *   token_ids[i]       = g_i
 *   expert_offsets[i]  = i - (first output row of g_i's key)
 *   session_ids_out[i] = session_ids[a] (or a when session_ids is NULL)
 *   micro_batch_ids_out[i] = micro_batch_ids[a] (or 0 when NULL)
 *   dynamic_scale[i]   = scale of slot g_i (INT8 only)
 * Rows i >= actual_token_num of the per-row outputs are NOT written.
 * group_list[j] = {key_j, count_j} for the j-th present key in ascending order,
 * then {0, 0} rows up to expert_num rows; actual_token_num = sum of counts.
 * ------------------------------------------------------------------------------------------ */
typedef struct ffnwb_batching_desc {
  /* maxOutShape {A, BS, topK+1, H}: A in (0,1024], BS > 0, K1 in (0,64], H > 0. */
  int64_t A, BS, K1, H;
  int64_t expert_num;    /* experts on this device over all layers, in (0, 8192] */
  int64_t layer_num;     /* in [0, expert_num]; 0 behaves as 1; expert_num % max(layer_num,1) == 0 */
  int32_t token_dtype;   /* FFNWB_DT_FP16, FFNWB_DT_BF16 or FFNWB_DT_INT8 */
  int32_t need_schedule; /* must be 0: the caller supplies mask / layer_ids itself */

  /* Inputs. */
  const void* token_data;    /* Y rows; row s starts at token_data + s*token_row_stride (bytes) */
  int64_t token_row_stride;  /* bytes; 0 = H*elt, or H+4 for INT8 with a packed scale */
  const float* token_scale;  /* INT8: NULL = scale packed at byte H of each token row
                                (the page's contiguous layout); else scale of slot s at
                                (char*)token_scale + s*scale_stride */
  int64_t scale_stride;      /* bytes; 0 = 4 for a separate array */
  const int32_t* expert_ids; /* [Y] expert id of each slot, indexed within its layer */
  const uint8_t* mask;       /* [Y] non-zero = slot masked; NULL = no slot masked */
  const int32_t* layer_ids;  /* [A] layer of each chunk; NULL = layer 0 */
  const int32_t* session_ids;     /* [A] or NULL */
  const int32_t* micro_batch_ids; /* [A] or NULL */

  /* Outputs (all required except err_count; dynamic_scale required for INT8 only). */
  void* y;                       /* [Y, H] dense, element type token_dtype */
  int32_t* session_ids_out;      /* [Y] */
  int32_t* micro_batch_ids_out;  /* [Y] */
  int32_t* token_ids;            /* [Y] */
  int32_t* expert_offsets;       /* [Y] */
  float* dynamic_scale;          /* [Y] */
  int64_t* group_list;           /* [expert_num, 2] */
  int64_t* actual_token_num;     /* [1] */
  int32_t* err_count;            /* [1] or NULL: number of unmasked slots whose expert or layer
                                    id was out of range (such slots are dropped) */

  /* Optional timing hooks (hipEvent_t), bound to the launch of the row-gather kernel: `begin`
     takes the kernel's start and `end` its completion, from the kernel's own dispatch on
     `stream`, so the span is the kernel alone and no event packet of its own is added to
     the stream.  A lone `begin` is recorded on `stream` before the kernel instead (a lone
     `end` is still bound), and under graph capture both are recorded around it.
     NULL = not recorded. */
  void* ev_gather_begin;
  void* ev_gather_end;
} ffnwb_batching_desc;

/* Validates *d and returns the workspace size in bytes (host only, no device work).
   Errors: FFNWB_ERR_PARAM_NULLPTR (d, ws_bytes or a required array NULL),
   FFNWB_ERR_PARAM_INVALID (a range above violated). */
int ffnwb_batching_workspace_size(const ffnwb_batching_desc* d, size_t* ws_bytes);

/* Validates again, then enqueues the batching on `stream`.  `workspace` must hold at
   least the queried size and be 256-byte aligned (FFNWB_ERR_WORKSPACE otherwise; NULL
   allowed when the size is 0). */
int ffnwb_batching(const ffnwb_batching_desc* d, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * FFN-worker batching from a ScheduleContext (aclnnFfnWorkerBatching API page:
 * "Function description" step 1; the scheduleContext, needSchedule and maxOutShape rows
 * of the parameter table; the usage example's packed ScheduleContext and FfnDataDesc).
 *
 * schedule_context points at the 1024-byte context in device memory.  The library reads
 * it on the device only (no host copy, no synchronisation), at the offsets of the packed
 * definition: CommonArea at 0 (u32 session_num, micro_batch_num, micro_batch_size,
 * selected_expert_num, expert_num at 0, 4, 8, 12, 16), FfnArea at 384 (u64
 * token_info_buf, token_info_buf_size, token_data_buf, token_data_buf_size,
 * polling_index at +0, +8, +16, +24, +32).  The two FfnArea buffers are device memory.
 *
 * Data area, with M = micro_batch_num and n = BS*K1: chunk (session s, micro-batch m)
 * is chunk number s*M + m.  Its FfnDataDesc -- int32 flag, int32 layer_id, int32
 * expert_ids[n] -- starts at byte (s*M + m) * (8 + 4n) of token_info; its n rows start at
 * row (s*M + m) * n of token_data, rows back to back, each H elements (INT8: H bytes then
 * the FP32 dynamic scale).
 *
 * One call batches micro-batch m = polling_index of every session: slot s*n + j is entry
 * j of session s's chunk.  need_schedule = 1: a chunk whose flag is not 1 takes no part
 * (its slots count as masked).  Each chunk's flag is read once, with an acquire load,
 * then its layer id; every slot of the chunk follows that one read, so a flag that a
 * producer sets during the call gives a chunk batched whole or not at all.  Nothing
 * waits for a flag.  need_schedule = 0: flags are not read.  From there the results are those of
 * ffnwb_batching on the flattened slots, with session id s, micro-batch id m and token
 * id s*n + j.
 *
 * The context must agree with the call: session_num = A, micro_batch_size = BS,
 * selected_expert_num = K1, expert_num * max(layer_num, 1) = the descriptor's
 * expert_num, 1 <= micro_batch_num <= 64, polling_index < micro_batch_num, both buffer
 * pointers non-NULL, token_info 4-byte and token_data 16-byte aligned, token_info at
 * least A*M*(8 + 4n) bytes and token_data at least A*M*n rows.  Otherwise nothing is read
 * from the data area, actual_token_num = 0, group_list is all {0, 0}, err_count = 0, and
 * *ctx_status holds the FFNWB_CTX_* bits of every failed check (0 when all pass).
 * The buffer pointers must address device memory of the stated sizes: they cannot be
 * checked beyond that.
 * ------------------------------------------------------------------------------------------ */
#define FFNWB_CTX_BYTES          1024
#define FFNWB_CTX_SHAPE          1  /* session_num / micro_batch_size / selected_expert_num / expert_num */
#define FFNWB_CTX_POLLING        2  /* micro_batch_num outside [1, 64], or polling_index >= it */
#define FFNWB_CTX_POINTER        4  /* a data-area pointer is NULL or misaligned */
#define FFNWB_CTX_BUFFER         8  /* a data-area buffer is smaller than the layout needs */

typedef struct ffnwb_batching_ctx_desc {
  /* maxOutShape {A, BS, topK+1, H}, expert_num, layer_num, token_dtype: as in
     ffnwb_batching_desc. */
  int64_t A, BS, K1, H;
  int64_t expert_num;
  int64_t layer_num;
  int32_t token_dtype;
  int32_t need_schedule;          /* 0 or 1 */
  const void* schedule_context;   /* device pointer to FFNWB_CTX_BYTES bytes, 8-byte aligned */

  /* Outputs: as in ffnwb_batching_desc, plus the context check. */
  void* y;
  int32_t* session_ids_out;
  int32_t* micro_batch_ids_out;
  int32_t* token_ids;
  int32_t* expert_offsets;
  float* dynamic_scale;           /* INT8 only */
  int64_t* group_list;
  int64_t* actual_token_num;
  int32_t* err_count;             /* or NULL */
  int32_t* ctx_status;            /* [1], required: 0 or FFNWB_CTX_* bits */

  /* Optional timing hooks around the row-gather kernel, as in ffnwb_batching_desc. */
  void* ev_gather_begin;
  void* ev_gather_end;
} ffnwb_batching_ctx_desc;

/* Validates the host-side fields of *d and returns the workspace size (host only).
   Errors: FFNWB_ERR_PARAM_NULLPTR (d, ws_bytes, schedule_context or a required output
   NULL), FFNWB_ERR_PARAM_INVALID (need_schedule not 0 or 1, or a range of
   ffnwb_batching_desc violated). */
int ffnwb_batching_ctx_workspace_size(const ffnwb_batching_ctx_desc* d, size_t* ws_bytes);

/* Validates again, then enqueues the context decode and the batching on `stream`. */
int ffnwb_batching_ctx(const ffnwb_batching_ctx_desc* d, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * MoE token unpermute with routing map (MoeTokenUnpermuteWithRoutingMap article).
 *
 * T = num_tokens, H = hidden, N = num_indices, E = num_experts.
 * Non-padded mode (padded_mode = 0): topK = N / T; slot i = t*topK + k reads permuted
 *   row r = sorted_indices[i]; slots with r outside [0, num_rows) (e.g. -1) are skipped.
 *     out[t] = RNE( sum_k  f32(x[r]) * w )        (FP32 products and sums, k ascending)
 *   with w = permute_probs[r] (weight_index 0) or permute_probs[i] (weight_index 1),
 *   w = 1 without probs.  permute_probs = probs^T compacted under routing_map^T
 *   (expert-major order of the (token, expert) pairs with a non-zero map entry),
 *   zero-padded to N.  out_index = stable argsort of the slots by sorted_indices,
 *   invalid slots first; permute_token_id = out_index / topK.
 * Padded mode (padded_mode = 1): capacity C = N / E.  permute_token_id / out_index =
 *   stable sort of sorted_indices (values / source positions); entries outside [0, T)
 *   sort after all valid ones and are not accumulated.  permute_probs[i] =
 *   probs[sorted_indices[i], i / C] (0 for invalid entries).
 *     out[t] = RNE( sum_{j : permute_token_id[j] == t, j ascending} f32(x[out_index[j]]) * w )
 *   with w = permute_probs[out_index[j]], or 1 without probs.
 * Every element of out is written (+0.0 where nothing accumulates).
 * ------------------------------------------------------------------------------------------ */
typedef struct moe_unpermute_desc {
  int32_t dtype;        /* permuted / unpermuted tokens: FFNWB_DT_FP16, _BF16 or _FP32 */
  int32_t probs_dtype;  /* = dtype, or FFNWB_DT_FP32 when dtype is BF16; ignored without probs */
  int32_t padded_mode;  /* 0 = token-slot layout, 1 = expert-capacity layout */
  int32_t weight_index; /* non-padded with probs: 0 = weight of the permuted row (default),
                           1 = weight of the slot */
  int64_t num_rows;     /* rows of permuted_tokens; must equal num_indices */
  int64_t hidden;       /* H > 0 */
  int64_t num_tokens;   /* T = restoreShape[0] (= probs rows when probs are given), >= 0 */
  int64_t num_experts;  /* E = probs columns, in (0, 8192]; 0 without probs */
  int64_t num_indices;  /* N = length of sorted_indices */

  /* Inputs. */
  const void* permuted_tokens;   /* [num_rows, H] */
  const int32_t* sorted_indices; /* [N] */
  const uint8_t* routing_map;    /* [T, E] INT8 {0,1} or BOOL, or NULL; NULL iff probs NULL */
  const void* probs;             /* [T, E] of probs_dtype, or NULL */

  /* Outputs. unpermuted_tokens is required; the other three may be NULL to skip them. */
  void* unpermuted_tokens;  /* [T, H] of dtype */
  int32_t* out_index;       /* [N] */
  int32_t* permute_token_id;/* [N] */
  void* permute_probs;      /* [N] of probs_dtype (only with probs) */

  /* Optional timing hooks (hipEvent_t), bound to the launch of the gather-reduce kernel: `begin`
     takes the kernel's start and `end` its completion, from the kernel's own dispatch on
     `stream`, so the span is the kernel alone and no event packet of its own is added to
     the stream.  A lone `begin` is recorded on `stream` before the kernel instead (a lone
     `end` is still bound), and under graph capture both are recorded around it.
     NULL = not recorded. */
  void* ev_reduce_begin;
  void* ev_reduce_end;

  /* Opt-in (with probs): leave out every term whose weight is 0 instead of adding
     0 * row -- the article's kernel copies a slot's row only when its prob is non-zero
     ("Kernel implementation").  The result is the same for finite rows; a zero-weight
     row holding inf or NaN no longer reaches the output; zero-weight rows are not read.
     Applied in both layouts.  0 = off (formula-faithful, the default). */
  int32_t skip_zero_weight;
  int32_t reserved0;        /* must be 0 */

  /* Optional auxiliary stream (hipStream_t, same device as `stream`) for the non-padded
     out_index / permute_token_id sort, which depends on sorted_indices only.  NULL (or
     equal to `stream`): the sort runs on `stream` with the rest of the call.  Otherwise
     both events (hipEvent_t, created by the caller, best with hipEventDisableTiming) are
     required: the library records aux_fork_event on `stream` (bound to the first kernel of
     the call when there is one), makes aux_stream wait for it, enqueues the sort on
     aux_stream, records aux_join_event there, and makes `stream` wait for it before the
     call returns, so all of the call's work is ordered before later work on `stream`.
     The events are re-recorded by every call: calls that may run at the same time must
     not share them (calls issued one after another from one thread may).  Ignored in
     padded mode and when out_index and permute_token_id are both NULL. */
  void* aux_stream;
  void* aux_fork_event;
  void* aux_join_event;
} moe_unpermute_desc;

/* Validates *d and returns the workspace size in bytes (host only, no device work).
   Errors: FFNWB_ERR_PARAM_NULLPTR (required pointer NULL, or aux_stream given without
   both events), FFNWB_ERR_PARAM_INVALID
   (dtype combination, routing_map/probs NULL mismatch, num_rows != N, N not a multiple
   of T (non-padded) or of E (padded with probs), sizes out of range),
   FFNWB_ERR_INNER_NULLPTR (topK > 512, or num_experts outside (0, 8192] with probs). */
int moe_unpermute_workspace_size(const moe_unpermute_desc* d, size_t* ws_bytes);

/* Validates again, then enqueues the unpermute on `stream`. */
int moe_unpermute(const moe_unpermute_desc* d, void* workspace, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
   serving loops, harnesses that forbid hipMalloc): moe_unpermute with its workspace taken
   from a static device array the library holds on each GPU it runs on, of
   FFNWB_NOALLOC_SCRATCH_BYTES, until the process ends.  The caller still passes every input
   and output in *d.  Same validation, kernels and results as moe_unpermute; in addition
   FFNWB_ERR_SCRATCH when moe_unpermute_workspace_size would return more than
   FFNWB_NOALLOC_SCRATCH_BYTES (returned before any device work).  The call itself
   allocates nothing; its first call on a GPU looks up that GPU's array address once.
   All calls on one GPU share that GPU's array: calls that may overlap in time on one GPU
   (on different streams, or from different threads) race and give undefined results;
   calls ordered on one stream are safe.  The array's contents between calls do not
   matter to the kernels. */
#define FFNWB_NOALLOC_SCRATCH_BYTES (16u << 20)
int moe_unpermute_noalloc(const moe_unpermute_desc* d, void* stream);

/* ------------------------------------------------------------------------------------------
 * MoE token permute with routing map: the step before the experts that the
 * MoeTokenUnpermuteWithRoutingMap article names in "Operator positioning" -- tokens
 * regrouped by expert, so that every expert reads its tokens contiguously, plus the
 * sorted_indices moe_unpermute takes back.  The page does not specify it further; the
 * outputs are the arrangement moe_unpermute's formulas invert.
 *
 * T = num_tokens, H = hidden, E = num_experts, N = num_out_rows.
 * Non-padded (padded_mode = 0): N a multiple of T, topK = N / T.
 *   Row r of permuted_tokens = the token of the r-th non-zero routing-map entry in
 *   expert-major order (expert ascending, then token ascending); rows past the number
 *   of non-zero entries are zero; entries past N are dropped.
 *   sorted_indices[t*topK + k] = the row of token t's k-th expert (experts ascending)
 *   for k < topK when that row exists (< N); -1 for every other slot.
 * Padded (padded_mode = 1): N = E * capacity.
 *   sorted_indices[e*C + j] = the j-th token (ascending) routed to expert e, for j below
 *   min(C, the expert's token count); -1 for the rest.  Row i of permuted_tokens = token
 *   row sorted_indices[i], zero where that is -1.  Tokens past the capacity are dropped.
 * Rows are moved as bytes.  Supported: E <= 8192 and T * E < 2^31.  Up to 256 experts with
 * ceil(T / 256) * E <= 16384 the order takes one launch after the map count; larger maps
 * take a four-launch order through a [T][E] table in the workspace (4 * T * E bytes).
 * ------------------------------------------------------------------------------------------ */
typedef struct moe_permute_desc {
  int32_t dtype;             /* element type of the rows: FFNWB_DT_FP16, _BF16, _FP32, or _INT8
                                (1-byte elements, no scale) */
  int32_t padded_mode;       /* 0 = token-slot layout, 1 = expert-capacity layout */
  int64_t num_tokens;        /* T >= 1 */
  int64_t hidden;            /* H > 0 elements per row */
  int64_t num_experts;       /* E in [1, 8192] */
  int64_t num_out_rows;      /* N >= 0 (see above) */
  int64_t capacity;          /* C >= 0, padded mode only */
  int64_t token_row_stride;  /* bytes between token rows; 0 = H * element size */

  /* Inputs. */
  const void* tokens;           /* [T] rows of H elements, token_row_stride apart */
  const uint8_t* routing_map;   /* [T, E] bytes, non-zero = the token is routed to the expert */

  /* Outputs (both required). */
  void* permuted_tokens;        /* [N, H] of dtype, dense */
  int32_t* sorted_indices;      /* [N] */

  /* Optional timing hooks (hipEvent_t), bound to the launch of the row-copy kernel: `begin`
     takes the kernel's start and `end` its completion, from the kernel's own dispatch on
     `stream`, so the span is the kernel alone and no event packet of its own is added to
     the stream.  A lone `begin` is recorded on `stream` before the kernel instead (a lone
     `end` is still bound), and under graph capture both are recorded around it.
     NULL = not recorded. */
  void* ev_copy_begin;
  void* ev_copy_end;
} moe_permute_desc;

/* Validates *d and returns the workspace size in bytes (host only, no device work).
   Errors: FFNWB_ERR_PARAM_NULLPTR (a pointer is NULL), FFNWB_ERR_PARAM_INVALID (dtype,
   padded_mode, sizes out of range or outside the supported set above, N not a multiple
   of T (non-padded) or not E * capacity (padded), stride below the row size). */
int moe_permute_workspace_size(const moe_permute_desc* d, size_t* ws_bytes);

/* Validates again, then enqueues the permute on `stream`. */
int moe_permute(const moe_permute_desc* d, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * MoeUpdateExpert (its README page: "Function description", the parameter table,
 * "Constraints").
 *
 * For every token t < BS and slot k < K with logical expert e = expert_ids[t*K + k]:
 *   balanced_expert_ids[t*K + k] = eplb_table[e*F + 1 + r],
 *     r = local_rank_id mod count (balance_mode 0, by rank) or t mod count (balance_mode
 *     1, by token), count = eplb_table[e*F]: each table row is [count, the instance ids
 *     of the expert's replicas].
 *   With scales: balanced_active_mask[t*K + k] = 1 when the token is active (active_mask
 *   NULL or active_mask[t] != 0) and NOT expert_scales[t*K + k] < pruning_threshold[k]
 *   (FP32 comparison: equal is kept, NaN is kept); 0 otherwise.
 * An expert id outside [0, moe_expert_num) or a count outside [1, F-1] gives -1, mask 0,
 * and is counted in *err_count.  Table rows are only read at columns 0 .. count.
 * ------------------------------------------------------------------------------------------ */
typedef struct moe_update_expert_desc {
  int64_t bs;               /* BS in (0, 512] */
  int64_t k;                /* K in (0, 16], K <= moe_expert_num */
  int64_t moe_expert_num;   /* E in (0, 1024] */
  int64_t table_cols;       /* F in [2, world_size + 1] */
  int64_t local_rank_id;    /* balance_mode 0: in [0, world_size) */
  int64_t world_size;       /* balance_mode 0: in [2, 768]; balance_mode 1: in [1, 768] */
  int32_t balance_mode;     /* 0 = distribute by rank, 1 = by token */
  int32_t id_dtype;         /* FFNWB_DT_INT32 or FFNWB_DT_INT64, for ids in and out */
  int32_t scale_dtype;      /* FFNWB_DT_FP16, _BF16 or _FP32; ignored without scales */
  int32_t reserved0;        /* must be 0 */

  /* Inputs (row-major; see the strides below). */
  const void* expert_ids;          /* [BS, K] of id_dtype */
  const int32_t* eplb_table;       /* [E, F] */
  const void* expert_scales;       /* [BS, K] of scale_dtype, or NULL */
  const float* pruning_threshold;  /* [K], or NULL; NULL exactly when expert_scales is */
  const uint8_t* active_mask;      /* [BS] bool, or NULL (= all active); only with scales */

  /* Outputs. */
  void* balanced_expert_ids;       /* [BS, K] of id_dtype, required */
  uint8_t* balanced_active_mask;   /* [BS, K] bool; required with scales, ignored without */
  int32_t* err_count;              /* [1] or NULL */

  /* Layouts (the parameter table allows non-contiguous tensors): strides in ELEMENTS, 0 =
     dense.  A 2-D tensor's elements along K (or F) are adjacent; its rows are the given
     stride apart, at least the row length.  The 1-D threshold and mask take an element
     stride >= 1. */
  int64_t expert_ids_stride;       /* between tokens of expert_ids (0 = K) */
  int64_t eplb_table_stride;       /* between experts of eplb_table (0 = F) */
  int64_t expert_scales_stride;    /* between tokens of expert_scales (0 = K) */
  int64_t threshold_stride;        /* between entries of pruning_threshold (0 = 1) */
  int64_t active_mask_stride;      /* between tokens of active_mask (0 = 1) */
  int64_t out_ids_stride;          /* between tokens of balanced_expert_ids (0 = K) */
  int64_t out_mask_stride;         /* between tokens of balanced_active_mask (0 = K) */
} moe_update_expert_desc;

/* Validates *d and returns the workspace size (0) (host only).  Errors:
   FFNWB_ERR_PARAM_NULLPTR (d, ws_bytes or a required pointer NULL),
   FFNWB_ERR_PARAM_INVALID (a range above violated, dtype codes, scales given without a
   threshold or the other way round, active_mask without scales, reserved0 != 0, a
   negative stride or a row stride below its row length). */
int moe_update_expert_workspace_size(const moe_update_expert_desc* d, size_t* ws_bytes);

/* Validates again, then enqueues the update on `stream` (one launch). */
int moe_update_expert(const moe_update_expert_desc* d, void* workspace, size_t ws_bytes, void* stream);

/* Human-readable name of a status code (static storage). */
const char* ffnwb_status_string(int status);

/* FFNWB_ABI_VERSION of the built library. */
int ffnwb_abi_version(void);

/* sizeof the descriptors as compiled into the library (binding self-check). */
size_t ffnwb_batching_desc_size(void);
size_t ffnwb_batching_ctx_desc_size(void);
size_t moe_unpermute_desc_size(void);
size_t moe_permute_desc_size(void);
size_t moe_update_expert_desc_size(void);

#ifdef __cplusplus
}
#endif

#endif /* FFNWB_H */

"""ctypes mirror of include/ffnwb.h (constants and the descriptor structs)."""

import ctypes

FFNWB_ABI_VERSION = 6

FFNWB_OK = 0
FFNWB_ERR_PARAM_NULLPTR = 161001
FFNWB_ERR_PARAM_INVALID = 161002
FFNWB_ERR_INNER_NULLPTR = 561103
FFNWB_ERR_WORKSPACE = 1
FFNWB_ERR_RUNTIME = 2
FFNWB_ERR_SCRATCH = 3
FFNWB_NOALLOC_SCRATCH_BYTES = 16 << 20

FFNWB_DT_FP16 = 0
FFNWB_DT_BF16 = 1
FFNWB_DT_INT8 = 2
FFNWB_DT_FP32 = 3
FFNWB_DT_INT32 = 4
FFNWB_DT_INT64 = 5

FFNWB_CTX_BYTES = 1024
FFNWB_CTX_SHAPE = 1
FFNWB_CTX_POLLING = 2
FFNWB_CTX_POINTER = 4
FFNWB_CTX_BUFFER = 8

_i64, _i32, _vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p


class BatchingDesc(ctypes.Structure):
    _fields_ = [
        ("A", _i64), ("BS", _i64), ("K1", _i64), ("H", _i64),
        ("expert_num", _i64), ("layer_num", _i64),
        ("token_dtype", _i32), ("need_schedule", _i32),
        ("token_data", _vp), ("token_row_stride", _i64),
        ("token_scale", _vp), ("scale_stride", _i64),
        ("expert_ids", _vp), ("mask", _vp), ("layer_ids", _vp),
        ("session_ids", _vp), ("micro_batch_ids", _vp),
        ("y", _vp), ("session_ids_out", _vp), ("micro_batch_ids_out", _vp),
        ("token_ids", _vp), ("expert_offsets", _vp), ("dynamic_scale", _vp),
        ("group_list", _vp), ("actual_token_num", _vp), ("err_count", _vp),
        ("ev_gather_begin", _vp), ("ev_gather_end", _vp),
    ]


class BatchingCtxDesc(ctypes.Structure):
    _fields_ = [
        ("A", _i64), ("BS", _i64), ("K1", _i64), ("H", _i64),
        ("expert_num", _i64), ("layer_num", _i64),
        ("token_dtype", _i32), ("need_schedule", _i32),
        ("schedule_context", _vp),
        ("y", _vp), ("session_ids_out", _vp), ("micro_batch_ids_out", _vp),
        ("token_ids", _vp), ("expert_offsets", _vp), ("dynamic_scale", _vp),
        ("group_list", _vp), ("actual_token_num", _vp), ("err_count", _vp), ("ctx_status", _vp),
        ("ev_gather_begin", _vp), ("ev_gather_end", _vp),
    ]


class UnpermuteDesc(ctypes.Structure):
    _fields_ = [
        ("dtype", _i32), ("probs_dtype", _i32), ("padded_mode", _i32), ("weight_index", _i32),
        ("num_rows", _i64), ("hidden", _i64), ("num_tokens", _i64), ("num_experts", _i64),
        ("num_indices", _i64),
        ("permuted_tokens", _vp), ("sorted_indices", _vp), ("routing_map", _vp), ("probs", _vp),
        ("unpermuted_tokens", _vp), ("out_index", _vp), ("permute_token_id", _vp),
        ("permute_probs", _vp),
        ("ev_reduce_begin", _vp), ("ev_reduce_end", _vp),
        ("skip_zero_weight", _i32), ("reserved0", _i32),
        ("aux_stream", _vp), ("aux_fork_event", _vp), ("aux_join_event", _vp),
    ]


class PermuteDesc(ctypes.Structure):
    _fields_ = [
        ("dtype", _i32), ("padded_mode", _i32),
        ("num_tokens", _i64), ("hidden", _i64), ("num_experts", _i64), ("num_out_rows", _i64),
        ("capacity", _i64), ("token_row_stride", _i64),
        ("tokens", _vp), ("routing_map", _vp),
        ("permuted_tokens", _vp), ("sorted_indices", _vp),
        ("ev_copy_begin", _vp), ("ev_copy_end", _vp),
    ]


class UpdateExpertDesc(ctypes.Structure):
    _fields_ = [
        ("bs", _i64), ("k", _i64), ("moe_expert_num", _i64), ("table_cols", _i64),
        ("local_rank_id", _i64), ("world_size", _i64),
        ("balance_mode", _i32), ("id_dtype", _i32), ("scale_dtype", _i32), ("reserved0", _i32),
        ("expert_ids", _vp), ("eplb_table", _vp), ("expert_scales", _vp), ("pruning_threshold", _vp),
        ("active_mask", _vp),
        ("balanced_expert_ids", _vp), ("balanced_active_mask", _vp), ("err_count", _vp),
        ("expert_ids_stride", _i64), ("eplb_table_stride", _i64), ("expert_scales_stride", _i64),
        ("threshold_stride", _i64), ("active_mask_stride", _i64), ("out_ids_stride", _i64),
        ("out_mask_stride", _i64),
    ]

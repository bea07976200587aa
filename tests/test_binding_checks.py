"""Host-only checks of the Python binding's argument validation.

The C descriptors carry raw pointers and sizes, so a tensor whose shape, element type or
layout disagrees with the sizes the call is built from would make a kernel read or write
outside it.  The binding rejects such calls with ValueError before any descriptor is
built; these tests run on CPU tensors (no call is launched).
"""

import pytest
import torch

import unpermute_ffnwb_batching_amd as F

i32, i64 = torch.int32, torch.int64


def _unpermute(**over):
    T, K, H, E = 8, 2, 16, 4
    args = dict(permuted_tokens=torch.zeros(T * K, H, dtype=torch.bfloat16),
                sorted_indices=torch.zeros(T * K, dtype=i32),
                routing_map=torch.zeros(T, E, dtype=torch.int8), probs=torch.zeros(T, E, dtype=torch.float32),
                padded_mode=False, restore_shape=(T, H))
    args.update(over)
    return F.UnpermuteCall(args.pop("permuted_tokens"), args.pop("sorted_indices"), args.pop("routing_map"),
                           args.pop("probs"), **args)


def test_unpermute_valid_call_builds():
    c = _unpermute()
    assert c.out["unpermuted"].shape == (8, 16)


@pytest.mark.parametrize("over", [
    dict(restore_shape=(8, 15)),                                     # hidden differs from the rows
    dict(sorted_indices=torch.zeros(16, dtype=i64)),                 # int64 indices
    dict(sorted_indices=torch.zeros(32, dtype=i32)[::2]),            # strided indices
    dict(sorted_indices=torch.zeros(4, 4, dtype=i32)),               # not 1-D
    dict(permuted_tokens=torch.zeros(16, 32, dtype=torch.bfloat16)[:, ::2]),   # strided rows
    dict(permuted_tokens=torch.zeros(16, 16, dtype=torch.int32)),    # element type
    dict(routing_map=torch.zeros(8, 5, dtype=torch.int8)),           # map shape != probs shape
    dict(probs=torch.zeros(7, 4)),                                   # probs rows != T
    dict(routing_map=torch.zeros(8, 4, dtype=torch.float32)),        # map element type
    dict(routing_map=None),                                          # probs without a map
    dict(out={"unpermuted": torch.zeros(8, 8, dtype=torch.bfloat16)}),       # output too small
    dict(out={"unpermuted": torch.zeros(8, 16, dtype=torch.float16)}),       # output type
    dict(out={"out_index": torch.zeros(15, dtype=i32)}),
    dict(out={"permute_probs": torch.zeros(16, dtype=torch.float16)}),       # probs type
    dict(out={"bogus": torch.zeros(1)}),
])
def test_unpermute_rejects(over):
    with pytest.raises(ValueError):
        _unpermute(**over)


def _batching(**over):
    A, BS, K1, H = 2, 4, 3, 8
    Y = A * BS * K1
    args = dict(token_data=torch.zeros(Y, H, dtype=torch.float16), expert_ids=torch.zeros(Y, dtype=i32),
                expert_num=16, layer_num=1, max_out_shape=(A, BS, K1, H), token_dtype=F.FFNWB_DT_FP16)
    args.update(over)
    return F.BatchingCall(args.pop("token_data"), args.pop("expert_ids"), **args)


def test_batching_valid_call_builds():
    assert _batching().out["y"].shape == (24, 8)
    # INT8 rows with the packed scale: H + 4 bytes a row
    _batching(token_data=torch.zeros(24, 12, dtype=torch.uint8), token_dtype=F.FFNWB_DT_INT8)


@pytest.mark.parametrize("over", [
    dict(token_data=torch.zeros(23, 8, dtype=torch.float16)),        # one row short
    dict(token_data=torch.zeros(24, 8, dtype=torch.uint8), token_dtype=F.FFNWB_DT_INT8),  # no room for the scale
    dict(token_data=torch.zeros(24, 8, dtype=torch.float16), token_row_stride=8),   # stride below the row
    dict(expert_ids=torch.zeros(24, dtype=i64)),
    dict(expert_ids=torch.zeros(23, dtype=i32)),
    dict(mask=torch.zeros(24, dtype=i32)),
    dict(layer_ids=torch.zeros(3, dtype=i32)),
    dict(session_ids=torch.zeros(2, dtype=i64)),
    dict(token_dtype=7),
    dict(out={"y": torch.zeros(24, 7, dtype=torch.float16)}),
    dict(out={"group_list": torch.zeros(16, 2, dtype=i32)}),
    dict(out={"token_ids": torch.zeros(48, dtype=i32)[::2]}),
])
def test_batching_rejects(over):
    with pytest.raises(ValueError):
        _batching(**over)


def _permute(**over):
    T, H, E = 8, 16, 4
    args = dict(tokens=torch.zeros(T, H, dtype=torch.bfloat16), routing_map=torch.zeros(T, E, dtype=torch.int8),
                num_out_rows=2 * T)
    args.update(over)
    return F.PermuteCall(args.pop("tokens"), args.pop("routing_map"), **args)


def test_permute_valid_call_builds():
    assert _permute().out["permuted_tokens"].shape == (16, 16)
    _permute(tokens=torch.zeros(8, 32, dtype=torch.bfloat16)[:, :16])   # strided rows are allowed


@pytest.mark.parametrize("over", [
    dict(tokens=torch.zeros(8, 32, dtype=torch.bfloat16)[:, ::2]),   # elements not dense
    dict(routing_map=torch.zeros(7, 4, dtype=torch.int8)),
    dict(routing_map=torch.zeros(8, 4, dtype=torch.float16)),
    dict(routing_map=torch.zeros(8, 8, dtype=torch.int8)[:, ::2]),
    dict(out={"permuted_tokens": torch.zeros(16, 8, dtype=torch.bfloat16)}),
    dict(out={"sorted_indices": torch.zeros(16, dtype=i64)}),
    dict(num_out_rows=None),
])
def test_permute_rejects(over):
    with pytest.raises(ValueError):
        _permute(**over)


def test_ctx_rejects_short_context_and_bad_outputs():
    ctx = torch.zeros(1024, dtype=torch.uint8)
    kw = dict(expert_num=16, layer_num=1, max_out_shape=(2, 4, 3, 8), token_dtype=F.FFNWB_DT_FP16)
    F.BatchingCtxCall(ctx, **kw)
    with pytest.raises(ValueError):
        F.BatchingCtxCall(torch.zeros(1000, dtype=torch.uint8), **kw)
    with pytest.raises(ValueError):
        F.BatchingCtxCall(ctx, out={"ctx_status": torch.zeros(2, dtype=i32)}, **kw)


def test_update_expert_accepts_row_strided_views_and_rejects_bad_layouts():
    ids = torch.zeros(8, 6, dtype=i32)[:, :4]
    table = torch.ones(16, 5, dtype=i32)[:, :3]
    c = F.UpdateExpertCall(ids, table, local_rank_id=0, world_size=2)
    assert c.desc.expert_ids_stride == 6 and c.desc.eplb_table_stride == 5
    with pytest.raises(ValueError):
        F.UpdateExpertCall(torch.zeros(8, 8, dtype=i32)[:, ::2], table, local_rank_id=0, world_size=2)
    with pytest.raises(ValueError):
        F.UpdateExpertCall(ids, torch.ones(16, 3, dtype=i64), local_rank_id=0, world_size=2)
    with pytest.raises(ValueError):
        F.UpdateExpertCall(ids, table, local_rank_id=0, world_size=2, expert_scales=torch.zeros(8, 4),
                           pruning_threshold=torch.zeros(5))

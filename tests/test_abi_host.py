"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
function include/ffnwb.h declares, its descriptor layout matches the binding, and
argument validation returns the documented status codes before any device work."""

import ctypes
import os
import re

import pytest

import unpermute_ffnwb_batching_amd as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x1000  # a non-NULL address; the workspace queries never dereference pointers


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "ffnwb.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\([^;]*\)\s*;", src, flags=re.M)))


def test_header_declares_the_expected_entry_points():
    names = _declared_functions()
    for n in ("ffnwb_batching_workspace_size", "ffnwb_batching", "ffnwb_batching_ctx_workspace_size",
              "ffnwb_batching_ctx", "moe_update_expert_workspace_size", "moe_update_expert",
              "moe_unpermute_workspace_size",
              "moe_unpermute", "moe_permute_workspace_size", "moe_permute", "ffnwb_status_string",
              "ffnwb_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = F.lib()
    for n in _declared_functions():
        assert hasattr(L, n), n


def test_descriptor_layout_and_version():
    L = F.lib()
    assert L.ffnwb_batching_desc_size() == ctypes.sizeof(F.BatchingDesc)
    assert L.moe_unpermute_desc_size() == ctypes.sizeof(F.UnpermuteDesc)
    assert L.moe_permute_desc_size() == ctypes.sizeof(F.PermuteDesc)
    assert L.ffnwb_batching_ctx_desc_size() == ctypes.sizeof(F.BatchingCtxDesc)
    assert L.moe_update_expert_desc_size() == ctypes.sizeof(F.UpdateExpertDesc)
    assert F.ffnwb_abi_version() == 6
    for st in (0, 161001, 161002, 561103, 1, 2):
        assert F.ffnwb_status_string(st).startswith("FFNWB_")


# ----------------------------------------------------------------------------- batching

def _batching_desc(**over):
    d = F.BatchingDesc()
    vals = dict(A=2, BS=8, K1=3, H=128, expert_num=16, layer_num=1, token_dtype=0, need_schedule=0)
    vals.update({k: v for k, v in over.items() if k in vals})
    for k, v in vals.items():
        setattr(d, k, v)
    for p in ("token_data", "expert_ids", "y", "session_ids_out", "micro_batch_ids_out", "token_ids",
              "expert_offsets", "dynamic_scale", "group_list", "actual_token_num"):
        setattr(d, p, FAKE)
    for k, v in over.items():
        if k not in vals:
            setattr(d, k, v)
    return d


def _bws(d):
    n = ctypes.c_size_t(0)
    st = F.lib().ffnwb_batching_workspace_size(ctypes.byref(d), ctypes.byref(n))
    return st, n.value


def test_batching_valid_and_small_path_needs_no_workspace():
    st, n = _bws(_batching_desc())
    assert st == 0 and n == 0                       # Y = 48 runs in one fused workgroup


@pytest.mark.parametrize("field", ["token_data", "expert_ids", "y", "session_ids_out", "micro_batch_ids_out",
                                   "token_ids", "expert_offsets", "group_list", "actual_token_num"])
def test_batching_required_pointers(field):
    assert _bws(_batching_desc(**{field: None}))[0] == F.FFNWB_ERR_PARAM_NULLPTR


def test_batching_int8_requires_dynamic_scale():
    assert _bws(_batching_desc(token_dtype=2, dynamic_scale=None))[0] == F.FFNWB_ERR_PARAM_NULLPTR
    assert _bws(_batching_desc(token_dtype=0, dynamic_scale=None))[0] == 0


@pytest.mark.parametrize("over", [
    dict(expert_num=0), dict(expert_num=8193), dict(A=0), dict(A=1025), dict(BS=0), dict(K1=0), dict(K1=65),
    dict(H=0), dict(token_dtype=3), dict(token_dtype=-1), dict(need_schedule=1), dict(need_schedule=2),
    dict(layer_num=-1), dict(layer_num=17), dict(expert_num=16, layer_num=3),
    dict(token_row_stride=255), dict(token_dtype=2, token_row_stride=130),
])
def test_batching_invalid_parameters(over):
    assert _bws(_batching_desc(**over))[0] == F.FFNWB_ERR_PARAM_INVALID


def test_batching_boundaries_accepted():
    for over in (dict(expert_num=8192), dict(A=1024), dict(K1=64), dict(layer_num=0), dict(layer_num=16),
                 dict(token_dtype=2, token_row_stride=132), dict(token_dtype=1)):
        assert _bws(_batching_desc(**over))[0] == 0, over


def test_batching_workspace_grows_with_slots():
    sizes = [_bws(_batching_desc(A=a, BS=64, K1=9, H=7168, expert_num=1024, layer_num=16))[1]
             for a in (4, 16, 64, 256)]
    assert all(a < b for a, b in zip(sizes, sizes[1:]))


def test_batching_launch_rejects_small_workspace_before_any_device_work():
    d = _batching_desc(A=64, BS=64, K1=9, H=7168, expert_num=1024, layer_num=16)
    st, n = _bws(d)
    assert st == 0 and n > 0
    assert F.lib().ffnwb_batching(ctypes.byref(d), None, ctypes.c_size_t(n), None) == F.FFNWB_ERR_WORKSPACE
    assert F.lib().ffnwb_batching(ctypes.byref(d), ctypes.c_void_p(FAKE), ctypes.c_size_t(n - 1),
                                  None) == F.FFNWB_ERR_WORKSPACE
    bad = _batching_desc(expert_num=0)
    assert F.lib().ffnwb_batching(ctypes.byref(bad), None, 0, None) == F.FFNWB_ERR_PARAM_INVALID


# ----------------------------------------------------------------------------- batching from a context

def _ctx_desc(**over):
    d = F.BatchingCtxDesc()
    vals = dict(A=2, BS=8, K1=3, H=128, expert_num=16, layer_num=1, token_dtype=0, need_schedule=1)
    vals.update({k: v for k, v in over.items() if k in vals})
    for k, v in vals.items():
        setattr(d, k, v)
    for p in ("schedule_context", "y", "session_ids_out", "micro_batch_ids_out", "token_ids", "expert_offsets",
              "dynamic_scale", "group_list", "actual_token_num", "ctx_status"):
        setattr(d, p, FAKE)
    for k, v in over.items():
        if k not in vals:
            setattr(d, k, v)
    return d


def _cws(d):
    n = ctypes.c_size_t(0)
    st = F.lib().ffnwb_batching_ctx_workspace_size(ctypes.byref(d), ctypes.byref(n))
    return st, n.value


def test_ctx_valid_needs_workspace_for_the_decoded_slots():
    st, n = _cws(_ctx_desc())
    assert st == 0 and n >= 48 * 5              # expert id + mask of each of the 48 slots
    assert _cws(_ctx_desc(need_schedule=0))[0] == 0


@pytest.mark.parametrize("field", ["schedule_context", "ctx_status", "y", "session_ids_out", "micro_batch_ids_out",
                                   "token_ids", "expert_offsets", "group_list", "actual_token_num"])
def test_ctx_required_pointers(field):
    assert _cws(_ctx_desc(**{field: None}))[0] == F.FFNWB_ERR_PARAM_NULLPTR


@pytest.mark.parametrize("over", [
    dict(need_schedule=2), dict(need_schedule=-1), dict(schedule_context=FAKE + 4), dict(A=0), dict(A=1025),
    dict(K1=65), dict(expert_num=0), dict(token_dtype=3), dict(expert_num=16, layer_num=3),
])
def test_ctx_invalid_parameters(over):
    assert _cws(_ctx_desc(**over))[0] == F.FFNWB_ERR_PARAM_INVALID


def test_ctx_launch_rejects_small_workspace_before_any_device_work():
    d = _ctx_desc()
    st, n = _cws(d)
    assert F.lib().ffnwb_batching_ctx(ctypes.byref(d), None, ctypes.c_size_t(n), None) == F.FFNWB_ERR_WORKSPACE
    assert F.lib().ffnwb_batching_ctx(ctypes.byref(d), ctypes.c_void_p(FAKE), ctypes.c_size_t(n - 1),
                                      None) == F.FFNWB_ERR_WORKSPACE


# ----------------------------------------------------------------------------- unpermute

def _unpermute_desc(probs=True, **over):
    d = F.UnpermuteDesc()
    vals = dict(dtype=1, probs_dtype=3, padded_mode=0, weight_index=0, num_rows=64, hidden=32,
                num_tokens=8, num_experts=4 if probs else 0, num_indices=64)
    vals.update({k: v for k, v in over.items() if k in vals})
    for k, v in vals.items():
        setattr(d, k, v)
    for p in ("permuted_tokens", "sorted_indices", "unpermuted_tokens", "out_index", "permute_token_id"):
        setattr(d, p, FAKE)
    if probs:
        d.routing_map = FAKE
        d.probs = FAKE
        d.permute_probs = FAKE
    for k, v in over.items():
        if k not in vals:
            setattr(d, k, v)
    return d


def _uws(d):
    n = ctypes.c_size_t(0)
    st = F.lib().moe_unpermute_workspace_size(ctypes.byref(d), ctypes.byref(n))
    return st, n.value


def test_unpermute_valid_cases():
    assert _uws(_unpermute_desc())[0] == 0
    assert _uws(_unpermute_desc(probs=False))[0] == 0
    assert _uws(_unpermute_desc(padded_mode=1, num_experts=4))[0] == 0
    assert _uws(_unpermute_desc(num_tokens=0, num_rows=0, num_indices=0))[0] == 0     # empty
    assert _uws(_unpermute_desc(dtype=1, probs_dtype=1))[0] == 0
    assert _uws(_unpermute_desc(dtype=0, probs_dtype=0))[0] == 0
    assert _uws(_unpermute_desc(dtype=3, probs_dtype=3))[0] == 0
    assert _uws(_unpermute_desc(num_tokens=1, num_rows=512, num_indices=512))[0] == 0  # topK = 512


@pytest.mark.parametrize("field", ["permuted_tokens", "sorted_indices", "unpermuted_tokens"])
def test_unpermute_required_pointers(field):
    assert _uws(_unpermute_desc(**{field: None}))[0] == F.FFNWB_ERR_PARAM_NULLPTR


def test_unpermute_optional_outputs_may_be_null():
    assert _uws(_unpermute_desc(out_index=None, permute_token_id=None, permute_probs=None))[0] == 0


@pytest.mark.parametrize("over", [
    dict(dtype=2), dict(dtype=7), dict(dtype=0, probs_dtype=3), dict(dtype=3, probs_dtype=1),
    dict(dtype=1, probs_dtype=0), dict(routing_map=None), dict(padded_mode=2), dict(weight_index=2),
    dict(hidden=0), dict(num_rows=63), dict(num_indices=65, num_rows=65), dict(num_tokens=-1),
    dict(num_tokens=0), dict(padded_mode=1, num_experts=5), dict(skip_zero_weight=2), dict(reserved0=1),
])
def test_unpermute_invalid_parameters(over):
    assert _uws(_unpermute_desc(**over))[0] == F.FFNWB_ERR_PARAM_INVALID


def test_unpermute_noalloc_rejects_calls_above_its_scratch_before_device_work():
    # T = 131072, topK = 8, E = 256 with the auxiliary outputs needs 26.5 MiB of workspace
    d = _unpermute_desc(num_tokens=131072, num_rows=131072 * 8, num_indices=131072 * 8, num_experts=256)
    st, n = _uws(d)
    assert st == 0 and n > F.FFNWB_NOALLOC_SCRATCH_BYTES
    assert F.lib().moe_unpermute_noalloc(ctypes.byref(d), None) == F.FFNWB_ERR_SCRATCH
    assert F.lib().moe_unpermute_noalloc(ctypes.byref(_unpermute_desc(dtype=7)), None) == F.FFNWB_ERR_PARAM_INVALID
    assert F.ffnwb_status_string(F.FFNWB_ERR_SCRATCH).startswith("FFNWB_ERR_SCRATCH")


@pytest.mark.parametrize("missing", ["aux_fork_event", "aux_join_event"])
def test_unpermute_aux_stream_needs_both_events(missing):
    d = _unpermute_desc(aux_stream=FAKE, aux_fork_event=FAKE, aux_join_event=FAKE)
    assert _uws(d)[0] == 0
    setattr(d, missing, None)
    assert _uws(d)[0] == F.FFNWB_ERR_PARAM_NULLPTR


def test_unpermute_probs_without_map_is_invalid():
    d = _unpermute_desc(probs=False)
    d.probs = FAKE
    d.probs_dtype = 3
    assert _uws(d)[0] == F.FFNWB_ERR_PARAM_INVALID


@pytest.mark.parametrize("over", [
    dict(num_tokens=1, num_rows=513, num_indices=513),     # topK = 513 > 512
    dict(num_experts=0), dict(num_experts=8193),
])
def test_unpermute_inner_nullptr_code(over):
    assert _uws(_unpermute_desc(**over))[0] == F.FFNWB_ERR_INNER_NULLPTR


def test_unpermute_workspace_skips_aux_sort_when_not_requested():
    full = _uws(_unpermute_desc(num_tokens=16384, num_rows=131072, num_indices=131072, num_experts=128))[1]
    lean = _uws(_unpermute_desc(num_tokens=16384, num_rows=131072, num_indices=131072, num_experts=128,
                                out_index=None, permute_token_id=None))[1]
    assert lean < full


# ----------------------------------------------------------------------------- permute

def _permute_desc(**over):
    d = F.PermuteDesc()
    vals = dict(dtype=1, padded_mode=0, num_tokens=64, hidden=32, num_experts=8, num_out_rows=128, capacity=0,
                token_row_stride=0)
    vals.update({k: v for k, v in over.items() if k in vals})
    for k, v in vals.items():
        setattr(d, k, v)
    for p in ("tokens", "routing_map", "permuted_tokens", "sorted_indices"):
        setattr(d, p, FAKE)
    for k, v in over.items():
        if k not in vals:
            setattr(d, k, v)
    return d


def _pws(d):
    n = ctypes.c_size_t(0)
    st = F.lib().moe_permute_workspace_size(ctypes.byref(d), ctypes.byref(n))
    return st, n.value


def test_permute_valid_cases():
    assert _pws(_permute_desc())[0] == 0
    for dt in (0, 1, 2, 3):
        assert _pws(_permute_desc(dtype=dt))[0] == 0
    assert _pws(_permute_desc(padded_mode=1, num_out_rows=8 * 20, capacity=20))[0] == 0
    assert _pws(_permute_desc(num_out_rows=0))[0] == 0                              # topK = 0
    assert _pws(_permute_desc(num_experts=256, num_tokens=16384, num_out_rows=16384 * 8))[0] == 0
    assert _pws(_permute_desc(token_row_stride=96))[0] == 0


@pytest.mark.parametrize("field", ["tokens", "routing_map", "permuted_tokens", "sorted_indices"])
def test_permute_required_pointers(field):
    assert _pws(_permute_desc(**{field: None}))[0] == F.FFNWB_ERR_PARAM_NULLPTR


@pytest.mark.parametrize("over", [
    dict(dtype=9), dict(padded_mode=3), dict(num_tokens=0), dict(hidden=0), dict(num_experts=0),
    dict(num_experts=8193), dict(num_out_rows=100),                   # not a multiple of T
    dict(padded_mode=1, num_out_rows=100, capacity=20),               # not E * C
    dict(num_experts=8192, num_tokens=262144, num_out_rows=262144),   # T * E >= 2^31
    dict(token_row_stride=63), dict(capacity=-1),
])
def test_permute_invalid_parameters(over):
    assert _pws(_permute_desc(**over))[0] == F.FFNWB_ERR_PARAM_INVALID


def test_permute_wide_maps_take_the_table_order():
    # more than 256 experts, or a tile histogram beyond one workgroup's LDS: the [T][E] table
    for T, E in ((64, 257), (16385, 256), (65536, 128), (1024, 8192)):
        st, n = _pws(_permute_desc(num_tokens=T, num_experts=E, num_out_rows=T * 2))
        assert st == 0 and n >= 4 * T * E, (T, E)
        st, n = _pws(_permute_desc(padded_mode=1, num_tokens=T, num_experts=E, num_out_rows=E * 3, capacity=3))
        assert st == 0 and n >= 4 * T * E, (T, E)


def test_permute_workspace():
    st, n = _pws(_permute_desc(num_tokens=16384, num_experts=128, num_out_rows=16384 * 8))
    assert st == 0 and n >= 4 * 16384 * 8            # source token of every row
    st, n = _pws(_permute_desc(padded_mode=1, num_tokens=8192, num_experts=64, num_out_rows=64 * 512, capacity=512))
    assert st == 0 and n >= 4 * 32 * 64 + 4 * 8192 * 64  # tile histogram, capacity row of every entry


def test_launch_rejects_misaligned_workspace_before_any_device_work():
    """The workspace must be 256-byte aligned (the kernels store 16-byte vectors into it)."""
    d = _permute_desc(padded_mode=1, num_tokens=8192, num_experts=64, num_out_rows=64 * 512, capacity=512)
    st, n = _pws(d)
    assert st == 0 and n > 0
    for off in (4, 16, 128):
        assert F.lib().moe_permute(ctypes.byref(d), ctypes.c_void_p(FAKE + off), ctypes.c_size_t(n + 256),
                                   None) == F.FFNWB_ERR_WORKSPACE
    b = _batching_desc(A=64, BS=64, K1=9, H=7168, expert_num=1024, layer_num=16)
    st, n = _bws(b)
    assert st == 0 and n > 0
    assert F.lib().ffnwb_batching(ctypes.byref(b), ctypes.c_void_p(FAKE + 8), ctypes.c_size_t(n + 256),
                                  None) == F.FFNWB_ERR_WORKSPACE
    u = _unpermute_desc()
    st, n = _uws(u)
    if n > 0:
        assert F.lib().moe_unpermute(ctypes.byref(u), ctypes.c_void_p(FAKE + 64), ctypes.c_size_t(n + 256),
                                     None) == F.FFNWB_ERR_WORKSPACE


# ----------------------------------------------------------------------------- expert update

def _ue_desc(scales=True, **over):
    d = F.UpdateExpertDesc()
    vals = dict(bs=512, k=8, moe_expert_num=256, table_cols=9, local_rank_id=3, world_size=64, balance_mode=0,
                id_dtype=4, scale_dtype=1, reserved0=0)
    vals.update({k: v for k, v in over.items() if k in vals})
    for k, v in vals.items():
        setattr(d, k, v)
    for p in ("expert_ids", "eplb_table", "balanced_expert_ids"):
        setattr(d, p, FAKE)
    if scales:
        for p in ("expert_scales", "pruning_threshold", "balanced_active_mask"):
            setattr(d, p, FAKE)
    for k, v in over.items():
        if k not in vals:
            setattr(d, k, v)
    return d


def _uews(d):
    n = ctypes.c_size_t(7)
    st = F.lib().moe_update_expert_workspace_size(ctypes.byref(d), ctypes.byref(n))
    return st, n.value


def test_update_expert_valid_needs_no_workspace():
    assert _uews(_ue_desc()) == (0, 0)
    assert _uews(_ue_desc(scales=False)) == (0, 0)
    assert _uews(_ue_desc(active_mask=FAKE))[0] == 0
    for over in (dict(bs=1, k=1, moe_expert_num=1), dict(k=16), dict(moe_expert_num=1024), dict(world_size=768),
                 dict(table_cols=65), dict(balance_mode=1, world_size=1, table_cols=2, local_rank_id=99),
                 dict(id_dtype=5), dict(scale_dtype=0), dict(scale_dtype=3), dict(local_rank_id=63)):
        assert _uews(_ue_desc(**over))[0] == 0, over


@pytest.mark.parametrize("field", ["expert_ids", "eplb_table", "balanced_expert_ids", "balanced_active_mask"])
def test_update_expert_required_pointers(field):
    assert _uews(_ue_desc(**{field: None}))[0] == F.FFNWB_ERR_PARAM_NULLPTR


@pytest.mark.parametrize("over", [
    dict(bs=0), dict(bs=513), dict(k=0), dict(k=17), dict(moe_expert_num=0), dict(moe_expert_num=1025),
    dict(k=8, moe_expert_num=7), dict(world_size=1), dict(world_size=769), dict(local_rank_id=-1),
    dict(local_rank_id=64), dict(table_cols=1), dict(table_cols=66), dict(balance_mode=2), dict(id_dtype=3),
    dict(id_dtype=0), dict(scale_dtype=4), dict(reserved0=1), dict(pruning_threshold=None),
    dict(expert_scales=None), dict(expert_ids_stride=-1), dict(expert_ids_stride=1),      # below the row
    dict(eplb_table_stride=2), dict(expert_scales_stride=3), dict(out_ids_stride=1), dict(out_mask_stride=5),
    dict(threshold_stride=-2), dict(active_mask_stride=-1), dict(expert_ids_stride=(1 << 20) + 1),
])
def test_update_expert_invalid_parameters(over):
    assert _uews(_ue_desc(**over))[0] == F.FFNWB_ERR_PARAM_INVALID


def test_update_expert_strides_accepted():
    d = _ue_desc(expert_ids_stride=100, eplb_table_stride=66, expert_scales_stride=9, threshold_stride=4,
                 active_mask_stride=3, out_ids_stride=8, out_mask_stride=1 << 20)
    assert _uews(d)[0] == 0


def test_update_expert_active_mask_needs_scales():
    assert _uews(_ue_desc(scales=False, active_mask=FAKE))[0] == F.FFNWB_ERR_PARAM_INVALID

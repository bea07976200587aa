"""Helpers for the GPU parity tests: move a seeded case to the device, run the HIP
library through its binding, bring the outputs back in the oracle's storage format,
and compare with the oracle."""

import numpy as np
import torch

import synth
import unpermute_ffnwb_batching_amd as F

# The oracle is imported only by the functions that compare with it, so that the
# benchmark can use the device-side helpers below without loading the oracle outside
# its CPU-baseline leg.

CANARY = 0xA5


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _canary(shape, dtype):
    nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    return torch.full((nbytes,), CANARY, dtype=torch.uint8, device="cuda").view(dtype).reshape(shape)


def _bytes(t):
    return t.contiguous().view(torch.uint8).cpu().numpy()


_TOKEN_TORCH = {0: torch.float16, 1: torch.bfloat16, 2: torch.int8}


# ----------------------------------------------------------------------------- batching

def oracle_batching(case):
    from oracle import ffn_worker_batching
    return ffn_worker_batching(
        case["token_bytes"], case["expert_ids"], case["expert_num"], case["layer_num"],
        (case["A"], case["BS"], case["K1"], case["H"]), case["token_dtype"],
        mask=case["mask"], layer_ids=case["layer_ids"], session_ids=case["session_ids"],
        micro_batch_ids=case["micro_batch_ids"], token_scale=case["token_scale"])


def prepare_batching(case, ev_gather=None):
    A, BS, K1, H = case["A"], case["BS"], case["K1"], case["H"]
    Y = A * BS * K1
    td = case["token_dtype"]
    out = {"y": _canary((Y, H), _TOKEN_TORCH[td]),
           "group_list": _canary((case["expert_num"], 2), torch.int64),
           "actual_token_num": _canary((1,), torch.int64),
           "err_count": _canary((1,), torch.int32)}
    for k in ("session_ids", "micro_batch_ids", "token_ids", "expert_offsets"):
        out[k] = _canary((Y,), torch.int32)
    if td == 2:
        out["dynamic_scale"] = _canary((Y,), torch.float32)
    opt = {k: (dev(case[k]) if case[k] is not None else None)
           for k in ("mask", "layer_ids", "session_ids", "micro_batch_ids", "token_scale")}
    return F.BatchingCall(dev(case["token_bytes"]), dev(case["expert_ids"]), expert_num=case["expert_num"],
                          layer_num=case["layer_num"], max_out_shape=(A, BS, K1, H), token_dtype=td,
                          token_row_stride=case["stride"], out=out, ev_gather=ev_gather, **opt)


def fetch_batching(call):
    o = call.out
    r = {"y": _bytes(o["y"]).reshape(o["y"].shape[0], -1)}
    for k, v in o.items():
        if k != "y":
            r[k] = v.cpu().numpy()
    return r


def run_batching(case):
    call = prepare_batching(case)
    call.run()
    torch.cuda.synchronize()
    return fetch_batching(call)


def check_batching(case, got, ref=None):
    ref = ref if ref is not None else oracle_batching(case)
    act = ref["actual_token_num"]
    Y = case["A"] * case["BS"] * case["K1"]
    assert int(got["actual_token_num"][0]) == act
    assert np.array_equal(got["group_list"], ref["group_list"])
    assert int(got["err_count"][0]) == ref["err_count"]
    assert np.array_equal(got["y"][:act], ref["y"]), "gathered rows differ"
    for k in ("token_ids", "expert_offsets", "session_ids", "micro_batch_ids"):
        assert np.array_equal(got[k][:act], ref[k]), k
    if case["token_dtype"] == 2:
        assert np.array_equal(got["dynamic_scale"][:act].view(np.uint32), ref["dynamic_scale"].view(np.uint32))
    # rows past actual_token_num are never written
    assert (got["y"][act:] == CANARY).all()
    canary32 = np.uint32(0xA5A5A5A5).view(np.int32)
    for k in ("token_ids", "expert_offsets", "session_ids", "micro_batch_ids"):
        assert (got[k][act:Y] == canary32).all(), k
    return ref


# ----------------------------------------------------------------------------- unpermute

def to_torch_elems(a, dt):
    if dt == synth.BF16:
        return dev(np.asarray(a).view(np.int16)).view(torch.bfloat16)
    return dev(a)


def from_torch_elems(t, dt):
    a = t.cpu()
    if dt == synth.BF16:
        return a.view(torch.int16).numpy().view(np.uint16)
    return a.numpy()


def oracle_unpermute(case, weight_index=0, skip_zero_weight=False):
    from oracle import moe_token_unpermute_with_routing_map
    return moe_token_unpermute_with_routing_map(
        case["permuted"], case["dtype"], case["sorted_indices"], case["padded_mode"], case["restore_shape"],
        routing_map=case["routing_map"], probs=case["probs"], probs_dtype=case["probs_dtype"],
        weight_index=weight_index, skip_zero_weight=skip_zero_weight)


def prepare_unpermute(case, weight_index=0, aux=True, ev_reduce=None, skip_zero_weight=False, aux_stream=None):
    T, H = case["restore_shape"]
    N = case["sorted_indices"].shape[0]
    x = to_torch_elems(case["permuted"], case["dtype"])
    probs = to_torch_elems(case["probs"], case["probs_dtype"]) if case["probs"] is not None else None
    rmap = dev(case["routing_map"]) if case["routing_map"] is not None else None
    out = {"unpermuted": _canary((T, H), x.dtype)}
    if aux:
        out["out_index"] = _canary((N,), torch.int32)
        out["permute_token_id"] = _canary((N,), torch.int32)
    if probs is not None:
        out["permute_probs"] = _canary((N,), probs.dtype)
    return F.UnpermuteCall(x, dev(case["sorted_indices"]), rmap, probs, padded_mode=case["padded_mode"],
                           restore_shape=(T, H), weight_index=weight_index, aux=aux, out=out, ev_reduce=ev_reduce,
                           skip_zero_weight=skip_zero_weight, aux_stream=aux_stream)


def fetch_unpermute(call, case):
    o = call.out
    r = {"unpermuted": from_torch_elems(o["unpermuted"], case["dtype"])}
    for k in ("out_index", "permute_token_id"):
        if k in o:
            r[k] = o[k].cpu().numpy()
    if "permute_probs" in o:
        r["permute_probs"] = from_torch_elems(o["permute_probs"], case["probs_dtype"])
    return r


def run_unpermute(case, weight_index=0, aux=True, skip_zero_weight=False):
    call = prepare_unpermute(case, weight_index, aux, skip_zero_weight=skip_zero_weight)
    call.run()
    torch.cuda.synchronize()
    return fetch_unpermute(call, case)


TOL = {synth.FP16: (1e-2, 1e-3), synth.BF16: (1e-2, 1e-3), synth.FP32: (1e-5, 1e-6)}


def check_unpermute(case, got, ref=None, weight_index=0, aux=True, bit_exact=True):
    from oracle import numerics as nm
    ref = ref if ref is not None else oracle_unpermute(case, weight_index)
    dt = case["dtype"]
    g = nm.to_f32(got["unpermuted"], dt)
    o = nm.to_f32(ref["unpermuted"], dt)
    rtol, atol = TOL[dt]
    # acceptance bar: bf16/fp16 within 1e-2 relative or 1e-3 absolute; fp32 within 1e-5 relative
    np.testing.assert_allclose(g, o, rtol=rtol, atol=atol)
    if bit_exact:
        # same FP32 operations in the same order as the oracle: identical bits
        gb = np.asarray(got["unpermuted"]).view(np.uint8)
        ob = np.asarray(ref["unpermuted"]).view(np.uint8)
        assert np.array_equal(gb, ob), "unpermuted differs in bits from the oracle"
    if aux:
        assert np.array_equal(got["out_index"], ref["out_index"])
        assert np.array_equal(got["permute_token_id"], ref["permute_token_id"])
    if case["probs"] is not None:
        assert np.array_equal(np.asarray(got["permute_probs"]).view(np.uint8),
                              np.asarray(ref["permute_probs"]).view(np.uint8))
    return ref


# ----------------------------------------------------------------------------- permute

_ELEM_TORCH = {synth.FP16: torch.float16, synth.BF16: torch.bfloat16, synth.FP32: torch.float32,
               synth.INT8: torch.int8}


def permute_tokens(case):
    """The [T, H] token rows of a permute case as stored (a strided view when padded)."""
    return case["tokens_full"][:, :case["H"]]


def oracle_permute(case):
    from oracle import moe_token_permute_with_routing_map
    return moe_token_permute_with_routing_map(permute_tokens(case), case["routing_map"], case["N"],
                                              padded_mode=case["padded"], capacity=case["C"])


def prepare_permute(case, ev_copy=None):
    full = case["tokens_full"]
    if case["dtype"] == synth.BF16:
        t = dev(full.view(np.int16)).view(torch.bfloat16)
    else:
        t = dev(full)
    tokens = t[:, :case["H"]]
    N = case["N"]
    out = {"permuted_tokens": _canary((N, case["H"]), _ELEM_TORCH[case["dtype"]]),
           "sorted_indices": _canary((N,), torch.int32)}
    return F.PermuteCall(tokens, dev(case["routing_map"]), padded_mode=case["padded"], num_out_rows=N,
                         capacity=case["C"] or 0, out=out, ev_copy=ev_copy)


def fetch_permute(call):
    pt = call.out["permuted_tokens"]
    return {"permuted_tokens": _bytes(pt).reshape(pt.shape[0], pt.shape[1] * pt.element_size()),
            "sorted_indices": call.out["sorted_indices"].cpu().numpy()}


def run_permute(case):
    call = prepare_permute(case)
    call.run()
    torch.cuda.synchronize()
    return fetch_permute(call)


def check_permute(case, got, ref=None):
    ref = ref if ref is not None else oracle_permute(case)
    assert np.array_equal(got["sorted_indices"], ref["sorted_indices"]), "sorted_indices differ"
    rb = np.ascontiguousarray(ref["permuted_tokens"]).view(np.uint8).reshape(got["permuted_tokens"].shape)
    assert np.array_equal(got["permuted_tokens"], rb), "permuted rows differ"
    return ref


# ----------------------------------------------------------------------------- batching from a ScheduleContext

def ctx_fields(area, info, data, polling):
    """Context fields that describe ``area`` uploaded at ``info`` / ``data`` (device tensors)."""
    L = max(area["layer_num"], 1)
    return dict(session_num=area["A"], micro_batch_num=area["M"], micro_batch_size=area["BS"],
                selected_expert_num=area["K1"], expert_num=area["expert_num"] // L,
                token_info_buf=info.data_ptr(), token_info_buf_size=info.numel(),
                token_data_buf=data.data_ptr(), token_data_buf_size=data.numel(), polling_index=polling)


def prepare_ctx(area, polling, need_schedule, ctx_over=None, ev_gather=None, ptr_shift=None, bufs=None):
    """Upload the data area (or use the device buffers ``bufs`` = (info, data) already
    holding it) and a context describing it (fields in ``ctx_over`` replaced, pointer
    fields in ``ptr_shift`` moved by that many bytes); outputs pre-filled with the
    canary."""
    A, BS, K1, H = area["A"], area["BS"], area["K1"], area["H"]
    Y = A * BS * K1
    td = area["token_dtype"]
    info, data = bufs if bufs is not None else (dev(area["info"]), dev(area["data"].reshape(-1)))
    f = ctx_fields(area, info, data, polling)
    f.update(ctx_over or {})
    for k, v in (ptr_shift or {}).items():
        f[k] += v
    ctx_bytes = synth.schedule_context(**f)
    out = {"y": _canary((Y, H), _TOKEN_TORCH[td]),
           "group_list": _canary((area["expert_num"], 2), torch.int64),
           "actual_token_num": _canary((1,), torch.int64),
           "err_count": _canary((1,), torch.int32), "ctx_status": _canary((1,), torch.int32)}
    for k in ("session_ids", "micro_batch_ids", "token_ids", "expert_offsets"):
        out[k] = _canary((Y,), torch.int32)
    if td == 2:
        out["dynamic_scale"] = _canary((Y,), torch.float32)
    call = F.BatchingCtxCall(dev(ctx_bytes), expert_num=area["expert_num"], layer_num=area["layer_num"],
                             max_out_shape=(A, BS, K1, H), token_dtype=td, need_schedule=need_schedule, out=out,
                             ev_gather=ev_gather)
    call._keep += [info, data]
    call.ctx_bytes = ctx_bytes
    call.need_schedule = need_schedule
    return call


def oracle_ctx(area, call):
    from oracle import ffn_worker_batching_from_context
    return ffn_worker_batching_from_context(call.ctx_bytes, area["info"], area["data"].reshape(-1),
                                            area["expert_num"], area["layer_num"],
                                            (area["A"], area["BS"], area["K1"], area["H"]), area["token_dtype"],
                                            call.need_schedule)


def check_ctx(area, call, got=None, ref=None):
    got = got if got is not None else fetch_batching(call)
    ref = ref if ref is not None else oracle_ctx(area, call)
    assert int(got["ctx_status"][0]) == ref["status"]
    check_batching(area, got, ref)
    return ref


# ----------------------------------------------------------------------------- expert update

def prepare_update_expert(case, rank=None, mode=None):
    ids = dev(case["expert_ids"])
    BS, K = case["expert_ids"].shape
    out = {"balanced_expert_ids": _canary((BS, K), ids.dtype), "err_count": _canary((1,), torch.int32)}
    scales = thr = active = None
    if case["expert_scales"] is not None:
        scales = to_torch_elems(case["expert_scales"], case["scale_dtype"])
        thr = dev(case["pruning_threshold"])
        out["balanced_active_mask"] = _canary((BS, K), torch.uint8).view(torch.bool)
        if case["active_mask"] is not None:
            active = dev(case["active_mask"])
    return F.UpdateExpertCall(ids, dev(case["eplb_table"]),
                              local_rank_id=case["local_rank_id"] if rank is None else rank,
                              world_size=case["world_size"], balance_mode=case["balance_mode"] if mode is None else mode,
                              expert_scales=scales, pruning_threshold=thr, active_mask=active, out=out)


def oracle_update_expert(case, rank=None, mode=None):
    from oracle import moe_update_expert
    from oracle import numerics as nm
    s = None if case["expert_scales"] is None else nm.to_f32(case["expert_scales"], case["scale_dtype"])
    return moe_update_expert(case["expert_ids"], case["eplb_table"],
                             case["local_rank_id"] if rank is None else rank, case["world_size"],
                             case["balance_mode"] if mode is None else mode, s, case["pruning_threshold"],
                             case["active_mask"])


def check_update_expert(case, call, rank=None, mode=None):
    ref = oracle_update_expert(case, rank, mode)
    o = call.out
    got_ids = o["balanced_expert_ids"].cpu().numpy()
    assert got_ids.dtype == ref["balanced_expert_ids"].dtype
    assert np.array_equal(got_ids, ref["balanced_expert_ids"])
    assert int(o["err_count"][0]) == ref["err_count"]
    if ref["balanced_active_mask"] is not None:
        m = o["balanced_active_mask"].view(torch.uint8).cpu().numpy()
        assert np.array_equal(m, ref["balanced_active_mask"].astype(np.uint8))
    return ref

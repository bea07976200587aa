"""Python binding of libffnwb (include/ffnwb.h): MoE token reordering on MI355X.

Argument marshalling only -- every step of both operations runs in the library's HIP
kernels.  PyTorch provides device memory and the current HIP stream.

The names mirror the C ABI:

* ``ffnwb_batching_workspace_size`` / ``ffnwb_batching``
* ``ffnwb_batching_ctx_workspace_size`` / ``ffnwb_batching_ctx`` (ScheduleContext input)
* ``moe_unpermute_workspace_size`` / ``moe_unpermute``
* ``moe_permute_workspace_size`` / ``moe_permute``
* ``moe_update_expert_workspace_size`` / ``moe_update_expert``
* ``ffnwb_status_string``, ``ffnwb_abi_version``

``ffnwb_batching``, ``moe_unpermute`` and ``moe_permute`` take torch tensors, allocate any
output or workspace the caller did not pass, fill the C descriptor and enqueue the call
on the current stream.  ``BatchingCall`` / ``UnpermuteCall`` / ``PermuteCall`` build the
descriptor once for repeated launches (benchmarks, graph capture).

The library must be built (``python -m unpermute_ffnwb_batching_amd.build``); importing
works without it, but every call then raises ``RuntimeError``: there is no fallback.
"""

import ctypes
import os

import torch  # loads the HIP runtime the library binds to (same soname)

from . import _abi
from ._abi import (FFNWB_OK, FFNWB_ERR_PARAM_NULLPTR, FFNWB_ERR_PARAM_INVALID,  # noqa: F401
                   FFNWB_ERR_INNER_NULLPTR, FFNWB_ERR_WORKSPACE, FFNWB_ERR_RUNTIME,
                   FFNWB_DT_FP16, FFNWB_DT_BF16, FFNWB_DT_INT8, FFNWB_DT_FP32,
                   FFNWB_CTX_BYTES, FFNWB_CTX_SHAPE, FFNWB_CTX_POLLING, FFNWB_CTX_POINTER,
                   FFNWB_CTX_BUFFER, FFNWB_DT_INT32, FFNWB_DT_INT64, BatchingDesc, BatchingCtxDesc,
                   UnpermuteDesc, PermuteDesc, UpdateExpertDesc)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libffnwb.so")
_lib = None


class FfnwbError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: status {status} ({ffnwb_status_string(status)})")
        self.status = status


def lib():
    """The loaded shared library (ctypes.CDLL); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(run python -m unpermute_ffnwb_batching_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        L.ffnwb_batching_workspace_size.argtypes = [ctypes.POINTER(BatchingDesc), ctypes.POINTER(sz)]
        L.ffnwb_batching.argtypes = [ctypes.POINTER(BatchingDesc), vp, sz, vp]
        L.ffnwb_batching_ctx_workspace_size.argtypes = [ctypes.POINTER(BatchingCtxDesc), ctypes.POINTER(sz)]
        L.ffnwb_batching_ctx.argtypes = [ctypes.POINTER(BatchingCtxDesc), vp, sz, vp]
        L.moe_unpermute_workspace_size.argtypes = [ctypes.POINTER(UnpermuteDesc), ctypes.POINTER(sz)]
        L.moe_unpermute.argtypes = [ctypes.POINTER(UnpermuteDesc), vp, sz, vp]
        L.moe_permute_workspace_size.argtypes = [ctypes.POINTER(PermuteDesc), ctypes.POINTER(sz)]
        L.moe_permute.argtypes = [ctypes.POINTER(PermuteDesc), vp, sz, vp]
        L.moe_update_expert_workspace_size.argtypes = [ctypes.POINTER(UpdateExpertDesc), ctypes.POINTER(sz)]
        L.moe_update_expert.argtypes = [ctypes.POINTER(UpdateExpertDesc), vp, sz, vp]
        for f in ("ffnwb_batching_workspace_size", "ffnwb_batching", "ffnwb_batching_ctx_workspace_size",
                  "ffnwb_batching_ctx", "moe_unpermute_workspace_size",
                  "moe_unpermute", "moe_permute_workspace_size", "moe_permute", "moe_update_expert_workspace_size",
                  "moe_update_expert", "ffnwb_abi_version"):
            getattr(L, f).restype = ctypes.c_int
        L.ffnwb_status_string.argtypes = [ctypes.c_int]
        L.ffnwb_status_string.restype = ctypes.c_char_p
        L.ffnwb_batching_desc_size.restype = sz
        L.ffnwb_batching_ctx_desc_size.restype = sz
        L.moe_unpermute_desc_size.restype = sz
        L.moe_permute_desc_size.restype = sz
        L.moe_update_expert_desc_size.restype = sz
        if L.ffnwb_batching_desc_size() != ctypes.sizeof(BatchingDesc) or \
                L.ffnwb_batching_ctx_desc_size() != ctypes.sizeof(BatchingCtxDesc) or \
                L.moe_unpermute_desc_size() != ctypes.sizeof(UnpermuteDesc) or \
                L.moe_permute_desc_size() != ctypes.sizeof(PermuteDesc) or \
                L.moe_update_expert_desc_size() != ctypes.sizeof(UpdateExpertDesc):
            raise RuntimeError("libffnwb descriptor layout does not match the Python binding")
        if L.ffnwb_abi_version() != _abi.FFNWB_ABI_VERSION:
            raise RuntimeError("libffnwb ABI version mismatch")
        _lib = L
    return _lib


def ffnwb_status_string(status):
    return lib().ffnwb_status_string(int(status)).decode()


def ffnwb_abi_version():
    return lib().ffnwb_abi_version()


_placeholders = {}


def _ptr(t):
    """Device address of a tensor; an empty tensor gets a valid placeholder address
    (the library never reads it: every size that would index it is 0)."""
    if t is None:
        return None
    if t.numel() == 0:
        key = str(t.device)
        if key not in _placeholders:
            _placeholders[key] = torch.empty(256, dtype=torch.uint8, device=t.device)
        return ctypes.c_void_p(_placeholders[key].data_ptr())
    return ctypes.c_void_p(t.data_ptr())


def _event_handle(ev):
    """hipEvent_t of a HipEvent (``.handle``) or of a torch.cuda.Event (``.cuda_event``)."""
    if ev is None:
        return None
    if hasattr(ev, "handle"):
        return ev.handle
    return ctypes.c_void_p(ev.cuda_event)


def _stream_handle(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ----------------------------------------------------------------------------- batching

_TOKEN_TORCH = {FFNWB_DT_FP16: torch.float16, FFNWB_DT_BF16: torch.bfloat16, FFNWB_DT_INT8: torch.int8}
_ELT = {FFNWB_DT_FP16: 2, FFNWB_DT_BF16: 2, FFNWB_DT_INT8: 1, FFNWB_DT_FP32: 4}


def ffnwb_batching_workspace_size(desc):
    n = ctypes.c_size_t(0)
    st = lib().ffnwb_batching_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st != FFNWB_OK:
        raise FfnwbError(st, "ffnwb_batching_workspace_size")
    return n.value


def _row_stride_bytes(t):
    return t.stride(0) * t.element_size() if t.dim() >= 2 else 0


class BatchingCall:
    """A prepared ffnwb_batching call: descriptor, outputs and workspace bound once.

    ``token_data`` is a device tensor whose dim-0 rows are the Y slots (any element
    type; its row stride in bytes is passed as token_row_stride).  Outputs are
    allocated unless given in ``out`` (a dict with any of the keys below).
    """

    OUT_KEYS = ("y", "group_list", "actual_token_num", "session_ids", "micro_batch_ids",
                "token_ids", "expert_offsets", "dynamic_scale", "err_count")

    def __init__(self, token_data, expert_ids, *, expert_num, layer_num, max_out_shape, token_dtype,
                 mask=None, layer_ids=None, session_ids=None, micro_batch_ids=None, token_scale=None,
                 token_row_stride=None, scale_stride=0, need_schedule=0, out=None, with_err_count=True,
                 workspace=None, ev_gather=None):
        A, BS, K1, H = (int(v) for v in max_out_shape)
        Y = A * BS * K1
        dev = token_data.device
        out = dict(out or {})
        i32 = dict(dtype=torch.int32, device=dev)
        tdt = _TOKEN_TORCH.get(int(token_dtype), torch.uint8)
        if "y" not in out:
            out["y"] = torch.empty((Y, H), dtype=tdt, device=dev)
        if "group_list" not in out:
            out["group_list"] = torch.empty((int(expert_num), 2), dtype=torch.int64, device=dev)
        if "actual_token_num" not in out:
            out["actual_token_num"] = torch.empty(1, dtype=torch.int64, device=dev)
        for k in ("session_ids", "micro_batch_ids", "token_ids", "expert_offsets"):
            if k not in out:
                out[k] = torch.empty(Y, **i32)
        if int(token_dtype) == FFNWB_DT_INT8 and "dynamic_scale" not in out:
            out["dynamic_scale"] = torch.empty(Y, dtype=torch.float32, device=dev)
        if with_err_count and "err_count" not in out:
            out["err_count"] = torch.empty(1, **i32)
        self.out = out
        self._keep = [token_data, expert_ids, mask, layer_ids, session_ids, micro_batch_ids, token_scale]

        d = BatchingDesc()
        d.A, d.BS, d.K1, d.H = A, BS, K1, H
        d.expert_num = int(expert_num)
        d.layer_num = int(layer_num)
        d.token_dtype = int(token_dtype)
        d.need_schedule = int(need_schedule)
        d.token_data = _ptr(token_data)
        d.token_row_stride = _row_stride_bytes(token_data) if token_row_stride is None else int(token_row_stride)
        d.token_scale = _ptr(token_scale)
        d.scale_stride = int(scale_stride)
        d.expert_ids = _ptr(expert_ids)
        d.mask = _ptr(mask)
        d.layer_ids = _ptr(layer_ids)
        d.session_ids = _ptr(session_ids)
        d.micro_batch_ids = _ptr(micro_batch_ids)
        d.y = _ptr(out["y"])
        d.session_ids_out = _ptr(out["session_ids"])
        d.micro_batch_ids_out = _ptr(out["micro_batch_ids"])
        d.token_ids = _ptr(out["token_ids"])
        d.expert_offsets = _ptr(out["expert_offsets"])
        d.dynamic_scale = _ptr(out.get("dynamic_scale"))
        d.group_list = _ptr(out["group_list"])
        d.actual_token_num = _ptr(out["actual_token_num"])
        d.err_count = _ptr(out.get("err_count"))
        if ev_gather is not None:
            d.ev_gather_begin = _event_handle(ev_gather[0])
            d.ev_gather_end = _event_handle(ev_gather[1])
        self.desc = d
        self.ws_bytes = ffnwb_batching_workspace_size(d)
        if workspace is None and self.ws_bytes:
            workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.workspace = workspace

    def set_gather_events(self, begin, end):
        self.desc.ev_gather_begin = _event_handle(begin)
        self.desc.ev_gather_end = _event_handle(end)

    def run(self, stream=None):
        ws = self.workspace
        st = lib().ffnwb_batching(ctypes.byref(self.desc), _ptr(ws), ctypes.c_size_t(self.ws_bytes),
                                  _stream_handle(stream))
        if st != FFNWB_OK:
            raise FfnwbError(st, "ffnwb_batching")
        return self.out


def ffnwb_batching(token_data, expert_ids, *, stream=None, **kw):
    """Run FFN-worker batching once; returns the dict of output tensors."""
    return BatchingCall(token_data, expert_ids, **kw).run(stream)


def ffnwb_batching_ctx_workspace_size(desc):
    n = ctypes.c_size_t(0)
    st = lib().ffnwb_batching_ctx_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st != FFNWB_OK:
        raise FfnwbError(st, "ffnwb_batching_ctx_workspace_size")
    return n.value


class BatchingCtxCall:
    """A prepared ffnwb_batching_ctx call.

    ``schedule_context`` is a device tensor holding the 1024 context bytes (8-byte
    aligned); the data area it points to is device memory the caller keeps alive.
    Outputs are allocated unless given in ``out``; ``ctx_status`` holds the context
    check after the call has run.
    """

    def __init__(self, schedule_context, *, expert_num, layer_num, max_out_shape, token_dtype, need_schedule=0,
                 out=None, with_err_count=True, workspace=None, ev_gather=None):
        A, BS, K1, H = (int(v) for v in max_out_shape)
        Y = A * BS * K1
        dev = schedule_context.device
        out = dict(out or {})
        i32 = dict(dtype=torch.int32, device=dev)
        if "y" not in out:
            out["y"] = torch.empty((Y, H), dtype=_TOKEN_TORCH[int(token_dtype)], device=dev)
        if "group_list" not in out:
            out["group_list"] = torch.empty((int(expert_num), 2), dtype=torch.int64, device=dev)
        if "actual_token_num" not in out:
            out["actual_token_num"] = torch.empty(1, dtype=torch.int64, device=dev)
        for k in ("session_ids", "micro_batch_ids", "token_ids", "expert_offsets"):
            if k not in out:
                out[k] = torch.empty(Y, **i32)
        if int(token_dtype) == FFNWB_DT_INT8 and "dynamic_scale" not in out:
            out["dynamic_scale"] = torch.empty(Y, dtype=torch.float32, device=dev)
        if with_err_count and "err_count" not in out:
            out["err_count"] = torch.empty(1, **i32)
        if "ctx_status" not in out:
            out["ctx_status"] = torch.empty(1, **i32)
        self.out = out
        self._keep = [schedule_context]

        d = BatchingCtxDesc()
        d.A, d.BS, d.K1, d.H = A, BS, K1, H
        d.expert_num = int(expert_num)
        d.layer_num = int(layer_num)
        d.token_dtype = int(token_dtype)
        d.need_schedule = int(need_schedule)
        d.schedule_context = _ptr(schedule_context)
        d.y = _ptr(out["y"])
        d.session_ids_out = _ptr(out["session_ids"])
        d.micro_batch_ids_out = _ptr(out["micro_batch_ids"])
        d.token_ids = _ptr(out["token_ids"])
        d.expert_offsets = _ptr(out["expert_offsets"])
        d.dynamic_scale = _ptr(out.get("dynamic_scale"))
        d.group_list = _ptr(out["group_list"])
        d.actual_token_num = _ptr(out["actual_token_num"])
        d.err_count = _ptr(out.get("err_count"))
        d.ctx_status = _ptr(out["ctx_status"])
        if ev_gather is not None:
            d.ev_gather_begin = _event_handle(ev_gather[0])
            d.ev_gather_end = _event_handle(ev_gather[1])
        self.desc = d
        self.ws_bytes = ffnwb_batching_ctx_workspace_size(d)
        if workspace is None and self.ws_bytes:
            workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.workspace = workspace

    def set_gather_events(self, begin, end):
        self.desc.ev_gather_begin = _event_handle(begin)
        self.desc.ev_gather_end = _event_handle(end)

    def run(self, stream=None):
        st = lib().ffnwb_batching_ctx(ctypes.byref(self.desc), _ptr(self.workspace), ctypes.c_size_t(self.ws_bytes),
                                      _stream_handle(stream))
        if st != FFNWB_OK:
            raise FfnwbError(st, "ffnwb_batching_ctx")
        return self.out


def ffnwb_batching_ctx(schedule_context, *, stream=None, **kw):
    """Run FFN-worker batching from a ScheduleContext once; returns the output tensors."""
    return BatchingCtxCall(schedule_context, **kw).run(stream)


# ----------------------------------------------------------------------------- unpermute

_FLOAT_CODE = {torch.float16: FFNWB_DT_FP16, torch.bfloat16: FFNWB_DT_BF16, torch.float32: FFNWB_DT_FP32}


def moe_unpermute_workspace_size(desc):
    n = ctypes.c_size_t(0)
    st = lib().moe_unpermute_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st != FFNWB_OK:
        raise FfnwbError(st, "moe_unpermute_workspace_size")
    return n.value


class UnpermuteCall:
    """A prepared moe_unpermute call.

    ``permuted_tokens`` [rows, H] (fp16 / bf16 / fp32), ``sorted_indices`` int32 [N],
    ``routing_map`` int8/bool [T, E] or None, ``probs`` [T, E] or None.
    ``aux`` False skips out_index / permute_token_id.  ``skip_zero_weight`` leaves out
    terms whose weight is 0 (opt-in; see include/ffnwb.h).
    """

    def __init__(self, permuted_tokens, sorted_indices, routing_map=None, probs=None, *, padded_mode,
                 restore_shape, weight_index=0, aux=True, out=None, workspace=None, ev_reduce=None,
                 skip_zero_weight=False):
        T, H = (int(v) for v in restore_shape)
        dev = permuted_tokens.device
        out = dict(out or {})
        N = sorted_indices.numel()
        if "unpermuted" not in out:
            out["unpermuted"] = torch.empty((T, H), dtype=permuted_tokens.dtype, device=dev)
        if aux:
            for k in ("out_index", "permute_token_id"):
                if k not in out:
                    out[k] = torch.empty(N, dtype=torch.int32, device=dev)
        if probs is not None and "permute_probs" not in out:
            out["permute_probs"] = torch.empty(N, dtype=probs.dtype, device=dev)
        self.out = out
        rm = routing_map
        if rm is not None and rm.dtype == torch.bool:
            rm = rm.view(torch.uint8)
        self._keep = [permuted_tokens, sorted_indices, rm, probs]

        d = UnpermuteDesc()
        d.dtype = _FLOAT_CODE.get(permuted_tokens.dtype, -1)
        d.probs_dtype = _FLOAT_CODE.get(probs.dtype, -1) if probs is not None else 0
        d.padded_mode = int(bool(padded_mode))
        d.weight_index = int(weight_index)
        d.skip_zero_weight = int(bool(skip_zero_weight))
        d.num_rows = permuted_tokens.shape[0]
        d.hidden = H if permuted_tokens.dim() < 2 else permuted_tokens.shape[1]
        d.num_tokens = T
        d.num_experts = probs.shape[1] if probs is not None else 0
        d.num_indices = N
        d.permuted_tokens = _ptr(permuted_tokens)
        d.sorted_indices = _ptr(sorted_indices)
        d.routing_map = _ptr(rm)
        d.probs = _ptr(probs)
        d.unpermuted_tokens = _ptr(out["unpermuted"])
        d.out_index = _ptr(out.get("out_index"))
        d.permute_token_id = _ptr(out.get("permute_token_id"))
        d.permute_probs = _ptr(out.get("permute_probs"))
        if ev_reduce is not None:
            d.ev_reduce_begin = _event_handle(ev_reduce[0])
            d.ev_reduce_end = _event_handle(ev_reduce[1])
        self.desc = d
        self.ws_bytes = moe_unpermute_workspace_size(d)
        if workspace is None and self.ws_bytes:
            workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.workspace = workspace

    def set_reduce_events(self, begin, end):
        self.desc.ev_reduce_begin = _event_handle(begin)
        self.desc.ev_reduce_end = _event_handle(end)

    def run(self, stream=None):
        st = lib().moe_unpermute(ctypes.byref(self.desc), _ptr(self.workspace), ctypes.c_size_t(self.ws_bytes),
                                 _stream_handle(stream))
        if st != FFNWB_OK:
            raise FfnwbError(st, "moe_unpermute")
        return self.out


def moe_unpermute(permuted_tokens, sorted_indices, routing_map=None, probs=None, *, stream=None, **kw):
    """Run the unpermute once; returns dict(unpermuted, out_index, permute_token_id, permute_probs)."""
    return UnpermuteCall(permuted_tokens, sorted_indices, routing_map, probs, **kw).run(stream)


# ----------------------------------------------------------------------------- permute

_ANY_CODE = {torch.float16: FFNWB_DT_FP16, torch.bfloat16: FFNWB_DT_BF16, torch.float32: FFNWB_DT_FP32,
             torch.int8: FFNWB_DT_INT8, torch.uint8: FFNWB_DT_INT8}


def moe_permute_workspace_size(desc):
    n = ctypes.c_size_t(0)
    st = lib().moe_permute_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st != FFNWB_OK:
        raise FfnwbError(st, "moe_permute_workspace_size")
    return n.value


class PermuteCall:
    """A prepared moe_permute call.

    ``tokens`` [T, H] (fp16 / bf16 / fp32 / int8 / uint8; rows may be strided),
    ``routing_map`` int8/uint8/bool [T, E].  Non-padded: ``num_out_rows`` = T * topK;
    padded: ``capacity`` C gives num_out_rows = E * C.
    """

    def __init__(self, tokens, routing_map, *, padded_mode=False, num_out_rows=None, capacity=0, out=None,
                 workspace=None, ev_copy=None):
        T, H = tokens.shape[0], tokens.shape[1]
        E = routing_map.shape[1]
        dev = tokens.device
        N = int(E * capacity) if padded_mode else int(num_out_rows)
        out = dict(out or {})
        if "permuted_tokens" not in out:
            out["permuted_tokens"] = torch.empty((N, H), dtype=tokens.dtype, device=dev)
        if "sorted_indices" not in out:
            out["sorted_indices"] = torch.empty(N, dtype=torch.int32, device=dev)
        self.out = out
        rm = routing_map.view(torch.uint8) if routing_map.dtype in (torch.bool, torch.int8) else routing_map
        self._keep = [tokens, rm]
        d = PermuteDesc()
        d.dtype = _ANY_CODE.get(tokens.dtype, -1)
        d.padded_mode = int(bool(padded_mode))
        d.num_tokens = T
        d.hidden = H
        d.num_experts = E
        d.num_out_rows = N
        d.capacity = int(capacity)
        d.token_row_stride = _row_stride_bytes(tokens)
        d.tokens = _ptr(tokens)
        d.routing_map = _ptr(rm)
        d.permuted_tokens = _ptr(out["permuted_tokens"])
        d.sorted_indices = _ptr(out["sorted_indices"])
        if ev_copy is not None:
            d.ev_copy_begin = _event_handle(ev_copy[0])
            d.ev_copy_end = _event_handle(ev_copy[1])
        self.desc = d
        self.ws_bytes = moe_permute_workspace_size(d)
        if workspace is None and self.ws_bytes:
            workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.workspace = workspace

    def set_copy_events(self, begin, end):
        self.desc.ev_copy_begin = _event_handle(begin)
        self.desc.ev_copy_end = _event_handle(end)

    def run(self, stream=None):
        st = lib().moe_permute(ctypes.byref(self.desc), _ptr(self.workspace), ctypes.c_size_t(self.ws_bytes),
                               _stream_handle(stream))
        if st != FFNWB_OK:
            raise FfnwbError(st, "moe_permute")
        return self.out


def moe_permute(tokens, routing_map, *, stream=None, **kw):
    """Run the forward permute once; returns dict(permuted_tokens, sorted_indices)."""
    return PermuteCall(tokens, routing_map, **kw).run(stream)


# ----------------------------------------------------------------------------- expert update

_ID_CODE = {torch.int32: FFNWB_DT_INT32, torch.int64: FFNWB_DT_INT64}


def moe_update_expert_workspace_size(desc):
    n = ctypes.c_size_t(0)
    st = lib().moe_update_expert_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st != FFNWB_OK:
        raise FfnwbError(st, "moe_update_expert_workspace_size")
    return n.value


class UpdateExpertCall:
    """A prepared moe_update_expert call.  ``expert_ids`` [BS, K] int32 / int64,
    ``eplb_table`` [E, F] int32, optional ``expert_scales`` [BS, K] (float16, bfloat16
    or float32) with ``pruning_threshold`` [K] float32, and optional ``active_mask`` [BS]
    bool, all dense device tensors."""

    def __init__(self, expert_ids, eplb_table, *, local_rank_id, world_size, balance_mode=0, expert_scales=None,
                 pruning_threshold=None, active_mask=None, out=None, with_err_count=True):
        BS, K = expert_ids.shape
        E, Fc = eplb_table.shape
        dev = expert_ids.device
        out = dict(out or {})
        if "balanced_expert_ids" not in out:
            out["balanced_expert_ids"] = torch.empty((BS, K), dtype=expert_ids.dtype, device=dev)
        if expert_scales is not None and "balanced_active_mask" not in out:
            out["balanced_active_mask"] = torch.empty((BS, K), dtype=torch.bool, device=dev)
        if with_err_count and "err_count" not in out:
            out["err_count"] = torch.empty(1, dtype=torch.int32, device=dev)
        self.out = out
        self._keep = [expert_ids, eplb_table, expert_scales, pruning_threshold, active_mask]
        d = UpdateExpertDesc()
        d.bs, d.k, d.moe_expert_num, d.table_cols = BS, K, E, Fc
        d.local_rank_id, d.world_size, d.balance_mode = int(local_rank_id), int(world_size), int(balance_mode)
        d.id_dtype = _ID_CODE.get(expert_ids.dtype, -1)
        d.scale_dtype = _FLOAT_CODE.get(expert_scales.dtype, -1) if expert_scales is not None else 0
        d.expert_ids = _ptr(expert_ids)
        d.eplb_table = _ptr(eplb_table)
        d.expert_scales = _ptr(expert_scales)
        d.pruning_threshold = _ptr(pruning_threshold)
        d.active_mask = _ptr(active_mask)
        d.balanced_expert_ids = _ptr(out["balanced_expert_ids"])
        d.balanced_active_mask = _ptr(out.get("balanced_active_mask"))
        d.err_count = _ptr(out.get("err_count"))
        self.desc = d
        moe_update_expert_workspace_size(d)   # validates

    def run(self, stream=None):
        st = lib().moe_update_expert(ctypes.byref(self.desc), None, ctypes.c_size_t(0), _stream_handle(stream))
        if st != FFNWB_OK:
            raise FfnwbError(st, "moe_update_expert")
        return self.out


def moe_update_expert(expert_ids, eplb_table, *, stream=None, **kw):
    """Run MoeUpdateExpert once; returns the dict of output tensors."""
    return UpdateExpertCall(expert_ids, eplb_table, **kw).run(stream)

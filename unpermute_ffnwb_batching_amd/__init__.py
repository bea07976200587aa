"""Python binding of libffnwb (include/ffnwb.h): MoE token reordering on MI355X.

Argument marshalling only -- every step of both operations runs in the library's HIP
kernels.  PyTorch provides device memory and the current HIP stream.

The names mirror the C ABI:

* ``ffnwb_batching_workspace_size`` / ``ffnwb_batching``
* ``ffnwb_batching_ctx_workspace_size`` / ``ffnwb_batching_ctx`` (ScheduleContext input)
* ``moe_unpermute_workspace_size`` / ``moe_unpermute`` / ``moe_unpermute_noalloc``
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

import contextlib
import ctypes
import os

import torch  # loads the HIP runtime the library binds to (same soname)

from . import _abi
from ._abi import (FFNWB_OK, FFNWB_ERR_PARAM_NULLPTR, FFNWB_ERR_PARAM_INVALID,  # noqa: F401
                   FFNWB_ERR_INNER_NULLPTR, FFNWB_ERR_WORKSPACE, FFNWB_ERR_RUNTIME, FFNWB_ERR_SCRATCH,
                   FFNWB_NOALLOC_SCRATCH_BYTES,
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
        L.moe_unpermute_noalloc.argtypes = [ctypes.POINTER(UnpermuteDesc), vp]
        L.moe_permute_workspace_size.argtypes = [ctypes.POINTER(PermuteDesc), ctypes.POINTER(sz)]
        L.moe_permute.argtypes = [ctypes.POINTER(PermuteDesc), vp, sz, vp]
        L.moe_update_expert_workspace_size.argtypes = [ctypes.POINTER(UpdateExpertDesc), ctypes.POINTER(sz)]
        L.moe_update_expert.argtypes = [ctypes.POINTER(UpdateExpertDesc), vp, sz, vp]
        for f in ("ffnwb_batching_workspace_size", "ffnwb_batching", "ffnwb_batching_ctx_workspace_size",
                  "ffnwb_batching_ctx", "moe_unpermute_workspace_size",
                  "moe_unpermute", "moe_unpermute_noalloc", "moe_permute_workspace_size", "moe_permute", "moe_update_expert_workspace_size",
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


def _on(stream):
    """Allocate under ``stream`` (the caching allocator then ties the blocks to it)."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _alloc_stream(device):
    return torch.cuda.current_stream(device) if device.type == "cuda" else None


def _record_on(tensors, stream, alloc_stream):
    """Mark tensors as used by ``stream`` when it is not the stream they were allocated
    on, so that the allocator does not hand their memory out before that work ends."""
    if stream is None or alloc_stream is None or stream == alloc_stream:
        return
    for t in tensors:
        if t is not None and t.numel() > 0:
            t.record_stream(stream)


# ----------------------------------------------------------------------------- argument checks
# The C descriptors carry raw pointers and sizes only, so the shapes, element types and
# layouts of the tensors behind them are checked here before any call is built.

def _req(cond, msg):
    if not cond:
        raise ValueError(msg)


def _check_tensor(t, name, device, dtypes=None, shape=None, contiguous=True):
    _req(isinstance(t, torch.Tensor), f"{name} must be a torch.Tensor")
    _req(t.device == device, f"{name} is on {t.device}, expected {device}")
    if dtypes is not None:
        _req(t.dtype in dtypes, f"{name} has dtype {t.dtype}, expected one of {tuple(dtypes)}")
    if shape is not None:
        _req(tuple(t.shape) == tuple(shape), f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if contiguous:
        _req(t.is_contiguous(), f"{name} must be contiguous")


def _check_numel(t, name, device, dtypes, numel):
    _check_tensor(t, name, device, dtypes)
    _req(t.numel() == numel, f"{name} has {t.numel()} elements, expected {numel}")


def _check_rows(t, name, device, dtypes):
    """A 2-D tensor whose elements along the last dimension are adjacent and whose rows
    do not overlap (any row stride at least the row length)."""
    _check_tensor(t, name, device, dtypes, contiguous=False)
    _req(t.dim() == 2 and (t.shape[1] <= 1 or t.stride(1) == 1) and (t.shape[0] <= 1 or t.stride(0) >= t.shape[1]),
         f"{name} must be 2-D with adjacent elements in each row (a row stride of at least the row length)")


def _span_bytes(t):
    """Bytes from t's first element to just past its last (0 for an empty tensor)."""
    if t.numel() == 0:
        return 0
    return (sum((n - 1) * st for n, st in zip(t.shape, t.stride())) + 1) * t.element_size()


_I32 = (torch.int32,)
_BYTES = (torch.uint8, torch.int8, torch.bool)


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
        _check_batching_inputs(token_data, expert_ids, mask, layer_ids, session_ids, micro_batch_ids, token_scale,
                               token_row_stride, scale_stride, A, Y, H, int(token_dtype))
        _check_batching_outputs(out, dev, Y, H, int(expert_num), tdt)
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
        self._alloc_stream = _alloc_stream(dev)

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
        _record_on([ws, *self.out.values()], stream, self._alloc_stream)
        return self.out


def _check_batching_inputs(token_data, expert_ids, mask, layer_ids, session_ids, micro_batch_ids, token_scale,
                           token_row_stride, scale_stride, A, Y, H, token_dtype):
    _req(isinstance(token_data, torch.Tensor), "token_data must be a torch.Tensor")
    dev = token_data.device
    _req(token_dtype in _TOKEN_TORCH, f"token_dtype {token_dtype} is not FP16, BF16 or INT8")
    _req(A > 0 and Y > 0 and H > 0, "max_out_shape entries must be positive")
    _check_numel(expert_ids, "expert_ids", dev, _I32, Y)
    if mask is not None:
        _check_numel(mask, "mask", dev, _BYTES, Y)
    for t, name in ((layer_ids, "layer_ids"), (session_ids, "session_ids"), (micro_batch_ids, "micro_batch_ids")):
        if t is not None:
            _check_numel(t, name, dev, _I32, A)
    elt = 1 if token_dtype == FFNWB_DT_INT8 else 2
    packed = token_dtype == FFNWB_DT_INT8 and token_scale is None
    payload = H * elt + (4 if packed else 0)
    stride = _row_stride_bytes(token_data) if token_row_stride is None else int(token_row_stride)
    if stride == 0:
        stride = payload
    _req(stride >= payload, f"token row stride {stride} is below the row's {payload} bytes")
    need = (Y - 1) * stride + payload
    _req(_span_bytes(token_data) >= need,
         f"token_data spans {_span_bytes(token_data)} bytes, the {Y} rows need {need}")
    if token_scale is not None:
        _check_tensor(token_scale, "token_scale", dev, (torch.float32,), contiguous=False)
        sst = int(scale_stride) or 4
        _req(_span_bytes(token_scale) >= (Y - 1) * sst + 4, "token_scale is too small for Y scales")


def _check_batching_outputs(out, dev, Y, H, expert_num, tdt, ctx=False):
    want = {"y": ((Y, H), (tdt,)), "group_list": ((expert_num, 2), (torch.int64,)),
            "actual_token_num": ((1,), (torch.int64,)), "err_count": ((1,), _I32),
            "dynamic_scale": ((Y,), (torch.float32,))}
    if ctx:
        want["ctx_status"] = ((1,), _I32)
    for k in ("session_ids", "micro_batch_ids", "token_ids", "expert_offsets"):
        want[k] = ((Y,), _I32)
    for k, t in out.items():
        _req(k in want, f"unknown output {k!r}")
        shape, dtypes = want[k]
        _check_tensor(t, f"out[{k!r}]", dev, dtypes, shape)


def ffnwb_batching(token_data, expert_ids, *, stream=None, **kw):
    """Run FFN-worker batching once on ``stream`` (default: the current stream); returns
    the dict of output tensors, allocated on that stream."""
    with _on(stream):
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
        _req(int(token_dtype) in _TOKEN_TORCH, f"token_dtype {token_dtype} is not FP16, BF16 or INT8")
        _req(A > 0 and Y > 0 and H > 0, "max_out_shape entries must be positive")
        _check_tensor(schedule_context, "schedule_context", dev)
        _req(schedule_context.numel() * schedule_context.element_size() >= FFNWB_CTX_BYTES,
             f"schedule_context must hold {FFNWB_CTX_BYTES} bytes")
        _check_batching_outputs(out, dev, Y, H, int(expert_num), _TOKEN_TORCH[int(token_dtype)], ctx=True)
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
        self._alloc_stream = _alloc_stream(dev)

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
        _record_on([self.workspace, *self.out.values()], stream, self._alloc_stream)
        return self.out


def ffnwb_batching_ctx(schedule_context, *, stream=None, **kw):
    """Run FFN-worker batching from a ScheduleContext once on ``stream`` (default: the
    current stream); returns the output tensors, allocated on that stream."""
    with _on(stream):
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
    terms whose weight is 0 (opt-in; see include/ffnwb.h).  ``aux_stream`` (a
    torch.cuda.Stream) runs the non-padded out_index / permute_token_id sort beside the
    rest of the call; the call owns the two events that fork and join it, so calls that
    may overlap need Call objects of their own.  ``workspace=False`` allocates no
    workspace, for a call that only runs through ``run_noalloc``.
    """

    def __init__(self, permuted_tokens, sorted_indices, routing_map=None, probs=None, *, padded_mode,
                 restore_shape, weight_index=0, aux=True, out=None, workspace=None, ev_reduce=None,
                 skip_zero_weight=False, aux_stream=None):
        T, H = (int(v) for v in restore_shape)
        _check_tensor(permuted_tokens, "permuted_tokens", permuted_tokens.device, tuple(_FLOAT_CODE))
        dev = permuted_tokens.device
        _req(permuted_tokens.dim() == 2, "permuted_tokens must be 2-D [rows, H]")
        _req(T >= 0 and H == permuted_tokens.shape[1],
             f"restore_shape {tuple(restore_shape)} does not match permuted_tokens' hidden size "
             f"{permuted_tokens.shape[1]}")
        _req(sorted_indices.dim() == 1, "sorted_indices must be 1-D")
        _check_tensor(sorted_indices, "sorted_indices", dev, _I32)
        _req((routing_map is None) == (probs is None), "routing_map and probs are given together or not at all")
        if probs is not None:
            _req(probs.dim() == 2 and probs.shape[0] == T, f"probs must be [T={T}, E]")
            _check_tensor(probs, "probs", dev, tuple(_FLOAT_CODE))
            _check_tensor(routing_map, "routing_map", dev, _BYTES, tuple(probs.shape))
        out = dict(out or {})
        N = sorted_indices.numel()
        want = {"unpermuted": ((T, H), (permuted_tokens.dtype,)), "out_index": ((N,), _I32),
                "permute_token_id": ((N,), _I32)}
        if probs is not None:
            want["permute_probs"] = ((N,), (probs.dtype,))
        for k, t in out.items():
            _req(k in want, f"unknown output {k!r}")
            _check_tensor(t, f"out[{k!r}]", dev, want[k][1], want[k][0])
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
        self._alloc_stream = _alloc_stream(dev)
        self.aux_stream = aux_stream
        self._aux_events = None

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
        if aux_stream is not None:
            from .hip_events import HipEvent, HIP_EVENT_DISABLE_TIMING, HIP_EVENT_DISABLE_SYSTEM_FENCE
            flags = HIP_EVENT_DISABLE_TIMING | HIP_EVENT_DISABLE_SYSTEM_FENCE
            self._aux_events = (HipEvent(flags), HipEvent(flags))
            d.aux_stream = ctypes.c_void_p(aux_stream.cuda_stream)
            d.aux_fork_event = self._aux_events[0].handle
            d.aux_join_event = self._aux_events[1].handle
        self.desc = d
        self.ws_bytes = moe_unpermute_workspace_size(d)
        if workspace is None and self.ws_bytes:
            workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.workspace = workspace if workspace is not False else None

    def run_noalloc(self, stream=None):
        """Runs the call through moe_unpermute_noalloc: the workspace is the library's
        per-GPU scratch array, and nothing is allocated."""
        st = lib().moe_unpermute_noalloc(ctypes.byref(self.desc), _stream_handle(stream))
        if st != FFNWB_OK:
            raise FfnwbError(st, "moe_unpermute_noalloc")
        return self.out

    def set_reduce_events(self, begin, end):
        self.desc.ev_reduce_begin = _event_handle(begin)
        self.desc.ev_reduce_end = _event_handle(end)

    def run(self, stream=None):
        st = lib().moe_unpermute(ctypes.byref(self.desc), _ptr(self.workspace), ctypes.c_size_t(self.ws_bytes),
                                 _stream_handle(stream))
        if st != FFNWB_OK:
            raise FfnwbError(st, "moe_unpermute")
        _record_on([self.workspace, *self.out.values()], stream, self._alloc_stream)
        if self.aux_stream is not None:
            # the sort's workspace and outputs are also used on the auxiliary stream
            _record_on([self.workspace, self.out.get("out_index"), self.out.get("permute_token_id")],
                       self.aux_stream, self._alloc_stream)
        return self.out


def moe_unpermute_noalloc(call, stream=None):
    """Runs a prepared UnpermuteCall through the no-allocation entry point."""
    return call.run_noalloc(stream)


def moe_unpermute(permuted_tokens, sorted_indices, routing_map=None, probs=None, *, stream=None, **kw):
    """Run the unpermute once on ``stream`` (default: the current stream); returns
    dict(unpermuted, out_index, permute_token_id, permute_probs), allocated on that stream."""
    with _on(stream):
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
        _req(isinstance(tokens, torch.Tensor) and tokens.dim() == 2, "tokens must be a 2-D tensor [T, H]")
        dev = tokens.device
        _check_tensor(tokens, "tokens", dev, tuple(_ANY_CODE), contiguous=False)
        _req(tokens.stride(1) == 1 and tokens.stride(0) >= tokens.shape[1],
             "tokens rows must be dense (stride 1 along H) and must not overlap")
        T, H = tokens.shape[0], tokens.shape[1]
        _req(isinstance(routing_map, torch.Tensor) and routing_map.dim() == 2 and routing_map.shape[0] == T,
             f"routing_map must be [T={T}, E]")
        _check_tensor(routing_map, "routing_map", dev, _BYTES)
        E = routing_map.shape[1]
        _req(bool(padded_mode) or num_out_rows is not None, "num_out_rows is required in non-padded mode")
        N = int(E * capacity) if padded_mode else int(num_out_rows)
        out = dict(out or {})
        want = {"permuted_tokens": ((N, H), (tokens.dtype,)), "sorted_indices": ((N,), _I32)}
        for k, t in out.items():
            _req(k in want, f"unknown output {k!r}")
            _check_tensor(t, f"out[{k!r}]", dev, want[k][1], want[k][0])
        if "permuted_tokens" not in out:
            out["permuted_tokens"] = torch.empty((N, H), dtype=tokens.dtype, device=dev)
        if "sorted_indices" not in out:
            out["sorted_indices"] = torch.empty(N, dtype=torch.int32, device=dev)
        self.out = out
        rm = routing_map.view(torch.uint8) if routing_map.dtype in (torch.bool, torch.int8) else routing_map
        self._keep = [tokens, rm]
        self._alloc_stream = _alloc_stream(dev)
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
        _record_on([self.workspace, *self.out.values()], stream, self._alloc_stream)
        return self.out


def moe_permute(tokens, routing_map, *, stream=None, **kw):
    """Run the forward permute once on ``stream`` (default: the current stream); returns
    dict(permuted_tokens, sorted_indices), allocated on that stream."""
    with _on(stream):
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
    or float32) with ``pruning_threshold`` [K] or [1, K] float32, and optional
    ``active_mask`` [BS] bool.  Any of them, and any output passed in ``out``, may be a
    strided view, as long as a 2-D tensor's elements along K (or F) are adjacent."""

    def __init__(self, expert_ids, eplb_table, *, local_rank_id, world_size, balance_mode=0, expert_scales=None,
                 pruning_threshold=None, active_mask=None, out=None, with_err_count=True):
        _req(isinstance(expert_ids, torch.Tensor) and expert_ids.dim() == 2, "expert_ids must be [BS, K]")
        dev = expert_ids.device
        BS, K = expert_ids.shape
        _check_rows(expert_ids, "expert_ids", dev, tuple(_ID_CODE))
        _req(isinstance(eplb_table, torch.Tensor) and eplb_table.dim() == 2, "eplb_table must be [E, F]")
        _check_rows(eplb_table, "eplb_table", dev, _I32)
        E, Fc = eplb_table.shape
        if expert_scales is not None:
            _req(tuple(expert_scales.shape) == (BS, K), f"expert_scales must be [{BS}, {K}]")
            _check_rows(expert_scales, "expert_scales", dev, tuple(_FLOAT_CODE))
            _req(pruning_threshold is not None, "expert_scales need pruning_threshold")
            _req(pruning_threshold.numel() == K and pruning_threshold.shape[-1] == K,
                 f"pruning_threshold must be [{K}] or [1, {K}]")
            _check_tensor(pruning_threshold, "pruning_threshold", dev, (torch.float32,), contiguous=False)
            if active_mask is not None:
                _req(tuple(active_mask.shape) == (BS,), f"active_mask must be [{BS}]")
                _check_tensor(active_mask, "active_mask", dev, _BYTES, contiguous=False)
        out = dict(out or {})
        want = {"balanced_expert_ids": ((BS, K), (expert_ids.dtype,)), "balanced_active_mask": ((BS, K), _BYTES),
                "err_count": ((1,), _I32)}
        for k, t in out.items():
            _req(k in want, f"unknown output {k!r}")
            if k == "err_count":
                _check_tensor(t, "out['err_count']", dev, _I32, (1,))
            else:
                _req(tuple(t.shape) == want[k][0], f"out[{k!r}] must be {want[k][0]}")
                _check_rows(t, f"out[{k!r}]", dev, want[k][1])
        if "balanced_expert_ids" not in out:
            out["balanced_expert_ids"] = torch.empty((BS, K), dtype=expert_ids.dtype, device=dev)
        if expert_scales is not None and "balanced_active_mask" not in out:
            out["balanced_active_mask"] = torch.empty((BS, K), dtype=torch.bool, device=dev)
        if with_err_count and "err_count" not in out:
            out["err_count"] = torch.empty(1, dtype=torch.int32, device=dev)
        self.out = out
        self._keep = [expert_ids, eplb_table, expert_scales, pruning_threshold, active_mask]
        self._alloc_stream = _alloc_stream(dev)
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
        # strides in elements; 0 (dense) where a dimension of size 1 leaves torch's stride free
        def rs(t):
            return t.stride(0) if t.shape[0] > 1 else 0
        d.expert_ids_stride = rs(expert_ids)
        d.eplb_table_stride = rs(eplb_table)
        if expert_scales is not None:
            d.expert_scales_stride = rs(expert_scales)
            d.threshold_stride = pruning_threshold.stride(-1) if K > 1 else 0
            if active_mask is not None:
                d.active_mask_stride = active_mask.stride(0) if BS > 1 else 0
        d.out_ids_stride = rs(out["balanced_expert_ids"])
        if "balanced_active_mask" in out:
            d.out_mask_stride = rs(out["balanced_active_mask"])
        self.desc = d
        moe_update_expert_workspace_size(d)   # validates

    def run(self, stream=None):
        st = lib().moe_update_expert(ctypes.byref(self.desc), None, ctypes.c_size_t(0), _stream_handle(stream))
        if st != FFNWB_OK:
            raise FfnwbError(st, "moe_update_expert")
        _record_on(list(self.out.values()), stream, self._alloc_stream)
        return self.out


def moe_update_expert(expert_ids, eplb_table, *, stream=None, **kw):
    """Run MoeUpdateExpert once on ``stream`` (default: the current stream); returns the
    dict of output tensors, allocated on that stream."""
    with _on(stream):
        return UpdateExpertCall(expert_ids, eplb_table, **kw).run(stream)

"""Oracle for the ScheduleContext front-end of FFN-worker batching (test
infrastructure only).

Source: the aclnnFfnWorkerBatching API page --
  * "Function description", step 1: what the attention workers send lands in a
    data area laid out as the ScheduleContext structure (CommonArea, ControlArea,
    AttentionArea, FfnArea); the op takes FfnArea's token_info_buf and
    token_data_buf for the tokens and their descriptors, and from them the layer,
    session, micro-batch and expert ids;
  * the parameter table: scheduleContext is an INT8 tensor of 1024 bytes;
    needSchedule 0 = batch without scanning the data, 1 = scan the data first;
    maxOutShape = {A, BS, topK+1, H};
  * the usage example: the packed definitions of FfnDataDesc (flag, layer_id,
    expert_ids[]) and ScheduleContext (the four areas, padded to 1024 bytes),
    token_info sized (4 * (K+1) * BS + sizeof(FfnDataDesc)) * M * A bytes and
    filled session by session, micro-batch by micro-batch, and token_data
    holding the rows of H elements.

Readings taken where the page is silent (each listed with its reason in the
design notes):
  * field offsets are those of the packed definition: CommonArea at 0
    (session_num, micro_batch_num, micro_batch_size, selected_expert_num,
    expert_num as u32 at 0, 4, 8, 12, 16), ControlArea at 128, AttentionArea at
    256, FfnArea at 384 (token_info_buf u64 at +0, its size at +8,
    token_data_buf at +16, its size at +24, polling_index at +32);
  * chunk (s, m) -- session s, micro-batch m -- is chunk number s*M + m: its
    descriptor starts at byte (s*M + m) * (8 + 4*BS*(K+1)) of token_info, its
    BS*(K+1) rows start at row (s*M + m) * BS*(K+1) of token_data; a row holds
    H elements (INT8: H bytes, then the FP32 scale), rows back to back;
  * one call batches micro-batch m = polling_index of every session, so its
    Y = A * BS * (K+1) slots are those of maxOutShape; slot s*BS*(K+1) + j is
    entry j of session s's chunk;
  * needSchedule = 1: a chunk takes part only when its flag is 1; its other
    slots count as masked.  needSchedule = 0: flags are not read;
  * the session id of a row is s, its micro-batch id m, its token id the slot
    number in the call;
  * the context must agree with the call (session_num = A, micro_batch_size = BS,
    selected_expert_num = K+1, expert_num * max(layerNum, 1) = expertNum,
    micro_batch_num in [1, 64], polling_index < micro_batch_num, both buffers
    non-null, token_info 4-byte and token_data 16-byte aligned, each buffer at
    least as large as the data area needs); otherwise nothing is read, no slot
    is batched, and the status says why (bits below);
  * the FfnArea's id tables and out_num, ControlArea and AttentionArea, and the
    token-size and schedule-mode fields of CommonArea are not used.

Pins (tests/test_oracle_schedule.py): the page's usage example with every
output in closed form; contexts and data areas serialised through a NumPy
structured type declared member by member like the page's struct (so NumPy,
not this file, computes the offsets), checked against the flat oracle on the
arrays the test started from; brute force over micro-batches and flags; every
status condition on its own.
"""

import struct

import numpy as np

from .batching import ffn_worker_batching
from .numerics import DT_INT8, elt_bytes

CTX_BYTES = 1024
STATUS_SHAPE = 1        # the context's sizes disagree with the call's arguments
STATUS_POLLING = 2      # micro_batch_num outside [1, 64], or polling_index >= micro_batch_num
STATUS_POINTER = 4      # a data-area pointer is null or misaligned
STATUS_BUFFER = 8       # a data-area buffer is smaller than the layout needs

_COMMON = 0
_FFN = 384


def _u32(ctx, off):
    return struct.unpack_from("<I", ctx, off)[0]


def _u64(ctx, off):
    return struct.unpack_from("<Q", ctx, off)[0]


def decode_schedule_context(ctx, token_info, token_data, expert_num, layer_num, max_out_shape,
                            token_dtype, need_schedule):
    """Turn a ScheduleContext and the contents of its data area into the flat
    batching problem.

    ctx        : 1024 bytes of the context (the pointers in it are addresses on the
                 device; only their value is examined here).
    token_info : uint8 contents of the buffer at ffn.token_info_buf.
    token_data : uint8 contents of the buffer at ffn.token_data_buf.
    Returns dict(status, token_bytes [Y, row], expert_ids [Y], mask [Y],
    layer_ids [A], micro_batch_ids [A], row_bytes).
    """
    ctx = bytes(bytearray(np.asarray(ctx, dtype=np.uint8).tobytes()))
    assert len(ctx) == CTX_BYTES
    A, BS, K1, H = (int(v) for v in max_out_shape)
    n = BS * K1                         # slots of one chunk
    Y = A * n
    row = H * elt_bytes(token_dtype) + (4 if token_dtype == DT_INT8 else 0)
    L = max(int(layer_num), 1)

    session_num = _u32(ctx, _COMMON + 0)
    M = _u32(ctx, _COMMON + 4)
    mbs = _u32(ctx, _COMMON + 8)
    sel = _u32(ctx, _COMMON + 12)
    per_layer = _u32(ctx, _COMMON + 16)
    info_ptr = _u64(ctx, _FFN + 0)
    info_size = _u64(ctx, _FFN + 8)
    data_ptr = _u64(ctx, _FFN + 16)
    data_size = _u64(ctx, _FFN + 24)
    polling = _u64(ctx, _FFN + 32)

    status = 0
    if session_num != A or mbs != BS or sel != K1 or per_layer * L != int(expert_num):
        status |= STATUS_SHAPE
    if not 1 <= M <= 64 or polling >= M:
        status |= STATUS_POLLING
    if info_ptr == 0 or data_ptr == 0 or info_ptr % 4 != 0 or data_ptr % 16 != 0:
        status |= STATUS_POINTER
    chunk_info = 8 + 4 * n
    if info_size < A * M * chunk_info or data_size < A * M * n * row:
        status |= STATUS_BUFFER

    token_bytes = np.zeros((Y, row), dtype=np.uint8)
    expert_ids = np.zeros(Y, dtype=np.int32)
    mask = np.ones(Y, dtype=np.uint8)
    layer_ids = np.zeros(A, dtype=np.int32)
    micro = np.full(A, polling if status == 0 else 0, dtype=np.int32)
    if status != 0:
        return dict(status=status, token_bytes=token_bytes, expert_ids=expert_ids, mask=mask,
                    layer_ids=layer_ids, micro_batch_ids=micro, row_bytes=row)

    info = np.asarray(token_info, dtype=np.uint8)
    data = np.asarray(token_data, dtype=np.uint8)
    m = int(polling)
    for s in range(A):
        c = s * M + m                   # chunk number in the data area
        base = c * chunk_info
        flag, layer = struct.unpack_from("<ii", info, base)
        if need_schedule == 1 and flag != 1:
            continue                    # not ready: its slots stay masked
        layer_ids[s] = layer
        for j in range(n):
            slot = s * n + j
            expert_ids[slot] = struct.unpack_from("<i", info, base + 8 + 4 * j)[0]
            mask[slot] = 0
            r0 = (c * n + j) * row
            token_bytes[slot] = data[r0:r0 + row]
    return dict(status=status, token_bytes=token_bytes, expert_ids=expert_ids, mask=mask,
                layer_ids=layer_ids, micro_batch_ids=micro, row_bytes=row)


def ffn_worker_batching_from_context(ctx, token_info, token_data, expert_num, layer_num, max_out_shape,
                                     token_dtype, need_schedule):
    """Batching as the page's interface states it: the ScheduleContext front-end,
    then steps 2-4 (ffn_worker_batching).  Returns that function's outputs plus
    ``status``."""
    d = decode_schedule_context(ctx, token_info, token_data, expert_num, layer_num, max_out_shape,
                                token_dtype, need_schedule)
    out = ffn_worker_batching(d["token_bytes"], d["expert_ids"], expert_num, layer_num, max_out_shape,
                              token_dtype, mask=d["mask"], layer_ids=d["layer_ids"],
                              micro_batch_ids=d["micro_batch_ids"])
    out["status"] = d["status"]
    return out

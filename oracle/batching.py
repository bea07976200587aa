"""Oracle for FFN-worker batching (test infrastructure only).

Source: the aclnnFfnWorkerBatching API page --
  * "Function description", steps 2-4: sort the per-slot expert IDs with masked
    slots forced to a large value, gather each token's hidden state (and in INT8
    mode its FP32 dynamic scale) by the sort's gather index, look up the
    session / micro-batch / token IDs, scan the sorted IDs for jump points to
    build group_list;
  * the calculation formula: gather_idx = sort(expert_ids_in),
    y[i] = token_data[gather_idx[i]], group_list[e] = [expert_id_e, count_e],
    actual_token_num = sum of the counts;
  * the parameter table (expertNum = experts per layer x layerNum,
    maxOutShape = {A, BS, topK+1, H}, tokenDtype 0/1/2, layerNum in
    [0, expertNum], per-layer independent expert indexing) and the output table;
  * "Constraints": INT8 data and its FP32 scale laid out contiguously; the op is
    deterministic.

Readings taken where the page is silent (each one is listed with its reason in
the design notes):
  * the sort is stable (ties keep slot order) -- the page calls the op
    deterministic, and only a stable order makes y / tokenIds unique;
  * a slot's sort key is ``layer * experts_per_layer + expert_id``; masked slots,
    and unmasked slots whose expert or layer id is out of range, get the
    sentinel ``expert_num`` and are not emitted (out-of-range ones are counted
    in ``err_count``);
  * the layer id belongs to a (session, micro-batch) chunk of BS*(K+1) slots,
    as in the data-area descriptor of the page's usage sample;
  * group_list is compact: one row per expert that received tokens, in
    ascending key order, then [0, 0] rows;
  * tokenIds is the gathered slot's index in token_data; sessionIds /
    microBatchIds come from optional per-chunk tables (default: the chunk
    index, and 0);
  * only the first actual_token_num rows of each per-row output are produced;
  * layerNum = 0 behaves like 1.

Pins (tests/test_oracle_batching.py): the page's own usage sample (all
outputs derived in closed form), an O(Y^2) brute-force selection on tiny
random inputs, a hand-worked two-layer example, and invariants on random inputs
(y is a permutation of the unmasked rows, counts sum to actual_token_num,
keys non-decreasing, offsets restart per group).
"""

import numpy as np

from .numerics import DT_FP16, DT_BF16, DT_INT8, elt_bytes


def ffn_worker_batching(token_bytes, expert_ids, expert_num, layer_num, max_out_shape,
                        token_dtype, mask=None, layer_ids=None, session_ids=None,
                        micro_batch_ids=None, token_scale=None):
    """Reference FFN-worker batching.

    token_bytes : uint8 [Y, stride] -- row ``s`` holds slot ``s``'s hidden state
        (H elements of ``token_dtype``); for INT8 rows with ``token_scale`` None,
        bytes [H, H+4) of each row hold the FP32 dynamic scale (packed layout).
    expert_ids  : int32 [Y]      per-slot expert id, indexed within its layer.
    mask        : uint8 [Y] or None; non-zero = slot masked (not emitted).
    layer_ids, session_ids, micro_batch_ids : int32 [A] or None (per chunk).
    token_scale : float32 [Y] or None -- separate-array INT8 scales.

    Returns a dict with ``actual_token_num`` (int), ``group_list`` int64
    [expert_num, 2], ``err_count`` (int), and the per-row outputs for rows
    [0, actual_token_num): ``y`` uint8 [actual, H*elt], ``session_ids``,
    ``micro_batch_ids``, ``token_ids``, ``expert_offsets`` (int32) and, for
    INT8, ``dynamic_scale`` (float32).
    """
    A, BS, K1, H = (int(v) for v in max_out_shape)
    Y = A * BS * K1
    chunk = BS * K1
    if token_dtype not in (DT_FP16, DT_BF16, DT_INT8):
        raise ValueError("token_dtype must be 0 (FP16), 1 (BF16) or 2 (INT8)")
    row_bytes = H * elt_bytes(token_dtype)
    token_bytes = np.asarray(token_bytes, dtype=np.uint8)
    assert token_bytes.shape[0] == Y and token_bytes.shape[1] >= row_bytes
    expert_ids = np.asarray(expert_ids, dtype=np.int64)
    assert expert_ids.shape == (Y,)

    L = max(int(layer_num), 1)
    per_layer = int(expert_num) // L
    sentinel = int(expert_num)

    # Step 2 of the page: per-slot sort key, masked slots forced to a large value.
    key = np.full(Y, sentinel, dtype=np.int64)
    err_count = 0
    for s in range(Y):
        if mask is not None and mask[s] != 0:
            continue
        a = s // chunk
        layer = int(layer_ids[a]) if (layer_ids is not None and layer_num >= 1) else 0
        e = int(expert_ids[s])
        if 0 <= e < per_layer and 0 <= layer < L:
            key[s] = layer * per_layer + e
        else:
            err_count += 1

    # gather_idx = sort(expert_ids_in): a stable argsort over the keys.
    gather_idx = np.argsort(key, kind="stable")

    # Step 4: per-expert token counts; actual_token_num is their sum.
    counts = np.bincount(key[key < sentinel], minlength=sentinel)
    actual = int(counts.sum())
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]])

    group_list = np.zeros((sentinel, 2), dtype=np.int64)
    present = np.nonzero(counts)[0]
    group_list[:len(present), 0] = present
    group_list[:len(present), 1] = counts[present]

    # Step 3: gather the rows (and scales) and look up the IDs for each output row.
    y = np.empty((actual, row_bytes), dtype=np.uint8)
    sess = np.empty(actual, dtype=np.int32)
    mb = np.empty(actual, dtype=np.int32)
    tok = np.empty(actual, dtype=np.int32)
    offs = np.empty(actual, dtype=np.int32)
    scale = np.empty(actual, dtype=np.float32) if token_dtype == DT_INT8 else None
    for i in range(actual):
        g = int(gather_idx[i])
        a = g // chunk
        y[i] = token_bytes[g, :row_bytes]
        tok[i] = g
        sess[i] = int(session_ids[a]) if session_ids is not None else a
        mb[i] = int(micro_batch_ids[a]) if micro_batch_ids is not None else 0
        offs[i] = i - int(starts[key[g]])
        if scale is not None:
            if token_scale is not None:
                scale[i] = np.float32(token_scale[g])
            else:
                scale[i] = token_bytes[g, H:H + 4].copy().view(np.float32)[0]

    out = dict(actual_token_num=actual, group_list=group_list, err_count=err_count,
               y=y, session_ids=sess, micro_batch_ids=mb, token_ids=tok,
               expert_offsets=offs)
    if scale is not None:
        out["dynamic_scale"] = scale
    return out

"""Seeded synthetic inputs for the MoE token-reordering path.

This module only draws random inputs; it holds none of the operations'
arithmetic.  Both the CPU oracle's tests and the HIP path's tests / benchmark
take their inputs from here, so the two sides always see identical bytes.

Element storage follows the oracle's convention: FP16 as ``numpy.float16``,
BF16 as ``numpy.uint16`` bit patterns (the top 16 bits of a float32 draw),
FP32 as ``numpy.float32``, INT8 as ``numpy.int8``.

Named workloads (the shapes and value distributions of the five standard
cases):

=====  ===========================================================================
case   recipe
=====  ===========================================================================
1      batching: A=2, BS=8, K+1=3 (Y=48), H=128 FP16 ~N(0,1); 16 experts, 1 layer;
       expert ids uniform [0,16); 5 slots masked
2      batching: A=16, BS=32, K+1=9 (Y=4608), H=7168 BF16 ~N(0,1); 256 experts;
       ids = perm[r], r ~ p(r) proportional to (r+1)^-1.1 (Zipf s=1.1), perm a
       random permutation of the experts; 230 slots masked (5%)
3      batching: A=64, BS=64, K+1=9 (Y=36864), H=7168 INT8 uniform [-127,127] with
       a packed FP32 scale ~U(1e-3,1e-1) per row (row stride H+4); 16 layers x
       64 experts (expertNum=1024); layer of chunk a = a mod 16; ids uniform
       [0,64); 7373 slots masked (20%)
4      unpermute, non-padded, FP32 probs: T=16384, topK=8, E=128, H=4096 BF16
       ~N(0,1) permuted rows [T*topK, H]; 13107 slots (10%) = -1; the valid slots
       read permuted rows given by a random permutation of [0, #valid); token t's
       routing-map row has (#valid slots of t) ones at random experts; probs =
       softmax of N(0,1) logits over those experts, 0 elsewhere
5      unpermute, padded, FP16 probs: E=64, capacity C=512 (rows = 32768),
       H=5120 FP16 ~N(0,1), T=8192; each expert's C sortedIndices entries are
       drawn from [0,T) without replacement; routing map = top-4 of N(0,1)
       logits per token; probs = FP16 softmax over the top-4, 0 elsewhere
=====  ===========================================================================

All masks and -1 sets are exact counts drawn without replacement, so byte
counts of a case are deterministic.
"""

import os

import numpy as np

FP16, BF16, INT8, FP32 = 0, 1, 2, 3
_ELT = {FP16: 2, BF16: 2, INT8: 1, FP32: 4}


_CHUNK = 1 << 22   # elements per independently seeded block of a large draw


def _convert_block(x, dt):
    if dt == FP16:
        return x.astype(np.float16)
    if dt == BF16:
        return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    if dt == FP32:
        return x
    raise ValueError(dt)


def _normal_elements(rng, shape, dt):
    """N(0,1) elements of type ``dt``.

    Large draws are split into blocks of ``_CHUNK`` elements, each with its own
    child generator spawned from ``rng``, and filled on a thread pool; the
    result depends only on the seed and the shape, not on the thread count.
    """
    n = int(np.prod(shape))
    if n <= _CHUNK:
        return _convert_block(rng.standard_normal(size=shape, dtype=np.float32), dt)
    out_dtype = {FP16: np.float16, BF16: np.uint16, FP32: np.float32}[dt]
    out = np.empty(n, dtype=out_dtype)
    nblk = (n + _CHUNK - 1) // _CHUNK
    children = rng.spawn(nblk)

    def fill(b):
        lo, hi = b * _CHUNK, min(n, (b + 1) * _CHUNK)
        out[lo:hi] = _convert_block(children[b].standard_normal(size=hi - lo, dtype=np.float32), dt)

    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(fill, range(nblk)))
    return out.reshape(shape)


def _softmax_rows(logits, keep):
    """Row softmax over the kept entries; rows with nothing kept are all zero."""
    any_kept = keep.any(axis=1, keepdims=True)
    z = np.where(keep, logits.astype(np.float64), -1e300)
    z = z - z.max(axis=1, keepdims=True)
    e = np.where(keep, np.exp(z), 0.0)
    s = np.where(any_kept, e.sum(axis=1, keepdims=True), 1.0)
    return e / s


# ----------------------------------------------------------------------------- batching

def batching_case(seed, A, BS, K1, H, expert_num, layer_num, token_dtype,
                  n_masked=0, expert_dist="uniform", zipf_s=1.1, layer_of_chunk=None,
                  n_bad_ids=0, with_id_tables=False, stride_pad=0, separate_scale=False):
    """Draw one batching input.

    Returns a dict: ``token_bytes`` uint8 [Y, stride] (row s = slot s; for INT8
    with ``separate_scale`` False the FP32 scale sits in bytes [H, H+4)),
    ``token_scale`` float32 [Y] or None, ``expert_ids`` int32 [Y], ``mask``
    uint8 [Y] or None, ``layer_ids`` / ``session_ids`` / ``micro_batch_ids``
    int32 [A] or None, plus the scalar parameters.
    """
    rng = np.random.default_rng(seed)
    Y = A * BS * K1
    L = max(layer_num, 1)
    per_layer = expert_num // L
    elt = _ELT[token_dtype]
    row = H * elt
    if token_dtype == INT8:
        data = rng.integers(-127, 128, size=(Y, H), dtype=np.int16).astype(np.int8)
        scale = rng.uniform(1e-3, 1e-1, size=Y).astype(np.float32)
        payload = data.view(np.uint8).reshape(Y, H)
        if separate_scale:
            stride = row + stride_pad
            tb = np.zeros((Y, stride), dtype=np.uint8)
            tb[:, :row] = payload
            token_scale = scale
        else:
            stride = row + 4 + stride_pad
            tb = np.zeros((Y, stride), dtype=np.uint8)
            tb[:, :row] = payload
            tb[:, row:row + 4] = scale.view(np.uint8).reshape(Y, 4)
            token_scale = None
    else:
        data = _normal_elements(rng, (Y, H), token_dtype)
        stride = row + stride_pad
        tb = np.zeros((Y, stride), dtype=np.uint8)
        tb[:, :row] = data.view(np.uint8).reshape(Y, row)
        token_scale = None

    if expert_dist == "uniform":
        ids = rng.integers(0, per_layer, size=Y).astype(np.int32)
    elif expert_dist == "zipf":
        p = (np.arange(per_layer, dtype=np.float64) + 1.0) ** (-zipf_s)
        p /= p.sum()
        r = rng.choice(per_layer, size=Y, p=p)
        perm = rng.permutation(per_layer)
        ids = perm[r].astype(np.int32)
    elif expert_dist == "modulo":
        ids = (np.arange(Y) % (BS * K1) % per_layer).astype(np.int32)
    else:
        raise ValueError(expert_dist)

    mask = None
    if n_masked:
        mask = np.zeros(Y, dtype=np.uint8)
        mask[rng.choice(Y, size=n_masked, replace=False)] = 1
    if n_bad_ids:
        bad = rng.choice(Y, size=n_bad_ids, replace=False)
        vals = rng.choice(np.array([-1, -7, per_layer, per_layer + 3, 1 << 30]), size=n_bad_ids)
        ids[bad] = vals.astype(np.int32)

    layer_ids = None
    if layer_num >= 1 and (layer_of_chunk is not None or L > 1):
        if layer_of_chunk == "mod":
            layer_ids = (np.arange(A) % L).astype(np.int32)
        else:
            layer_ids = rng.integers(0, L, size=A).astype(np.int32)
    session_ids = micro_batch_ids = None
    if with_id_tables:
        session_ids = rng.integers(0, 1 << 20, size=A).astype(np.int32)
        micro_batch_ids = rng.integers(0, 64, size=A).astype(np.int32)

    return dict(token_bytes=tb, token_scale=token_scale, expert_ids=ids, mask=mask,
                layer_ids=layer_ids, session_ids=session_ids, micro_batch_ids=micro_batch_ids,
                A=A, BS=BS, K1=K1, H=H, expert_num=expert_num, layer_num=layer_num,
                token_dtype=token_dtype, stride=stride)


def batching_config(n):
    """The named batching workloads 1-3 (see the module table)."""
    if n == 1:
        return batching_case(1, A=2, BS=8, K1=3, H=128, expert_num=16, layer_num=1,
                             token_dtype=FP16, n_masked=5)
    if n == 2:
        return batching_case(2, A=16, BS=32, K1=9, H=7168, expert_num=256, layer_num=1,
                             token_dtype=BF16, n_masked=230, expert_dist="zipf")
    if n == 3:
        return batching_case(3, A=64, BS=64, K1=9, H=7168, expert_num=1024, layer_num=16,
                             token_dtype=INT8, n_masked=7373, layer_of_chunk="mod")
    raise ValueError(n)


# ----------------------------------------------------------------------------- unpermute

def unpermute_nonpadded_case(seed, T, K, E, H, dtype, probs_dtype=None, n_empty=0,
                             with_probs=True, rows_mode="compact"):
    """Non-padded (token-slot) input: sortedIndices [T*K], permuted rows [T*K, H].

    ``rows_mode`` "compact": the valid slots read a random permutation of rows
    [0, #valid); "slots": they read a random permutation of their own slot
    indices.
    """
    rng = np.random.default_rng(seed)
    N = T * K
    x = _normal_elements(rng, (N, H), dtype)
    sI = np.full(N, -1, dtype=np.int32)
    empty = np.zeros(N, dtype=bool)
    if n_empty:
        empty[rng.choice(N, size=n_empty, replace=False)] = True
    valid_slots = np.nonzero(~empty)[0]
    if rows_mode == "compact":
        sI[valid_slots] = rng.permutation(valid_slots.shape[0]).astype(np.int32)
    else:
        sI[valid_slots] = rng.permutation(valid_slots).astype(np.int32)
    routing_map = probs = None
    if with_probs:
        n_t = (~empty).reshape(T, K).sum(axis=1)
        routing_map = np.zeros((T, E), dtype=np.int8)
        for t in range(T):
            if n_t[t]:
                routing_map[t, rng.choice(E, size=int(n_t[t]), replace=False)] = 1
        logits = rng.standard_normal(size=(T, E))
        p = _softmax_rows(logits, routing_map != 0)
        probs = _probs_storage(p, probs_dtype)
    return dict(permuted=x, dtype=dtype, sorted_indices=sI, routing_map=routing_map,
                probs=probs, probs_dtype=probs_dtype if with_probs else None,
                padded_mode=False, restore_shape=(T, H), T=T, K=K, E=E, H=H)


def unpermute_padded_case(seed, E, C, T, H, dtype, probs_dtype=None, topk=4,
                          with_probs=True, n_invalid=0):
    """Padded (expert-capacity) input: sortedIndices [E*C] of token ids."""
    rng = np.random.default_rng(seed)
    N = E * C
    x = _normal_elements(rng, (N, H), dtype)
    sI = np.empty(N, dtype=np.int32)
    for e in range(E):
        sI[e * C:(e + 1) * C] = rng.choice(T, size=C, replace=C > T)
    if n_invalid:
        pos = rng.choice(N, size=n_invalid, replace=False)
        sI[pos] = rng.choice(np.array([-1, T, T + 5, -3]), size=n_invalid).astype(np.int32)
    routing_map = probs = None
    if with_probs:
        logits = rng.standard_normal(size=(T, E))
        k = min(topk, E)
        top = np.argsort(-logits, axis=1, kind="stable")[:, :k]
        routing_map = np.zeros((T, E), dtype=np.int8)
        np.put_along_axis(routing_map, top, 1, axis=1)
        p = _softmax_rows(logits, routing_map != 0)
        probs = _probs_storage(p, probs_dtype)
    return dict(permuted=x, dtype=dtype, sorted_indices=sI, routing_map=routing_map,
                probs=probs, probs_dtype=probs_dtype if with_probs else None,
                padded_mode=True, restore_shape=(T, H), T=T, E=E, C=C, H=H)


def _probs_storage(p, dt):
    p32 = p.astype(np.float32)
    if dt == FP32:
        return p32
    if dt == FP16:
        return p32.astype(np.float16)
    if dt == BF16:
        return (p32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    raise ValueError(dt)


def unpermute_config(n):
    """The named unpermute workloads 4 and 5 (see the module table)."""
    if n == 4:
        return unpermute_nonpadded_case(4, T=16384, K=8, E=128, H=4096, dtype=BF16,
                                        probs_dtype=FP32, n_empty=13107)
    if n == 5:
        return unpermute_padded_case(5, E=64, C=512, T=8192, H=5120, dtype=FP16,
                                     probs_dtype=FP16, topk=4)
    raise ValueError(n)


def permute_case(seed, T, K, E, H, dtype, padded=False, C=None, n_t=None, route="uniform", row_pad=0):
    """Forward-permute input: tokens [T, H] (optionally inside rows of H + row_pad
    elements), a routing map [T, E] with n_t[t] distinct experts per token (drawn in
    [0, K] unless given; route "uniform" picks experts uniformly, "skew" favours
    low-numbered experts), and the output size N = T*K (non-padded) or E*C (padded)."""
    rng = np.random.default_rng(seed)
    x = _normal_elements(rng, (T, H + row_pad), dtype) if dtype != INT8 else \
        rng.integers(-127, 128, size=(T, H + row_pad)).astype(np.int8)
    if n_t is None:
        n_t = rng.integers(0, K + 1, size=T)
    n_t = np.minimum(np.asarray(n_t), E)
    rmap = np.zeros((T, E), dtype=np.int8)
    if route == "skew":
        w = 1.0 / np.arange(1, E + 1) ** 1.2
        w /= w.sum()
    for t in range(T):
        if n_t[t] == 0:
            continue
        if route == "skew":
            rmap[t, rng.choice(E, size=int(n_t[t]), replace=False, p=w)] = 1
        else:
            rmap[t, rng.choice(E, size=int(n_t[t]), replace=False)] = 1
    N = (E * C if C is not None else 0) if padded else T * K
    return dict(tokens_full=x, H=H, dtype=dtype, routing_map=rmap, padded=padded, C=C, N=N, T=T, E=E, K=K)


def permute_config():
    """Forward permute at the non-padded unpermute workload's shape (T=16384, topK=8,
    E=128, H=4096 BF16): every token routed to 8 distinct uniform experts."""
    return permute_case(6, T=16384, K=8, E=128, H=4096, dtype=BF16, n_t=np.full(16384, 8))


def permute_padded_config():
    """Padded forward permute at the padded unpermute workload's shape (E=64, C=512,
    T=8192, H=5120 FP16): every token routed to 4 distinct uniform experts."""
    return permute_case(7, T=8192, K=4, E=64, H=5120, dtype=FP16, padded=True, C=512, n_t=np.full(8192, 4))


def config(n):
    return batching_config(n) if n <= 3 else unpermute_config(n)


# ----------------------------------------------------------------------------- schedule context

def _ctx_dtype():
    """The usage example's packed ScheduleContext, declared member by member (a NumPy
    structured type without alignment padding, as the definition is packed)."""
    r = lambda name, n: (name, "i1", (n,))
    common = [("session_num", "<u4"), ("micro_batch_num", "<u4"), ("micro_batch_size", "<u4"),
              ("selected_expert_num", "<u4"), ("expert_num", "<u4"), ("attn_to_ffn_token_size", "<u4"),
              ("ffn_to_attn_token_size", "<u4"), ("schedule_mode", "<i4"), r("reserve0", 96)]
    control = [("run_flag", "<i4"), r("reserve2", 124)]
    ffn = [("token_info_buf", "<u8"), ("token_info_buf_size", "<u8"), ("token_data_buf", "<u8"),
           ("token_data_buf_size", "<u8"), ("polling_index", "<u8"), r("reserve3", 88),
           ("layer_ids_buf", "<u8"), ("layer_ids_buf_size", "<u8"), ("session_ids_buf", "<u8"),
           ("session_ids_buf_size", "<u8"), ("micro_batch_ids_buf", "<u8"), ("micro_batch_ids_buf_size", "<u8"),
           ("expert_ids_buf", "<u8"), ("expert_ids_buf_size", "<u8"), ("out_num", "<u4"), r("reserve4", 60)]
    attention = [("token_info_buf", "<u8"), ("token_info_buf_size", "<u8"), ("token_data_buf", "<u8"),
                 ("token_data_buf_size", "<u8"), ("micro_batch_id", "<u4"), r("reserve5", 92)]
    return np.dtype([("common", common), ("control", control), ("attention", attention), ("ffn", ffn),
                     r("reserve6", 384)])


CTX_DTYPE = _ctx_dtype()


def ffn_data_desc_dtype(n_ids):
    """The usage example's packed FfnDataDesc with its trailing expert-id array sized."""
    return np.dtype([("flag", "<i4"), ("layer_id", "<i4"), ("expert_ids", "<i4", (n_ids,))])


def schedule_context(session_num, micro_batch_num, micro_batch_size, selected_expert_num, expert_num,
                     token_info_buf, token_info_buf_size, token_data_buf, token_data_buf_size,
                     polling_index=0, schedule_mode=0, run_flag=1, token_sizes=(512, 512)):
    """The 1024 context bytes, filled like the usage example fills them."""
    c = np.zeros((), dtype=CTX_DTYPE)
    cm = c["common"]
    cm["session_num"], cm["micro_batch_num"] = session_num, micro_batch_num
    cm["micro_batch_size"], cm["selected_expert_num"] = micro_batch_size, selected_expert_num
    cm["expert_num"] = expert_num
    cm["attn_to_ffn_token_size"], cm["ffn_to_attn_token_size"] = token_sizes
    cm["schedule_mode"] = schedule_mode
    c["control"]["run_flag"] = run_flag
    f = c["ffn"]
    f["token_info_buf"], f["token_info_buf_size"] = token_info_buf, token_info_buf_size
    f["token_data_buf"], f["token_data_buf_size"] = token_data_buf, token_data_buf_size
    f["polling_index"] = polling_index
    return np.frombuffer(c.tobytes(), dtype=np.uint8).copy()


def schedule_area(seed, A, M, BS, K1, H, expert_num, layer_num, token_dtype, n_not_ready=0, n_bad_ids=0,
                  bad_layers=0):
    """The attention->FFN data area of A sessions x M micro-batches: ``info`` (the
    FfnDataDesc of every chunk, session-major, as uint8 bytes) and ``data`` (uint8
    [A*M*BS*K1, row]: each chunk's BS*K1 rows in chunk order; an INT8 row is H bytes
    then its FP32 scale).  ``n_not_ready`` chunks get a flag other than 1; ids uniform
    within the layer, ``n_bad_ids`` of them out of range; ``bad_layers`` chunks get an
    out-of-range layer id."""
    rng = np.random.default_rng(seed)
    nch, n = A * M, BS * K1
    L = max(layer_num, 1)
    per_layer = expert_num // L
    row = H * _ELT[token_dtype] + (4 if token_dtype == INT8 else 0)
    rows = nch * n
    if token_dtype == INT8:
        data = np.empty((rows, row), dtype=np.uint8)
        data[:, :H] = rng.integers(-127, 128, size=(rows, H), dtype=np.int16).astype(np.int8).view(np.uint8)
        data[:, H:] = rng.uniform(1e-3, 1e-1, size=rows).astype(np.float32).view(np.uint8).reshape(rows, 4)
    else:
        data = _normal_elements(rng, (rows, H), token_dtype).view(np.uint8).reshape(rows, row)
    flags = np.ones(nch, dtype=np.int32)
    if n_not_ready:
        flags[rng.choice(nch, size=n_not_ready, replace=False)] = rng.choice(
            np.array([0, 2, -1], dtype=np.int32), size=n_not_ready)
    layers = rng.integers(0, L, size=nch).astype(np.int32)
    if bad_layers:
        layers[rng.choice(nch, size=bad_layers, replace=False)] = L
    ids = rng.integers(0, per_layer, size=(nch, n)).astype(np.int32)
    if n_bad_ids:
        flat = ids.reshape(-1)
        bad = rng.choice(flat.size, size=n_bad_ids, replace=False)
        flat[bad] = rng.choice(np.array([-1, per_layer, per_layer + 9, 1 << 30], dtype=np.int32), size=n_bad_ids)
    desc = np.zeros(nch, dtype=ffn_data_desc_dtype(n))
    desc["flag"], desc["layer_id"], desc["expert_ids"] = flags, layers, ids
    info = np.frombuffer(desc.tobytes(), dtype=np.uint8).copy()
    return dict(info=info, data=data, flags=flags, layers=layers, expert_ids=ids, row=row,
                A=A, M=M, BS=BS, K1=K1, H=H, expert_num=expert_num, layer_num=layer_num,
                token_dtype=token_dtype)


# ----------------------------------------------------------------------------- expert update

def eplb_table(rng, E, world_size, place_per_rank, F):
    """An expert-placement table: W*P physical instances, each hosting one logical
    expert; every expert has at least one instance, the W*P - E spare instances go to
    random experts as extra replicas (at most F - 1 per expert).  Row e = [count,
    distinct instance ids, then -1 padding]."""
    n_inst = world_size * place_per_rank
    assert E <= n_inst <= E * (F - 1)
    inst = rng.permutation(n_inst).astype(np.int32)
    rows = [[int(inst[e])] for e in range(E)]
    for i in inst[E:]:
        while True:
            e = int(rng.integers(0, E))
            if len(rows[e]) < F - 1:
                rows[e].append(int(i))
                break
    table = np.full((E, F), -1, dtype=np.int32)
    for e, r in enumerate(rows):
        table[e, 0] = len(r)
        table[e, 1:1 + len(r)] = r
    return table


def update_expert_case(seed, BS, K, E, world_size, place_per_rank, F=None, local_rank_id=0, balance_mode=0,
                       id_dtype=np.int32, scale_dtype=None, n_active=None, keep_frac=0.8, n_bad_ids=0):
    """MoeUpdateExpert input: each token's K distinct logical experts (uniform), the
    placement table, and optionally descending softmax scales of the token's experts
    with a per-slot threshold that prunes about 1 - keep_frac of the slots, and an
    active mask whose first n_active tokens are true."""
    rng = np.random.default_rng(seed)
    F = F if F is not None else world_size + 1
    table = eplb_table(rng, E, world_size, place_per_rank, F)
    ids = np.stack([rng.choice(E, size=K, replace=False) for _ in range(BS)]).astype(id_dtype)
    if n_bad_ids:
        flat = ids.reshape(-1)
        bad = rng.choice(flat.size, size=n_bad_ids, replace=False)
        flat[bad] = rng.choice(np.array([-1, E, E + 7]), size=n_bad_ids).astype(id_dtype)
    scales = thr = active = None
    if scale_dtype is not None:
        logits = rng.standard_normal((BS, K))
        p = np.exp(logits - logits.max(axis=1, keepdims=True))
        p = -np.sort(-(p / p.sum(axis=1, keepdims=True)), axis=1)
        scales = _probs_storage(p, scale_dtype)
        thr = np.quantile(p, 1.0 - keep_frac, axis=0).astype(np.float32)
        if n_active is not None:
            active = np.zeros(BS, dtype=bool)
            active[:n_active] = True
    return dict(expert_ids=ids, eplb_table=table, expert_scales=scales, scale_dtype=scale_dtype,
                pruning_threshold=thr, active_mask=active, local_rank_id=local_rank_id, world_size=world_size,
                balance_mode=balance_mode, BS=BS, K=K, E=E, F=F)

"""Oracle for MoE token unpermute with routing map (test infrastructure only).

Source: the article "MoeTokenUnpermuteWithRoutingMap 算子全解析" (pptc.cn) --
  * section "Function description and formulas": the derived sizes
    (topK_num = rows // tokens, numExperts / numTokens from probs' shape,
    capacity = len(sortedIndices) // numExperts) and the four branches
    (padded x has-probs);
  * "Supplementary notes": shapes and value ranges of every input and output;
  * "Kernel implementation": the padded kernel reads the prob of position pos at
    flat address sortedIndices[pos] * num_experts + pos / capacity; the
    non-padded kernel skips slots whose index is outside [0, rows), computes
    in float and converts back with round-to-nearest-even.

Arithmetic follows the article's kernel description: every element is widened
to FP32, multiplied by its FP32 weight (one rounding), added to an FP32
accumulator that starts at +0.0 (one rounding), in a fixed order, and the sum is
rounded once to the output type.

Readings taken where the article is silent, garbled or self-contradictory
(listed with reasons in the design notes):
  * lost operators: the accumulating assignments are "+=";
  * branch 1's garbled prob line means permuteProbs[i] = probs[sI[i], i // C]
    (the padded kernel's flat address says the same);
  * branch 2 applies each weight once; the weight of the slot that reads
    permuted row r is permuteProbs[r] ("W2", default: rows are multiplied by
    their compacted probs, which is the expert-major order masked_select
    produces).  ``weight_index=1`` selects the literal last line of branch 2,
    permuteProbs[slot] ("W1");
  * permuteProbs is zero-padded to len(sortedIndices) (its documented length);
    if the routing map holds more ones than that, the excess is dropped;
  * order of accumulation: ascending slot (non-padded); ascending permuted row
    within a token (padded, i.e. a stable sort);
  * padded mode: entries of sortedIndices outside [0, tokens) are not
    accumulated, sort after every valid entry (stable), and get weight 0;
  * non-padded outIndex = stable argsort of sortedIndices with invalid slots
    (outside [0, rows)) first, and permuteTokenId = outIndex // topK -- the
    only reading that fits the documented value ranges of both outputs.  Where
    the empty slots go (first) is the reading itself and stays unpinned; the
    rest (order by row index, stability, an index >= rows counted as empty) is
    pinned by a hand-worked example;
  * zero weights are multiplied in, not skipped, unless ``skip_zero_weight`` is set:
    then, as the article's kernel description has it (each slot's row is copied only
    when its index is valid and its prob is non-zero), terms with weight 0 are left
    out -- the same result for finite rows, different where a zero-weight row holds
    inf or NaN.  The skip is applied in both layouts.

Pins (tests/test_oracle_unpermute.py): the article's padded {2,2} example
(formula result; the article's printed "all 2" claim contradicts its own
formula), closed forms (permute-then-unpermute identities, softmax-weighted
recombination), brute force against torch index_add_ in float64 within the FP32
error bound, property checks of the auxiliary outputs, hand-worked examples of
both weight indices on permuted (non-identity) sortedIndices, where W1 and W2
give different sums, and of the non-padded auxiliary order with -1 and an index
>= rows, and for the zero-weight skip: equality with the formula on finite rows
and two worked examples where a zero-weight row holds NaN / inf.
"""

import numpy as np

from .numerics import to_f32, from_f32, storage_dtype


def moe_token_unpermute_with_routing_map(permuted_tokens, tokens_dtype, sorted_indices,
                                         padded_mode, restore_shape, routing_map=None,
                                         probs=None, probs_dtype=None, weight_index=0,
                                         skip_zero_weight=False):
    """Reference unpermute.

    permuted_tokens : [rows, H] stored as ``tokens_dtype`` (see numerics).
    sorted_indices  : int32 [N].
    restore_shape   : (tokens, H).
    routing_map     : int8/bool [tokens, experts] or None (None iff probs None).
    probs           : [tokens, experts] stored as ``probs_dtype`` or None.

    Returns dict(unpermuted [tokens, H] in tokens_dtype, out_index int32 [N],
    permute_token_id int32 [N], permute_probs [N] in probs_dtype or None).
    """
    x = to_f32(permuted_tokens, tokens_dtype)
    rows, H = x.shape
    T, H2 = (int(v) for v in restore_shape)
    assert H2 == H
    sI = np.asarray(sorted_indices, dtype=np.int64)
    N = sI.shape[0]
    has_probs = probs is not None
    assert (routing_map is None) == (probs is None)
    if has_probs:
        pf = to_f32(probs, probs_dtype)
        assert pf.shape[0] == T
        E = pf.shape[1]
    acc = np.zeros((T, H), dtype=np.float32)  # starts at +0.0

    if padded_mode:
        # Branches 1 and 3: permuteTokenId, outIndex = sortedIndices.sort()
        valid = (sI >= 0) & (sI < T)
        key = np.where(valid, sI, T)
        out_index = np.argsort(key, kind="stable")
        permute_token_id = sI[out_index]
        permute_probs = None
        if has_probs:
            C = N // E
            w = np.zeros(N, dtype=np.float32)
            for i in range(N):
                if valid[i]:
                    w[i] = pf[sI[i], i // C]
            permute_probs = from_f32(w, probs_dtype)
            w = to_f32(permute_probs, probs_dtype)
        # unpermuted[permuteTokenId[j]] += permutedTokens[outIndex[j]] (* weight)
        for j in range(N):
            t = int(permute_token_id[j])
            r = int(out_index[j])
            if not (0 <= t < T):
                continue
            if has_probs:
                if skip_zero_weight and w[r] == 0:
                    continue  # the kernel copies a row only when its prob is non-zero
                acc[t] = acc[t] + x[r] * w[r]
            else:
                acc[t] = acc[t] + x[r]
    else:
        # Branches 2 and 4.
        K = N // T
        permute_probs = None
        if has_probs:
            # permuteProbs = probs.T.maskedSelect(routingMap.T): expert-major order.
            sel = np.asarray(pf).T[np.asarray(routing_map).T != 0]
            P = np.zeros(N, dtype=np.float32)
            n = min(sel.shape[0], N)
            P[:n] = sel[:n]
            permute_probs = from_f32(P, probs_dtype)
            P = to_f32(permute_probs, probs_dtype)
        for t in range(T):
            for k in range(K):
                i = t * K + k
                r = int(sI[i])
                if not (0 <= r < rows):
                    continue  # -1 (or any out-of-range index) marks an empty slot
                if has_probs:
                    w = P[r] if weight_index == 0 else P[i]
                    if skip_zero_weight and w == 0:
                        continue  # the kernel copies a row only when its prob is non-zero
                    acc[t] = acc[t] + x[r] * w
                else:
                    acc[t] = acc[t] + x[r]
        valid = (sI >= 0) & (sI < rows)
        key = np.where(valid, sI + 1, 0)
        out_index = np.argsort(key, kind="stable")
        permute_token_id = out_index // max(K, 1)

    out = from_f32(acc, tokens_dtype).astype(storage_dtype(tokens_dtype), copy=False)
    return dict(unpermuted=out,
                out_index=out_index.astype(np.int32),
                permute_token_id=permute_token_id.astype(np.int32),
                permute_probs=permute_probs)

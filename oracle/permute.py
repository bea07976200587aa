"""Oracle for the forward MoE token permute with routing map (test infrastructure only).

Source: the MoeTokenUnpermuteWithRoutingMap article --
  * "Operator positioning": the permute step regroups the original tokens, by the
    routing map, into an expert-grouped compact layout (permutedTokens), so that
    every expert reads its tokens contiguously; the unpermute later uses
    sortedIndices to return each result to its token;
  * "Function description and formulas", branches 1-4: the unpermute contract the
    permute's outputs feed -- non-padded: token t's slot t*topK + k reads permuted
    row sortedIndices[t*topK + k] (rows outside [0, rows) mark an empty slot);
    padded: capacity entry i of expert i // C holds token sortedIndices[i];
  * the same section's weight layout (permuteProbs = probs.T masked by routingMap.T):
    permuted rows are in expert-major order of the routing map's non-zero entries.

The page names the forward op and its role only.  The readings below define its
outputs as the arrangement the unpermute's formulas invert (each listed with its
reason in the design notes):
  * non-padded, N = T * topK output rows: row r holds the token of the r-th
    non-zero map entry in expert-major order (expert ascending, then token
    ascending); rows past the number of non-zero entries are zero; entries past N
    are dropped;
  * non-padded sortedIndices[t*topK + k] = the row of token t's k-th non-zero
    expert (experts ascending), for k below the token's expert count and topK;
    every other slot is -1;
  * padded, capacity C, N = E * C rows: expert e's block holds its first C tokens
    in ascending order; sortedIndices[e*C + j] = that token, -1 for the unused
    capacity (whose rows are zero); tokens beyond the capacity are dropped.

Rows are moved as bytes: any element type works.

Pins (tests/test_oracle_permute.py): round trips through the unpermute oracle
(permute then unpermute without probs gives n_t * x bit-exactly, and x exactly for
one expert per token; with softmax weights it gives x within the FP32 bound), an
independent construction from torch.nonzero of the transposed map, and brute
force on tiny inputs.
"""

import numpy as np


def moe_token_permute_with_routing_map(tokens, routing_map, num_out_rows, padded_mode=False, capacity=None):
    """Reference forward permute.

    tokens       : [T, H] array of any element type (moved as bytes).
    routing_map  : [T, E] array; non-zero = token routed to the expert.
    num_out_rows : N; non-padded: a multiple of T (topK = N // T); padded: E * capacity.
    Returns dict(permuted_tokens [N, H] like tokens, sorted_indices int32 [N]).
    """
    tokens = np.asarray(tokens)
    rmap = np.asarray(routing_map) != 0
    T, E = rmap.shape
    assert tokens.shape[0] == T
    H = tokens.shape[1]
    N = int(num_out_rows)
    permuted = np.zeros((N, H), dtype=tokens.dtype)
    sorted_indices = np.full(N, -1, dtype=np.int32)
    if padded_mode:
        C = int(capacity)
        assert N == E * C
        for e in range(E):
            j = 0
            for t in range(T):
                if rmap[t, e] and j < C:
                    sorted_indices[e * C + j] = t
                    permuted[e * C + j] = tokens[t]
                    j += 1
        return dict(permuted_tokens=permuted, sorted_indices=sorted_indices)
    assert T > 0 and N % T == 0
    K = N // T
    # expert-major walk of the non-zero entries: row r <- token of the r-th entry
    row_of = {}
    r = 0
    for e in range(E):
        for t in range(T):
            if rmap[t, e]:
                if r < N:
                    permuted[r] = tokens[t]
                    row_of[(t, e)] = r
                r += 1
    # token t's k-th expert (ascending) -> its row
    for t in range(T):
        k = 0
        for e in range(E):
            if rmap[t, e]:
                if k < K and (t, e) in row_of:
                    sorted_indices[t * K + k] = row_of[(t, e)]
                k += 1
    return dict(permuted_tokens=permuted, sorted_indices=sorted_indices)

"""Oracle for MoeUpdateExpert (test infrastructure only).

Source: the MoeUpdateExpert README page --
  * "Function description": for unbalanced load, map each token's topK logical
    expert ids to physical expert instances, and prune a token's experts by a
    threshold on their scales;
  * the parameter table: expertIds (BS, K); eplbTable (moeExpertNum, F), row e =
    [count, instance_1 .. instance_count] with count in [1, worldSize] and distinct
    instance ids in [0, worldSize * place_per_rank); expertScales (BS, K), descending
    within a token, given together with pruningThreshold (K,) or (1, K); activeMask
    (BS,), true = the token takes part, trues before falses, only with the scales;
    localRankId; worldSize; balanceMode 0 = distribute by rank, 1 = by token;
    outputs balancedExpertIds (BS, K), the instance each of a token's experts maps
    to, and balancedActiveMask (BS, K), valid when scales and threshold are given;
  * "Constraints": 0 < BS <= 512, 0 < K <= 16 and K <= moeExpertNum, moeExpertNum in
    (0, 1024], F in [2, worldSize + 1]; worldSize in [2, 768] and localRankId in
    [0, worldSize) when balanceMode is 0.

Readings taken where the page is silent (each listed with its reason in the design
notes):
  * the instance of (token t, slot k) with logical expert e is eplbTable[e, 1 + r],
    r = localRankId mod count (balanceMode 0) or t mod count (balanceMode 1):
    mode 0 sends all of a rank's tokens for e to one replica, different ranks to
    different replicas in turn; mode 1 spreads a rank's tokens over the replicas;
  * pruning is per element: slot k of token t stays active when the token is active
    and scale[t, k] >= threshold[k] (a scale below the threshold is pruned); the
    descending order of the scales is a caller guarantee the rule does not need;
  * the mapping does not depend on pruning or activity: every slot is mapped;
  * an expert id outside [0, moeExpertNum), or a table count outside [1, F - 1],
    maps to -1, is counted in err_count, and is inactive in the mask.

Pins (tests/test_oracle_update_expert.py): a count of 1 everywhere reduces to a
plain table lookup (NumPy fancy indexing); the chosen instance is always one of the
expert's listed instances; balanceMode 0 gives one instance per (rank, expert) and,
over all ranks, uses each replica floor(W/count) or ceil(W/count) times; balanceMode
1 ignores the rank and, over count consecutive tokens routed to e, uses each replica
once; the mask against NumPy's elementwise comparison; error cases by hand.  The
exact replica index is a reading of the page: beyond these invariants its parity is
unpinned.
"""

import numpy as np


def moe_update_expert(expert_ids, eplb_table, local_rank_id, world_size, balance_mode,
                      expert_scales=None, pruning_threshold=None, active_mask=None):
    """Reference MoeUpdateExpert.

    expert_ids       : int [BS, K] logical expert ids.
    eplb_table       : int32 [E, F]; row e = [count, instance ids ...].
    expert_scales    : float32 [BS, K] (values of the FP16 / BF16 / FP32 scales) or None.
    pruning_threshold: float32 [K] or None (given iff expert_scales is).
    active_mask      : bool [BS] or None (only with the scales).
    Returns dict(balanced_expert_ids [BS, K] like expert_ids, balanced_active_mask
    bool [BS, K] or None, err_count).
    """
    ids = np.asarray(expert_ids)
    table = np.asarray(eplb_table, dtype=np.int64)
    BS, K = ids.shape
    E, F = table.shape
    out = np.empty((BS, K), dtype=ids.dtype)
    ok = np.ones((BS, K), dtype=bool)
    err = 0
    for t in range(BS):
        for k in range(K):
            e = int(ids[t, k])
            if not 0 <= e < E:
                out[t, k], ok[t, k] = -1, False
                err += 1
                continue
            count = int(table[e, 0])
            if not 1 <= count <= F - 1:
                out[t, k], ok[t, k] = -1, False
                err += 1
                continue
            r = (int(local_rank_id) if balance_mode == 0 else t) % count
            out[t, k] = table[e, 1 + r]
    mask = None
    if expert_scales is not None:
        s = np.asarray(expert_scales, dtype=np.float32)
        thr = np.asarray(pruning_threshold, dtype=np.float32).reshape(-1)
        mask = np.zeros((BS, K), dtype=bool)
        for t in range(BS):
            if active_mask is not None and not active_mask[t]:
                continue
            for k in range(K):
                mask[t, k] = ok[t, k] and not (s[t, k] < thr[k])
    return dict(balanced_expert_ids=out, balanced_active_mask=mask, err_count=err)

"""Pins for the MoeUpdateExpert oracle (CPU only).

  * count = 1 everywhere: a plain table lookup (NumPy fancy indexing);
  * the chosen instance is always one of the expert's listed instances;
  * balanceMode 0: one instance per (rank, expert), independent of the token; over
    all ranks each replica serves floor(W/count) or ceil(W/count) of them;
  * balanceMode 1: independent of the rank; over count consecutive tokens routed to
    an expert, each replica serves one;
  * the pruning mask against NumPy's elementwise comparison, with the active mask;
  * out-of-range ids and counts map to -1 and are counted.
"""

import numpy as np
import pytest

import synth
from oracle import numerics as nm
from oracle.update_expert import moe_update_expert


def _case(**kw):
    base = dict(BS=40, K=4, E=12, world_size=6, place_per_rank=3)
    base.update(kw)
    return synth.update_expert_case(5, **base)


def _run(c, rank=None, mode=None):
    s = None if c["expert_scales"] is None else nm.to_f32(c["expert_scales"], c["scale_dtype"])
    return moe_update_expert(c["expert_ids"], c["eplb_table"], c["local_rank_id"] if rank is None else rank,
                             c["world_size"], c["balance_mode"] if mode is None else mode, s,
                             c["pruning_threshold"], c["active_mask"])


@pytest.mark.parametrize("mode", [0, 1])
def test_single_instance_is_a_table_lookup(mode):
    c = _case(E=18, world_size=6, place_per_rank=3)         # 18 instances: count 1 everywhere
    assert (c["eplb_table"][:, 0] == 1).all()
    out = _run(c, rank=4, mode=mode)
    assert np.array_equal(out["balanced_expert_ids"], c["eplb_table"][c["expert_ids"], 1])
    assert out["err_count"] == 0 and out["balanced_active_mask"] is None


@pytest.mark.parametrize("mode,id_dtype", [(0, np.int32), (1, np.int64)])
def test_instance_is_one_of_the_experts_replicas(mode, id_dtype):
    c = _case(id_dtype=id_dtype)
    out = _run(c, rank=2, mode=mode)["balanced_expert_ids"]
    assert out.dtype == id_dtype
    t = c["eplb_table"]
    for (tok, k), inst in np.ndenumerate(out):
        e = c["expert_ids"][tok, k]
        assert inst in t[e, 1:1 + t[e, 0]]


def test_by_rank_one_replica_per_rank_and_balanced_over_ranks():
    c = _case(BS=64, world_size=7, place_per_rank=4, E=10, F=8)
    t, W = c["eplb_table"], c["world_size"]
    use = {}
    for r in range(W):
        out = _run(c, rank=r, mode=0)["balanced_expert_ids"]
        for e in range(c["E"]):
            chosen = set(out[c["expert_ids"] == e].tolist())
            assert len(chosen) <= 1                       # the same replica for every token
            for i in chosen:
                use.setdefault(e, []).append(i)
    for e, used in use.items():
        n = t[e, 0]
        counts = [used.count(int(i)) for i in t[e, 1:1 + n]]
        if len(used) == W:                                # every rank routed a token to e
            assert max(counts) - min(counts) <= 1 and sum(counts) == W


def test_by_token_ignores_the_rank_and_cycles_over_replicas():
    c = _case(BS=60, E=5, world_size=4, place_per_rank=4, F=5)
    a = _run(c, rank=0, mode=1)["balanced_expert_ids"]
    b = _run(c, rank=3, mode=1)["balanced_expert_ids"]
    assert np.array_equal(a, b)
    # every expert routed from all tokens: tokens t..t+count-1 use each replica once
    ids = np.tile(np.arange(5, dtype=np.int32)[None, :4], (60, 1))
    c2 = dict(c, expert_ids=ids, K=4)
    out = _run(c2, rank=1, mode=1)["balanced_expert_ids"]
    t = c["eplb_table"]
    for e in range(4):
        n = t[e, 0]
        for t0 in range(0, 60 - n + 1):
            assert sorted(out[t0:t0 + n, e].tolist()) == sorted(t[e, 1:1 + n].tolist())


@pytest.mark.parametrize("dt", [synth.FP16, synth.BF16, synth.FP32])
def test_pruning_mask_is_elementwise(dt):
    c = _case(BS=50, K=6, E=16, world_size=8, place_per_rank=3, scale_dtype=dt, n_active=35, keep_frac=0.6)
    out = _run(c)["balanced_active_mask"]
    s = nm.to_f32(c["expert_scales"], dt)
    expect = (s >= c["pruning_threshold"][None, :]) & c["active_mask"][:, None]
    assert np.array_equal(out, expect)
    assert 0 < out.sum() < out.size and not out[35:].any()


def test_equal_to_threshold_is_kept_and_nan_is_kept():
    c = _case(BS=3, K=2, E=4, world_size=2, place_per_rank=2, scale_dtype=synth.FP32)
    c["expert_scales"] = np.array([[0.5, 0.25], [0.5, 0.2], [np.nan, 0.3]], np.float32)
    c["pruning_threshold"] = np.array([0.5, 0.25], np.float32)
    out = _run(c)["balanced_active_mask"]
    assert out.tolist() == [[True, True], [True, False], [True, True]]


def test_bad_ids_and_counts_map_to_minus_one():
    c = _case(BS=6, K=2, E=4, world_size=2, place_per_rank=3, F=3, scale_dtype=synth.FP32, keep_frac=1.0)
    c["expert_ids"] = np.array([[0, 4], [-1, 1], [2, 3], [3, 0], [1, 2], [0, 1]], np.int32)
    c["eplb_table"] = c["eplb_table"].copy()
    c["eplb_table"][2, 0] = 0                 # count below 1
    c["eplb_table"][3, 0] = 3                 # count above F - 1 = 2
    out = _run(c)
    ids = out["balanced_expert_ids"]
    bad = [(0, 1), (1, 0), (2, 0), (2, 1), (3, 0), (4, 1)]
    assert sorted(map(tuple, np.argwhere(ids == -1).tolist())) == bad
    assert out["err_count"] == 6
    assert not out["balanced_active_mask"][ids == -1].any()
    assert (ids[ids != -1] >= 0).all()

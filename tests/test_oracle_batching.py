"""Pins for the batching oracle (CPU only).

Each test checks the oracle against something other than itself:
  * the API page's usage sample, with every output derived in closed form;
  * a hand-worked two-layer example;
  * an O(Y^2) brute-force selection (a different algorithm from the oracle's
    library argsort) on tiny random inputs;
  * invariants that any correct batching satisfies.
"""

import json
import os

import numpy as np
import pytest

import synth
from oracle import ffn_worker_batching

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _run(case):
    return ffn_worker_batching(
        case["token_bytes"], case["expert_ids"], case["expert_num"], case["layer_num"],
        (case["A"], case["BS"], case["K1"], case["H"]), case["token_dtype"],
        mask=case["mask"], layer_ids=case["layer_ids"], session_ids=case["session_ids"],
        micro_batch_ids=case["micro_batch_ids"], token_scale=case["token_scale"])


def test_api_page_usage_sample_closed_form():
    g = json.load(open(os.path.join(GOLD, "ffn_worker_batching_usage_sample.json")))["inputs"]
    A, BS, K1, H = g["session_num_A"], g["micro_batch_size_BS"], g["selected_expert_num_K_plus_1"], g["hidden_H"]
    E = g["expert_num"]
    Y = A * BS * K1
    ids = (np.arange(BS * K1) % E).astype(np.int32)          # expert_id = i % expert_num
    ids = np.tile(ids, A)
    tb = np.full((Y, H), g["token_data_element_int16"], dtype=np.int16).view(np.uint8).reshape(Y, 2 * H)
    out = ffn_worker_batching(tb, ids, E, g["layer_num"], (A, BS, K1, H), g["token_dtype"],
                              layer_ids=np.array([g["chunk_layer_id"]] * A, dtype=np.int32))
    # Closed form: every slot is valid, 72 slots over 8 experts, 9 slots each.
    assert out["actual_token_num"] == 72
    assert out["group_list"].tolist() == [[e, 9] for e in range(8)]
    j = np.arange(72)
    # Output row j belongs to expert j // 9; it is that expert's (j % 9)-th slot,
    # i.e. slot (j // 9) + 8 * (j % 9).
    assert out["token_ids"].tolist() == ((j // 9) + 8 * (j % 9)).tolist()
    assert out["expert_offsets"].tolist() == (j % 9).tolist()
    assert (out["session_ids"] == 0).all() and (out["micro_batch_ids"] == 0).all()
    assert (out["y"].view(np.uint16) == 1).all()
    assert out["err_count"] == 0


def test_hand_worked_two_layer_example():
    # 2 chunks (A=2) of BS*K1 = 1*3 slots, 2 layers x 2 experts (expert_num=4).
    # chunk 0 is layer 1, chunk 1 is layer 0.
    # slot:        0  1  2 | 3  4  5
    # expert id:   1  0  1 | 0  1  5(bad)
    # mask:        0  0  1 | 0  0  0
    # key = layer*2 + id:  3  2  masked | 0  1  invalid
    # sorted (key, slot): (0,3) (1,4) (2,1) (3,0)
    H = 2
    tb = np.arange(6 * 4, dtype=np.uint8).reshape(6, 4)
    out = ffn_worker_batching(tb, np.array([1, 0, 1, 0, 1, 5], np.int32), 4, 2, (2, 1, 3, H), 0,
                              mask=np.array([0, 0, 1, 0, 0, 0], np.uint8),
                              layer_ids=np.array([1, 0], np.int32),
                              session_ids=np.array([70, 80], np.int32),
                              micro_batch_ids=np.array([7, 8], np.int32))
    assert out["actual_token_num"] == 4
    assert out["err_count"] == 1
    assert out["group_list"].tolist() == [[0, 1], [1, 1], [2, 1], [3, 1]]
    assert out["token_ids"].tolist() == [3, 4, 1, 0]
    assert out["expert_offsets"].tolist() == [0, 0, 0, 0]
    assert out["session_ids"].tolist() == [80, 80, 70, 70]
    assert out["micro_batch_ids"].tolist() == [8, 8, 7, 7]
    assert out["y"].tolist() == [tb[3].tolist(), tb[4].tolist(), tb[1].tolist(), tb[0].tolist()]


def test_compact_group_list_with_gaps():
    # experts 0..7 in one layer; only experts 2 and 6 receive slots.
    ids = np.array([6, 2, 6, 6, 2, 2, 6, 2], np.int32)
    tb = np.zeros((8, 2), np.uint8)
    out = ffn_worker_batching(tb, ids, 8, 1, (1, 8, 1, 1), 0)
    assert out["group_list"].tolist() == [[2, 4], [6, 4]] + [[0, 0]] * 6
    assert out["token_ids"].tolist() == [1, 4, 5, 7, 0, 2, 3, 6]
    assert out["expert_offsets"].tolist() == [0, 1, 2, 3, 0, 1, 2, 3]


def _brute_force(case):
    """Selection by smallest (key, slot), one output row at a time."""
    A, BS, K1 = case["A"], case["BS"], case["K1"]
    L = max(case["layer_num"], 1)
    per = case["expert_num"] // L
    chunk = BS * K1
    Y = A * BS * K1
    cand = []
    for s in range(Y):
        if case["mask"] is not None and case["mask"][s]:
            continue
        lay = int(case["layer_ids"][s // chunk]) if case["layer_ids"] is not None else 0
        e = int(case["expert_ids"][s])
        if 0 <= e < per and 0 <= lay < L:
            cand.append((lay * per + e, s))
    picked = []
    remaining = list(cand)
    while remaining:
        best = remaining[0]
        for c in remaining[1:]:
            if c[0] < best[0] or (c[0] == best[0] and c[1] < best[1]):
                best = c
        picked.append(best)
        remaining.remove(best)
    return picked


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_selection_tiny(seed):
    rng = np.random.default_rng(100 + seed)
    A, BS, K1 = int(rng.integers(1, 4)), int(rng.integers(1, 5)), int(rng.integers(1, 5))
    layer_num = int(rng.integers(0, 4))
    L = max(layer_num, 1)
    expert_num = L * int(rng.integers(1, 6))
    Y = A * BS * K1
    case = synth.batching_case(seed, A, BS, K1, H=3, expert_num=expert_num, layer_num=layer_num,
                               token_dtype=synth.FP16, n_masked=int(rng.integers(0, Y // 2 + 1)),
                               n_bad_ids=int(rng.integers(0, min(3, Y) + 1)),
                               with_id_tables=bool(seed % 2))
    if case["layer_ids"] is not None and seed % 3 == 0:
        case["layer_ids"][0] = L + 2  # an out-of-range layer id: whole chunk invalid
    out = _run(case)
    picked = _brute_force(case)
    assert out["actual_token_num"] == len(picked)
    assert out["token_ids"].tolist() == [s for _, s in picked]
    # group_list: distinct keys in first-appearance order of the selection, with counts
    keys = [k for k, _ in picked]
    uniq = []
    for k in keys:
        if not uniq or uniq[-1][0] != k:
            uniq.append([k, 0])
        uniq[-1][1] += 1
    gl = out["group_list"].tolist()
    assert gl[:len(uniq)] == uniq and all(r == [0, 0] for r in gl[len(uniq):])
    # expert offsets count up from 0 inside each run of equal keys
    exp_off, prev, run = [], None, 0
    for k in keys:
        run = run + 1 if k == prev else 0
        exp_off.append(run)
        prev = k
    assert out["expert_offsets"].tolist() == exp_off
    chunk = BS * K1
    for i, (_, s) in enumerate(picked):
        assert out["y"][i].tobytes() == case["token_bytes"][s, :6].tobytes()
        sess = case["session_ids"][s // chunk] if case["session_ids"] is not None else s // chunk
        mb = case["micro_batch_ids"][s // chunk] if case["micro_batch_ids"] is not None else 0
        assert out["session_ids"][i] == sess and out["micro_batch_ids"][i] == mb


@pytest.mark.parametrize("n", [1, 2])
def test_invariants_named_cases(n):
    case = synth.batching_config(n)
    out = _run(case)
    Y = case["A"] * case["BS"] * case["K1"]
    unmasked = np.nonzero(case["mask"] == 0)[0] if case["mask"] is not None else np.arange(Y)
    act = out["actual_token_num"]
    assert act == unmasked.size
    assert out["group_list"][:, 1].sum() == act
    tok = out["token_ids"]
    # y is a permutation of the unmasked rows, row i = token_data[token_ids[i]]
    assert sorted(tok.tolist()) == unmasked.tolist()
    row = case["H"] * 2
    assert np.array_equal(out["y"], case["token_bytes"][tok, :row])
    # keys (expert ids) non-decreasing, offsets restart per group, stable inside groups
    ex = case["expert_ids"][tok]
    assert (np.diff(ex) >= 0).all()
    starts = np.r_[0, np.nonzero(np.diff(ex))[0] + 1]
    for a, b in zip(starts, np.r_[starts[1:], act]):
        assert out["expert_offsets"][a:b].tolist() == list(range(b - a))
        assert (np.diff(tok[a:b]) > 0).all()


def test_int8_packed_and_separate_scale_agree():
    packed = synth.batching_case(7, A=3, BS=4, K1=3, H=40, expert_num=12, layer_num=3,
                                 token_dtype=synth.INT8, n_masked=5)
    sep = synth.batching_case(7, A=3, BS=4, K1=3, H=40, expert_num=12, layer_num=3,
                              token_dtype=synth.INT8, n_masked=5, separate_scale=True)
    a, b = _run(packed), _run(sep)
    assert np.array_equal(a["y"], b["y"])
    assert np.array_equal(a["dynamic_scale"].view(np.uint32), b["dynamic_scale"].view(np.uint32))
    # the scale travels with its row
    assert np.array_equal(a["dynamic_scale"], sep["token_scale"][a["token_ids"]])

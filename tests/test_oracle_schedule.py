"""Pins for the ScheduleContext front-end oracle (CPU only).

  * the page's usage example, every output in closed form;
  * contexts and data areas serialised through NumPy structured types declared
    member by member like the page's packed structs (NumPy computes the offsets),
    against the flat batching oracle run on the arrays the data area was built
    from, picked out here by (session, micro-batch) without any byte offsets;
  * flags: needSchedule 1 drops exactly the chunks whose flag is not 1,
    needSchedule 0 reads no flag;
  * every status condition on its own, and the exact-size boundary.
"""

import json
import os

import numpy as np
import pytest

import synth
from oracle import ffn_worker_batching
from oracle.schedule import (STATUS_BUFFER, STATUS_POINTER, STATUS_POLLING, STATUS_SHAPE,
                             ffn_worker_batching_from_context)

GOLD = os.path.join(os.path.dirname(__file__), "golden")
INFO_PTR, DATA_PTR = 0x7f00_0000_0000, 0x7f10_0000_0000


def _ctx(area, polling=0, **over):
    A, M, BS, K1 = area["A"], area["M"], area["BS"], area["K1"]
    L = max(area["layer_num"], 1)
    kw = dict(session_num=A, micro_batch_num=M, micro_batch_size=BS, selected_expert_num=K1,
              expert_num=area["expert_num"] // L, token_info_buf=INFO_PTR, token_info_buf_size=area["info"].size,
              token_data_buf=DATA_PTR, token_data_buf_size=area["data"].size, polling_index=polling)
    kw.update(over)
    return synth.schedule_context(**kw)


def _run(area, ctx, need_schedule, layer_num=None):
    a = area
    return ffn_worker_batching_from_context(ctx, a["info"], a["data"].reshape(-1), a["expert_num"],
                                            a["layer_num"] if layer_num is None else layer_num,
                                            (a["A"], a["BS"], a["K1"], a["H"]), a["token_dtype"], need_schedule)


def _flat(area, m, need_schedule):
    """The flat problem of micro-batch m, taken from the generator's per-chunk arrays."""
    A, M, n = area["A"], area["M"], area["BS"] * area["K1"]
    rows = area["data"].reshape(A, M, n, -1)[:, m].reshape(A * n, -1)
    ids = area["expert_ids"].reshape(A, M, n)[:, m].reshape(-1)
    layers = area["layers"].reshape(A, M)[:, m]
    ready = area["flags"].reshape(A, M)[:, m] == 1
    mask = np.repeat(~ready if need_schedule else np.zeros(A, bool), n).astype(np.uint8)
    out = ffn_worker_batching(rows, ids, area["expert_num"], area["layer_num"],
                              (A, area["BS"], area["K1"], area["H"]), area["token_dtype"], mask=mask,
                              layer_ids=np.where(mask.reshape(A, n)[:, 0] == 1, 0, layers).astype(np.int32),
                              micro_batch_ids=np.full(A, m, np.int32))
    return out


def _same(got, ref):
    assert got["actual_token_num"] == ref["actual_token_num"]
    assert got["err_count"] == ref["err_count"]
    assert np.array_equal(got["group_list"], ref["group_list"])
    for k in ("y", "session_ids", "micro_batch_ids", "token_ids", "expert_offsets"):
        assert np.array_equal(got[k], ref[k]), k
    if "dynamic_scale" in ref:
        assert np.array_equal(got["dynamic_scale"].view(np.uint32), ref["dynamic_scale"].view(np.uint32))


def test_api_page_usage_example_through_the_context():
    g = json.load(open(os.path.join(GOLD, "ffn_worker_batching_usage_sample.json")))["inputs"]
    A, M, BS, K1 = g["session_num_A"], g["micro_batch_num_M"], g["micro_batch_size_BS"], g["selected_expert_num_K_plus_1"]
    E, H = g["expert_num"], g["hidden_H"]
    n = BS * K1
    desc = np.zeros(A * M, dtype=synth.ffn_data_desc_dtype(n))
    desc["flag"], desc["layer_id"] = g["chunk_flag"], g["chunk_layer_id"]
    desc["expert_ids"] = np.arange(n) % E
    info = np.frombuffer(desc.tobytes(), np.uint8)
    data = np.full(A * M * n * H, g["token_data_element_int16"], np.int16).view(np.uint8)
    ctx = synth.schedule_context(A, M, BS, K1, E, INFO_PTR, info.size, DATA_PTR, data.size)
    out = ffn_worker_batching_from_context(ctx, info, data, E, g["layer_num"], (A, BS, K1, H), g["token_dtype"],
                                           g["need_schedule"])
    j = np.arange(n)
    assert out["status"] == 0 and out["actual_token_num"] == n and out["err_count"] == 0
    assert out["group_list"].tolist() == [[e, n // E] for e in range(E)]
    assert np.array_equal(out["token_ids"], j // K1 + E * (j % K1))
    assert np.array_equal(out["expert_offsets"], j % K1)
    assert not out["session_ids"].any() and not out["micro_batch_ids"].any()
    assert np.array_equal(out["y"].view(np.int16), np.ones((n, H), np.int16))


CASES = [
    # (dtype, A, M, BS, K1, H, experts, layers, polling, need_schedule, not_ready, bad_ids, bad_layers)
    (synth.FP16, 3, 1, 4, 3, 8, 16, 1, 0, 0, 0, 0, 0),
    (synth.BF16, 4, 3, 2, 5, 6, 12, 3, 2, 1, 4, 3, 0),
    (synth.INT8, 5, 2, 3, 2, 7, 8, 2, 1, 1, 3, 2, 2),
    (synth.FP16, 2, 4, 5, 2, 4, 9, 0, 3, 0, 5, 1, 0),      # layerNum = 0: layer ids not used
    (synth.BF16, 6, 64, 1, 1, 2, 4, 1, 63, 1, 100, 0, 0),  # M = 64, last micro-batch
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_matches_the_flat_oracle(case):
    dt, A, M, BS, K1, H, E, Ln, pol, ns, nr, nb, bl = case
    area = synth.schedule_area(40 + A * M, A, M, BS, K1, H, E, Ln, dt, n_not_ready=nr, n_bad_ids=nb,
                               bad_layers=bl)
    got = _run(area, _ctx(area, pol), ns)
    assert got["status"] == 0
    _same(got, _flat(area, pol, ns))


def test_every_micro_batch_is_reachable():
    area = synth.schedule_area(7, 3, 5, 2, 3, 4, 6, 1, synth.FP16)
    rows = area["data"].reshape(3, 5, 6, -1)
    for m in range(5):
        out = _run(area, _ctx(area, m), 0)
        assert out["actual_token_num"] == 18 and (out["micro_batch_ids"] == m).all()
        for i, t in enumerate(out["token_ids"]):
            s, j = divmod(int(t), 6)
            assert np.array_equal(out["y"][i], rows[s, m, j])


def test_flags_decide_only_under_need_schedule():
    area = synth.schedule_area(8, 4, 2, 3, 3, 4, 8, 1, synth.BF16, n_not_ready=5)
    for m in range(2):
        ready = area["flags"].reshape(4, 2)[:, m] == 1
        on = _run(area, _ctx(area, m), 1)
        off = _run(area, _ctx(area, m), 0)
        assert on["actual_token_num"] == 9 * int(ready.sum())
        assert set((on["token_ids"] // 9).tolist()) == set(np.nonzero(ready)[0].tolist())
        assert off["actual_token_num"] == 36
        # with every flag set, the scan changes nothing
    full = dict(area, flags=np.ones_like(area["flags"]))
    desc = np.frombuffer(area["info"].tobytes(), dtype=synth.ffn_data_desc_dtype(9)).copy()
    desc["flag"] = 1
    full["info"] = np.frombuffer(desc.tobytes(), np.uint8)
    _same(_run(full, _ctx(full, 1), 1), _run(area, _ctx(area, 1), 0))


def _status_case():
    return synth.schedule_area(9, 2, 3, 2, 2, 8, 8, 2, synth.INT8)


@pytest.mark.parametrize("over,bit", [
    (dict(session_num=3), STATUS_SHAPE),
    (dict(micro_batch_size=1), STATUS_SHAPE),
    (dict(selected_expert_num=3), STATUS_SHAPE),
    (dict(expert_num=8), STATUS_SHAPE),            # per layer: 8 // 2 = 4 expected
    (dict(micro_batch_num=0), STATUS_POLLING),
    (dict(micro_batch_num=65), STATUS_POLLING | STATUS_BUFFER),   # 65 micro-batches would not fit either
    (dict(polling_index=3), STATUS_POLLING),
    (dict(token_info_buf=0), STATUS_POINTER),
    (dict(token_data_buf=0), STATUS_POINTER),
    (dict(token_info_buf=INFO_PTR + 2), STATUS_POINTER),
    (dict(token_data_buf=DATA_PTR + 8), STATUS_POINTER),
    (dict(token_info_buf_size=2 * 3 * (8 + 4 * 4) - 1), STATUS_BUFFER),
    (dict(token_data_buf_size=2 * 3 * 4 * (8 + 4) - 1), STATUS_BUFFER),
])
def test_status_conditions(over, bit):
    area = _status_case()
    kw = {k: v for k, v in over.items() if k != "polling_index"}
    out = _run(area, _ctx(area, over.get("polling_index", 1), **kw), 1)
    assert out["status"] == bit
    assert out["actual_token_num"] == 0 and not out["group_list"].any() and out["err_count"] == 0


def test_exact_buffer_sizes_are_enough():
    area = _status_case()
    assert area["info"].size == 2 * 3 * (8 + 4 * 4) and area["data"].size == 2 * 3 * 4 * (8 + 4)
    out = _run(area, _ctx(area, 2), 0)
    assert out["status"] == 0 and out["actual_token_num"] + out["err_count"] == 8

"""GPU parity of ffnwb_batching_ctx (batching fed by a ScheduleContext) against the
oracle: the context check word, and every output bit-exact (rows past
actual_token_num stay unwritten)."""

import json
import os

import numpy as np
import pytest
import torch

import synth
from _gpu import check_ctx, dev, fetch_batching, prepare_ctx, prepare_batching

pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _run(area, polling, need_schedule, ctx_over=None, ptr_shift=None):
    call = prepare_ctx(area, polling, need_schedule, ctx_over, ptr_shift=ptr_shift)
    call.run()
    torch.cuda.synchronize()
    return call


def test_api_page_usage_example():
    g = json.load(open(os.path.join(GOLD, "ffn_worker_batching_usage_sample.json")))["inputs"]
    A, M, BS, K1 = g["session_num_A"], g["micro_batch_num_M"], g["micro_batch_size_BS"], g["selected_expert_num_K_plus_1"]
    E, H, n = g["expert_num"], g["hidden_H"], g["micro_batch_size_BS"] * g["selected_expert_num_K_plus_1"]
    desc = np.zeros(A * M, dtype=synth.ffn_data_desc_dtype(n))
    desc["flag"], desc["layer_id"], desc["expert_ids"] = g["chunk_flag"], g["chunk_layer_id"], np.arange(n) % E
    area = dict(info=np.frombuffer(desc.tobytes(), np.uint8).copy(),
                data=np.full((A * M * n, H), g["token_data_element_int16"], np.int16).view(np.uint8),
                flags=desc["flag"], layers=desc["layer_id"], expert_ids=desc["expert_ids"], row=2 * H,
                A=A, M=M, BS=BS, K1=K1, H=H, expert_num=E, layer_num=g["layer_num"], token_dtype=g["token_dtype"])
    print("context: the API page's usage example", flush=True)
    call = _run(area, 0, g["need_schedule"])
    check_ctx(area, call)
    got = fetch_batching(call)
    j = np.arange(n)
    assert np.array_equal(got["token_ids"], j // K1 + E * (j % K1))
    assert np.array_equal(got["group_list"], np.array([[e, n // E] for e in range(E)]))


CASES = [
    # (dtype, A, M, BS, K1, H, experts, layers, polling, need_schedule, not_ready, bad_ids, bad_layers)
    (synth.FP16, 3, 1, 4, 3, 8, 16, 1, 0, 0, 0, 0, 0),
    (synth.BF16, 4, 3, 2, 5, 6, 12, 3, 2, 1, 4, 3, 0),          # odd rows: 4-byte copies
    (synth.INT8, 5, 2, 3, 2, 7, 8, 2, 1, 1, 3, 2, 2),           # 1-byte copies, packed scales
    (synth.FP16, 2, 4, 5, 2, 4, 9, 0, 3, 0, 5, 1, 0),           # layerNum = 0
    (synth.BF16, 6, 64, 1, 1, 2, 4, 1, 63, 1, 100, 0, 0),       # M = 64, last micro-batch
    (synth.BF16, 16, 2, 32, 9, 256, 256, 1, 1, 1, 3, 10, 0),    # Y = 4608: one-launch slot order
    (synth.INT8, 64, 2, 16, 9, 64, 1024, 16, 0, 1, 20, 50, 3),  # Y = 9216: rank / scan / gather path
    (synth.FP16, 1024, 1, 1, 1, 8, 8192, 1, 0, 1, 200, 0, 0),   # A = 1024, 8192 experts
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_matches_the_oracle(case):
    dt, A, M, BS, K1, H, E, Ln, pol, ns, nr, nb, bl = case
    area = synth.schedule_area(60 + A * M, A, M, BS, K1, H, E, Ln, dt, n_not_ready=nr, n_bad_ids=nb,
                               bad_layers=bl)
    print(f"context case {case}", flush=True)
    check_ctx(area, _run(area, pol, ns))


def test_same_rows_as_the_flat_entry_point():
    # the context path must equal ffnwb_batching on the same slots laid out flat
    area = synth.schedule_area(71, 16, 3, 32, 9, 512, 256, 1, synth.BF16, n_not_ready=4, n_bad_ids=7)
    m = 2
    print("context vs flat entry point", flush=True)
    call = _run(area, m, 1)
    A, n = 16, 32 * 9
    ready = area["flags"].reshape(A, 3)[:, m] == 1
    flat = dict(token_bytes=area["data"].reshape(A, 3, n, -1)[:, m].reshape(A * n, -1).copy(),
                token_scale=None, expert_ids=area["expert_ids"].reshape(A, 3, n)[:, m].reshape(-1).copy(),
                mask=np.repeat(~ready, n).astype(np.uint8), layer_ids=None, session_ids=None,
                micro_batch_ids=np.full(A, m, np.int32), A=A, BS=32, K1=9, H=512, expert_num=256, layer_num=1,
                token_dtype=synth.BF16, stride=1024)
    fcall = prepare_batching(flat)
    fcall.run()
    torch.cuda.synchronize()
    a, b = fetch_batching(call), fetch_batching(fcall)
    for k in b:
        assert np.array_equal(a[k], b[k]), k


def _status_area():
    return synth.schedule_area(9, 2, 3, 2, 2, 8, 8, 2, synth.INT8)


@pytest.mark.parametrize("over,pol", [
    (dict(session_num=3), 1), (dict(micro_batch_size=1), 1), (dict(selected_expert_num=3), 1),
    (dict(expert_num=8), 1), (dict(micro_batch_num=0), 1), (dict(micro_batch_num=65), 1), ({}, 3),
    (dict(token_info_buf=0), 1), (dict(token_data_buf=0), 1), ("info+2", 1), ("data+8", 1),
    (dict(token_info_buf_size=2 * 3 * (8 + 4 * 4) - 1), 1), (dict(token_data_buf_size=2 * 3 * 4 * (8 + 4) - 1), 1),
])
def test_rejected_contexts_read_nothing(over, pol):
    # every check runs on the device; a failed one leaves the data area unread
    area = _status_area()
    shift = None
    if isinstance(over, str):
        # a misaligned pointer into the uploaded buffer (the decode rejects it unread)
        key = "token_info_buf" if over.startswith("info") else "token_data_buf"
        shift, over = {key: int(over.split("+")[1])}, {}
    print(f"context rejected: {over} {shift} polling {pol}", flush=True)
    call = _run(area, pol, 1, over, shift)
    ref = check_ctx(area, call)
    assert ref["status"] != 0 and ref["actual_token_num"] == 0


def test_exact_sizes_and_repeated_calls():
    area = synth.schedule_area(10, 8, 4, 16, 9, 128, 64, 2, synth.FP16, n_not_ready=6, n_bad_ids=5)
    print("context: consecutive calls at every polling index", flush=True)
    for m in (3, 0, 2, 1):
        for ns in (1, 0):
            check_ctx(area, _run(area, m, ns))


def test_named_workload_shape_with_four_micro_batches():
    # the BF16 batching workload's slots and rows (A=16, BS=32, K+1=9, H=7168, 256 experts)
    # as micro-batch 3 of 4, with three sessions not ready
    area = synth.schedule_area(12, 16, 4, 32, 9, 7168, 256, 1, synth.BF16, n_not_ready=12)
    print("context: A=16 M=4 BS=32 K+1=9 H=7168 bf16", flush=True)
    check_ctx(area, _run(area, 3, 1))


def test_flags_set_during_the_decode_give_whole_chunks():
    # A producer on a second stream rewrites every chunk's flag (a bounded run of copies of
    # random 0/1 patterns) while batching calls run on the current stream, with no
    # synchronisation between the two streams.  Whatever each call saw, every chunk must
    # come out batched whole (all its slots, keyed with its own layer) or not at all.
    A, BS, K1, H, E, Ln = 64, 16, 9, 8, 64, 4
    n, El = BS * K1, E // Ln
    area = synth.schedule_area(81, A, 1, BS, K1, H, E, Ln, synth.FP16)
    words = area["info"].view(np.int32).reshape(A, 2 + n)
    words[:, 1] = 1 + np.arange(A) % (Ln - 1)   # every chunk on a layer other than 0
    info, data = dev(area["info"]), dev(area["data"].reshape(-1))
    flags = info.view(torch.int32)[0::2 + n]
    g = torch.Generator().manual_seed(5)
    patterns = dev(torch.randint(0, 2, (64, A), generator=g, dtype=torch.int32).numpy())
    calls = [prepare_ctx(area, 0, 1, bufs=(info, data)) for _ in range(48)]
    prod = torch.cuda.Stream()
    torch.cuda.synchronize()
    print("context: flags rewritten on a second stream during 48 calls", flush=True)
    torch.cuda._sleep(50_000_000)          # both streams start together once this ends (bounded spin)
    prod.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(prod):
        for i in range(600):
            flags.copy_(patterns[i % 64])
    for c in calls:
        c.run()
    torch.cuda.synchronize()
    ids = area["expert_ids"].reshape(A, n)
    layer = words[:, 1]
    seen = set()
    for ci, c in enumerate(calls):
        got = fetch_batching(c)
        act = int(got["actual_token_num"][0])
        tok = got["token_ids"][:act].astype(np.int64)
        chunk = tok // n
        counts = np.bincount(chunk, minlength=A)
        assert set(np.unique(counts)) <= {0, n}, f"call {ci}: a chunk was batched in part"
        seen.add(tuple(counts // n))
        # the key of every output row, from group_list, against its chunk's layer and id
        gl = got["group_list"]
        key = np.repeat(gl[:, 0], gl[:, 1])[:act]
        assert np.array_equal(key, layer[chunk] * El + ids[chunk, tok % n]), f"call {ci}: wrong keys"
        assert np.array_equal(got["y"][:act], area["data"][tok]), f"call {ci}: wrong rows"
        assert int(got["ctx_status"][0]) == 0 and int(got["err_count"][0]) == 0
    print(f"distinct ready patterns seen: {len(seen)}", flush=True)

"""GPU parity of ffnwb_batching against the oracle (bit-exact for every output)."""

import numpy as np
import pytest

import synth
from _gpu import check_batching, prepare_batching, fetch_batching, run_batching, oracle_batching

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [1, 2, 3])
def test_named_cases_full_size(n):
    case = synth.batching_config(n)
    print(f"batching case {n}", flush=True)
    check_batching(case, run_batching(case))


RANDOM = [
    # (A, BS, K1, H, experts, layers, dtype, masked, bad, tables, stride_pad, separate_scale)
    (1, 1, 1, 1, 1, 1, synth.FP16, 0, 0, False, 0, False),          # a single slot
    (1, 4, 2, 3, 5, 0, synth.BF16, 8, 0, False, 0, False),          # everything masked, odd H
    (3, 5, 7, 64, 12, 3, synth.FP16, 20, 6, True, 0, False),        # small fused path
    (2, 40, 9, 136, 64, 4, synth.BF16, 100, 9, True, 32, False),   # general path, padded stride
    (8, 16, 9, 100, 256, 1, synth.FP16, 30, 0, False, 6, False),   # 4-byte rows (VEC4), ragged tail
    (5, 33, 3, 37, 40, 2, synth.BF16, 0, 3, False, 2, False),      # byte-path rows
    (16, 16, 9, 512, 1024, 16, synth.INT8, 400, 17, True, 0, False),   # INT8 packed scale
    (16, 16, 9, 520, 64, 1, synth.INT8, 100, 0, False, 8, True),       # INT8 separate scale
    (6, 8, 8, 256, 8192, 8, synth.BF16, 10, 0, False, 0, False),       # max experts
    (2, 100, 64, 16, 5000, 1, synth.FP16, 999, 30, False, 0, False),   # K+1 = 64, 5000 keys
    (1024, 2, 1, 8, 16, 1, synth.FP16, 0, 0, True, 0, False),          # A = 1024 chunks
    (64, 512, 9, 16, 256, 2, synth.FP16, 1000, 10, True, 0, False),    # Y = 294912: multi-launch sort
    (16, 64, 8, 32, 2048, 4, synth.BF16, 700, 11, True, 0, False),     # Y = 8192, 2048 keys: one-workgroup order at its limits
    (16, 32, 9, 64, 4096, 2, synth.FP16, 300, 5, True, 0, False),      # 4096 keys: range-partitioned order
    (16, 128, 8, 64, 8192, 8, synth.BF16, 900, 7, True, 0, False),     # Y = 16384, 8192 keys: placement by 4096-slot tiles
    (64, 128, 8, 16, 1024, 16, synth.INT8, 3000, 9, True, 0, False),   # Y = 65536: placement at its 64-tile limit
    (65, 128, 8, 16, 512, 2, synth.FP16, 2000, 4, False, 0, False),    # Y = 66560: 65 tiles, rank / scan / gather
]


@pytest.mark.parametrize("params", RANDOM, ids=[str(i) for i in range(len(RANDOM))])
def test_random_shapes(params):
    A, BS, K1, H, E, L, dt, masked, bad, tables, pad, sep = params
    Y = A * BS * K1
    case = synth.batching_case(1000 + A * 7 + H, A, BS, K1, H, E, L, dt, n_masked=min(masked, Y),
                               n_bad_ids=min(bad, Y - min(masked, Y)), with_id_tables=tables,
                               stride_pad=pad, separate_scale=sep)
    print(f"batching random {params}", flush=True)
    check_batching(case, run_batching(case))


def test_zipf_skew_and_layer_gaps():
    case = synth.batching_case(77, 32, 32, 9, 128, 512, 8, synth.BF16, n_masked=500,
                               expert_dist="zipf", zipf_s=1.6, layer_of_chunk="mod")
    check_batching(case, run_batching(case))


@pytest.mark.parametrize("A", [8, 32])
def test_one_expert_takes_every_slot(A):
    # one key holds nearly every slot (A = 8: one-launch order, A = 32: multi-launch sort)
    case = synth.batching_case(78, A, 64, 9, 256, 64, 1, synth.BF16, n_masked=100)
    case["expert_ids"][:] = 9
    case["expert_ids"][::97] = 3
    check_batching(case, run_batching(case))


def test_deterministic_and_reusable_call():
    case = synth.batching_config(2)
    call = prepare_batching(case)
    call.run()
    import torch
    torch.cuda.synchronize()
    a = fetch_batching(call)
    call.run()   # same workspace and outputs again
    torch.cuda.synchronize()
    b = fetch_batching(call)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    check_batching(case, b)


def test_usage_sample_of_the_api_page():
    A, BS, K1, H, E = 1, 8, 9, 4096, 8
    case = synth.batching_case(0, A, BS, K1, H, E, 1, synth.FP16, expert_dist="modulo")
    case["token_bytes"][:] = np.frombuffer(np.int16(1).tobytes() * (BS * K1 * H), np.uint8).reshape(72, -1)
    case["layer_ids"] = np.zeros(A, np.int32)
    got = run_batching(case)
    ref = check_batching(case, got)
    assert ref["actual_token_num"] == 72
    j = np.arange(72)
    assert got["token_ids"][:72].tolist() == ((j // 9) + 8 * (j % 9)).tolist()

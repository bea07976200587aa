"""GPU parity of moe_unpermute against the oracle: the acceptance tolerance and, since
the kernels use the oracle's FP32 operation order without fused multiply-adds, identical
bits; index and prob outputs are bit-exact."""

import numpy as np
import pytest
import torch

import synth
from _gpu import check_unpermute, prepare_unpermute, fetch_unpermute, run_unpermute, oracle_unpermute

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [4, 5])
def test_named_cases_full_size(n):
    case = synth.unpermute_config(n)
    print(f"unpermute case {n}", flush=True)
    check_unpermute(case, run_unpermute(case))


NONPAD = [
    # (T, K, E, H, dtype, probs dtype, n_empty, with_probs, rows_mode)
    (1, 1, 1, 8, synth.FP32, synth.FP32, 0, True, "compact"),
    (7, 3, 5, 24, synth.FP16, synth.FP16, 4, True, "slots"),
    (64, 8, 16, 4096, synth.BF16, synth.FP32, 50, True, "compact"),
    (40, 4, 9, 136, synth.BF16, synth.BF16, 0, True, "slots"),
    (33, 5, 12, 19, synth.FP16, synth.FP16, 30, True, "compact"),     # odd H: element path
    (50, 6, 1, 64, synth.FP32, None, 60, False, "slots"),              # branch 4, no probs
    (3000, 8, 64, 32, synth.BF16, synth.FP32, 2000, True, "compact"),  # aux order needs 2 LSD passes
    (40000, 8, 64, 16, synth.BF16, synth.FP32, 30000, True, "compact"),  # 320000 slots
    (20000, 4, 129, 16, synth.BF16, synth.FP32, 5000, True, "compact"),  # 79 tiles x 17 column ranges
    (300, 4, 1100, 16, synth.BF16, synth.FP32, 100, True, "compact"),    # E > 1024: three-launch compaction
    (70000, 2, 64, 8, synth.FP16, synth.FP16, 20000, True, "slots"),     # 274 tiles x 64 > 16384 words: the same
    (2, 512, 600, 16, synth.FP16, synth.FP16, 100, True, "slots"),    # topK = 512
    (1000, 2, 300, 264, synth.FP32, synth.FP32, 0, True, "compact"),
]


@pytest.mark.parametrize("params", NONPAD, ids=[str(i) for i in range(len(NONPAD))])
def test_nonpadded_random(params):
    T, K, E, H, dt, pdt, empty, wp, mode = params
    case = synth.unpermute_nonpadded_case(500 + T + K, T=T, K=K, E=E, H=H, dtype=dt, probs_dtype=pdt,
                                          n_empty=empty, with_probs=wp, rows_mode=mode)
    print(f"unpermute nonpadded {params}", flush=True)
    check_unpermute(case, run_unpermute(case))


PAD = [
    # (E, C, T, H, dtype, probs dtype, topk, with_probs, n_invalid)
    (1, 1, 1, 8, synth.FP32, synth.FP32, 1, True, 0),
    (2, 1, 2, 2, synth.FP32, synth.FP32, 2, True, 0),
    (8, 40, 100, 264, synth.FP16, synth.FP16, 3, True, 5),
    (16, 64, 50, 128, synth.BF16, synth.FP32, 2, True, 0),     # capacity > tokens (with replacement)
    (4, 33, 200, 21, synth.BF16, synth.BF16, 1, True, 7),     # odd H
    (6, 10, 30, 64, synth.FP16, None, 0, False, 3),           # branch 3, no probs
    (4, 8, 25000, 32, synth.FP32, synth.FP32, 2, True, 2),    # 25001 keys, 32 entries
    (64, 4500, 20000, 8, synth.FP16, synth.FP16, 4, True, 10),  # 288000 entries: multi-launch sort, one pass
    (64, 4500, 30000, 8, synth.FP32, synth.FP32, 4, True, 10),  # 288000 entries, 30001 keys: LSD passes
]


@pytest.mark.parametrize("params", PAD, ids=[str(i) for i in range(len(PAD))])
def test_padded_random(params):
    E, C, T, H, dt, pdt, topk, wp, inv = params
    case = synth.unpermute_padded_case(900 + E + C, E=E, C=C, T=T, H=H, dtype=dt, probs_dtype=pdt, topk=topk,
                                       with_probs=wp, n_invalid=inv)
    print(f"unpermute padded {params}", flush=True)
    check_unpermute(case, run_unpermute(case))


def test_padded_skewed_tokens():
    # two tokens hold every capacity entry: one ordering workgroup owns them all and its
    # waves read their slices again instead of keeping per-wave lists
    case = synth.unpermute_padded_case(36, E=16, C=2048, T=4096, H=64, dtype=synth.BF16, probs_dtype=synth.FP32)
    rng = np.random.default_rng(36)
    case["sorted_indices"] = rng.choice(np.array([5, 6], np.int32), size=case["sorted_indices"].shape[0])
    case["sorted_indices"][:7] = -1
    print("unpermute padded skewed", flush=True)
    check_unpermute(case, run_unpermute(case))


def test_article_padded_example():
    case = dict(permuted=np.ones((2, 2), np.float32), dtype=synth.FP32,
                sorted_indices=np.array([1, 1], np.int32), routing_map=np.ones((2, 2), np.int8),
                probs=np.ones((2, 2), np.float32), probs_dtype=synth.FP32, padded_mode=True,
                restore_shape=(2, 2))
    got = run_unpermute(case)
    check_unpermute(case, got)
    assert got["unpermuted"].tolist() == [[0.0, 0.0], [2.0, 2.0]]


def test_weight_index_slot_reading():
    case = synth.unpermute_nonpadded_case(31, T=200, K=4, E=32, H=256, dtype=synth.BF16,
                                          probs_dtype=synth.FP32, n_empty=90)
    check_unpermute(case, run_unpermute(case, weight_index=1), oracle_unpermute(case, 1), weight_index=1)


def test_aux_outputs_skipped():
    case = synth.unpermute_nonpadded_case(32, T=128, K=8, E=64, H=512, dtype=synth.FP16,
                                          probs_dtype=synth.FP16, n_empty=100)
    check_unpermute(case, run_unpermute(case, aux=False), aux=False)
    pcase = synth.unpermute_padded_case(33, E=8, C=64, T=300, H=256, dtype=synth.FP16, probs_dtype=synth.FP16)
    check_unpermute(pcase, run_unpermute(pcase, aux=False), aux=False)


def test_empty_inputs():
    # no slots at all for some tokens, and no entries at all
    case = synth.unpermute_nonpadded_case(34, T=16, K=2, E=4, H=64, dtype=synth.FP16, probs_dtype=synth.FP16,
                                          n_empty=32)
    check_unpermute(case, run_unpermute(case))
    empty = dict(permuted=np.zeros((0, 64), np.float16), dtype=synth.FP16, sorted_indices=np.zeros(0, np.int32),
                 routing_map=None, probs=None, probs_dtype=None, padded_mode=True, restore_shape=(5, 64))
    got = run_unpermute(empty)
    assert (got["unpermuted"].view(np.uint16) == 0).all()
    nz = dict(empty, padded_mode=False, restore_shape=(0, 64))
    run_unpermute(nz)


def test_deterministic_repeat():
    case = synth.unpermute_padded_case(35, E=16, C=128, T=1000, H=512, dtype=synth.BF16, probs_dtype=synth.FP32)
    call = prepare_unpermute(case)
    call.run()
    torch.cuda.synchronize()
    a = fetch_unpermute(call, case)
    call.run()
    torch.cuda.synchronize()
    b = fetch_unpermute(call, case)
    for k in a:
        assert np.array_equal(np.asarray(a[k]).view(np.uint8), np.asarray(b[k]).view(np.uint8)), k
    check_unpermute(case, b)


def test_nondefault_streams_and_back_to_back_calls():
    # the auxiliary order runs on a library side stream joined back to the caller's stream;
    # check results on two user streams with calls in flight together
    cases = [synth.unpermute_nonpadded_case(40 + i, T=500, K=4, E=32, H=256, dtype=synth.BF16,
                                            probs_dtype=synth.FP32, n_empty=150) for i in range(2)]
    refs = [oracle_unpermute(c) for c in cases]
    calls = [prepare_unpermute(c) for c in cases]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for _ in range(3):
        for call, st in zip(calls, streams):
            with torch.cuda.stream(st):
                call.run(st)
    torch.cuda.synchronize()
    for c, call, ref in zip(cases, calls, refs):
        check_unpermute(c, fetch_unpermute(call, c), ref)


# ----------------------------------------------------------------------------- zero-weight skip

SKIP = [
    ("padded", dict(E=16, C=64, T=1000, H=512, dtype=synth.FP16, probs_dtype=synth.FP16)),
    ("padded", dict(E=8, C=40, T=300, H=24, dtype=synth.BF16, probs_dtype=synth.FP32)),
    ("padded", dict(E=4, C=33, T=200, H=21, dtype=synth.FP32, probs_dtype=synth.FP32)),   # element path
    ("nonpadded", dict(T=400, K=4, E=32, H=256, dtype=synth.BF16, probs_dtype=synth.FP32, n_empty=300,
                       rows_mode="slots")),                                             # rows past nnz weigh 0
]


def _skip_case(kind, kw, seed):
    if kind == "padded":
        return synth.unpermute_padded_case(seed, **kw)
    return synth.unpermute_nonpadded_case(seed, **kw)


@pytest.mark.parametrize("poison", [False, True])
@pytest.mark.parametrize("params", SKIP, ids=[str(i) for i in range(len(SKIP))])
def test_zero_weight_skip(params, poison):
    kind, kw = params
    case = _skip_case(kind, kw, 61 + len(kw))
    # zero a third of the probs (half of those as -0.0) so that routed entries weigh 0
    rng = np.random.default_rng(62)
    pr = case["probs"].copy()
    bits = pr.view(np.uint32 if pr.itemsize == 4 else np.uint16)
    pick = rng.random(pr.shape) < 1 / 3
    neg = rng.random(pr.shape) < 0.5
    bits[pick] = 0
    bits[pick & neg] = 0x80000000 if pr.itemsize == 4 else 0x8000
    case = dict(case, probs=pr)
    if poison:
        # NaN in every permuted row whose weight is 0: the skip must keep them out
        ref0 = oracle_unpermute(case)
        from oracle import numerics as nm
        w = nm.to_f32(ref0["permute_probs"], case["probs_dtype"])
        zero_rows = np.nonzero(w == 0)[0] if kind == "padded" else \
            np.array([r for r in range(len(w)) if w[r] == 0], np.int64)
        nan_bits = {synth.FP16: np.float16("nan"), synth.FP32: np.float32("nan")}
        x = case["permuted"].copy()
        if case["dtype"] == synth.BF16:
            x[zero_rows] = np.uint16(0x7fc0)
        else:
            x[zero_rows] = nan_bits[case["dtype"]]
        case = dict(case, permuted=x)
    print(f"unpermute skip {kind} {kw} poison={poison}", flush=True)
    ref = oracle_unpermute(case, skip_zero_weight=True)
    got = run_unpermute(case, skip_zero_weight=True)
    check_unpermute(case, got, ref)


def test_zero_weight_skip_full_size_padded():
    case = synth.unpermute_config(5)
    print("unpermute padded workload with the zero-weight skip", flush=True)
    check_unpermute(case, run_unpermute(case, skip_zero_weight=True), oracle_unpermute(case, skip_zero_weight=True))

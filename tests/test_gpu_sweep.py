"""A seeded sweep of random shapes for batching, unpermute and permute, each checked
against the oracle.

The hand-picked GPU cases cover every path and limit one at a time. This sweep draws
combinations of them from fixed seeds (element types, odd and large rows, key counts,
layers, masks, bad ids, strided rows, probs types, empty slots, invalid capacity
entries, skewed routing), so the same shapes run every time.  The non-padded unpermute
cases also make several slots read the same row: equal keys for the stable auxiliary
order, which the generators alone never produce.
"""

import numpy as np
import pytest

import synth
from _gpu import check_batching, check_permute, check_unpermute, run_batching, run_permute, run_unpermute

pytestmark = pytest.mark.gpu

_DT = (synth.FP16, synth.BF16, synth.INT8)
# unpermute (token, probs) element types: equal, or BF16 tokens with FP32 probs
_PAIRS = ((synth.FP16, synth.FP16), (synth.BF16, synth.BF16), (synth.BF16, synth.FP32), (synth.FP32, synth.FP32))


def _batching_cases(n):
    rng = np.random.default_rng(20241)
    out = []
    while len(out) < n:
        A = int(rng.choice([1, 2, 3, 16, 64, 200]))
        BS = int(rng.integers(1, 33))
        K1 = int(rng.choice([1, 2, 3, 9, 17, 64]))
        Y = A * BS * K1
        if Y > 40000:
            continue
        H = int(rng.choice([1, 3, 8, 64, 100, 257, 1024]))
        dt = int(rng.choice(_DT))
        L = int(rng.choice([0, 1, 2, 4, 16]))
        per = int(rng.choice([1, 3, 8, 64, 300]))
        expert_num = per * max(L, 1)
        if expert_num > 8192:
            continue
        out.append(dict(seed=int(rng.integers(1 << 30)), A=A, BS=BS, K1=K1, H=H, expert_num=expert_num,
                        layer_num=L, token_dtype=dt, n_masked=int(rng.integers(0, Y + 1)),
                        expert_dist=str(rng.choice(["uniform", "zipf", "modulo"])),
                        n_bad_ids=int(min(Y, rng.integers(0, 6))), with_id_tables=bool(rng.random() < 0.5),
                        stride_pad=int(rng.choice([0, 0, 4, 12])),
                        separate_scale=bool(dt == synth.INT8 and rng.random() < 0.5)))
    return out


@pytest.mark.parametrize("params", _batching_cases(12), ids=[str(i) for i in range(12)])
def test_batching_sweep(params):
    p = dict(params)
    seed = p.pop("seed")
    case = synth.batching_case(seed, **p)
    print(f"batching sweep {params}", flush=True)
    check_batching(case, run_batching(case))


def _nonpadded_cases(n):
    rng = np.random.default_rng(20242)
    out = []
    for _ in range(n):
        T = int(rng.choice([1, 5, 64, 300, 1000, 3000]))
        E = int(rng.choice([1, 4, 9, 32, 128, 300]))
        K = int(rng.integers(1, min(E, 16) + 1))
        dt, pdt = _PAIRS[int(rng.integers(len(_PAIRS)))]
        out.append(dict(seed=int(rng.integers(1 << 30)), T=T, K=K, E=E, H=int(rng.choice([4, 19, 64, 136, 300])),
                        dtype=dt, probs_dtype=pdt,
                        n_empty=int(rng.integers(0, T * K + 1)), with_probs=bool(rng.random() < 0.8),
                        rows_mode=str(rng.choice(["compact", "slots"])), n_dup=int(rng.integers(0, 8))))
    return out


@pytest.mark.parametrize("params", _nonpadded_cases(10), ids=[str(i) for i in range(10)])
def test_unpermute_nonpadded_sweep(params):
    p = dict(params)
    seed, n_dup = p.pop("seed"), p.pop("n_dup")
    case = synth.unpermute_nonpadded_case(seed, **p)
    sI = case["sorted_indices"]
    valid = np.nonzero(sI >= 0)[0]
    if n_dup and valid.size >= 2:
        # several slots read the same row (equal keys in the auxiliary order)
        rng = np.random.default_rng(seed)
        src = rng.choice(valid, size=n_dup)
        dst = rng.choice(valid, size=n_dup)
        sI[dst] = sI[src]
    print(f"unpermute non-padded sweep {params}", flush=True)
    check_unpermute(case, run_unpermute(case))


def _padded_cases(n):
    rng = np.random.default_rng(20243)
    out = []
    for _ in range(n):
        E = int(rng.choice([1, 2, 8, 64]))
        dt, pdt = _PAIRS[int(rng.integers(len(_PAIRS)))]
        out.append(dict(seed=int(rng.integers(1 << 30)), E=E, C=int(rng.choice([1, 7, 64, 300])),
                        T=int(rng.choice([1, 10, 200, 3000])), H=int(rng.choice([4, 21, 64, 520])),
                        dtype=dt, probs_dtype=pdt,
                        topk=int(rng.integers(1, E + 1)), with_probs=bool(rng.random() < 0.8),
                        n_invalid=int(rng.integers(0, 20))))
    return out


@pytest.mark.parametrize("params", _padded_cases(8), ids=[str(i) for i in range(8)])
def test_unpermute_padded_sweep(params):
    p = dict(params)
    seed = p.pop("seed")
    p["n_invalid"] = min(p["n_invalid"], p["E"] * p["C"])
    case = synth.unpermute_padded_case(seed, **p)
    print(f"unpermute padded sweep {params}", flush=True)
    check_unpermute(case, run_unpermute(case))


def _permute_cases(n):
    rng = np.random.default_rng(20244)
    out = []
    for _ in range(n):
        E = int(rng.choice([1, 4, 9, 32, 128, 256]))
        T = int(rng.choice([1, 7, 256, 513, 2000]))
        padded = bool(rng.random() < 0.4)
        out.append(dict(seed=int(rng.integers(1 << 30)), T=T, K=int(rng.integers(1, min(E, 8) + 1)), E=E,
                        H=int(rng.choice([1, 13, 64, 130])), dtype=int(rng.choice(_DT + (synth.FP32,))),
                        padded=padded, C=int(rng.choice([1, 5, 100])) if padded else None,
                        route=str(rng.choice(["uniform", "skew"])), row_pad=int(rng.choice([0, 0, 3]))))
    return out


@pytest.mark.parametrize("params", _permute_cases(8), ids=[str(i) for i in range(8)])
def test_permute_sweep(params):
    p = dict(params)
    seed = p.pop("seed")
    case = synth.permute_case(seed, **p)
    print(f"permute sweep {params}", flush=True)
    check_permute(case, run_permute(case))

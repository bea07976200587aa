"""Pins for the unpermute oracle (CPU only).

  * the article's padded {2,2} example (formula result);
  * closed forms: permute-then-unpermute without probs gives n_t * x[t] (exactly
    x[t] for topK = 1); a padded unpermute with sortedIndices a permutation of
    the tokens gives the inverse permutation exactly; a consistent permute with
    softmax probs recombines to x[t] (this pins the W2 weight index and the
    expert-major masked_select order, in both modes);
  * brute force: torch index_add_ in float64 (a library scatter-add), with the
    oracle inside the FP32 accumulation error bound plus one output rounding;
  * properties of out_index / permute_token_id / permute_probs.
"""

import json
import os

import numpy as np
import pytest
import torch

import synth
from oracle import moe_token_unpermute_with_routing_map as unpermute
from oracle import numerics as nm

GOLD = os.path.join(os.path.dirname(__file__), "golden")
TDT = {nm.DT_FP16: torch.float16, nm.DT_BF16: torch.bfloat16, nm.DT_FP32: torch.float32}


def _torch_f32(a, dt):
    if dt == nm.DT_BF16:
        return torch.from_numpy(np.asarray(a).view(np.int16).copy()).view(torch.bfloat16).float()
    return torch.from_numpy(np.asarray(a).copy()).float()


def _torch_round(x64, dt):
    """float64 tensor -> stored numpy array of type dt via torch's conversions."""
    t = x64.to(torch.float32).to(TDT[dt])
    if dt == nm.DT_BF16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _run(case, weight_index=0):
    return unpermute(case["permuted"], case["dtype"], case["sorted_indices"], case["padded_mode"],
                     case["restore_shape"], routing_map=case["routing_map"], probs=case["probs"],
                     probs_dtype=case["probs_dtype"], weight_index=weight_index)


# ------------------------------------------------------------------ the article's example

def test_article_padded_example():
    g = json.load(open(os.path.join(GOLD, "moe_unpermute_padded_example.json")))["inputs"]
    x = np.array(g["permuted_tokens_fp32"], np.float32).reshape(g["permuted_tokens_shape"])
    out = unpermute(x, nm.DT_FP32, np.array(g["sorted_indices_int32"], np.int32), g["padded_mode"],
                    tuple(g["restore_shape"]),
                    routing_map=np.array(g["routing_map_int8"], np.int8).reshape(g["routing_map_int8_shape"]),
                    probs=np.array(g["probs_fp32"], np.float32).reshape(g["probs_fp32_shape"]),
                    probs_dtype=nm.DT_FP32)
    # Derived by hand from branch 1: E = 2 experts, N = 2 entries, capacity C = 1.
    # permuteProbs[i] = probs[sI[i], i // 1] = [probs[1,0], probs[1,1]] = [1, 1];
    # sorting sI = [1, 1] gives permuteTokenId = [1, 1], outIndex = [0, 1];
    # token 1 accumulates rows 0 and 1 (each 1 * 1); token 0 receives nothing.
    assert out["unpermuted"].tolist() == [[0.0, 0.0], [2.0, 2.0]]
    assert out["permute_token_id"].tolist() == [1, 1]
    assert out["out_index"].tolist() == [0, 1]
    assert out["permute_probs"].tolist() == [1.0, 1.0]


# ------------------------------------------------------------------ closed forms

def _consistent_permute(rng, T, K, E, H, dt, topk_dist=None):
    """Forward permute built here from a routing map: expert-major rows."""
    x = synth._normal_elements(rng, (T, H), dt)
    n_t = rng.integers(0, K + 1, size=T) if topk_dist is None else topk_dist
    rmap = np.zeros((T, E), np.int8)
    for t in range(T):
        rmap[t, rng.choice(E, size=int(n_t[t]), replace=False)] = 1
    rows, slot_of = [], {}
    for e in range(E):
        for t in range(T):
            if rmap[t, e]:
                slot_of[(t, e)] = len(rows)
                rows.append(t)
    N = T * K
    permuted = np.zeros((N, H), dtype=x.dtype)
    permuted[:len(rows)] = x[rows]
    sI = np.full(N, -1, np.int32)
    for t in range(T):
        for k, e in enumerate(np.nonzero(rmap[t])[0]):
            sI[t * K + k] = slot_of[(t, e)]
    return x, permuted, sI, rmap, n_t


@pytest.mark.parametrize("dt", [nm.DT_FP16, nm.DT_BF16, nm.DT_FP32])
def test_permute_then_unpermute_no_probs_is_count_times_x(dt):
    rng = np.random.default_rng(3)
    T, K, E, H = 37, 4, 6, 19
    x, permuted, sI, _, n_t = _consistent_permute(rng, T, K, E, H, dt)
    out = unpermute(permuted, dt, sI, False, (T, H))
    # tokens with no expert keep the zero-initialised output (+0.0, hence the + 0.0)
    expect = _torch_round(_torch_f32(x, dt).double() * torch.from_numpy(n_t.astype(np.float64))[:, None] + 0.0, dt)
    assert np.array_equal(np.asarray(out["unpermuted"]).view(np.uint8), np.asarray(expect).view(np.uint8))


def test_topk1_round_trip_is_identity():
    rng = np.random.default_rng(4)
    T, E, H = 50, 7, 33
    x, permuted, sI, _, _ = _consistent_permute(rng, T, 1, E, H, nm.DT_BF16,
                                                topk_dist=np.ones(50, np.int64))
    out = unpermute(permuted, nm.DT_BF16, sI, False, (T, H))
    assert np.array_equal(out["unpermuted"], x)


def test_padded_permutation_inverse_exact():
    rng = np.random.default_rng(5)
    T, H, E = 48, 10, 4            # E * C = T, so sI can be a permutation of the tokens
    x = synth._normal_elements(rng, (T, H), nm.DT_FP16)
    sI = rng.permutation(T).astype(np.int32)
    out = unpermute(x, nm.DT_FP16, sI, True, (T, H))
    inv = np.empty(T, np.int64)
    inv[sI] = np.arange(T)
    assert np.array_equal(out["unpermuted"].view(np.uint16), x[inv].view(np.uint16))
    assert out["permute_token_id"].tolist() == list(range(T))
    assert out["out_index"].tolist() == inv.tolist()


def _softmax_probs(rng, rmap, dt):
    logits = rng.standard_normal(rmap.shape)
    p = synth._softmax_rows(logits, rmap != 0)
    return synth._probs_storage(p, dt)


@pytest.mark.parametrize("dt,pdt", [(nm.DT_FP32, nm.DT_FP32), (nm.DT_BF16, nm.DT_FP32),
                                    (nm.DT_FP16, nm.DT_FP16)])
def test_weighted_recombination_nonpadded_W2(dt, pdt):
    rng = np.random.default_rng(6)
    T, K, E, H = 40, 3, 8, 16
    n_t = rng.integers(1, K + 1, size=T)
    x, permuted, sI, rmap, _ = _consistent_permute(rng, T, K, E, H, dt, topk_dist=n_t)
    probs = _softmax_probs(rng, rmap, pdt)
    out = unpermute(permuted, dt, sI, False, (T, H), routing_map=rmap, probs=probs, probs_dtype=pdt)
    psum = nm.to_f32(probs, pdt).astype(np.float64).sum(axis=1)
    expect = nm.to_f32(x, dt).astype(np.float64) * psum[:, None]
    tol = 1e-5 if dt == nm.DT_FP32 else 1e-2
    np.testing.assert_allclose(nm.to_f32(out["unpermuted"], dt), expect, rtol=tol, atol=tol * 0.1)


def test_weighted_recombination_padded():
    rng = np.random.default_rng(7)
    T, E, H, k = 30, 5, 12, 2
    x = synth._normal_elements(rng, (T, H), nm.DT_FP32)
    rmap = np.zeros((T, E), np.int8)
    for t in range(T):
        rmap[t, rng.choice(E, size=k, replace=False)] = 1
    probs = _softmax_probs(rng, rmap, nm.DT_FP32)
    C = int(rmap.sum(axis=0).max()) + 2
    sI = np.empty(E * C, np.int32)
    for e in range(E):
        toks = list(np.nonzero(rmap[:, e])[0])
        pad = int(np.nonzero(rmap[:, e] == 0)[0][0])   # a token with zero prob for expert e
        sI[e * C:(e + 1) * C] = toks + [pad] * (C - len(toks))
    permuted = x[sI]
    out = unpermute(permuted, nm.DT_FP32, sI, True, (T, H), routing_map=rmap, probs=probs,
                    probs_dtype=nm.DT_FP32)
    np.testing.assert_allclose(out["unpermuted"], x, rtol=1e-5, atol=1e-6)


def test_W1_equals_W2_on_identity_indices():
    rng = np.random.default_rng(8)
    case = synth.unpermute_nonpadded_case(8, T=12, K=3, E=5, H=7, dtype=nm.DT_FP32,
                                          probs_dtype=nm.DT_FP32)
    case["sorted_indices"] = np.arange(36, dtype=np.int32)
    case["sorted_indices"][rng.choice(36, 5, replace=False)] = -1
    a, b = _run(case, 0), _run(case, 1)
    assert np.array_equal(a["unpermuted"], b["unpermuted"])


# ------------------------------------------------------------------ brute force vs torch

def _fp32_error_bound(terms_abs_sum, nterms, dt, exact):
    u32 = 2.0 ** -24
    acc_err = (2 * nterms + 1) * u32 * terms_abs_sum
    ulp_half = {nm.DT_FP32: 2.0 ** -24, nm.DT_FP16: 2.0 ** -11, nm.DT_BF16: 2.0 ** -8}[dt]
    tiny = {nm.DT_FP32: 1e-45, nm.DT_FP16: 6e-8, nm.DT_BF16: 1e-40}[dt]
    return acc_err * (1 + ulp_half) + ulp_half * np.abs(exact) + tiny


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("padded", [False, True])
@pytest.mark.parametrize("with_probs", [False, True])
def test_against_torch_index_add_fp64(seed, padded, with_probs):
    rng = np.random.default_rng(200 + seed)
    dt = [nm.DT_FP16, nm.DT_BF16, nm.DT_FP32][seed % 3]
    pdt = (nm.DT_FP32 if (dt == nm.DT_BF16 and seed % 2) else dt) if with_probs else None
    H = int(rng.integers(1, 40))
    if padded:
        E, T = int(rng.integers(1, 6)), int(rng.integers(1, 30))
        C = int(rng.integers(1, 12))
        case = synth.unpermute_padded_case(seed, E=E, C=C, T=T, H=H, dtype=dt, probs_dtype=pdt,
                                           topk=int(rng.integers(1, E + 1)), with_probs=with_probs,
                                           n_invalid=int(rng.integers(0, 3)) if E * C > 2 else 0)
    else:
        T, K, E = int(rng.integers(1, 30)), int(rng.integers(1, 6)), int(rng.integers(1, 10))
        K = min(K, E) if with_probs else K
        case = synth.unpermute_nonpadded_case(seed, T=T, K=K, E=E, H=H, dtype=dt, probs_dtype=pdt,
                                              n_empty=int(rng.integers(0, T * K + 1)),
                                              with_probs=with_probs,
                                              rows_mode=["compact", "slots"][seed % 2])
    out = _run(case)
    x = _torch_f32(case["permuted"], dt).double()
    sI = torch.from_numpy(case["sorted_indices"].astype(np.int64))
    N, T = sI.numel(), case["restore_shape"][0]
    rows = x.shape[0]
    if padded:
        valid = (sI >= 0) & (sI < T)
        dst, src = sI[valid], torch.arange(N)[valid]
        if with_probs:
            pf = _torch_f32(case["probs"], pdt).double()
            C = N // pf.shape[1]
            w = torch.zeros(N, dtype=torch.float64)
            w[valid] = pf[sI[valid], torch.arange(N)[valid] // C]
            wsrc = w[src]
    else:
        K = N // T
        valid = (sI >= 0) & (sI < rows)
        slots = torch.arange(N)[valid]
        dst, src = slots // K, sI[valid]
        if with_probs:
            pf = _torch_f32(case["probs"], pdt).double()
            sel = torch.masked_select(pf.t(), torch.from_numpy(case["routing_map"]).t() != 0)
            P = torch.zeros(N, dtype=torch.float64)
            P[:min(N, sel.numel())] = sel[:N]
            wsrc = P[src]
    terms = x[src] * (wsrc[:, None] if with_probs else 1.0)
    exact = torch.zeros((T, x.shape[1]), dtype=torch.float64).index_add_(0, dst, terms)
    abs_sum = torch.zeros_like(exact).index_add_(0, dst, terms.abs())
    cnt = torch.zeros(T, dtype=torch.float64).index_add_(0, dst, torch.ones(dst.numel(), dtype=torch.float64))
    got = nm.to_f32(out["unpermuted"], dt).astype(np.float64)
    bound = _fp32_error_bound(abs_sum.numpy(), cnt.numpy()[:, None], dt, exact.numpy())
    err = np.abs(got - exact.numpy())
    assert (err <= bound).all(), float((err - bound).max())
    if with_probs:
        pp = nm.to_f32(out["permute_probs"], pdt).astype(np.float64)
        ref = (w if padded else P).numpy()
        assert np.array_equal(pp, ref)


# ------------------------------------------------------------------ auxiliary outputs

@pytest.mark.parametrize("padded", [False, True])
def test_aux_outputs_properties(padded):
    if padded:
        case = synth.unpermute_padded_case(9, E=6, C=7, T=20, H=3, dtype=nm.DT_FP16,
                                           probs_dtype=nm.DT_FP16, n_invalid=4)
    else:
        case = synth.unpermute_nonpadded_case(9, T=20, K=4, E=9, H=3, dtype=nm.DT_FP16,
                                              probs_dtype=nm.DT_FP16, n_empty=17)
    out = _run(case)
    sI = case["sorted_indices"].astype(np.int64)
    N, T = sI.size, case["restore_shape"][0]
    oi, pt = out["out_index"].astype(np.int64), out["permute_token_id"].astype(np.int64)
    assert sorted(oi.tolist()) == list(range(N))               # a permutation of [0, N)
    if padded:
        key = np.where((sI >= 0) & (sI < T), sI, T)
        assert np.array_equal(pt, sI[oi])
    else:
        K = N // T
        key = np.where((sI >= 0) & (sI < N), sI + 1, 0)
        assert np.array_equal(pt, oi // K) and pt.min() >= 0 and pt.max() <= T - 1
    ks = key[oi]
    assert (np.diff(ks) >= 0).all()                              # sorted by key
    same = np.diff(ks) == 0
    assert (np.diff(oi)[same] > 0).all()                         # stable among equal keys
    ts = torch.sort(torch.from_numpy(key), stable=True)
    assert np.array_equal(ts.indices.numpy(), oi)


# ------------------------------------------------------------------ opt-in zero-weight skip

@pytest.mark.parametrize("padded", [False, True])
def test_zero_weight_skip_matches_the_formula_on_finite_rows(padded):
    # 0 * x = +-0 and acc + (+-0) = acc for any acc reachable from +0.0, so leaving the
    # term out cannot change a finite result
    if padded:
        case = synth.unpermute_padded_case(41, E=8, C=16, T=40, H=12, dtype=nm.DT_BF16, probs_dtype=nm.DT_FP32)
    else:
        case = synth.unpermute_nonpadded_case(42, T=30, K=4, E=8, H=12, dtype=nm.DT_FP16, probs_dtype=nm.DT_FP16,
                                              n_empty=20)
    args = (case["permuted"], case["dtype"], case["sorted_indices"], case["padded_mode"], case["restore_shape"])
    kw = dict(routing_map=case["routing_map"], probs=case["probs"], probs_dtype=case["probs_dtype"])
    a = unpermute(*args, **kw)
    b = unpermute(*args, skip_zero_weight=True, **kw)
    assert np.array_equal(np.asarray(a["unpermuted"]).view(np.uint8), np.asarray(b["unpermuted"]).view(np.uint8))


def test_zero_weight_skip_padded_worked_example():
    # expert 0 holds tokens 0 and 1, expert 1 tokens 0 and 2; token 1's row has weight 0
    # and holds NaN / inf: the skip leaves it out, the formula propagates it
    nan, inf = np.float32("nan"), np.float32("inf")
    x = np.array([[2, 4], [nan, inf], [8, 8], [3, 5]], np.float32)
    sI = np.array([0, 1, 0, 2], np.int32)
    probs = np.array([[0.5, 0.25], [0.0, 0.0], [0.0, 1.0]], np.float32)
    rmap = (probs != 0).astype(np.int8)
    out = unpermute(x, nm.DT_FP32, sI, True, (3, 2), routing_map=rmap, probs=probs, probs_dtype=nm.DT_FP32,
                    skip_zero_weight=True)
    assert out["unpermuted"].tolist() == [[3.0, 4.0], [0.0, 0.0], [3.0, 5.0]]
    with np.errstate(invalid="ignore"):  # inf * 0
        plain = unpermute(x, nm.DT_FP32, sI, True, (3, 2), routing_map=rmap, probs=probs, probs_dtype=nm.DT_FP32)
    assert np.isnan(plain["unpermuted"][1]).all()


def test_zero_weight_skip_nonpadded_worked_example():
    # map [[1,1],[1,0]]: expert-major weights P = [p00, p10, p01, 0]; slot 3 reads row 3,
    # whose weight is the zero padding of P
    nan = np.float32("nan")
    x = np.array([[2, 2], [4, 6], [6, 2], [nan, nan]], np.float32)
    sI = np.array([0, 2, 1, 3], np.int32)
    probs = np.array([[0.5, 0.5], [1.0, 0.0]], np.float32)
    rmap = np.array([[1, 1], [1, 0]], np.int8)
    out = unpermute(x, nm.DT_FP32, sI, False, (2, 2), routing_map=rmap, probs=probs, probs_dtype=nm.DT_FP32,
                    skip_zero_weight=True)
    assert out["unpermuted"].tolist() == [[4.0, 2.0], [4.0, 6.0]]
    plain = unpermute(x, nm.DT_FP32, sI, False, (2, 2), routing_map=rmap, probs=probs, probs_dtype=nm.DT_FP32)
    assert np.isnan(plain["unpermuted"][1]).all()


# ------------------------------------------------------------------ hand-worked weight-index and order pins

def test_W1_and_W2_worked_example_with_permuted_indices():
    # Non-padded, T = 2 tokens, topK = 2 (N = 4), E = 2 experts, H = 2, FP32.
    # routing map [[1, 1], [1, 0]], probs [[0.25, 0.75], [1.0, 0]]: the expert-major
    # masked select lists (t0,e0), (t1,e0), (t0,e1), so P = [0.25, 1.0, 0.75, 0] (zero pad).
    # sortedIndices = [2, 0, 1, -1]: token 0 reads rows 2 and 0, token 1 reads row 1.
    x = np.array([[1, 2], [10, 20], [100, 200], [1000, 2000]], np.float32)
    sI = np.array([2, 0, 1, -1], np.int32)
    probs = np.array([[0.25, 0.75], [1.0, 0.0]], np.float32)
    rmap = np.array([[1, 1], [1, 0]], np.int8)
    kw = dict(routing_map=rmap, probs=probs, probs_dtype=nm.DT_FP32)
    w2 = unpermute(x, nm.DT_FP32, sI, False, (2, 2), weight_index=0, **kw)
    w1 = unpermute(x, nm.DT_FP32, sI, False, (2, 2), weight_index=1, **kw)
    assert w2["permute_probs"].tolist() == [0.25, 1.0, 0.75, 0.0]
    # W2, weight of the permuted row r = sI[i]: token 0 = x2*P[2] + x0*P[0]
    # = [75, 150] + [0.25, 0.5]; token 1 = x1*P[1] = [10, 20]
    assert w2["unpermuted"].tolist() == [[75.25, 150.5], [10.0, 20.0]]
    # W1, weight of the slot i (the literal last line of branch 2): token 0 =
    # x2*P[0] + x0*P[1] = [25, 50] + [1, 2]; token 1 = x1*P[2] = [7.5, 15]
    assert w1["unpermuted"].tolist() == [[26.0, 52.0], [7.5, 15.0]]


def test_nonpadded_aux_order_worked_example():
    # Non-padded, T = 3, topK = 2 (N = rows = 6).  sortedIndices = [4, -1, 6, 1, 4, 0]:
    # slot 1 holds -1 and slot 2 holds 6 = rows, both outside [0, rows), so both are empty
    # slots.  Empty slots take the lowest key (the position of -1 is the design's reading,
    # since -1 leaves the slot-index range unchanged); the others sort by row index.
    # Keys [5, 0, 0, 2, 5, 1] -> stable order: slots 1, 2 (key 0), 5 (row 0), 3 (row 1),
    # 0, 4 (row 4, in slot order).
    x = np.arange(12, dtype=np.float32).reshape(6, 2)
    sI = np.array([4, -1, 6, 1, 4, 0], np.int32)
    out = unpermute(x, nm.DT_FP32, sI, False, (3, 2))
    assert out["out_index"].tolist() == [1, 2, 5, 3, 0, 4]
    assert out["permute_token_id"].tolist() == [0, 1, 2, 1, 0, 2]
    # token 0 = x4 (slot 1 empty); token 1 = x1 (slot 2 out of range, skipped);
    # token 2 = x4 + x0
    assert out["unpermuted"].tolist() == [[8.0, 9.0], [2.0, 3.0], [8.0, 10.0]]

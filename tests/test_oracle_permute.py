"""Pins for the forward permute oracle (CPU only).

  * round trips through the unpermute oracle: permute then non-padded unpermute
    without probs gives n_t * x exactly (x exactly for one expert per token); with
    softmax weights over each token's experts it gives x within the FP32 bound; a
    padded permute then padded unpermute gives n_t * x exactly;
  * an independent construction from library routines: torch.nonzero of the
    transposed map lists the entries expert-major, torch.cumsum along a token's row
    ranks its experts;
  * brute force of the padded capacity blocks, and the drop rules.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import numerics as nm
from oracle import moe_token_unpermute_with_routing_map as unpermute
from oracle.permute import moe_token_permute_with_routing_map as permute


def _map(rng, T, E, n_t):
    rmap = np.zeros((T, E), np.int8)
    for t in range(T):
        rmap[t, rng.choice(E, size=int(n_t[t]), replace=False)] = 1
    return rmap


def _torch_round(x64, dt):
    t32 = torch.from_numpy(np.asarray(x64, np.float64)).to(torch.float32)
    if dt == nm.DT_FP32:
        return t32.numpy()
    if dt == nm.DT_FP16:
        return t32.to(torch.float16).numpy()
    return t32.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("dt", [nm.DT_FP16, nm.DT_BF16, nm.DT_FP32])
def test_round_trip_without_probs_is_count_times_x(dt):
    rng = np.random.default_rng(11)
    T, K, E, H = 41, 4, 9, 13
    x = synth._normal_elements(rng, (T, H), dt)
    n_t = rng.integers(0, K + 1, size=T)
    rmap = _map(rng, T, E, n_t)
    p = permute(x, rmap, T * K)
    out = unpermute(p["permuted_tokens"], dt, p["sorted_indices"], False, (T, H))
    expect = _torch_round(nm.to_f32(x, dt).astype(np.float64) * n_t[:, None] + 0.0, dt)
    assert np.array_equal(np.asarray(out["unpermuted"]).view(np.uint8), np.asarray(expect).view(np.uint8))


def test_one_expert_per_token_round_trip_is_identity():
    rng = np.random.default_rng(12)
    T, E, H = 64, 5, 21
    x = synth._normal_elements(rng, (T, H), nm.DT_BF16)
    rmap = _map(rng, T, E, np.ones(T, np.int64))
    p = permute(x, rmap, T)
    out = unpermute(p["permuted_tokens"], nm.DT_BF16, p["sorted_indices"], False, (T, H))
    assert np.array_equal(out["unpermuted"], x)


@pytest.mark.parametrize("dt,pdt", [(nm.DT_FP32, nm.DT_FP32), (nm.DT_BF16, nm.DT_FP32), (nm.DT_FP16, nm.DT_FP16)])
def test_round_trip_with_softmax_weights_is_x(dt, pdt):
    rng = np.random.default_rng(13)
    T, K, E, H = 37, 3, 7, 10
    n_t = rng.integers(1, K + 1, size=T)
    rmap = _map(rng, T, E, n_t)
    x = synth._normal_elements(rng, (T, H), dt)
    logits = rng.standard_normal(rmap.shape)
    probs = synth._probs_storage(synth._softmax_rows(logits, rmap != 0), pdt)
    p = permute(x, rmap, T * K)
    out = unpermute(p["permuted_tokens"], dt, p["sorted_indices"], False, (T, H), routing_map=rmap, probs=probs,
                    probs_dtype=pdt)
    psum = nm.to_f32(probs, pdt).astype(np.float64).sum(axis=1)
    expect = nm.to_f32(x, dt).astype(np.float64) * psum[:, None]
    tol = 1e-5 if dt == nm.DT_FP32 else 1e-2
    np.testing.assert_allclose(nm.to_f32(out["unpermuted"], dt), expect, rtol=tol, atol=tol * 0.1)


@pytest.mark.parametrize("T,K,E,extra", [(30, 2, 6, 0), (25, 3, 4, 2), (17, 1, 9, 1), (12, 5, 3, 0)])
def test_matches_a_torch_nonzero_construction(T, K, E, extra):
    # extra > 0 routes some tokens to more than K experts: their later slots are dropped
    rng = np.random.default_rng(100 + T)
    n_t = np.minimum(rng.integers(0, K + 1 + extra, size=T), E)
    rmap = _map(rng, T, E, n_t)
    x = rng.integers(0, 256, size=(T, 6)).astype(np.uint8)
    N = T * K
    got = permute(x, rmap, N)
    m = torch.from_numpy(rmap != 0)
    pairs = torch.nonzero(m.t())                 # (expert, token), expert-major
    rank = torch.cumsum(m.to(torch.int64), dim=1) - 1   # rank of each expert within its token's row
    perm = np.zeros((N, 6), np.uint8)
    sI = np.full(N, -1, np.int32)
    for r, (e, t) in enumerate(pairs.tolist()):
        if r >= N:
            break
        perm[r] = x[t]
        k = int(rank[t, e])
        if k < K:
            sI[t * K + k] = r
    assert np.array_equal(got["permuted_tokens"], perm)
    assert np.array_equal(got["sorted_indices"], sI)


def test_rows_past_N_are_dropped():
    rng = np.random.default_rng(14)
    T, E = 10, 4
    rmap = np.ones((T, E), np.int8)             # 40 entries, N = 20
    x = np.arange(T * 3, dtype=np.float32).reshape(T, 3)
    got = permute(x, rmap, 2 * T)
    # expert-major: experts 0 and 1 fill the 20 rows
    assert np.array_equal(got["permuted_tokens"][:10], x)
    assert np.array_equal(got["permuted_tokens"][10:], x)
    sI = got["sorted_indices"].reshape(T, 2)
    assert sI[:, 0].tolist() == list(range(10)) and sI[:, 1].tolist() == list(range(10, 20))


@pytest.mark.parametrize("T,E,C", [(20, 4, 3), (9, 3, 9), (30, 5, 8)])
def test_padded_capacity_blocks_brute_force(T, E, C):
    rng = np.random.default_rng(200 + T)
    rmap = (rng.random((T, E)) < 0.35).astype(np.int8)
    x = rng.integers(0, 256, size=(T, 5)).astype(np.uint8)
    got = permute(x, rmap, E * C, padded_mode=True, capacity=C)
    for e in range(E):
        toks = [t for t in range(T) if rmap[t, e]][:C]
        blk = got["sorted_indices"][e * C:(e + 1) * C]
        assert blk[:len(toks)].tolist() == toks
        assert (blk[len(toks):] == -1).all()
        rows = got["permuted_tokens"][e * C:(e + 1) * C]
        assert np.array_equal(rows[:len(toks)], x[toks])
        assert (rows[len(toks):] == 0).all()


def test_padded_round_trip_is_count_times_x():
    # at most 5 experts per token: a sequential FP32 sum of up to 5 copies of x is the
    # rounded product (2x and 4x are exact), so n_t * x is exact
    rng = np.random.default_rng(15)
    T, E, H = 24, 5, 9
    rmap = (rng.random((T, E)) < 0.4).astype(np.int8)
    C = int(rmap.sum(axis=0).max())            # no token dropped
    x = synth._normal_elements(rng, (T, H), nm.DT_FP32)
    p = permute(x, rmap, E * C, padded_mode=True, capacity=C)
    out = unpermute(p["permuted_tokens"], nm.DT_FP32, p["sorted_indices"], True, (T, H))
    n_t = rmap.sum(axis=1).astype(np.float64)
    expect = (x.astype(np.float64) * n_t[:, None] + 0.0).astype(np.float32)
    assert np.array_equal(out["unpermuted"], expect)

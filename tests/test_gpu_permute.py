"""GPU parity of moe_permute against the oracle (bit-exact rows and indices), and GPU
round trips permute -> unpermute against their closed forms."""

import numpy as np
import pytest
import torch

import synth
from _gpu import (check_permute, fetch_permute, prepare_permute, run_permute, permute_tokens, dev,
                  to_torch_elems, from_torch_elems)
import unpermute_ffnwb_batching_amd as F

pytestmark = pytest.mark.gpu


def test_named_workload_full_size():
    case = synth.permute_config()
    print("permute T=16384 topK=8 E=128 H=4096 bf16", flush=True)
    check_permute(case, run_permute(case))


def test_padded_named_workload_full_size():
    case = synth.permute_padded_config()
    print("permute padded E=64 C=512 T=8192 H=5120 fp16", flush=True)
    check_permute(case, run_permute(case))


NONPAD = [
    # (T, K, E, H, dtype, route, row_pad, n_t override)
    (1, 1, 1, 8, synth.FP32, "uniform", 0, None),
    (37, 4, 9, 13, synth.FP16, "uniform", 0, None),          # E not a multiple of 4: byte map loads; odd H
    (300, 2, 64, 128, synth.BF16, "skew", 0, None),
    (513, 8, 128, 64, synth.BF16, "uniform", 0, None),        # several 256-token tiles, ragged tail
    (200, 3, 16, 33, synth.INT8, "uniform", 5, None),         # 1-byte elements, strided rows, byte copies
    (1000, 2, 32, 72, synth.FP32, "skew", 4, "more"),         # tokens with more experts than slots
    (256, 1, 4, 16, synth.FP16, "uniform", 0, "all"),         # every token to all experts: rows dropped past N
    (77, 5, 256, 24, synth.BF16, "uniform", 0, None),         # E = 256
    (64, 3, 12, 8, synth.FP16, "uniform", 0, "none"),         # empty map: zero rows, -1 slots
    # four-launch order through the [T][E] table (more than 256 experts, or large maps)
    (4096, 8, 512, 64, synth.BF16, "uniform", 0, None),       # E = 512
    (300, 70, 300, 24, synth.FP32, "skew", 0, "more"),        # E not a multiple of 4, topK = 70 > 64
    (2000, 3, 1000, 16, synth.INT8, "uniform", 3, None),      # byte rows, strided tokens
    (40, 300, 512, 8, synth.BF16, "uniform", 0, "all300"),    # 300 rows per token: the list is copied in two parts
    (50, 200, 8192, 8, synth.FP16, "uniform", 0, None),       # the most experts
    (9000, 2, 260, 32, synth.FP16, "skew", 0, "more"),        # 260 experts: rows dropped past N
]


@pytest.mark.parametrize("params", NONPAD, ids=[str(i) for i in range(len(NONPAD))])
def test_nonpadded(params):
    T, K, E, H, dt, route, pad, mode = params
    rng = np.random.default_rng(T + E)
    n_t = None
    if mode == "more":
        n_t = rng.integers(0, K + 3, size=T)
    elif mode == "all":
        n_t = np.full(T, E)
    elif mode == "none":
        n_t = np.zeros(T, np.int64)
    elif mode == "all300":
        n_t = np.full(T, 300)
    case = synth.permute_case(700 + T + E, T=T, K=K, E=E, H=H, dtype=dt, route=route, row_pad=pad, n_t=n_t)
    print(f"permute non-padded {params}", flush=True)
    check_permute(case, run_permute(case))


PAD = [
    # (T, E, C, H, dtype, topK)
    (100, 8, 40, 24, synth.FP16, 3),       # enough capacity
    (500, 16, 20, 64, synth.BF16, 2),      # capacity overflow: tokens dropped
    (300, 6, 1, 9, synth.INT8, 2),         # C = 1, byte copies
    (700, 64, 48, 128, synth.FP32, 4),     # three tiles
    (50, 5, 0, 8, synth.FP16, 1),          # C = 0: nothing to write
    (300, 256, 30, 16, synth.BF16, 200),   # up to 200 experts per token: four 64-entry table chunks
    (150, 200, 64, 24, synth.FP16, 130),   # partial last table chunk (200 = 3*64 + 8)
    (90, 130, 20, 8, synth.INT8, 100),     # E not a multiple of 4 (byte map loads) with partial chunks
    # four-launch order through the [T][E] table
    (4096, 512, 64, 32, synth.BF16, 8),    # E = 512
    (64, 512, 64, 8, synth.FP16, 300),     # 300 capacity rows per token: the list is copied in two parts
    (3000, 1000, 7, 24, synth.FP32, 5),    # capacity overflow over 1000 experts
    (5000, 301, 40, 13, synth.INT8, 4),    # E not a multiple of 4, byte rows
]


@pytest.mark.parametrize("params", PAD, ids=[str(i) for i in range(len(PAD))])
def test_padded(params):
    T, E, C, H, dt, k = params
    case = synth.permute_case(800 + T + E, T=T, K=k, E=E, H=H, dtype=dt, padded=True, C=C)
    print(f"permute padded {params}", flush=True)
    check_permute(case, run_permute(case))


def test_repeat_is_bit_identical():
    case = synth.permute_case(901, T=600, K=4, E=32, H=256, dtype=synth.BF16, route="skew")
    call = prepare_permute(case)
    call.run()
    torch.cuda.synchronize()
    a = fetch_permute(call)
    call.run()
    torch.cuda.synchronize()
    b = fetch_permute(call)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    check_permute(case, b)


def _gpu_unpermute(permuted, sI, dt, T, H, rmap=None, probs=None, padded=False):
    out = F.moe_unpermute(permuted, sI, rmap, probs, padded_mode=padded, restore_shape=(T, H), aux=False)
    torch.cuda.synchronize()
    return out["unpermuted"]


def test_round_trip_without_probs_is_count_times_x():
    # permute then unpermute on the GPU: each token's row summed once per expert (<= 4,
    # so the FP32 sums are the rounded products)
    T, K, E, H = 3000, 4, 64, 256
    case = synth.permute_case(902, T=T, K=K, E=E, H=H, dtype=synth.BF16)
    call = prepare_permute(case)
    call.run()
    back = _gpu_unpermute(call.out["permuted_tokens"], call.out["sorted_indices"], synth.BF16, T, H)
    x = to_torch_elems(permute_tokens(case).copy(), synth.BF16).float().cpu()
    n_t = torch.from_numpy(case["routing_map"].sum(axis=1).astype(np.float32))
    expect = (x.double() * n_t.double()[:, None] + 0.0).float().to(torch.bfloat16)
    assert torch.equal(back.cpu().view(torch.int16), expect.view(torch.int16))


@pytest.mark.parametrize("pdt", [synth.FP32, synth.BF16])
def test_round_trip_with_softmax_weights_is_x(pdt):
    # the unpermute's default weight reading (each permuted row times its compacted prob)
    # recombines softmax-weighted expert copies into the token itself
    T, K, E, H = 2000, 4, 32, 128
    rng = np.random.default_rng(903)
    case = synth.permute_case(903, T=T, K=K, E=E, H=H, dtype=synth.BF16, n_t=rng.integers(1, K + 1, size=T))
    rmap = case["routing_map"]
    p = synth._probs_storage(synth._softmax_rows(rng.standard_normal(rmap.shape), rmap != 0), pdt)
    call = prepare_permute(case)
    call.run()
    back = _gpu_unpermute(call.out["permuted_tokens"], call.out["sorted_indices"], synth.BF16, T, H,
                          rmap=dev(rmap), probs=to_torch_elems(p, pdt))
    from oracle import numerics as nm
    psum = nm.to_f32(p, pdt).astype(np.float64).sum(axis=1)
    x = nm.to_f32(permute_tokens(case), synth.BF16).astype(np.float64)
    got = nm.to_f32(from_torch_elems(back, synth.BF16), synth.BF16)
    np.testing.assert_allclose(got, x * psum[:, None], rtol=1e-2, atol=1e-3)


def test_padded_round_trip_is_count_times_x():
    T, E, H = 1200, 16, 64
    case = synth.permute_case(904, T=T, K=3, E=E, H=H, dtype=synth.FP32, padded=True, C=None)
    C = int(case["routing_map"].sum(axis=0).max())   # no token dropped
    case["C"], case["N"] = C, E * C
    call = prepare_permute(case)
    call.run()
    back = _gpu_unpermute(call.out["permuted_tokens"], call.out["sorted_indices"], synth.FP32, T, H, padded=True)
    x = permute_tokens(case).astype(np.float64)
    n_t = case["routing_map"].sum(axis=1).astype(np.float64)
    assert np.array_equal(back.cpu().numpy(), (x * n_t[:, None] + 0.0).astype(np.float32))


def _permute_indices(rmap, N, padded, C=None):
    """sorted_indices from library routines (torch.nonzero lists entries expert-major,
    cumsum ranks a token's experts), independent of the oracle's loops."""
    m = torch.from_numpy(rmap != 0)
    T, E = m.shape
    e_idx, t_idx = torch.nonzero(m.t(), as_tuple=True)       # expert-major entry order
    out = torch.full((N,), -1, dtype=torch.int64)
    if padded:
        place = torch.cumsum(m.t().long(), dim=1) - 1           # rank of t within expert e
        p = place[e_idx, t_idx]
        keep = p < C
        out[e_idx[keep] * C + p[keep]] = t_idx[keep]
        return out.numpy()
    K = N // T
    row = torch.full((T, E), -1, dtype=torch.int64)
    row[t_idx, e_idx] = torch.arange(e_idx.numel())
    k = torch.cumsum(m.long(), dim=1) - 1                        # rank of e within token t
    tt, ee = torch.nonzero(m, as_tuple=True)
    kk = k[tt, ee]
    r = row[tt, ee]
    keep = kk < K
    out[tt[keep] * K + kk[keep]] = torch.where(r[keep] < N, r[keep], torch.full_like(r[keep], -1))
    return out.numpy()


@pytest.mark.parametrize("T,E,padded", [(4096, 512, False), (65536, 128, False), (4096, 512, True),
                                        (65536, 128, True)])
def test_table_order_round_trip_is_count_times_x(T, E, padded):
    # the four-launch order at E = 512 and at T = 65536 (256 tiles x 128 experts): the
    # permute's indices against a construction from library routines, then permute ->
    # unpermute gives every token's row once per expert it kept, exactly
    H, K = 64, 4
    rng = np.random.default_rng(905 + T + E)
    n_t = rng.integers(0, K + 1, size=T)
    rmap = np.zeros((T, E), np.int8)
    for t in np.nonzero(n_t)[0]:
        rmap[t, rng.choice(E, size=int(n_t[t]), replace=False)] = 1
    x = synth._normal_elements(rng, (T, H), synth.FP32)
    tokens = dev(x)
    C = int(rmap.sum(axis=0).max()) - 1 if padded else 0   # one token dropped from the fullest expert
    N = E * C if padded else T * K
    call = F.PermuteCall(tokens, dev(rmap), padded_mode=padded, num_out_rows=N, capacity=C)
    print(f"permute table order T={T} E={E} padded={padded}", flush=True)
    call.run()
    torch.cuda.synchronize()
    sI = call.out["sorted_indices"].cpu().numpy()
    assert np.array_equal(sI, _permute_indices(rmap, N, padded, C))
    back = _gpu_unpermute(call.out["permuted_tokens"], call.out["sorted_indices"], synth.FP32, T, H, padded=padded)
    if padded:
        kept = np.bincount(sI[sI >= 0], minlength=T).astype(np.float64)
    else:
        kept = (sI.reshape(T, K) >= 0).sum(axis=1).astype(np.float64)
    assert np.array_equal(back.cpu().numpy(), (x.astype(np.float64) * kept[:, None] + 0.0).astype(np.float32))

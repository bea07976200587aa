"""GPU parity of moe_update_expert against the oracle: instance ids, the pruning mask
and the error count, all bit-exact."""

import numpy as np
import pytest
import torch

import synth
from _gpu import check_update_expert, prepare_update_expert

pytestmark = pytest.mark.gpu


def _run(case, rank=None, mode=None):
    call = prepare_update_expert(case, rank, mode)
    call.run()
    torch.cuda.synchronize()
    return call


CASES = [
    # (BS, K, E, world, place, F, id dtype, scale dtype, active tokens, mode, rank)
    (512, 8, 256, 64, 5, 9, np.int32, synth.BF16, 400, 0, 37),     # the measured workload
    (512, 8, 256, 64, 5, 9, np.int32, synth.BF16, 400, 1, 0),
    (512, 16, 1024, 128, 8, 2, np.int64, synth.FP16, None, 0, 127),  # the largest sizes, one replica each
    (300, 5, 40, 16, 4, 17, np.int64, synth.FP32, 123, 1, 5),
    (77, 3, 12, 6, 3, 7, np.int32, None, None, 0, 2),               # no scales: ids only
    (1, 1, 1, 2, 1, 3, np.int32, synth.FP32, 1, 0, 1),              # the smallest
    (64, 4, 8, 768, 1, 769, np.int32, synth.BF16, 50, 0, 767),      # 768 ranks, 96 replicas per expert
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_matches_the_oracle(case):
    BS, K, E, W, P, Fc, idt, sdt, na, mode, rank = case
    c = synth.update_expert_case(90 + BS + K, BS, K, E, W, P, F=Fc, local_rank_id=rank, balance_mode=mode,
                                 id_dtype=idt, scale_dtype=sdt, n_active=na)
    print(f"update expert {case}", flush=True)
    check_update_expert(c, _run(c))


def test_every_rank_and_both_modes():
    c = synth.update_expert_case(3, 128, 6, 32, 12, 4, F=8, scale_dtype=synth.FP32, n_active=100)
    print("update expert: every rank, both modes", flush=True)
    for mode in (0, 1):
        for rank in range(12):
            check_update_expert(c, _run(c, rank, mode), rank, mode)


def test_bad_ids_counts_and_edge_scales():
    c = synth.update_expert_case(4, 32, 4, 16, 8, 3, F=5, scale_dtype=synth.FP32, n_active=20, n_bad_ids=9)
    t = c["eplb_table"].copy()
    t[3, 0], t[5, 0], t[7, 0] = 0, 5, -2          # counts outside [1, F - 1]
    s = c["expert_scales"].copy()
    s[0, 0], s[1, 1] = np.nan, c["pruning_threshold"][1]   # NaN kept, equal kept
    c = dict(c, eplb_table=t, expert_scales=s)
    print("update expert: bad ids and counts, NaN and equal scales", flush=True)
    ref = check_update_expert(c, _run(c))
    assert ref["err_count"] > 9


def test_repeat_is_bit_identical():
    c = synth.update_expert_case(6, 256, 8, 64, 16, 5, F=9, id_dtype=np.int64, scale_dtype=synth.BF16, n_active=200)
    call = prepare_update_expert(c)
    call.run()
    torch.cuda.synchronize()
    a = {k: v.clone() for k, v in call.out.items()}
    call.run()
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k].view(torch.uint8), call.out[k].view(torch.uint8)), k
    check_update_expert(c, call)


def test_strided_views_of_every_input_and_output():
    # the parameter table allows non-contiguous tensors: every input and output a view
    # into a wider buffer (row strides for the 2-D tensors, an element stride for the
    # threshold and the mask), against the oracle on the same values
    import unpermute_ffnwb_batching_amd as F
    from _gpu import dev, oracle_update_expert, to_torch_elems
    for mode, idt, sdt in ((0, np.int32, synth.BF16), (1, np.int64, synth.FP32)):
        c = synth.update_expert_case(7 + mode, 200, 6, 48, 16, 5, F=9, local_rank_id=11, balance_mode=mode,
                                     id_dtype=idt, scale_dtype=sdt, n_active=150, n_bad_ids=5)
        BS, K = c["expert_ids"].shape
        E, Fc = c["eplb_table"].shape
        ids_w = np.full((BS, K + 5), -7, dtype=idt)
        ids_w[:, 2:2 + K] = c["expert_ids"]
        tab_w = np.full((E, Fc + 3), 99999, np.int32)
        tab_w[:, :Fc] = c["eplb_table"]
        sc = to_torch_elems(c["expert_scales"], sdt)
        sc_w = torch.zeros((BS, K + 2), dtype=sc.dtype, device="cuda")
        sc_w[:, 1:1 + K] = sc
        thr_w = torch.full((3 * K,), 1e30, dtype=torch.float32, device="cuda")
        thr_w[::3] = dev(c["pruning_threshold"])
        act_w = torch.zeros((2 * BS,), dtype=torch.bool, device="cuda")
        act_w[::2] = dev(c["active_mask"])
        out_ids_w = torch.full((BS, K + 4), -5, dtype=torch.int32 if idt == np.int32 else torch.int64, device="cuda")
        out_mask_w = torch.full((BS, 2 * K), 7, dtype=torch.uint8, device="cuda")
        out = {"balanced_expert_ids": out_ids_w[:, 3:3 + K], "balanced_active_mask": out_mask_w[:, 1:1 + K].view(torch.bool),
               "err_count": torch.zeros(1, dtype=torch.int32, device="cuda")}
        call = F.UpdateExpertCall(dev(ids_w)[:, 2:2 + K], dev(tab_w)[:, :Fc], local_rank_id=c["local_rank_id"],
                                  world_size=c["world_size"], balance_mode=mode, expert_scales=sc_w[:, 1:1 + K],
                                  pruning_threshold=thr_w[::3], active_mask=act_w[::2], out=out)
        print(f"update expert, strided views, mode {mode}", flush=True)
        call.run()
        torch.cuda.synchronize()
        ref = oracle_update_expert(c)
        assert np.array_equal(out_ids_w[:, 3:3 + K].cpu().numpy(), ref["balanced_expert_ids"])
        assert np.array_equal(out_mask_w[:, 1:1 + K].cpu().numpy(), ref["balanced_active_mask"].astype(np.uint8))
        assert int(out["err_count"][0]) == ref["err_count"]
        # the bytes around the views stay untouched
        ow = out_ids_w.cpu().numpy()
        assert (ow[:, :3] == -5).all() and (ow[:, 3 + K:] == -5).all()
        om = out_mask_w.cpu().numpy()
        assert (om[:, :1] == 7).all() and (om[:, 1 + K:] == 7).all()

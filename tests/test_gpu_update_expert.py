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

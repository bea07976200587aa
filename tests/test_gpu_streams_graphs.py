"""Calls on several streams at once, and calls captured in a HIP graph.

  * two non-padded unpermutes (one with its auxiliary order on a caller-supplied
    auxiliary stream, one without) and a batching, launched on three streams without
    synchronising between them, each checked against the oracle;
  * a one-shot helper run on a side stream, its outputs and workspace allocated there,
    followed by allocations on the current stream before that work has finished;
  * every entry point captured into one graph, replayed three times with new input
    data copied into the captured inputs (and eager work in between), every replay
    checked against the oracle for the data it saw.
"""

import numpy as np
import pytest
import torch

import synth
from _gpu import (check_batching, check_ctx, check_permute, check_unpermute, check_update_expert, dev,
                  fetch_batching, fetch_permute, fetch_unpermute, oracle_batching, oracle_ctx, oracle_permute,
                  oracle_unpermute, prepare_batching, prepare_ctx, prepare_permute, prepare_unpermute,
                  prepare_update_expert)

pytestmark = pytest.mark.gpu


def test_concurrent_calls_on_three_streams():
    u1 = synth.unpermute_nonpadded_case(31, T=2048, K=4, E=32, H=512, dtype=synth.BF16, probs_dtype=synth.FP32,
                                        n_empty=900)
    u2 = synth.unpermute_nonpadded_case(32, T=1500, K=8, E=64, H=256, dtype=synth.FP16, probs_dtype=synth.FP16,
                                        n_empty=2000)
    bt = synth.batching_case(33, 16, 32, 9, 1024, 256, 1, synth.BF16, n_masked=300)
    aux = torch.cuda.Stream()
    calls = [prepare_unpermute(u1, aux_stream=aux), prepare_unpermute(u2), prepare_batching(bt)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in calls]
    print("three streams, no synchronisation between them", flush=True)
    for _ in range(3):
        for call, st in zip(calls, streams):
            call.run(st)
    torch.cuda.synchronize()
    check_unpermute(u1, fetch_unpermute(calls[0], u1))
    check_unpermute(u2, fetch_unpermute(calls[1], u2))
    check_batching(bt, fetch_batching(calls[2]))


def test_one_shot_helper_on_a_side_stream():
    # The helper allocates its workspace on the stream it runs on.  The side stream is
    # held back by a bounded spin, so the call's kernels run late; the current stream
    # meanwhile allocates and fills buffers of the workspace's size.  Had the workspace
    # been taken from the current stream's pool and freed on return, those buffers could
    # reuse it while the call still writes there.
    import unpermute_ffnwb_batching_amd as F
    case = synth.unpermute_nonpadded_case(34, T=4096, K=8, E=64, H=1024, dtype=synth.BF16, probs_dtype=synth.FP32,
                                          n_empty=3000)
    x = dev(case["permuted"].view(np.int16)).view(torch.bfloat16)
    sI, rmap, probs = dev(case["sorted_indices"]), dev(case["routing_map"]), dev(case["probs"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    kw = dict(padded_mode=False, restore_shape=(4096, 1024))
    with torch.cuda.stream(side):
        ws_bytes = F.UnpermuteCall(x, sI, rmap, probs, **kw).ws_bytes
    assert ws_bytes > 0
    print(f"one-shot unpermute on a side stream (workspace {ws_bytes} B), then allocations on the current "
          "stream", flush=True)
    with torch.cuda.stream(side):
        torch.cuda._sleep(20_000_000)
    out = F.moe_unpermute(x, sI, rmap, probs, stream=side, **kw)
    junk = [torch.full((ws_bytes,), 7, dtype=torch.uint8, device="cuda") for _ in range(4)]
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    got = {"unpermuted": out["unpermuted"].view(torch.int16).cpu().numpy().view(np.uint16),
           "out_index": out["out_index"].cpu().numpy(), "permute_token_id": out["permute_token_id"].cpu().numpy(),
           "permute_probs": out["permute_probs"].cpu().numpy()}
    check_unpermute(case, got)
    assert all(int(j.min()) == 7 == int(j.max()) for j in junk)


def _refill(t, a):
    """Copy host array `a` into the captured device tensor `t` (same bytes)."""
    src = torch.from_numpy(np.ascontiguousarray(a)).view(torch.uint8).reshape(-1)
    t.view(torch.uint8).reshape(-1).copy_(src.to(t.device))


def test_every_entry_point_in_one_graph_replayed_with_new_inputs():
    seeds = [(41, 42, 43, 44, 45, 46), (51, 52, 53, 54, 55, 56), (61, 62, 63, 64, 65, 66)]

    def cases(sd):
        return dict(
            bt=synth.batching_case(sd[0], 8, 16, 9, 256, 64, 1, synth.BF16, n_masked=100),
            un=synth.unpermute_nonpadded_case(sd[1], T=1024, K=4, E=32, H=256, dtype=synth.BF16,
                                              probs_dtype=synth.FP32, n_empty=400),
            up=synth.unpermute_padded_case(sd[2], E=16, C=64, T=700, H=128, dtype=synth.FP16,
                                           probs_dtype=synth.FP16),
            pm=synth.permute_case(sd[3], T=900, K=4, E=32, H=128, dtype=synth.BF16),
            ue=synth.update_expert_case(sd[4], 256, 8, 64, 16, 5, F=9, local_rank_id=3, scale_dtype=synth.BF16,
                                        n_active=200),
            cx=synth.schedule_area(sd[5], 8, 3, 16, 9, 128, 64, 1, synth.FP16, n_not_ready=4),
        )

    c0 = cases(seeds[0])
    aux = torch.cuda.Stream()
    calls = dict(bt=prepare_batching(c0["bt"]), un=prepare_unpermute(c0["un"], aux_stream=aux),
                 up=prepare_unpermute(c0["up"]),
                 pm=prepare_permute(c0["pm"]), ue=prepare_update_expert(c0["ue"]),
                 cx=prepare_ctx(c0["cx"], 2, 1))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    print("capturing every entry point into one graph", flush=True)
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for call in calls.values():
                call.run(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep, sd in enumerate(seeds):
        c = cases(sd)
        if rep > 0:
            # new data into the tensors the graph captured
            k = calls["bt"]._keep
            _refill(k[0], c["bt"]["token_bytes"]), _refill(k[1], c["bt"]["expert_ids"]), _refill(k[2], c["bt"]["mask"])
            for key in ("un", "up"):
                uk = calls[key]._keep
                _refill(uk[0], c[key]["permuted"]), _refill(uk[1], c[key]["sorted_indices"])
                _refill(uk[2], c[key]["routing_map"]), _refill(uk[3], c[key]["probs"])
            pk = calls["pm"]._keep
            _refill(pk[0], c["pm"]["tokens_full"][:, :c["pm"]["H"]]), _refill(pk[1], c["pm"]["routing_map"])
            ek = calls["ue"]._keep
            _refill(ek[0], c["ue"]["expert_ids"]), _refill(ek[1], c["ue"]["eplb_table"])
            _refill(ek[2], c["ue"]["expert_scales"]), _refill(ek[3], c["ue"]["pruning_threshold"])
            _refill(ek[4], c["ue"]["active_mask"])
            xk = calls["cx"]._keep
            _refill(xk[1], c["cx"]["info"]), _refill(xk[2], c["cx"]["data"].reshape(-1))
            # eager work between replays
            torch.ones(1 << 20, device="cuda").mul_(3.0).sum().item()
        torch.cuda.synchronize()
        print(f"replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        check_batching(c["bt"], fetch_batching(calls["bt"]))
        check_unpermute(c["un"], fetch_unpermute(calls["un"], c["un"]))
        check_unpermute(c["up"], fetch_unpermute(calls["up"], c["up"]))
        check_permute(c["pm"], fetch_permute(calls["pm"]))
        check_update_expert(c["ue"], calls["ue"])
        check_ctx(c["cx"], calls["cx"])

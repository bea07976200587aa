"""GPU parity of moe_unpermute_noalloc (the entry point that allocates nothing: its
workspace is the library's per-GPU scratch array) against moe_unpermute on the same
inputs, through the C ABI.  Two calls in a row on the scratch, the second smaller than
the first, in both layouts; every output bit-identical to moe_unpermute's, and within
the unpermute's tolerance of the oracle."""

import numpy as np
import pytest
import torch

import synth
import unpermute_ffnwb_batching_amd as F
from _gpu import check_unpermute, fetch_unpermute, prepare_unpermute

pytestmark = pytest.mark.gpu


def _same(a, b):
    for k in b:
        assert np.array_equal(np.asarray(a[k]).view(np.uint8), np.asarray(b[k]).view(np.uint8)), k


def _pair(case, aux_stream=None):
    """(outputs of moe_unpermute, outputs of moe_unpermute_noalloc) for one case."""
    ref_call = prepare_unpermute(case)
    na_call = prepare_unpermute(case, aux_stream=aux_stream)
    ref_call.run()
    torch.cuda.synchronize()
    na_call.run_noalloc()
    torch.cuda.synchronize()
    return fetch_unpermute(ref_call, case), fetch_unpermute(na_call, case)


@pytest.mark.parametrize("padded", [False, True])
def test_noalloc_matches_moe_unpermute_on_two_calls_in_a_row(padded):
    if padded:
        big = synth.unpermute_padded_case(91, E=64, C=512, T=8192, H=512, dtype=synth.FP16, probs_dtype=synth.FP16,
                                          n_invalid=300)
        small = synth.unpermute_padded_case(92, E=8, C=33, T=100, H=40, dtype=synth.BF16, probs_dtype=synth.FP32)
    else:
        big = synth.unpermute_nonpadded_case(93, T=16384, K=8, E=128, H=512, dtype=synth.BF16,
                                             probs_dtype=synth.FP32, n_empty=13107)
        small = synth.unpermute_nonpadded_case(94, T=700, K=3, E=16, H=72, dtype=synth.FP16, probs_dtype=synth.FP16,
                                               n_empty=200)
    for name, case in (("first, larger", big), ("second, smaller", small)):
        print(f"noalloc {'padded' if padded else 'non-padded'} {name}", flush=True)
        ref, got = _pair(case)
        _same(got, ref)
        check_unpermute(case, got)


def test_noalloc_with_an_auxiliary_stream_then_without_probs():
    case = synth.unpermute_nonpadded_case(95, T=4096, K=8, E=64, H=256, dtype=synth.FP32, probs_dtype=synth.FP32,
                                          n_empty=2000)
    print("noalloc non-padded with an auxiliary stream", flush=True)
    ref, got = _pair(case, aux_stream=torch.cuda.Stream())
    _same(got, ref)
    check_unpermute(case, got)
    small = synth.unpermute_nonpadded_case(96, T=300, K=2, E=8, H=16, dtype=synth.FP16, probs_dtype=None,
                                           n_empty=50, with_probs=False)
    print("noalloc non-padded without probs, smaller", flush=True)
    ref, got = _pair(small)
    _same(got, ref)
    check_unpermute(small, got)


def test_noalloc_rejects_a_call_larger_than_the_scratch():
    # T = 131072, topK = 8, E = 256 with the auxiliary outputs needs 26.5 MiB of workspace
    d = F.UnpermuteDesc()
    T, K, E = 131072, 8, 256
    d.dtype, d.probs_dtype, d.num_rows, d.hidden, d.num_tokens, d.num_experts, d.num_indices = \
        F.FFNWB_DT_BF16, F.FFNWB_DT_FP32, T * K, 64, T, E, T * K
    x = torch.empty(1, device="cuda")
    for f in ("permuted_tokens", "sorted_indices", "unpermuted_tokens", "out_index", "permute_token_id",
              "routing_map", "probs", "permute_probs"):
        setattr(d, f, x.data_ptr())
    import ctypes
    n = ctypes.c_size_t(0)
    assert F.lib().moe_unpermute_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0
    assert n.value > F.FFNWB_NOALLOC_SCRATCH_BYTES
    assert F.lib().moe_unpermute_noalloc(ctypes.byref(d), None) == F.FFNWB_ERR_SCRATCH

"""Timing hooks bound to the timed kernel's launch.

Every entry point that takes hooks runs with both hooks given and with only the end
hook (both bound to the kernel's dispatch).  Its results still match the oracle, and the
bound span is positive, finite and shorter than the whole call measured on the host
around a synchronisation.
"""

import time

import numpy as np
import pytest
import torch

import synth
from _gpu import (check_batching, check_permute, check_unpermute, fetch_batching, fetch_permute, fetch_unpermute,
                  prepare_batching, prepare_permute, prepare_unpermute)
from unpermute_ffnwb_batching_amd.hip_events import HipEvent

pytestmark = pytest.mark.gpu


def _timed(call, begin, end):
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    call.run(torch.cuda.current_stream())
    torch.cuda.synchronize()
    host_ms = (time.perf_counter() - t0) * 1e3
    if begin is not None:
        ms = begin.elapsed_ms(end)
        assert np.isfinite(ms) and 0.0 < ms <= host_ms, (ms, host_ms)
    else:
        end.synchronize()


@pytest.mark.parametrize("both", [True, False], ids=["bound", "end-only"])
def test_hooks_unpermute(both):
    for case in (synth.unpermute_nonpadded_case(71, T=2048, K=4, E=32, H=512, dtype=synth.BF16,
                                                probs_dtype=synth.FP32, n_empty=700),
                 synth.unpermute_padded_case(72, E=16, C=64, T=700, H=256, dtype=synth.FP16,
                                             probs_dtype=synth.FP16)):
        b, e = HipEvent(), HipEvent()
        call = prepare_unpermute(case, ev_reduce=(b if both else None, e))
        print(f"unpermute hooks both={both} padded={case.get('padded')}", flush=True)
        _timed(call, b if both else None, e)
        check_unpermute(case, fetch_unpermute(call, case))


@pytest.mark.parametrize("both", [True, False], ids=["bound", "end-only"])
def test_hooks_batching(both):
    for case in (synth.batching_case(73, 16, 32, 9, 1024, 256, 1, synth.BF16, n_masked=300),   # one-launch order
                 synth.batching_case(74, 64, 64, 9, 256, 1024, 16, synth.INT8, n_masked=5000),  # rank / scan / gather
                 synth.batching_case(75, 2, 8, 3, 128, 16, 1, synth.FP16, n_masked=5)):         # one workgroup
        b, e = HipEvent(), HipEvent()
        call = prepare_batching(case, ev_gather=(b if both else None, e))
        print(f"batching hooks both={both} Y={case['A'] * case['BS'] * case['K1']}", flush=True)
        _timed(call, b if both else None, e)
        check_batching(case, fetch_batching(call))


@pytest.mark.parametrize("both", [True, False], ids=["bound", "end-only"])
def test_hooks_permute(both):
    for case in (synth.permute_case(76, T=900, K=4, E=32, H=128, dtype=synth.BF16),
                 synth.permute_case(77, T=300, K=2, E=8, H=64, dtype=synth.FP16, padded=True, C=64)):
        b, e = HipEvent(), HipEvent()
        call = prepare_permute(case, ev_copy=(b if both else None, e))
        print(f"permute hooks both={both}", flush=True)
        _timed(call, b if both else None, e)
        check_permute(case, fetch_permute(call))

"""Pins for the oracle's element conversions against torch's CPU conversions."""

import numpy as np
import pytest
import torch

from oracle import numerics as nm


def _interesting_f32():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 32, size=200000, dtype=np.uint64).astype(np.uint32)
    # exact ties at every exponent, both parities of the kept lsb
    hi = rng.integers(0, 1 << 16, size=4096, dtype=np.uint64).astype(np.uint32)
    ties = (hi << np.uint32(16)) | np.uint32(0x8000)
    near = np.concatenate([ties - np.uint32(1), ties + np.uint32(1)])
    special = np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7F7FFFFF,
                        0xFF7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x00000001, 0x807FFFFF,
                        0x00008000, 0x00018000, 0x3F808000, 0x3F818000], dtype=np.uint32)
    allbits = np.concatenate([bits, ties, near, special])
    f = allbits.view(np.float32)
    return f[~np.isnan(f)]


def test_bf16_rne_matches_torch():
    f = _interesting_f32()
    ours = nm.f32_to_bf16_bits(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    mism = np.nonzero(ours != ref)[0]
    assert mism.size == 0, (f[mism[:5]], ours[mism[:5]], ref[mism[:5]])


def test_bf16_nan_stays_nan_and_widening_is_exact():
    nan_bits = np.array([0x7FC00000, 0xFFC00001, 0x7F800001], dtype=np.uint32).view(np.float32)
    out = nm.bf16_bits_to_f32(nm.f32_to_bf16_bits(nan_bits))
    assert np.isnan(out).all()
    b = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    w = nm.bf16_bits_to_f32(b)
    ref = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    same = (w.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(w) & np.isnan(ref))
    assert same.all()


def test_fp16_rne_matches_torch():
    f = _interesting_f32()
    ours = nm.from_f32(f, nm.DT_FP16)
    ref = torch.from_numpy(f.copy()).to(torch.float16).numpy()
    assert (ours.view(np.uint16) == ref.view(np.uint16)).all()


@pytest.mark.parametrize("dt", [nm.DT_FP16, nm.DT_BF16, nm.DT_FP32])
def test_roundtrip_of_representable_values(dt):
    rng = np.random.default_rng(1)
    x = rng.standard_normal(1000).astype(np.float32)
    stored = nm.from_f32(x, dt)
    again = nm.from_f32(nm.to_f32(stored, dt), dt)
    assert np.array_equal(np.asarray(stored).view(np.uint8), np.asarray(again).view(np.uint8))

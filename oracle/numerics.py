"""Element-type conversions used by the oracle (test infrastructure only).

The unpermute article (MoeTokenUnpermuteWithRoutingMap, section "Kernel
implementation", non-padded kernel) states that non-FP32 inputs are converted
to float for the multiply-by-prob and the add, and that the result is converted
back to the original type with round-to-nearest-even (CAST_RINT).  This module
provides those two conversions for the three floating element types the
article lists (FLOAT16, BFLOAT16, FLOAT32).

Storage conventions (identical for inputs and outputs of the oracle):

* FP16 -> ``numpy.float16`` arrays;
* BF16 -> ``numpy.uint16`` arrays holding the raw bfloat16 bit patterns
  (NumPy has no bfloat16 type);
* FP32 -> ``numpy.float32`` arrays.

Pins (tests/test_oracle_numerics.py): the bfloat16 rounding is checked against
torch's CPU ``float32 -> bfloat16`` conversion on ties, overflow, subnormals,
infinities and NaN; FP16 uses NumPy's IEEE conversion, also checked against
torch.
"""

import numpy as np

# Element-type codes.  The batching API page numbers its token types
# 0 = FP16, 1 = BF16, 2 = INT8 (+ FP32 dynamic scale); the unpermute side adds FP32.
DT_FP16 = 0
DT_BF16 = 1
DT_INT8 = 2
DT_FP32 = 3

_ELT_BYTES = {DT_FP16: 2, DT_BF16: 2, DT_INT8: 1, DT_FP32: 4}


def elt_bytes(dt):
    return _ELT_BYTES[dt]


def bf16_bits_to_f32(bits):
    """bfloat16 bit patterns (uint16) -> float32 (exact: bf16 is the top half of f32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def f32_to_bf16_bits(x):
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even.

    Written from the definition of RNE on the binary representation: the 16
    discarded low bits are compared with one half-ulp of the kept part; exact
    halves go to the neighbour whose last kept bit is 0.  Carries propagate
    into the exponent, so values past the largest bf16 round to infinity.
    NaN inputs map to a quiet NaN with the input's sign.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    hi = u >> np.uint64(16)
    lo = u & np.uint64(0xFFFF)
    half = np.uint64(0x8000)
    round_up = (lo > half) | ((lo == half) & ((hi & np.uint64(1)) == np.uint64(1)))
    out = hi + round_up.astype(np.uint64)
    is_nan = np.isnan(x)
    if is_nan.any():
        sign = (u >> np.uint64(31)) & np.uint64(1)
        out = np.where(is_nan, (sign << np.uint64(15)) | np.uint64(0x7FC0), out)
    return out.astype(np.uint16)


def to_f32(a, dt):
    """Stored element array of type ``dt`` -> float32 values (exact widening)."""
    if dt == DT_FP16:
        return np.asarray(a, dtype=np.float16).astype(np.float32)
    if dt == DT_BF16:
        return bf16_bits_to_f32(a)
    if dt == DT_FP32:
        return np.asarray(a, dtype=np.float32)
    raise ValueError(f"unsupported float type code {dt}")


def from_f32(x, dt):
    """float32 values -> stored array of type ``dt`` with one RNE rounding."""
    x = np.asarray(x, dtype=np.float32)
    if dt == DT_FP16:
        with np.errstate(over="ignore"):  # out-of-range values become +-inf
            return x.astype(np.float16)  # IEEE binary32 -> binary16, ties to even
    if dt == DT_BF16:
        return f32_to_bf16_bits(x)
    if dt == DT_FP32:
        return x.copy()
    raise ValueError(f"unsupported float type code {dt}")


def storage_dtype(dt):
    """NumPy dtype used to store elements of type ``dt`` in the oracle."""
    return {DT_FP16: np.float16, DT_BF16: np.uint16, DT_FP32: np.float32,
            DT_INT8: np.int8}[dt]

"""bfloat16 <-> float32 conversion on bit patterns (oracle; test infrastructure).

bfloat16 is the upper half of an IEEE binary32.  Conversion from float32
rounds to nearest with ties to even, the rounding the LS-docs page assumes when
it calls the store dtype bf16 ("How it works": non-quantised tensors keep the
store dtype).  NaN stays NaN (quiet).
"""
import numpy as np


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16, returned as uint16 bit patterns (RNE)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), r)
    return r


def bf16_bits_to_f32(b):
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(b):
    return bf16_bits_to_f32(b).astype(np.float64)


def round_to_bf16(x):
    """float32 -> nearest bfloat16 value, returned as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))

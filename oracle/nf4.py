"""NF4 blockwise quantization of the streamed base (oracle; test infrastructure).

What the pages fix: the frozen base is rewritten once, offline, one shard per
decoder layer, quantising to NF4 as it goes, which makes the store about four
times smaller than bf16 (LS-docs "Shard cache"; About; LS-docs "Turn it on").
The pages do not print the codebook, the block rule or the packing.  Readings
taken here (the pages leave each open):

1. Codebook: the NormalFloat-4 construction of the QLoRA paper (Dettmers et
   al., 2023): 8 positive normal quantiles and 7 negative ones, with one
   exact zero, normalised so the extremes are -1 and +1.  The quantile levels
   run from delta = ((1 - 1/30) + (1 - 1/32)) / 2 to 1/2.  Evaluated in
   float64 and rounded once to float32.
2. Blocks: 64 consecutive elements of the row-major weight [n_out, n_in]
   (n_in % 64 == 0, so a block never crosses a row); one float32 absmax per
   block (no second-level quantisation of the absmax).
3. Code: n = x / absmax rounded once to float32 (IEEE division), then the
   index of the nearest codebook value, nearest measured exactly; an exact
   tie goes to the lower index.  An all-zero block has absmax 0 and every
   code is the zero code (7).
4. Packing: byte b of a row holds element 2b in its high nibble and element
   2b+1 in its low nibble.
5. Dequantize: w = bf16(fp32(c[code] * absmax)) on the bf16 path; the float32
   product itself on the float32 path.
"""
import numpy as np
from scipy.stats import norm

from .bf16 import bf16_bits_to_f32, f32_to_bf16_bits

BLOCK = 64


def codebook():
    """The 16 NF4 levels as float32, ascending (reading 1)."""
    delta = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0))
    positive = norm.ppf(np.linspace(delta, 0.5, 9)[:-1])       # 8 levels > 0
    negative = -norm.ppf(np.linspace(delta, 0.5, 8)[:-1])      # 7 levels < 0
    levels = np.sort(np.concatenate([negative, [0.0], positive]))
    levels = levels / levels.max()
    return levels.astype(np.float32)


def _check_shape(n_out, n_in):
    if n_in % BLOCK != 0 or n_out < 0:
        raise ValueError(f"NF4 needs n_in % {BLOCK} == 0, got {n_out}x{n_in}")


def nearest_code(n):
    """float32 normalised values -> index of the nearest level (reading 3).

    |n - c_j| is exact in float64 because both are float32 numbers; argmin
    returns the first minimum, so an exact tie goes to the lower index."""
    cb = codebook().astype(np.float64)
    dist = np.abs(np.asarray(n, dtype=np.float32).astype(np.float64)[..., None] - cb)
    return np.argmin(dist, axis=-1).astype(np.uint8)


def quantize(w_bits):
    """bf16 weight bits [n_out, n_in] -> (packed uint8 [n_out, n_in/2], absmax f32 [n_out, n_in/64]).

    Raises ValueError on a non-finite input or a bad shape.
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    return _quantize_rows(w_bits, bf16_bits_to_f32)


def quantize_f32(w):
    """A float32 weight [n_out, n_in] -> (packed, absmax), by the same readings
    2-4 applied to its float32 values (a float32 holding a bf16 value gives the
    bf16 result)."""
    w = np.asarray(w, dtype=np.float32)
    return _quantize_rows(w, lambda x: x)


def _quantize_rows(w, to_f32):
    n_out, n_in = w.shape
    _check_shape(n_out, n_in)
    packed = np.empty((n_out, n_in // 2), dtype=np.uint8)
    absmax = np.empty((n_out, n_in // BLOCK), dtype=np.float32)
    rows = max(1, (1 << 20) // max(1, n_in))          # bound the [.., 16] distance tensor
    for r0 in range(0, n_out, rows):
        x = to_f32(w[r0:r0 + rows]).reshape(-1, n_in // BLOCK, BLOCK)
        if not np.isfinite(x).all():
            raise ValueError("non-finite value in NF4 quantize input")
        a = np.max(np.abs(x), axis=-1)                           # exact in float32
        n = np.zeros_like(x)
        np.divide(x, a[..., None], out=n, where=a[..., None] > 0)  # float32 IEEE division
        code = nearest_code(n).reshape(-1, n_in)
        packed[r0:r0 + rows] = (code[:, 0::2] << 4) | code[:, 1::2]
        absmax[r0:r0 + rows] = a
    return packed, absmax


def unpack_codes(packed):
    """packed uint8 [n_out, n_in/2] -> codes uint8 [n_out, n_in] (reading 4)."""
    packed = np.asarray(packed, dtype=np.uint8)
    codes = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    codes[:, 0::2] = packed >> 4
    codes[:, 1::2] = packed & 0x0F
    return codes


def dequantize_f32(packed, absmax):
    """Dequantized weight as float32: fp32(c[code] * absmax) (reading 5, float32 path)."""
    codes = unpack_codes(packed)
    n_out, n_in = codes.shape
    _check_shape(n_out, n_in)
    cb = codebook()
    vals = cb[codes].reshape(n_out, n_in // BLOCK, BLOCK)
    prod = vals * np.asarray(absmax, dtype=np.float32)[..., None]   # float32 multiply, RNE
    return prod.reshape(n_out, n_in).astype(np.float32)


def dequantize_bf16_bits(packed, absmax):
    """Dequantized weight as bf16 bit patterns: bf16(fp32(c[code] * absmax)) (reading 5)."""
    return f32_to_bf16_bits(dequantize_f32(packed, absmax))


def dequantize_bf16_f64(packed, absmax):
    """The bf16 dequantized weight widened to float64, the operand of every GEMM."""
    return bf16_bits_to_f32(dequantize_bf16_bits(packed, absmax)).astype(np.float64)

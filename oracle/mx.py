"""MXFP8 weight quantization, reference implementation. TEST INFRASTRUCTURE
ONLY: imported by the tests, the smoke check and the benchmark's CPU-baseline
leg, never by the GPU library.

What the pages fix (paper "Dory1.0-4B: A Looped Normalized-GPT", section
Quantization, Post-Training Quantization): an MXFP8 checkpoint made by
post-training quantization with standard maximum scaling, weight-only
(W8A16: activations stay 16-bit), applied to every weight matrix except the
token embeddings and the LM head; vectors and scalars stay in high precision.

Readings where the pages are silent (each applied below):
  M1  MXFP8 is the microscaling format of the OCP MX specification: blocks of
      32 consecutive elements along the reduction (input) dimension of a
      weight matrix [out, in] share one power-of-two scale (E8M0: an 8-bit
      biased exponent, value 2^(code - 127)); elements are FP8 E4M3 (1 sign,
      4 exponent bits with bias 7, 3 mantissa bits; no infinities; the only
      NaN encodings are S.1111.111; largest finite value 448; subnormals
      m * 2^-9).
  M2  "Standard maximum scaling": the block's shared exponent is
      floor(log2(max |w|)) - 8, 8 being the exponent of E4M3's largest power
      of two, so the block maximum lands in [256, 512) before rounding.
      Shared exponents are clamped to at least -126, so that every scale is a
      normal float32 (a block whose maximum is below 2^-118, all-zero blocks
      included, uses 2^-126).
  M3  Elements w / 2^shared are rounded to the nearest E4M3 value, ties to
      the even encoding, and values beyond 448 saturate to +-448 (the block
      maximum can reach 511.99 after scaling). The sign of a value that
      rounds to zero is kept (-0 is 0x80).

Dequantization is exact in bfloat16: an E4M3 value has at most 4
significant bits, and multiplying by a power of two in the float32 range
keeps it representable.
"""
import numpy as np

BLOCK = 32
E4M3_MAX = 448.0
MIN_SHARED_EXP = -126


def e4m3_value(code) -> np.ndarray:
    """float64 value of E4M3 codes (uint8 array or int); NaN for 0x7F/0xFF."""
    c = np.asarray(code, dtype=np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


# Finite non-negative codes 0x00 .. 0x7E and their values, increasing.
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = e4m3_value(_POS_CODES)
assert np.all(np.diff(_POS_VALUES) > 0)


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code of each float64 value: ties to the even code,
    saturating at 448, sign kept (reading M3)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")   # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(np.signbit(x), code | 0x80, code)
    return code.astype(np.uint8)


def shared_exponent(amax) -> np.ndarray:
    """floor(log2(amax)) - 8, clamped to >= -126 (readings M2)."""
    amax = np.asarray(amax, dtype=np.float64)
    mant, ex = np.frexp(amax)            # amax = mant * 2^ex, mant in [0.5, 1)
    fl = ex.astype(np.int64) - 1         # floor(log2(amax)) for amax > 0
    se = np.where(amax > 0, fl - 8, MIN_SHARED_EXP)
    return np.maximum(se, MIN_SHARED_EXP)


def quantize(w) -> tuple:
    """w [N, K] (K a multiple of 32) -> (codes uint8 [N, K], scale codes
    uint8 [N, K / 32]) with scale value 2^(code - 127)."""
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    assert K % BLOCK == 0
    blocks = w.reshape(N, K // BLOCK, BLOCK)
    se = shared_exponent(np.max(np.abs(blocks), axis=2))
    scaled = blocks * np.exp2(-se.astype(np.float64))[..., None]   # exact
    codes = e4m3_encode(scaled).reshape(N, K)
    return codes, (se + 127).astype(np.uint8)


def dequantize(codes, scales) -> np.ndarray:
    """float64 [N, K] = E4M3 value x 2^(scale - 127) per block."""
    codes = np.asarray(codes)
    N, K = codes.shape
    v = e4m3_value(codes).reshape(N, K // BLOCK, BLOCK)
    sc = np.exp2(np.asarray(scales, dtype=np.float64) - 127.0)
    return (v * sc[..., None]).reshape(N, K)


# Weight matrices that the quantized model stores in MXFP8 (section
# Quantization: all weight matrices but the token embeddings and LM head).
QUANTIZED = ("w_qkvg", "w_o", "w_upgate", "w_down")


def quantized_weight_fn(weight):
    """Wraps an OracleModel weight callable so that every quantized matrix is
    replaced by its MXFP8 round trip (W8A16: the forward pass then runs on
    the dequantized values)."""
    cache = {}

    def fn(name):
        if name.split(".")[-1] in QUANTIZED:
            if name not in cache:
                cache[name] = dequantize(*quantize(weight(name)))
            return cache[name]
        return weight(name)
    return fn

"""Number formats and the elementwise specification used by the oracle.

Test infrastructure only (see oracle/__init__.py). Written from the
definitions of the formats, not from any library's conversion code.

* bf16: the upper 16 bits of an IEEE binary32; rounding from any binary64 or
  binary32 value to bf16 is a single round-to-nearest-even at 8 significant
  bits, with bf16 subnormals below 2^-126 spaced 2^-133.
* e4m3: the OCP 8-bit floating point format E4M3 ("FN": no infinities, one NaN
  pattern per sign). Exponent bias 7, 3 mantissa bits, largest finite 448,
  subnormals k * 2^-9. Encoding is round-to-nearest-even; magnitudes above
  448 saturate to 448 (the quantizer never produces them, see quant.py).
* exp32 / silu32: the fp32 exponential and SiLU that every SwiGLU in this
  project evaluates, defined as a fixed sequence of IEEE binary32 operations
  (each + - * / rounded to nearest-even, no fused multiply-add):

    x   <- clamp(x, -86, 88)
    n   <- rint(x * LOG2E)                    (round half to even)
    r   <- (x - n * LN2_HI) - n * LN2_LO      (Cody & Waite argument reduction,
                                               "Software Manual for the
                                               Elementary Functions", 1980)
    p   <- 1 + r*(1 + r*(1/2 + r*(1/6 + r*(1/24 + r*(1/120 + r*(1/720 + r/5040))))))
                                              (degree-7 Taylor polynomial,
                                               coefficients rounded to fp32)
    exp32(x) <- p * 2^n                       (exact: n in [-124, 127])
    silu32(g) <- g / (1 + exp32(-g))

  The pages fix no exp; a bit-exact FP8 quantizer needs both sides to take
  the SiLU in the same arithmetic, so this sequence is the definition. Its
  accuracy against the true exp is pinned by the tests (within 2 ulp over
  every finite bf16 input in range).
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------- bf16 -----


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 patterns -> float32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)


def to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64/float32 values to bf16 (nearest-even, one rounding) -> uint16 patterns.

    The value is split as m * 2^e with 0.5 <= |m| < 1; a bf16 in that binade has
    spacing 2^(e-8), and below 2^-126 the spacing stays 2^-133 (subnormals).
    Finite inputs only.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("to_bf16: non-finite input")
    _, e = np.frexp(x)
    q = np.ldexp(1.0, np.maximum(e, -125) - 8)
    r = np.rint(x / q) * q                       # exact: x/q and the product are exact
    if np.any(np.abs(r) > 3.3895313892515355e38):
        raise ValueError("to_bf16: overflow")
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Value of x after rounding to bf16, as float64."""
    return bf16_to_f64(to_bf16(x))


# ---------------------------------------------------------------- e4m3 -----

E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 E4M3FN codes -> float64 values (0x7F/0xFF decode to NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    mant = c & 0x7
    val = np.where(ex == 0, mant * 2.0 ** -9, (1.0 + mant / 8.0) * np.ldexp(1.0, ex - 7))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """float32/float64 values -> E4M3FN codes, round-to-nearest-even, saturating to +-448.

    In the binade [2^k, 2^(k+1)), k >= -6, codes are spaced 2^(k-3); below
    2^-6 they are subnormal with spacing 2^-9. The sign bit is kept (-0 -> 0x80).
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.isnan(v)):
        raise ValueError("e4m3_encode: NaN input")
    neg = np.signbit(v)
    a = np.abs(v)
    _, e = np.frexp(a)                      # a in [2^(e-1), 2^e)
    k = np.maximum(e - 1, -6)               # binade exponent, subnormals share 2^-6's spacing
    q = np.ldexp(1.0, k - 3)
    r = np.rint(a / q) * q                  # round half to even on the code grid
    r = np.minimum(r, E4M3_MAX)
    # encode the exact grid value r
    _, er = np.frexp(r)
    kr = er - 1
    normal = r >= 2.0 ** -6
    exp_field = np.where(normal, kr + 7, 0)
    mant = np.where(normal, r / np.ldexp(1.0, np.where(normal, kr, 0)) * 8.0 - 8.0, r / 2.0 ** -9)
    code = (exp_field.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)
    code = np.where(r == 0, 0, code)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


# ------------------------------------------------------- exp32 / silu32 -----

F32 = np.float32
LOG2E = F32(1.4426950408889634)
LN2_HI = F32(0.693145751953125)          # 15 significant bits: n * LN2_HI is exact for |n| < 512
LN2_LO = F32(1.4286067653301870e-06)     # ln 2 - LN2_HI, rounded to fp32
EXP_LO = F32(-86.0)
EXP_HI = F32(88.0)
TAYLOR = [F32(1.0 / f) for f in (1.0, 1.0, 2.0, 6.0, 24.0, 120.0, 720.0, 5040.0)]


def exp32(x: np.ndarray) -> np.ndarray:
    """The project's fp32 exponential (see module docstring); float32 in, float32 out."""
    x = np.asarray(x, dtype=F32)
    x = np.minimum(np.maximum(x, EXP_LO), EXP_HI)
    n = np.rint(x * LOG2E)
    r = (x - n * LN2_HI) - n * LN2_LO
    p = TAYLOR[7]
    for c in TAYLOR[6::-1]:
        p = c + r * p
    p = p.astype(F32)
    two_n = np.ldexp(F32(1.0), n.astype(np.int32)).astype(F32)
    return (p * two_n).astype(F32)


def silu32(g: np.ndarray) -> np.ndarray:
    """g / (1 + exp32(-g)), every step in fp32."""
    g = np.asarray(g, dtype=F32)
    d = (F32(1.0) + exp32(-g)).astype(F32)
    return (g / d).astype(F32)

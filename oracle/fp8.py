"""E4M3 / UE8M0 / bf16 codecs (CPU oracle; test infrastructure only).

The pages name the element format only as OCP FP8 and the MX scale only as
"OCP UE8M0" (Fish Audio X post, section "Custom kernels for the shapes TTS
actually uses"; fish.audio blog, section "Estrategia de cuantización FP8").
The bit-level definitions below follow the public OCP OFP8 specification
(E4M3: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no infinities;
S.1111.111 is NaN) and the OCP MX v1.0 specification (E8M0: an unsigned
8-bit biased exponent, value 2**(E-127), 0xFF is NaN).

Readings where the pages are silent (each listed in the design notes):

* Conversion to E4M3 is round-to-nearest, ties to the even code, with one
  rounding from the exact input value, and SATURATES: magnitudes at or above
  448 (and infinities) become +-448 instead of NaN.
* The sign of zero is kept: negative values that round to zero give 0x80.
* NaN input gives 0x7F with its sign bit.

All arithmetic here is float64 (every fp32 / bf16 value is exact in it).
"""

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN_POS = 0x7F


def e4m3_decode_table():
    """Value of each of the 256 E4M3 codes as float64 (NaN for S.1111.111).

    Built from the bit fields: exponent field e (bias 7) and mantissa m.
    e == 0 is subnormal: (-1)^s * 2^-6 * m/8; otherwise
    (-1)^s * 2^(e-7) * (1 + m/8).
    """
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if (c >> 7) & 1 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = s * (2.0 ** -6) * (m / 8.0)
        else:
            vals[c] = s * (2.0 ** (e - 7)) * (1.0 + m / 8.0)
    return vals


_TABLE = e4m3_decode_table()


def e4m3_decode(codes):
    """Decode uint8 codes to float64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v):
    """Encode real values (float64 array of any shape) to E4M3 codes; large
    arrays are processed in pieces to bound memory.  See _e4m3_encode_flat."""
    v = np.asarray(v, dtype=np.float64)
    flat = v.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    step = 1 << 13
    for i in range(0, flat.size, step):
        out[i:i + step] = _e4m3_encode_flat(flat[i:i + step])
    return out.reshape(v.shape)


def _e4m3_encode_flat(v):
    """Encode real values (given exactly, e.g. fp32 values held in float64)
    to E4M3 codes with a single round-to-nearest-even, saturating at 448.

    Method: the representable magnitudes in the binade [2^e, 2^(e+1)) for
    e >= -6 are spaced 2^(e-3); below 2^-6 the subnormals continue the grid
    of 2^-9.  So |v| is divided (exactly, by a power of two) by the local
    spacing q, rounded to the nearest integer n with ties to even (np.rint),
    and n is turned back into exponent and mantissa fields.  n is even
    exactly when the mantissa field is even, so ties go to the even code.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    sign = np.signbit(v).astype(np.uint8) << 7
    nan = np.isnan(v)
    sat = (a >= E4M3_MAX) & ~nan  # includes +-inf
    finite = ~(nan | sat)
    af = np.where(finite, a, 1.0)
    # frexp: af = f * 2**E with f in [0.5, 1)  =>  floor(log2(af)) = E - 1
    _, E = np.frexp(af)
    e = np.maximum(E.astype(np.int64) - 1, -6)
    e = np.where(af == 0.0, -6, e)
    n = np.rint(np.ldexp(af, (3 - e).astype(np.int32)))  # af / 2^(e-3), exact
    n = n.astype(np.int64)
    # n in [8, 16] for the normal branch; [0, 8] when e == -6 and af < 2^-6
    carry = n == 16
    exp_field = np.where(n >= 8, e + 7 + carry, 0)
    man_field = np.where(n >= 8, np.where(carry, 0, n - 8), n)
    code = ((exp_field << 3) | man_field).astype(np.uint8)
    code = np.where(sat, np.uint8(0x7E), code)
    code = np.where(nan, np.uint8(E4M3_NAN_POS), code)
    return (code | sign).astype(np.uint8)


# --------------------------------------------------------------------------
# UE8M0 (OCP MX v1.0 shared scale)
# --------------------------------------------------------------------------

def ue8m0_decode(e):
    """Value 2^(E-127) of an E8M0 byte (0xFF is NaN)."""
    e = np.asarray(e, dtype=np.int64)
    out = np.ldexp(1.0, (e - 127).astype(np.int32))
    return np.where(e == 0xFF, np.nan, out)


def floor_log2(a):
    """floor(log2(a)) for finite a > 0, exactly, from the binary exponent
    (np.frexp also handles subnormals); never through a floating log."""
    _, E = np.frexp(np.asarray(a, dtype=np.float64))
    return E.astype(np.int64) - 1


# --------------------------------------------------------------------------
# bf16
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def to_bf16(v):
    """Round float64 values to the bf16 grid, nearest with ties to even, from
    the exact value (a single rounding).  Returns float64 values on the grid.

    bf16 has 8 significant bits and the fp32 exponent range: in the binade
    [2^e, 2^(e+1)) the spacing is 2^(e-7) for e >= -126; below 2^-126 the
    subnormal spacing 2^-133 continues.  Magnitudes that round past the
    largest finite value (2^128 - 2^120) become infinity.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    fin = np.isfinite(a) & (a > 0)
    af = np.where(fin, a, 1.0)
    _, E = np.frexp(af)
    e = np.maximum(E.astype(np.int64) - 1, -126)
    n = np.rint(np.ldexp(af, (7 - e).astype(np.int32)))
    r = np.ldexp(n, (e - 7).astype(np.int32))
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    r = np.where(fin, r, a)
    return np.copysign(r, v)


def f64_to_bf16_bits(v):
    """RNE-round float64 values to bf16 and return the uint16 bit patterns."""
    r = to_bf16(v).astype(np.float32)  # exact: r is on the bf16 grid
    return (r.view(np.uint32) >> 16).astype(np.uint16)

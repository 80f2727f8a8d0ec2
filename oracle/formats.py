"""Number formats used by the layer step, decoded from their bit fields in fp64.

Test infrastructure: see the package docstring for who may import this.
"""

import numpy as np


def bf16_round(x):
    """Round fp64 values to the nearest bfloat16 value (ties to even), returned as fp64.

    bfloat16 keeps 8 significant bits and fp32's exponent range.  The cache stores K/V
    in this type ([RT] ``unsupported``: KV cache dtypes other than BF16 are refused) and
    the draft head produces its logits in it ([RT] ``unsupported``: BF16 head dtype).
    The rounding is done directly from fp64 (no intermediate fp32 step).
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    finite = np.isfinite(x) & (x != 0)
    v = x[finite]
    _, e = np.frexp(np.abs(v))          # |v| = m * 2**e with m in [0.5, 1)
    e = np.maximum(e, -125)             # below 2**-126 the quantum stays 2**-133
    quantum = np.ldexp(1.0, e - 8)      # 8 significant bits
    r = np.rint(v / quantum) * quantum  # np.rint rounds half to even
    r[np.abs(r) >= np.ldexp(1.0, 128)] = np.inf * np.sign(r[np.abs(r) >= np.ldexp(1.0, 128)])
    out[finite] = r
    return out


def e2m1_decode(nibbles):
    """Value of 4-bit E2M1 codes [OCP, FP4 E2M1]: 1 sign, 2 exponent (bias 1), 1 mantissa.

    exponent field 0 is subnormal: 0.5 * m; otherwise 2**(e-1) * (1 + m/2).
    Magnitudes: 0, 0.5, 1, 1.5, 2, 3, 4, 6.
    """
    c = np.asarray(nibbles).astype(np.int64) & 0xF
    s = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, (e - 1)))
    return s * mag


def e4m3_decode(codes):
    """Value of 8-bit E4M3FN codes [OCP, FP8 E4M3]: 1 sign, 4 exponent (bias 7), 3 mantissa.

    exponent field 0 is subnormal: 2**-6 * m/8; otherwise 2**(e-7) * (1 + m/8).
    There is no infinity; 0x7F and 0xFF are NaN.  Largest finite magnitude 448.
    """
    c = np.asarray(codes).astype(np.int64) & 0xFF
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 0xF) & (m == 7), np.nan, mag)
    return s * mag


def unpack_nibbles(packed):
    """Split packed E2M1 bytes [..., K/2] into codes [..., K]: the low nibble is the
    even element, the high nibble the odd one (a layout reading; the pages do not
    print the packing)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def dequant_nvfp4(packed_codes, scale_codes, gscale):
    """Block-scaled FP4 weight matrix [N, K] in fp64.

    W[n, k] = e2m1(code[n, k]) * e4m3(scale[n, k // 16]) * gscale.  The routed experts
    run on FP4 weights ([RT] module list: expert_tp for the routed NVFP4 experts;
    [DEC] module docstring: the NVFP4 layers' experts); one E4M3 scale per 16
    consecutive weights along the reduction dimension and one fp32 scale per matrix
    is this implementation's reading of that format.
    """
    codes = unpack_nibbles(packed_codes)
    n, k = codes.shape
    sc = np.asarray(scale_codes)
    assert sc.shape == (n, k // 16), (sc.shape, n, k)
    w = e2m1_decode(codes) * np.repeat(e4m3_decode(sc), 16, axis=1)
    return w * float(gscale)

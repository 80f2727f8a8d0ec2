"""Pins of the oracle's number formats against published tables and library decoders."""

import os

import numpy as np
import torch

from oracle import formats

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _table(name):
    rows = []
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(line.split())
    return rows


def test_e2m1_matches_ocp_table():
    for code, value in _table("e2m1_table.txt"):
        got = formats.e2m1_decode(int(code, 2))
        assert got == float(value) and np.signbit(got) == value.startswith("-"), (code, got)


def test_e2m1_embeds_in_e4m3_via_torch():
    # An E2M1 value with exponent field e > 0 and mantissa m is the E4M3 value with exponent
    # field e - 1 + 7 and mantissa m << 2; e = 0, m = 1 (0.5) is E4M3 exponent 6.  torch's
    # float8_e4m3fn decoder is the library reference.
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        if e == 0 and m == 0:
            continue
        if e == 0:
            code = (s << 7) | (6 << 3)
        else:
            code = (s << 7) | ((e - 1 + 7) << 3) | (m << 2)
        ref = torch.tensor([code], dtype=torch.uint8).view(torch.float8_e4m3fn).float().item()
        assert formats.e2m1_decode(c) == ref


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = formats.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_e4m3_specials_table():
    for code, value in _table("e4m3_specials.txt"):
        got = formats.e4m3_decode(int(code, 16))
        if value == "nan":
            assert np.isnan(got)
        else:
            assert got == float(value), (code, got)


def test_bf16_round_matches_torch_on_fp32_values():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.float32([0.0, -0.0, 1.0, 3.0e38, 1e-40, -7e-39])]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    got = formats.bf16_round(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_round_ties_to_even_and_no_double_rounding():
    one = 1.0
    assert formats.bf16_round(one + 2.0 ** -8) == 1.0                    # tie -> even (1.0)
    assert formats.bf16_round(one + 3 * 2.0 ** -8) == one + 2.0 ** -6    # tie -> even
    # just above the tie: direct fp64 rounding goes up; fp64 -> fp32 -> bf16 would not
    assert formats.bf16_round(one + 2.0 ** -8 + 2.0 ** -30) == one + 2.0 ** -7
    assert formats.bf16_round(-(one + 2.0 ** -8 + 2.0 ** -30)) == -(one + 2.0 ** -7)


def test_unpack_low_nibble_first():
    codes = formats.unpack_nibbles(np.array([[0x71, 0x0F]], dtype=np.uint8))
    assert codes.tolist() == [[1, 7, 15, 0]]


def test_dequant_block_scales_and_gscale():
    rng = np.random.default_rng(2)
    n, k = 3, 64
    packed = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7E, (n, k // 16), dtype=np.uint8)
    w = formats.dequant_nvfp4(packed, scales, 2.0)
    # element-by-element from the bit fields: nibble order, block index k // 16, gscale
    for i in range(n):
        for j in range(k):
            byte = packed[i, j // 2]
            code = (byte & 0xF) if j % 2 == 0 else (byte >> 4)
            want = formats.e2m1_decode(code) * formats.e4m3_decode(scales[i, j // 16]) * 2.0
            assert w[i, j] == want
    # a block of code 2 (value 1.0) exposes the scale itself
    ones = np.full((1, 16 // 2), 0x22, dtype=np.uint8)
    sc = np.array([[0x38]], dtype=np.uint8)        # E4M3 1.0
    assert np.all(formats.dequant_nvfp4(ones, sc, 1.0) == 1.0)


def test_dequant_products_exact_in_bf16():
    # E2M1 (<= 2 significant bits) x E4M3 (<= 4) has <= 6 significant bits, so every
    # product with gscale 1 is a bf16 value: rounding to bf16 changes nothing.
    v2 = formats.e2m1_decode(np.arange(16))
    v8 = formats.e4m3_decode(np.arange(256))
    v8 = v8[np.isfinite(v8)]
    prod = (v2[:, None] * v8[None, :]).ravel()
    assert np.array_equal(formats.bf16_round(prod), prod)

"""Pins of the oracle's number formats (E4M3FN encode/decode, bf16 rounding).

The oracle's encoder is checked against: hand-worked codes (golden file), an exhaustive
nearest-value search, and torch's independent float8_e4m3fn / bfloat16 casts.
"""
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_hand_cases.txt")


def _parse_value(s: str) -> float:
    s = s.strip()
    neg = s.startswith("-")
    if neg:
        s = s[1:]
    if "*" in s:
        a, b = s.split("*")
        v = float(a) * 2.0 ** int(b.split("^")[1])
    elif s.startswith("2^"):
        v = 2.0 ** int(s[2:])
    else:
        v = float(s)
    return -v if neg else v


def _golden_cases():
    out = []
    with open(GOLDEN) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            parts = line.split()
            out.append((_parse_value(parts[0]), int(parts[1], 16), parts[0]))
    return out


@pytest.mark.parametrize("value,code,text", _golden_cases())
def test_e4m3_hand_cases(orc, value, code, text):
    got = orc.e4m3_encode(value)
    assert got == code, f"{text}: got {got:#04x}, want {code:#04x}"


def test_e4m3_decode_matches_torch(orc):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = orc.e4m3_decode_table()
    for c in range(256):
        if c in (0x7F, 0xFF):
            assert math.isnan(mine[c]) and math.isnan(ref[c])
        else:
            assert mine[c] == ref[c], hex(c)


def _interesting_values(g, n):
    # every code value, every midpoint between neighbouring codes, their float32 neighbours,
    # plus random magnitudes spanning the subnormal..saturation range
    codes = torch.arange(0x7F, dtype=torch.int32).to(torch.uint8)
    table = np.unique(codes.view(torch.float8_e4m3fn).to(torch.float64).numpy())
    mids = (table[1:] + table[:-1]) / 2.0
    base = np.concatenate([table, mids]).astype(np.float32)
    up = np.nextafter(base, np.float32(np.inf))
    dn = np.nextafter(base, np.float32(-np.inf))
    rnd = (np.exp2(g.uniform(-12, 9, n)) * g.uniform(1, 2, n)).astype(np.float32)
    vals = np.concatenate([base, up, dn, rnd])
    vals = vals[np.abs(vals) <= 464.0]
    return np.concatenate([vals, -vals]).astype(np.float32)


def test_e4m3_encode_matches_torch_cast(orc):
    # torch's cast rounds to nearest even and saturates up to 464 (it returns NaN above),
    # so it is an independent check for |y| <= 464.
    vals = _interesting_values(np.random.default_rng(1), 20000)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = orc.e4m3_encode_array(vals)
    bad = np.nonzero(mine != ref)[0]
    assert bad.size == 0, [(float(vals[i]), hex(mine[i]), hex(ref[i])) for i in bad[:5]]


def test_e4m3_encode_matches_bruteforce(orc):
    vals = _interesting_values(np.random.default_rng(2), 3000)
    extra = np.array([448.0, 449.0, 1e6, -1e30, 0.0, -0.0, 1e-30, -1e-30], np.float32)
    for v in np.concatenate([vals, extra]):
        assert orc.e4m3_encode(float(v)) == orc.e4m3_encode_bruteforce(float(v)), float(v)


def test_e4m3_saturates_instead_of_nan(orc):
    for v in (448.0, 450.0, 464.0, 465.0, 1e10, float("inf")):
        assert orc.e4m3_encode(v) == 0x7E
        assert orc.e4m3_encode(-v) == 0xFE


def test_bf16_rounding_matches_torch_for_fp32_inputs(orc):
    g = np.random.default_rng(3)
    f = (g.standard_normal(5000) * np.exp2(g.uniform(-30, 30, 5000))).astype(np.float32)
    # exact ties: bf16 keeps 8 significant bits, so set bit 15 alone below the cut
    ties = ((f.view(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    vals = np.concatenate([f, ties, np.float32([1.0, -1.0, 0.0, -0.0, 3e38, -3e38])])
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for v, r in zip(vals, ref):
        assert orc.bf16_from_double(float(v)) == int(r), float(v)


def test_bf16_rounding_from_double_is_single_rounding(orc):
    # 1 + 2^-8 is a tie between 1.0 and 1 + 2^-7; a hair above it must round up.  Going via
    # float32 first would land exactly on the tie and round down (double rounding).
    assert orc.bf16_from_double(1.0 + 2.0 ** -8) == 0x3F80
    assert orc.bf16_from_double(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    assert orc.bf16_from_double(1.0 + 3 * 2.0 ** -8) == 0x3F82
    assert orc.bf16_from_double(-(1.0 + 2.0 ** -8 + 2.0 ** -40)) == 0xBF81
    assert orc.bf16_from_double(2.0 ** 128) == 0x7F80
    assert orc.bf16_value(0x3F81) == 1.0 + 2.0 ** -7

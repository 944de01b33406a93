"""Pins of the oracle's scalar formats against definitions outside the oracle.

* E2M1 and E4M3 values are re-derived here from their bit layouts (sign,
  exponent, mantissa, bias) -- the format definitions, not the oracle's code.
* E4M3 rounding is checked against torch's float8_e4m3fn CPU cast (a library
  routine: round-to-nearest-even with subnormals).
* E2M1 rounding is checked against a brute-force nearest-value search with the
  half-to-even rule stated on mantissa bits.
* The E4M3 saturation limit 448 is the value "Building Custom TensorRT-LLM
  Plugins for Low-Latency FP8 Inference at Scale" gives for E4M3 ("Fusing the
  Kernel in CUDA" and "Production Pitfalls" 2); see tests/golden/formats.txt.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "formats.txt")


def _golden():
    vals = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    return vals


def e2m1_from_bits(n):
    """E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent 0 is subnormal."""
    s = -1.0 if n & 8 else 1.0
    e = (n >> 1) & 3
    m = n & 1
    if e == 0:
        return s * m * 0.5
    return s * (1 + m / 2) * 2.0 ** (e - 1)


def e4m3_from_bits(b):
    """E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa; S.1111.111 is NaN, no inf."""
    s = -1.0 if b & 0x80 else 1.0
    e = (b >> 3) & 15
    m = b & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return s * (m / 8) * 2.0 ** -6
    return s * (1 + m / 8) * 2.0 ** (e - 7)


def test_e2m1_decode_matches_bit_definition_and_grid(oracle):
    g = _golden()
    grid = sorted(float(v) for v in g["e2m1_magnitudes"].split(","))
    mags = sorted({abs(e2m1_from_bits(n)) for n in range(16)})
    assert mags == grid
    for n in range(16):
        want = e2m1_from_bits(n)
        got = oracle.e2m1_decode(n)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), n


def test_e4m3_decode_exhaustive(oracle):
    tq = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        want = e4m3_from_bits(b)
        got = oracle.e4m3_decode(b)
        if math.isnan(want):
            assert math.isnan(got) and math.isnan(tq[b])
        else:
            assert got == want == tq[b], b


def test_e4m3_max_is_448(oracle):
    g = _golden()
    assert oracle.e4m3_decode(0x7E) == float(g["e4m3_max"]) == 448.0
    assert oracle.e4m3_encode(448.0) == 0x7E


def _e4m3_sweep():
    pos = [e4m3_from_bits(b) for b in range(0x7F)]
    xs = set()
    for i, v in enumerate(pos):
        xs.add(v)
        if i + 1 < len(pos):
            mid = (v + pos[i + 1]) / 2
            for t in (mid, np.nextafter(np.float32(mid), np.float32(0)),
                      np.nextafter(np.float32(mid), np.float32(1e9))):
                xs.add(float(np.float32(t)))
    rng = np.random.default_rng(123)
    xs.update(float(v) for v in (rng.random(20000) * 448).astype(np.float32))
    xs.update(float(v) for v in np.exp(rng.uniform(-25, 6, 20000)).astype(np.float32))
    return sorted(v for v in xs if 0 <= v <= 448)


def test_e4m3_encode_matches_torch_cast(oracle):
    xs = np.array(_e4m3_sweep(), np.float32)
    tb = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(x)) for x in xs], np.uint8)
    bad = np.nonzero(got != tb)[0]
    assert bad.size == 0, [(float(xs[i]), int(got[i]), int(tb[i])) for i in bad[:5]]


def test_e4m3_encode_saturates_and_round_trips(oracle):
    for x in [448.0, 449.0, 463.9, 464.0, 480.0, 1e6, 3.4e38, float("inf")]:
        assert oracle.e4m3_encode(x) == 0x7E
    for b in range(0x7F):  # every finite non-negative code encodes to itself
        assert oracle.e4m3_encode(e4m3_from_bits(b)) == b
    assert oracle.e4m3_encode(0.0) == 0 and oracle.e4m3_encode(-0.0) == 0
    # below half the smallest subnormal rounds to 0; exactly half ties to even (0)
    assert oracle.e4m3_encode(2.0 ** -10) == 0
    assert oracle.e4m3_encode(1.5 * 2.0 ** -10) == 1


def brute_e2m1(v):
    """Nearest of the 8 magnitudes; on a tie the code whose mantissa bit is 0."""
    sign = 8 if math.copysign(1.0, v) < 0 else 0
    m = Fraction(abs(v))                     # exact distances, no absorption
    cands = []
    for n in range(8):
        cands.append((abs(m - Fraction(e2m1_from_bits(n))), n & 1, n))
    cands.sort()
    return sign | cands[0][2]


def test_e2m1_encode_brute_force_sweep(oracle):
    pts = [0.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.5, 1, 1.5, 2, 3, 4]
    xs = set()
    for p in pts:
        f = np.float32(p)
        xs.update([float(f), float(np.nextafter(f, np.float32(0))), float(np.nextafter(f, np.float32(10)))])
    rng = np.random.default_rng(7)
    xs.update(float(v) for v in (rng.random(30000) * 7).astype(np.float32))
    xs.update([1e-30, 1e-45, 7.0, 100.0, 3.4e38])
    for x in sorted(xs):
        for s in (1.0, -1.0):
            v = s * x
            assert oracle.e2m1_encode(v) == brute_e2m1(v), v
    assert oracle.e2m1_encode(float("inf")) == 7
    assert oracle.e2m1_encode(-0.0) == 8


def test_input_decoding_matches_torch(oracle):
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 1 << 16, 4000, dtype=np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]          # finite bf16 only
    bf = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    for b, want in zip(bits, bf):
        assert oracle.lib().oracle_input_to_float(int(b), 0) == want
    bits = rng.integers(0, 1 << 16, 4000, dtype=np.uint16)
    bits = bits[((bits >> 10) & 0x1F) != 0x1F]
    hf = torch.from_numpy(bits.view(np.int16)).view(torch.float16).float().numpy()
    for b, want in zip(bits, hf):
        assert oracle.lib().oracle_input_to_float(int(b), 1) == want

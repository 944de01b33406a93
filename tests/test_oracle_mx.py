"""Pins of the MXFP4 oracle (E8M0 block scales over 32 elements) that do not
come from the oracle itself.

The variant is the UE8M0_SF switch of the block helper in "perf: optimize
per-token nvfp4 quantization kernel" (review); the readings (32-element blocks,
the scale rounded up to a power of two, the NVFP4 global scale kept) are listed
at the top of oracle/nvfp4_oracle.c.  Pins:

* E8M0 decode and round-up encode against the closed form from frexp;
* hand-worked blocks and a hand-worked per-token row (tests/golden/mx_worked_example.txt);
* invariants: no element saturates, the block maximum lands in [3, 6], the
  per-element error bound of the E2M1 grid, on-grid round trip when every
  scale is a power of two, sign equivariance;
* the fp64 MX GEMM reference against a scalar triple loop that decodes every
  nibble and scale byte from the format definitions;
* the tile layout: reshape version against the element-by-element loops and
  hand-computed positions.
"""
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mx_worked_example.txt")
GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _golden():
    d = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split("=", 1)
            d[k.strip()] = [t.strip() for t in v.split(",")]
    return d


def ceil_log2_byte(x: float) -> int:
    """Closed form: 127 + ceil(log2 x) from frexp, clamped to the finite E8M0 codes."""
    if not (x <= 2.0 ** 127):
        return 254
    if x <= 2.0 ** -127:
        return 0
    m, e = math.frexp(x)          # x = m * 2^e, m in [0.5, 1)
    c = e - 1 if m == 0.5 else e
    return max(0, min(254, c + 127))


def test_e8m0_decode(oracle):
    for b in range(255):
        assert oracle.e8m0_decode(b) == math.ldexp(1.0, b - 127)
    assert math.isnan(oracle.e8m0_decode(255))


def test_e8m0_encode_up_closed_form(oracle):
    rng = np.random.default_rng(7)
    xs = [0.0, 1.0, 2.0, 0.75, 448.0, 2.0 ** -127, 2.0 ** -126, 2.0 ** 127, 3e38,
          float(np.float32(2.0 ** -127) * np.float32(1.5)), 1e-45, float("inf"), float("nan")]
    xs += [float(np.float32(v)) for v in np.exp(rng.uniform(-87, 87, 2000))]
    xs += [float(np.nextafter(np.float32(2.0 ** e), np.float32(np.inf))) for e in range(-120, 120, 7)]
    xs += [float(np.nextafter(np.float32(2.0 ** e), np.float32(0))) for e in range(-120, 120, 7)]
    for x in xs:
        b = oracle.e8m0_encode_up(x)
        assert b == ceil_log2_byte(x), x
        if 0 < b < 254 and not math.isnan(x):
            assert math.ldexp(1.0, b - 127) >= x > math.ldexp(1.0, b - 128)


def _nib(codes, i):
    return (codes[i // 2] >> (4 * (i % 2))) & 15


@pytest.mark.parametrize("name", ["A", "B", "C", "D", "E1", "E2"])
def test_hand_worked_blocks(oracle, name):
    g = _golden()
    y = np.zeros(32, np.float32)
    vals = [float(v) for v in g[name + ".y"]]
    y[:len(vals)] = vals
    ge, gd = (float(v) for v in g[name + ".g"])
    sf, c, codes = oracle.mx_quantize_block(y, ge, gd)
    want = [int(v, 16) for v in g[name + ".codes"]]
    assert sf == int(g[name + ".sf"][0], 16)
    assert codes.tolist() == want + [0] * (16 - len(want))
    if name == "D":
        assert c == 0.0


def test_hand_worked_row(oracle):
    g = _golden()
    row = np.zeros(64, np.float32)
    b0 = [float(v) for v in g["row.b0"]]
    b1 = [float(v) for v in g["row.b1"]]
    row[:len(b0)] = b0
    row[32:32 + len(b1)] = b1
    q = oracle.mx_quantize(torch.from_numpy(row[None]).to(torch.bfloat16))
    assert q["g_dec"][0] == np.float32(2.0 ** -9)
    assert q["sf"][0].tolist() == [int(v, 16) for v in g["row.sf"]]
    c0 = [int(v, 16) for v in g["row.codes_b0"]]
    c1 = [int(v, 16) for v in g["row.codes_b1"]]
    assert q["codes"][0].tolist() == c0 + [0] * (16 - len(c0)) + c1 + [0] * (16 - len(c1))


def _deq(codes, n=32):
    return np.array([(-1 if _nib(codes, i) & 8 else 1) * GRID[_nib(codes, i) & 7] for i in range(n)])


def test_block_invariants(oracle):
    """No saturation, block max coded in [3, 6], error within half a grid step."""
    rng = np.random.default_rng(11)
    for t in range(400):
        y = (rng.standard_normal(32) * np.exp(rng.uniform(-8, 8))).astype(np.float32)
        amax = float(np.max(np.abs(y)))
        ge, gd = oracle.global_scale(amax * float(np.exp(rng.uniform(0, 3))))
        sf, c, codes = oracle.mx_quantize_block(y, ge, gd)
        assert c > 0
        v = y.astype(np.float64) / c
        assert np.max(np.abs(v)) <= 6.0 * (1 + 2 ** -20)           # nothing clipped
        q = _deq(codes)
        assert 3.0 <= np.max(np.abs(q)) <= 6.0                    # scale is the smallest power of two
        step = np.where(np.abs(v) < 2, 0.5, np.where(np.abs(v) < 4, 1.0, 2.0))
        assert np.all(np.abs(q - v) <= step / 2 + 1e-6 * np.abs(v))
        # sign equivariance
        sf2, c2, codes2 = oracle.mx_quantize_block(-y, ge, gd)
        assert sf2 == sf and c2 == c
        assert all((_nib(codes2, i) ^ 8) == _nib(codes, i) for i in range(32))


def test_on_grid_round_trip(oracle):
    """Group amax 2688 * 2^m makes g_enc = 2^-m and g_dec powers of two; a block
    whose maximum is 6 * 2^t then has the power-of-two scale 2^(t-m), so on-grid
    values (grid * 2^t) return exactly.  Block 0 holds only the row maximum,
    which lands on v = 2688/512 = 5.25 and is coded 6."""
    rng = np.random.default_rng(3)
    k = 256
    rows = []
    for r in range(6):
        m = int(rng.integers(-6, 6))
        x = np.zeros(k, np.float64)
        x[0] = 2688 * 2.0 ** m
        for b in range(1, k // 32):
            s = int(rng.integers(-8, 0))            # block max 3072 * 2^(s+m) < 2688 * 2^m
            q = rng.choice(GRID, 32) * rng.choice([-1, 1], 32)
            q[rng.integers(0, 32)] = 6.0
            x[32 * b:32 * b + 32] = q * 2.0 ** (s + m) * 512
        rows.append(x)
    X = torch.tensor(np.array(rows), dtype=torch.float32).to(torch.bfloat16)
    assert torch.equal(X.float().double(), torch.tensor(np.array(rows)))   # exact in bf16
    q = oracle.mx_quantize(X)
    deq = oracle.dequant_mx(q["codes"], q["sf"], q["g_dec"])
    want = np.array(rows)
    assert np.array_equal(deq[:, 32:], want[:, 32:])
    assert np.array_equal(deq[:, 0], want[:, 0] / 2688 * 3072)
    assert not deq[:, 1:32].any()


def test_zero_block_inside_a_row_keeps_signed_zero_codes(oracle):
    """An all-zero block (alternating -0 / +0) next to a block with maximum 3:
    g_dec = 3/2688, the zero block's scale is the smallest E8M0 value (byte 0,
    2^-127), its combined scale 2^-127 * 3/2688 is a binary32 subnormal, so the
    encode factor 1/c overflows to +inf -- and every zero element must still get
    the zero code with its own sign (reading of the NVFP4 zero rule, kept for MX),
    not the code of 0 * inf."""
    x = np.zeros((1, 64), np.float32)
    x[0, 0:32:4] = -0.0            # -0 and +0 in both nibble positions of the bytes
    x[0, 3:32:4] = -0.0
    x[0, 32:] = np.linspace(-3.0, 3.0, 32)
    xt = torch.from_numpy(x).to(torch.bfloat16)
    assert xt[0, 0].item() == 0.0 and math.copysign(1.0, xt[0, 0].item()) < 0
    q = oracle.mx_quantize(xt)
    assert q["sf"][0, 0] == 0
    c0 = np.float32(oracle.e8m0_decode(0)) * np.float32(q["g_dec"][0])
    assert 0.0 < c0 < np.finfo(np.float32).tiny
    with np.errstate(over="ignore"):
        assert np.isinf(np.float32(1.0) / c0)
    want = np.where(np.signbit(x[0, :32]), 8, 0).astype(np.uint8)
    codes = q["codes"][0, :16]
    assert np.array_equal(codes & 0xF, want[0::2]) and np.array_equal(codes >> 4, want[1::2])


def test_group_scale_per_tensor_equals_per_row_when_maxima_match(oracle):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 128)).astype(np.float32)
    x[:, 0] = 3.0
    X = torch.from_numpy(x).to(torch.bfloat16)
    a = oracle.mx_quantize(X, group_rows=1)
    b = oracle.mx_quantize(X, group_rows=4)
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["sf"], b["sf"])
    assert np.all(a["g_dec"] == b["g_dec"][0])


def test_mx_gemm_ref_against_scalar_loops(oracle):
    rng = np.random.default_rng(9)
    B, N, K = 3, 5, 64
    ac = rng.integers(0, 256, (B, K // 2), dtype=np.uint8)
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    asf = rng.integers(120, 135, (B, K // 32), dtype=np.uint8)
    wsf = rng.integers(120, 135, (N, K // 32), dtype=np.uint8)
    ag = rng.uniform(0.5, 2, B).astype(np.float32)
    wg = np.float32(0.375)
    y = oracle.mx_gemm_ref(ac, asf, ag, wc, wsf, wg)

    def val(codes, sf, g, r, k):
        n = (int(codes[r, k // 2]) >> (4 * (k % 2))) & 15
        mag = GRID[n & 7] * (-1 if n & 8 else 1)
        return mag * 2.0 ** (int(sf[r, k // 32]) - 127) * float(g)

    for b in range(B):
        for n in range(N):
            s = sum(val(ac, asf, ag[b], b, k) * val(wc, wsf, wg, n, k) for k in range(K))
            assert y[b, n] == pytest.approx(s, rel=1e-12, abs=1e-300)


def test_mx_tile_layout(oracle):
    rng = np.random.default_rng(1)
    for R, K in [(32, 128), (45, 256), (64, 384)]:
        codes = rng.integers(0, 256, (R, K // 2), dtype=np.uint8)
        sf = rng.integers(0, 255, (R, K // 32), dtype=np.uint8)
        ct, st = oracle.mx_tile(codes, sf)
        lt, ls = oracle.mx_tile_loops(codes, sf)
        assert np.array_equal(ct, lt) and np.array_equal(st, ls)
        G = (R + 31) // 32
        assert ct.size == G * 32 * K // 2 and st.size == G * 32 * K // 32
        # hand-computed positions: row 33 (G 1, r 1), k 64..95 (c 1, h 0) and
        # k 96..127 (h 1); block 5 of row 33 = chunk 1, j 0, h 1
        if R >= 34:
            nch = K // 64
            t = (1 * nch + 1) * 64 + 1
            assert ct[16 * t:16 * t + 16].tolist() == codes[33, 32:48].tolist()
            t = (1 * nch + 1) * 64 + 33
            assert ct[16 * t:16 * t + 16].tolist() == codes[33, 48:64].tolist()
            t = (1 * (K // 128) + 1) * 64 + 33
            assert st[2 * t] == sf[33, 5] and st[2 * t + 1] == sf[33, 7]
        # padding rows are zero
        if R % 32:
            pad = ct.reshape(G, K // 64, 2, 32, 16)[G - 1, :, :, R % 32:]
            assert not pad.any()

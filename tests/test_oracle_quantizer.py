"""Pins of the oracle quantizer that do not come from the oracle itself.

* a hand-worked example (tests/golden/quant_worked_example.txt);
* a closed-form round trip: with a row maximum of 2688*2^m every scale in the
  chain is a power of two, so on-grid inputs must return their exact codes,
  scale bytes and scales;
* invariants any correct implementation of the two-level scheme satisfies:
  block-max element at +-6, E4M3 448 for the block holding the row maximum,
  the per-element error bound, scale and sign equivariance, per-tensor and
  per-row agreement when every row has the same maximum, zero rows.

The scheme: 16-element blocks with an FP8-E4M3 scale and an FP32 global scale
("Fused Nvfp4 GEMM All Reduce Plugin", Baked-weight inputs), a per-token global
for activations ("perf: optimize per-token nvfp4 quantization kernel",
description), E4M3 saturation at 448 ("Building Custom TensorRT-LLM Plugins for
Low-Latency FP8 Inference at Scale", "Fusing the Kernel in CUDA").
"""
import math
import os

import numpy as np
import pytest
import torch

import synth_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant_worked_example.txt")
GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _read_golden():
    d = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split("=", 1)
            d[k.strip()] = [t.strip() for t in v.split(",")]
    return d


def e4m3_code_of_pow2(e: int) -> int:
    """Bit pattern of 2^e in E4M3FN (format definition, bias 7)."""
    if e >= -6:
        return (e + 7) << 3
    return 1 << (e + 9)          # subnormal m/8 * 2^-6 with m = 2^(e+9)


def e2m1_code(q: float) -> int:
    mag = GRID.index(abs(q))
    return mag | (8 if math.copysign(1.0, q) < 0 else 0)


def test_hand_worked_example(oracle):
    g = _read_golden()
    row = torch.tensor([[float(v) for v in g["row"]]], dtype=torch.bfloat16)
    q = oracle.quantize(row)
    assert [int(v, 16) for v in g["codes"]] == q["codes"][0].tolist()
    assert [int(v, 16) for v in g["sf"]] == q["sf"][0].tolist()
    assert q["g_dec"][0] == np.float32(1.0) / np.float32(448.0)
    assert abs(q["scale"][0, 0] - 1.0) < 3e-7 and abs(q["scale"][0, 1] - 0.5) < 2e-7


@pytest.mark.parametrize("m", [-20, -3, 0, 5, 20])
def test_closed_form_round_trip(oracle, m):
    rng = np.random.default_rng(100 + m)
    nblocks = 24
    vals = np.zeros((2, nblocks * 16), np.float64)
    want_codes = np.zeros((2, nblocks * 16), np.uint8)
    want_sf = np.zeros((2, nblocks), np.uint8)
    want_c = np.zeros((2, nblocks), np.float64)
    for r in range(2):
        for b in range(nblocks):
            qs = rng.choice(GRID, 16) * rng.choice([-1.0, 1.0], 16)
            qs[rng.integers(16)] = 6.0 * rng.choice([-1.0, 1.0])   # block max is 6 * scale
            if b == 0:
                # the block holding the row maximum 2688*2^m: values q*448*2^m
                scale = 448.0 * 2.0 ** m
                want_sf[r, b] = 0x7E
                want_c[r, b] = float(np.float32(448.0) * (np.float32(2.0 ** m)))
            else:
                p = m + int(rng.integers(-9, 9))                    # 2^(p-m) in E4M3 range
                scale = 2.0 ** p
                want_sf[r, b] = e4m3_code_of_pow2(p - m)
                want_c[r, b] = 2.0 ** p
            vals[r, b * 16:(b + 1) * 16] = qs * scale
            want_codes[r, b * 16:(b + 1) * 16] = [e2m1_code(q) for q in qs]
    x = torch.from_numpy(vals).to(torch.bfloat16)
    assert torch.equal(x.double(), torch.from_numpy(vals))          # exact in bf16
    q = oracle.quantize(x)
    nib = oracle.unpack_codes(q["codes"])
    assert np.array_equal(nib, want_codes)
    assert np.array_equal(q["sf"], want_sf)
    assert np.all(q["g_dec"] == np.float32(2.0 ** m))
    assert np.array_equal(q["scale"].astype(np.float64), want_c)


def _random_rows(rows=64, k=512, seed=0, outliers=True):
    return si.bf16_normal((rows, k), 1.0, 99, 0, seed,
                          outlier_frac=0.01 if outliers else 0.0, outlier_scale=50.0)


def test_block_and_row_max_invariants(oracle):
    x = _random_rows()
    q = oracle.quantize(x)
    y = x.float().numpy().reshape(x.shape[0], -1, 16)
    nib = oracle.unpack_codes(q["codes"]).reshape(y.shape)
    sfd = oracle.e4m3_table()[q["sf"]]
    for r in range(y.shape[0]):
        rowmax_block = int(np.argmax(np.abs(y[r]).max(axis=1)))
        assert q["sf"][r, rowmax_block] == 0x7E
        for b in range(y.shape[1]):
            if sfd[r, b] >= 2.0 ** -6:
                i = int(np.argmax(np.abs(y[r, b])))
                assert nib[r, b, i] & 7 == 7, (r, b)


def _half_gap(v):
    v = abs(v)
    if v <= 2.0:
        return 0.25
    if v <= 4.0:
        return 0.5
    if v <= 6.0:
        return 1.0
    return v - 6.0


def test_error_bound(oracle):
    x = _random_rows(rows=32, k=256, seed=1)
    q = oracle.quantize(x)
    y = x.double().numpy()
    deq = oracle.dequant_act(q["codes"], q["scale"])
    c = np.repeat(q["scale"].astype(np.float64), 16, axis=1)
    g_dec = q["g_dec"].astype(np.float64)
    for r in range(y.shape[0]):
        for k in range(y.shape[1]):
            if c[r, k] == 0:
                # block scale rounded to 0: the block max is below 6*2^-10*g_dec
                assert abs(y[r, k]) <= 6 * 2.0 ** -10 * g_dec[r] * (1 + 1e-6)
                continue
            v = y[r, k] / c[r, k]
            bound = c[r, k] * (_half_gap(v) + (abs(v) + 6.0) * 2.0 ** -21)
            assert abs(y[r, k] - deq[r, k]) <= bound, (r, k)


@pytest.mark.parametrize("p", [-7, 3, 11])
def test_scale_equivariance(oracle, p):
    x = _random_rows(rows=16, k=256, seed=2)
    xs = (x.double() * 2.0 ** p).to(torch.bfloat16)
    assert torch.equal(xs.double(), x.double() * 2.0 ** p)
    a, b = oracle.quantize(x), oracle.quantize(xs)
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["sf"], b["sf"])
    assert np.array_equal(a["g_dec"].astype(np.float64) * 2.0 ** p, b["g_dec"].astype(np.float64))
    assert np.array_equal(a["scale"].astype(np.float64) * 2.0 ** p, b["scale"].astype(np.float64))


def test_sign_equivariance(oracle):
    x = _random_rows(rows=16, k=256, seed=3)
    a, b = oracle.quantize(x), oracle.quantize(-x)
    assert np.array_equal(a["codes"] ^ 0x88, b["codes"])
    assert np.array_equal(a["sf"], b["sf"]) and np.array_equal(a["g_dec"], b["g_dec"])


def test_zero_and_constant_rows(oracle):
    x = torch.zeros((3, 64), dtype=torch.bfloat16)
    x[1] = 3.0
    x[2] = -0.375
    q = oracle.quantize(x)
    assert np.all(q["codes"][0] == 0) and np.all(q["sf"][0] == 0) and np.all(q["scale"][0] == 0)
    assert q["g_dec"][0] == np.float32(1.0) / np.float32(np.finfo(np.float32).max)
    assert np.all(q["codes"][1] == 0x77) and np.all(q["sf"][1] == 0x7E)
    assert np.all(q["codes"][2] == 0xFF) and np.all(q["sf"][2] == 0x7E)


def test_row_whose_encode_factor_overflows(oracle):
    """Row maximum 2^-133 (the smallest bf16 subnormal): 2688/amax overflows,
    so g_enc = FLT_MAX and g_dec = 1/FLT_MAX rounds to 2^-128; the block scale
    (2^-133/6)*FLT_MAX = 10923*2^-21 lies between the E4M3 subnormals 2*2^-9
    and 3*2^-9 (nearer 3); c = 3*2^-137 is exact, 1/c overflows to +inf.  The
    non-zero element saturates to code 7 and zero elements keep zero codes
    with their own sign."""
    x = np.zeros((1, 16), np.uint16)
    x[0, 0] = 0x0001                 # +2^-133
    x[0, 5] = 0x8000                 # -0
    q = oracle.quantize(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16))
    assert q["g_dec"][0] == np.float32(2.0 ** -128)
    assert q["sf"][0, 0] == 0x03
    assert q["scale"][0, 0] == np.float32(3 * 2.0 ** -137)
    nib = np.stack([q["codes"][0] & 0xF, q["codes"][0] >> 4], axis=1).reshape(-1)
    want = np.zeros(16, np.uint8)
    want[0], want[5] = 7, 8
    assert nib.tolist() == want.tolist()


def test_per_tensor_equals_per_row_when_row_maxima_agree(oracle):
    x = _random_rows(rows=8, k=128, seed=4, outliers=False).double()
    x[:, 5] = 1000.0                       # every row has the same maximum
    x = x.to(torch.bfloat16)
    a = oracle.quantize(x, group_rows=1)
    b = oracle.quantize(x, group_rows=8)
    assert b["g_dec"].shape == (1,) and np.all(a["g_dec"] == b["g_dec"][0])
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["sf"], b["sf"])
    assert np.array_equal(a["scale"], b["scale"])


def test_per_tensor_uses_tensor_max(oracle):
    x = _random_rows(rows=8, k=128, seed=5).double()
    amax = float(x.abs().max())
    q = oracle.quantize(x.to(torch.bfloat16), group_rows=8)
    assert q["g_dec"][0] == np.float32(1.0) / (np.float32(2688.0) / np.float32(amax))


def test_activation_fused_matches_quantize_of_bf16_exact_activation(oracle):
    # ReLU^2 of bf16 values with <= 4 significant bits is exact in bf16, so
    # quantizing relu2(x) computed by hand must equal the fused path.
    rng = np.random.default_rng(6)
    mant = rng.integers(0, 4, (4, 64)) + 4               # 3-bit significands
    vals = mant * 2.0 ** rng.integers(-6, 4, (4, 64)) * rng.choice([-1, 1], (4, 64))
    x = torch.from_numpy(vals).to(torch.bfloat16)
    y = torch.from_numpy(np.maximum(vals, 0.0) ** 2).to(torch.bfloat16)
    assert torch.equal(y.double(), torch.from_numpy(np.maximum(vals, 0.0) ** 2))
    a = oracle.quantize(x, act=oracle.ACT_RELU2)
    b = oracle.quantize(y)
    for k in ("codes", "sf", "g_dec", "scale"):
        assert np.array_equal(a[k], b[k]), k


def test_swiglu_layout_gate_then_up(oracle):
    # gate = first half, up = second half: with gate = +large the output is
    # exactly up (silu(g) = g, then times u is not exact), so use u = 1.0
    # and check y = silu(g) on the gate half only.
    g = torch.tensor([[3.0, -2.0, 0.5, 100.0] * 4], dtype=torch.bfloat16)
    u = torch.ones_like(g)
    x = torch.cat([g, u], dim=1)
    y = oracle.activation(x, oracle.ACT_SWIGLU)
    for j in range(16):
        gv = float(g[0, j])
        assert y[0, j] == np.float32(oracle.swiglu_f32(gv, 1.0))
        assert abs(y[0, j] - gv / (1 + math.exp(-gv))) <= 4e-7 * max(1.0, abs(gv))


def test_rejects_bad_arguments(oracle):
    with pytest.raises(ValueError):
        oracle.quantize(torch.zeros((2, 24), dtype=torch.bfloat16))          # K % 16 != 0
    with pytest.raises(ValueError):
        oracle.quantize(torch.zeros((3, 32), dtype=torch.bfloat16), group_rows=2)


def test_combined_scale_is_dequantize_product_of_stored_scales(oracle):
    # The activation scale is the DequantizeLinear product of the two stored
    # scales ("Fused Nvfp4 GEMM All Reduce Plugin": activation_scale is the
    # combined FP32 scale from DequantizeLinear): one binary32 product of the
    # decoded E4M3 byte and the emitted FP32 global.
    x = _random_rows(rows=16, k=256, seed=7)
    q = oracle.quantize(x)
    sfd = oracle.e4m3_table()[q["sf"]].astype(np.float32)
    prod = sfd * q["g_dec"][:, None]
    assert np.array_equal(prod, q["scale"])


@pytest.mark.parametrize("m", [-4, 0, 6])
def test_block_scale_rounds_half_to_even(oracle, m):
    # With the row maximum 2688*2^m the global is exactly 2^-m, so a block
    # whose maximum is 6*t*2^m asks for the E4M3 value nearest to t.  Put t on
    # midpoints between adjacent E4M3 values and one bf16 step either side.
    def e4(b):
        e, mm = (b >> 3) & 15, b & 7
        return (mm / 8) * 2.0 ** -6 if e == 0 else (1 + mm / 8) * 2.0 ** (e - 7)
    def bf16_step(v, d):                     # neighbouring bf16 value
        b = torch.tensor([v], dtype=torch.bfloat16).view(torch.int16)
        return float((b + d).view(torch.bfloat16).double())
    cases = []
    for lo in (0x02, 0x07, 0x30, 0x38, 0x39, 0x44, 0x51):
        mid = (e4(lo) + e4(lo + 1)) / 2
        even = lo if lo % 2 == 0 else lo + 1
        a = 6.0 * mid * 2.0 ** m
        for amax_b, want in ((a, even), (bf16_step(a, -1), lo), (bf16_step(a, 1), lo + 1)):
            cases.append((amax_b, want))
    row = np.zeros(16 * (len(cases) + 1))
    row[0] = 2688.0 * 2.0 ** m
    for i, (amax_b, _) in enumerate(cases):
        row[16 * (i + 1)] = amax_b
    x = torch.from_numpy(row[None, :]).to(torch.bfloat16)
    assert torch.equal(x.double()[0], torch.from_numpy(row))
    q = oracle.quantize(x)
    assert q["g_dec"][0] == np.float32(2.0 ** m)
    assert [int(v) for v in q["sf"][0, 1:]] == [w for _, w in cases]

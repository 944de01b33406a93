"""Saturation / zero-code diagnostics of the oracle quantizer on the synthetic
workloads (CPU), with the two scale-chain properties checked in
quant_diagnostics: every normal-scale block holds a +-6 code, and with per-row
global scales every nonzero row has a 448 block scale.

A planted mistake fails them: the block scale computed from the decode factor
instead of the encode factor leaves blocks without a +-6 code.
"""
import numpy as np
import pytest
import torch

import synth_inputs as si
from quant_diagnostics import report, stats


def test_prefill_activations(oracle):
    a, _ = si.gemm_inputs("C3", N=16)
    q = oracle.quantize(a[:64])
    s = stats(q["codes"], q["sf"])
    report("C3 activations (64 rows, oracle)", s)
    assert s["normal_blocks_without_max_code"] == 0
    assert s["nonzero_rows_without_448"] == 0
    # ~N(0,1) data: no zero or subnormal block scales; a row's 448 block is one of 512
    assert s["zero_scale_share"] == 0.0 and s["subnormal_scale_share"] == 0.0
    assert 0.0 < s["scale_448_share"] < 0.01


def test_swiglu_outputs(oracle):
    x = si.swiglu_input(rows=16)
    q = oracle.quantize(x, act=oracle.ACT_SWIGLU, want_scale=False)
    s = stats(q["codes"], q["sf"])
    report("C4 SwiGLU (16 rows, oracle)", s)
    assert s["normal_blocks_without_max_code"] == 0
    assert s["nonzero_rows_without_448"] == 0
    # SwiGLU of N(0,1) pairs is concentrated near zero: a third of the codes or more are +-0
    assert s["zero_code_share"] > 0.25


def test_degenerate_rows(oracle):
    # zero row, constant row, a row with one huge outlier (its other blocks get
    # subnormal or zero scales), a row of tiny values
    k = 256
    rows = torch.zeros(4, k)
    rows[1] = 1.5
    rows[2, :] = 1e-3
    rows[2, 7] = 3e4
    rows[3] = 1e-20
    q = oracle.quantize(rows.to(torch.bfloat16))
    s = stats(q["codes"], q["sf"])
    report("degenerate rows (oracle)", s)
    assert s["normal_blocks_without_max_code"] == 0
    assert s["nonzero_rows_without_448"] == 0
    n = q["codes"]
    assert np.all(n[0] == 0) and np.all(q["sf"][0] == 0)          # zero row: zero codes, zero scales
    assert np.all(q["sf"][1] == 0x7E)                               # constant row: every block at 448
    assert s["subnormal_scale_share"] > 0 or s["zero_scale_share"] > 0.25


def test_planted_scale_mistake_is_caught():
    # the block scale computed from the wrong grid maximum (amax_b / 4 instead
    # of amax_b / 6) maps each block maximum to ~4, not 6: the diagnostic flags it
    rng = np.random.default_rng(0)
    v = rng.standard_normal((8, 64)).astype(np.float32)
    amax = np.abs(v).max(axis=1)[:, None, None]
    g_enc = 448.0 * 6.0 / amax
    blocks = v.reshape(8, 4, 16)
    bmax = np.abs(blocks).max(axis=-1, keepdims=True)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])

    def quantize(grid_max):
        sf = torch.tensor(bmax / grid_max * g_enc).to(torch.float8_e4m3fn)
        dec = sf.float().numpy() / g_enc
        x = np.abs(blocks) / dec
        idx = np.abs(x[..., None] - grid).argmin(-1)
        flat = (idx | ((blocks < 0) << 3)).reshape(8, 64).astype(np.uint8)
        return stats((flat[:, 0::2] | (flat[:, 1::2] << 4)).astype(np.uint8), sf.view(torch.uint8).numpy().reshape(8, 4))

    assert quantize(6.0)["normal_blocks_without_max_code"] == 0
    assert quantize(4.0)["normal_blocks_without_max_code"] > 0    # the planted mistake

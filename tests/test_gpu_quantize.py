"""GPU parity of the quantizer (nvfp4_quantize / nvfp4_act_quant) against the
oracle: codes, E4M3 bytes, FP32 globals and combined scales must match
bit-for-bit.

Workloads: per-token activations of the prefill GEMM ([4096, 8192] bf16
~N(0,1)), fused SwiGLU + quantize ([8192, 2x14336] bf16 with 1% outliers x50,
"Building Custom TensorRT-LLM Plugins for Low-Latency FP8 Inference at Scale",
"The Cost of Non-Fused Quantization"), per-tensor and per-expert weights.  At
full size the oracle checks sampled rows; small cases check everything.
"""
import numpy as np
import pytest
import torch

import synth_inputs as si
from quant_diagnostics import report, stats

pytestmark = pytest.mark.gpu

ACTS = {"none": 0, "swiglu": 1, "relu2": 2}


@pytest.fixture(scope="module")
def nv():
    import nvfp4_block_scaled_quantize_amd as nv
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return nv


def _cmp(got: dict, want: dict):
    for k in ("codes", "sf", "g_dec", "scale"):
        if want.get(k) is None or got.get(k) is None:
            continue
        g = got[k].cpu().numpy()
        w = want[k]
        if g.dtype == np.float32:
            g = g.view(np.uint32); w = w.view(np.uint32)
        bad = np.argwhere(g != w)
        assert bad.size == 0, "%s mismatch at %s (got %s want %s)" % (
            k, bad[:3].tolist(), g[tuple(bad[0])], w[tuple(bad[0])])


def _gpu_quant(nv, x, act, group_rows=1):
    xd = x.cuda()
    if act == "none":
        out = nv.quantize(xd, group_rows=group_rows)
    else:
        assert group_rows == 1
        out = nv.act_quant(xd, act)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("act", ["none", "swiglu", "relu2"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("rows,k_out", [(1, 16), (3, 32), (37, 48), (5, 256), (9, 1040), (4, 4096),
                                         (2, 14336), (1, 32768), (3, 32784)])
def test_small_shapes_bit_exact(nv, oracle, act, dtype, rows, k_out):
    k_in = 2 * k_out if act == "swiglu" else k_out
    x32 = si.normal_f32((rows, k_in), 1.0, 90, 0, seed=rows * 7 + k_out,
                        outlier_frac=0.01, outlier_scale=50.0)
    x = torch.from_numpy(x32).to(dtype)
    want = oracle.quantize(x, act=ACTS[act])
    got = _gpu_quant(nv, x, act)
    _cmp(got, want)


@pytest.mark.parametrize("group", ["tensor", "expert4"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_per_tensor_and_per_expert(nv, oracle, group, dtype):
    rows, k = 64, 384
    x = torch.from_numpy(si.normal_f32((rows, k), 0.02, 91, 1, seed=3)).to(dtype)
    gr = rows if group == "tensor" else rows // 4
    want = oracle.quantize(x, group_rows=gr)
    got = _gpu_quant(nv, x, "none", group_rows=gr)
    _cmp(got, want)


def test_edge_rows(nv, oracle):
    k = 64
    x = torch.zeros((8, k), dtype=torch.bfloat16)
    x[1] = 3.0                                    # constant row
    x[2] = -0.0                                   # negative zeros
    x[3, 5] = 7.5                                 # single non-zero
    x[3, 16:32:3] = -0.0                          # signed zeros in an all-zero block of that row
    x[4] = torch.tensor(np.full(k, 1e-39, np.float32)).to(torch.bfloat16)   # subnormal bf16
    x[5, :16] = torch.tensor(np.linspace(-1e-38, 1e-38, 16, dtype=np.float32)).to(torch.bfloat16)
    x[6] = torch.tensor(np.geomspace(1e-30, 1e30, k, dtype=np.float32)).to(torch.bfloat16)
    x[7] = torch.from_numpy(si.normal_f32((k,), 1.0, 92, 0)).to(torch.bfloat16)
    for act in ("none", "relu2", "swiglu"):
        xx = torch.cat([x, x], dim=1) if act == "swiglu" else x
        if act == "relu2":
            xx = xx.clone(); xx[6] = 0            # squares of 1e30 overflow (outside the contract)
        if act == "swiglu":
            xx = xx.clone(); xx[6] = torch.linspace(-100, 100, 2 * k).to(torch.bfloat16)
        want = oracle.quantize(xx, act=ACTS[act])
        got = _gpu_quant(nv, xx, act)
        _cmp(got, want)


def test_misaligned_input_takes_scalar_path(nv, oracle):
    rows, k = 6, 160
    base = torch.from_numpy(si.normal_f32((rows * k + 1,), 1.0, 93, 0)).to(torch.bfloat16).cuda()
    x = base[1:].view(rows, k)                    # 2-byte offset: not 16-byte aligned
    assert x.data_ptr() % 16 != 0
    want = oracle.quantize(x.cpu())
    got = nv.quantize(x)
    torch.cuda.synchronize()
    _cmp(got, want)
    xs = torch.cat([x, x], dim=1).contiguous()
    base2 = torch.empty(xs.numel() + 8, dtype=torch.bfloat16, device="cuda")
    xm = base2[8 - 1:8 - 1 + xs.numel()].view_as(xs)
    xm.copy_(xs)
    want = oracle.quantize(xs.cpu(), act=1)
    got = nv.act_quant(xm, "swiglu")
    torch.cuda.synchronize()
    _cmp(got, want)


def test_full_size_swiglu_sampled_rows(nv, oracle):
    c = si.CONFIGS["C4"]
    x = si.swiglu_input()
    got = nv.act_quant(x.cuda(), "swiglu")
    torch.cuda.synchronize()
    rows = [0, 1, 2, 777, 4095, 4096, 6000, c["rows"] - 1]
    want = oracle.quantize(x[rows], act=1)
    for k in ("codes", "sf", "scale"):
        g = got[k].cpu().numpy()[rows]
        w = want[k]
        if g.dtype == np.float32:
            g, w = g.view(np.uint32), w.view(np.uint32)
        assert np.array_equal(g, w), k
    assert np.array_equal(got["g_dec"].cpu().numpy()[rows].view(np.uint32), want["g_dec"].view(np.uint32))
    # every row: the block holding the row maximum has scale byte 448 (0x7E);
    # every normal-scale block of the whole output holds a +-6 code
    sf = got["sf"].cpu().numpy()
    assert np.all(sf.max(axis=1) == 0x7E)
    d = stats(got["codes"].cpu().numpy(), sf)
    report("C4 SwiGLU [8192, 14336] (GPU, all rows)", d)
    assert d["normal_blocks_without_max_code"] == 0 and d["nonzero_rows_without_448"] == 0


def test_full_size_prefill_activations_sampled_rows(nv, oracle):
    a, _ = si.gemm_inputs("C3", N=16)
    got = nv.quantize(a.cuda())
    torch.cuda.synchronize()
    rows = [0, 5, 1000, 2047, 4095]
    want = oracle.quantize(a[rows])
    for k in ("codes", "sf", "scale"):
        g = got[k].cpu().numpy()[rows]
        w = want[k]
        if g.dtype == np.float32:
            g, w = g.view(np.uint32), w.view(np.uint32)
        assert np.array_equal(g, w), k
    d = stats(got["codes"].cpu().numpy(), got["sf"].cpu().numpy())
    report("C3 activations [4096, 8192] (GPU, all rows)", d)
    assert d["normal_blocks_without_max_code"] == 0 and d["nonzero_rows_without_448"] == 0


def test_deterministic_and_concurrent_streams(nv, oracle):
    x1 = torch.from_numpy(si.normal_f32((64, 2048), 1.0, 94, 0)).to(torch.bfloat16)
    x2 = torch.from_numpy(si.normal_f32((64, 4096), 1.0, 94, 1)).to(torch.bfloat16)
    d1, d2 = x1.cuda(), x2.cuda()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            o1 = nv.act_quant(d1, "swiglu", stream=s1)
        with torch.cuda.stream(s2):
            o2 = nv.quantize(d2, stream=s2)
        outs.append((o1, o2))
    torch.cuda.synchronize()
    w1 = oracle.quantize(x1, act=1)
    w2 = oracle.quantize(x2)
    for o1, o2 in outs:
        _cmp(o1, w1)
        _cmp(o2, w2)


def test_no_scale_output_and_empty(nv, oracle):
    x = torch.from_numpy(si.normal_f32((4, 64), 1.0, 95, 0)).to(torch.bfloat16)
    got = nv.quantize(x.cuda(), want_scale=False)
    torch.cuda.synchronize()
    want = oracle.quantize(x)
    _cmp(got, want)
    e = nv.quantize(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"))
    assert e["codes"].shape == (0, 32)


def _one_gate_per_row(patterns: np.ndarray, torch_dtype):
    """Rows of one 16-block whose SwiGLU output is silu(g) * 1 at position 0
    and silu(0) * 1 = 0 elsewhere: the row amax, hence the stored global
    1 / (2688 / amax), exposes |silu(g)| and the code exposes its sign."""
    n = patterns.size
    x = np.zeros((n, 32), np.uint16)
    x[:, 0] = patterns
    one = 0x3F80 if torch_dtype == torch.bfloat16 else 0x3C00
    x[:, 16:] = one
    return torch.from_numpy(x.view(np.int16)).view(torch_dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_swiglu_every_finite_gate_value(nv, oracle, dtype):
    """silu over every finite 16-bit gate value: bf16 runs the tabulated path
    (more than 1024 rows), fp16 the direct evaluation."""
    p = np.arange(65536, dtype=np.uint32)
    if dtype == torch.bfloat16:
        finite = ((p >> 7) & 0xFF) != 0xFF
    else:
        finite = ((p >> 10) & 0x1F) != 0x1F
    x = _one_gate_per_row(p[finite].astype(np.uint16), dtype)
    want = oracle.quantize(x, act=1)
    got = _gpu_quant(nv, x, "swiglu")
    _cmp(got, want)


@pytest.mark.parametrize("rows,k_out", [(1100, 272), (1030, 16384), (1024, 16), (1030, 24576)])
def test_swiglu_tabulated_path_shapes(nv, oracle, rows, k_out):
    """Persistent tabulated SwiGLU kernel: ragged last wave, three units per
    lane, exactly the row threshold; every row compared."""
    x32 = si.normal_f32((rows, 2 * k_out), 1.0, 96, 0, seed=rows + k_out,
                        outlier_frac=0.01, outlier_scale=50.0)
    x = torch.from_numpy(x32).to(torch.bfloat16)
    want = oracle.quantize(x, act=1)
    got = _gpu_quant(nv, x, "swiglu")
    _cmp(got, want)

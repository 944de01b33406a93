"""GPU parity of nvfp4_gemm against the fp64 oracle on the same quantized
operands: relative Frobenius error <= 1e-3 (the operands are bit-identical;
the only differences are the FP16 rounding of the activation operand, fp32
accumulation order and the FP16 output rounding).

Operand contract: "Fused Nvfp4 GEMM All Reduce Plugin", Baked-weight inputs
(activation FP4 [B,K], activation_scale FP32 [B,1,K/16], weight FP4 [N,K],
weight FP8 [N,K/16], scalar FP32 global) and Output (FP16 [B,N]).  Operands are
produced by the oracle quantizer from seeded bf16 data (activations ~N(0,1)
per token, weights ~N(0,0.02) per tensor), never by the GPU path.
"""
import numpy as np
import pytest
import torch

import synth_inputs as si

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module")
def nv():
    import nvfp4_block_scaled_quantize_amd as nv
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return nv


def _operands(oracle, a, w):
    qa = oracle.quantize(a)
    qw = oracle.quantize(w, group_rows=w.shape[0])
    return qa, qw


def _run(nv, qa, qw, **kw):
    y = nv.gemm(torch.from_numpy(qa["codes"]).cuda(), torch.from_numpy(qa["scale"]).cuda(),
                torch.from_numpy(qw["codes"]).cuda(), torch.from_numpy(qw["sf"]).cuda(),
                torch.from_numpy(qw["g_dec"][:1]).cuda(), **kw)
    torch.cuda.synchronize()
    return y.cpu().double().numpy()


def _ref(oracle, qa, qw, rows=None):
    return oracle.gemm_ref(qa["codes"], qa["scale"], qw["codes"], qw["sf"], qw["g_dec"][0], rows=rows)


@pytest.mark.parametrize("B,N,K", [(16, 256, 256),                      # quantize + GEMM workload
                                   (1, 96, 32), (5, 100, 160), (3, 33, 4096 + 32),
                                   (16, 64, 2048), (17, 64, 64), (37, 300, 96), (64, 512, 1024),
                                   (300, 260, 544)])
def test_small_shapes(nv, oracle, B, N, K):
    a = si.bf16_normal((B, K), 1.0, 80, 0, seed=B + N + K)
    w = si.bf16_normal((N, K), 0.02, 80, 1, seed=B + N + K)
    qa, qw = _operands(oracle, a, w)
    y = _run(nv, qa, qw)
    ref = _ref(oracle, qa, qw)
    err = oracle.rel_fro(y, ref)
    assert err <= TOL, err


@pytest.mark.parametrize("B", [1, 4, 8])
def test_decode_full_size(nv, oracle, B):
    c = si.CONFIGS["C2"]
    a, w = si.gemm_inputs("C2", B=B)
    qa, qw = _operands(oracle, a, w)
    y = _run(nv, qa, qw)
    ref = _ref(oracle, qa, qw)
    err = oracle.rel_fro(y, ref)
    assert y.shape == (B, c["N"])
    assert err <= TOL, err


@pytest.fixture(scope="module")
def prefill_operands(oracle):
    a, w = si.gemm_inputs("C3")
    return _operands(oracle, a, w)


def test_prefill_full_size_sampled_rows(nv, oracle, prefill_operands):
    qa, qw = prefill_operands
    y = _run(nv, qa, qw)
    rows = [0, 1, 255, 256, 1000, 2047, 3071, 4095]
    ref = _ref(oracle, qa, qw, rows=rows)
    err = oracle.rel_fro(y[rows], ref)
    assert err <= TOL, err
    assert np.all(np.isfinite(y))


def test_identity_weights_return_activations(nv, oracle):
    B, K = 24, 128
    a = si.bf16_normal((B, K), 1.0, 81, 0)
    qa = oracle.quantize(a)
    nib = np.where(np.eye(K) > 0, 2, 0).astype(np.uint8)          # code 2 = 1.0
    qw = {"codes": (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8),
          "sf": np.full((K, K // 16), 0x38, np.uint8),                # E4M3 1.0
          "g_dec": np.ones(1, np.float32)}
    y = _run(nv, qa, qw)
    A = oracle.dequant_act(qa["codes"], qa["scale"])
    assert np.allclose(y, A, rtol=2e-3, atol=1e-6)


def test_zero_activations_and_workspace_reuse(nv, oracle):
    B, N, K = 40, 64, 256
    a = torch.zeros((B, K), dtype=torch.bfloat16)
    w = si.bf16_normal((N, K), 0.02, 82, 1)
    qa, qw = _operands(oracle, a, w)
    ws = torch.empty(nv.gemm_workspace_size(B, N, K), dtype=torch.uint8, device="cuda")
    y = _run(nv, qa, qw, workspace=ws)
    assert np.all(y == 0)


def test_deterministic(nv, oracle):
    a, w = si.gemm_inputs("C1")
    qa, qw = _operands(oracle, a, w)
    y1 = _run(nv, qa, qw)
    y2 = _run(nv, qa, qw)
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("B", [4, 64])
def test_external_weight_mode_matches_baked(nv, oracle, B):
    # "Fused Nvfp4 GEMM All Reduce Plugin", external-weight mode: same operands
    # by registered resource id -> the same kernels, bit-identical output
    N, K = 256, 512
    a = si.bf16_normal((B, K), 1.0, 0, 0, 31)
    wsrc = si.bf16_normal((N, K), 0.02, 0, 1, 31)
    dev = "cuda"
    qa = nv.quantize(a.to(dev))
    qw = nv.quantize(wsrc.to(dev), group_rows=N, want_scale=False)
    y0 = nv.gemm(qa["codes"], qa["scale"], qw["codes"], qw["sf"], qw["g_dec"])
    nv.register_weight(41, qw["codes"], qw["sf"])
    try:
        y1 = nv.gemm_external(qa["codes"], qa["scale"], 41, N, qw["g_dec"])
        torch.cuda.synchronize()
        assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
        with pytest.raises(nv.Nvfp4Error):
            nv.gemm_external(qa["codes"], qa["scale"], 41, N + 32, qw["g_dec"])   # N differs
    finally:
        nv.unregister_weight(41, torch.cuda.current_device())
    with pytest.raises(nv.Nvfp4Error):
        nv.gemm_external(qa["codes"], qa["scale"], 41, N, qw["g_dec"])


def test_prefill_path_past_4gib_of_fp16_activations(nv, oracle):
    # B*K*2 > 4 GiB: the copy offsets of the prefill kernel must not wrap
    # (rows past 32768 are checked); ragged in B (not a multiple of 128) and N
    B, N, K = 33024, 96, 65536
    d = si.random_nvfp4_operands(B, N, K, seed=5)
    dev = "cuda"
    t = {k: torch.from_numpy(v).to(dev) for k, v in d.items()}
    y = nv.gemm(t["a_codes"], t["a_scale"], t["w_codes"], t["w_sf"], t["w_g"])
    torch.cuda.synchronize()
    rows = [0, 127, 128, 32767, 32768, 32900, B - 1]
    got = y[rows].cpu().double().numpy()
    ref = oracle.gemm_ref(d["a_codes"], d["a_scale"], d["w_codes"], d["w_sf"], d["w_g"][0], rows=rows)
    assert oracle.rel_fro(got, ref) <= TOL
    del t, y
    torch.cuda.empty_cache()


@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (8192, 4096)])
def test_pretile_matches_oracle(nv, oracle, N, K):
    d = si.random_nvfp4_operands(1, N, K, seed=N + K)
    dev = "cuda"
    t = nv.pretile_weight(torch.from_numpy(d["w_codes"]).to(dev), torch.from_numpy(d["w_sf"]).to(dev))
    torch.cuda.synchronize()
    wt, st = oracle.pretile_weight(d["w_codes"], d["w_sf"])
    assert np.array_equal(t["codes"].cpu().numpy(), wt)
    assert np.array_equal(t["sf"].cpu().numpy(), st)


@pytest.mark.parametrize("B,N,K", [(1, 8192, 4096), (4, 48, 384), (16, 64, 256), (17, 48, 384),
                                   (300, 528, 640), (64, 512, 1024)])
def test_gemm_pretiled_matches_untiled(nv, oracle, B, N, K):
    # decode (B <= 16) and prefill kernels on the pre-tiled layout: the same
    # products in the same order as on [N, K/2] weights -> bit-identical
    d = si.random_nvfp4_operands(B, N, K, seed=B * 7 + N + K)
    dev = "cuda"
    t = {k: torch.from_numpy(v).to(dev) for k, v in d.items()}
    y0 = nv.gemm(t["a_codes"], t["a_scale"], t["w_codes"], t["w_sf"], t["w_g"])
    wt = nv.pretile_weight(t["w_codes"], t["w_sf"])
    y1 = nv.gemm_pretiled(t["a_codes"], t["a_scale"], wt, t["w_g"])
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    ref = oracle.gemm_ref(d["a_codes"], d["a_scale"], d["w_codes"], d["w_sf"], d["w_g"][0],
                          rows=list(range(min(B, 8))))
    assert oracle.rel_fro(y1[:min(B, 8)].cpu().double().numpy(), ref) <= TOL

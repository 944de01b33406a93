"""GPU parity at the shapes the benchmark runs, boundary paths and robustness.

- Full C3 prefill (B=4096, K=8192, N=8192): both weight layouts against the
  fp64 oracle over EVERY row (relative Frobenius per row <= 1e-3, plus an
  element-wise bound), at the shape where the XCD-aware tile order is active;
  the same order at a small K; the MXFP4 GEMM at its remap-active shape.
- Weight quantization as the benchmark does it, bit-exact against the oracle:
  C3 and C2 weights per tensor (1024 / 512 partial maxima), C5 fc1 and fc2 per
  expert, and the full C3 activations per token.
- Boundary paths: activation codes at a 2-byte offset (decode kernel's byte
  loads), weights at odd offsets and K % 32 == 16 (byte-load paths, results
  bit-identical to the aligned path where one exists), per-tensor
  quantization of an input at a 2-byte offset (scalar path with partials).
- MoE routing lists above 4096 (token, expert) pairs, and an expert with more
  than 65536 tokens.
- Canary bytes around every output buffer of every entry point, and the
  number of kernels each call launches (the "numGpuOps" test aid of "Nvfp4 A16
  Blackwell Moe Runner"), counted by capturing the call into a HIP graph.

Operands and expected values come from the oracle or from seeded synthetic
generators only ("Fused Nvfp4 GEMM All Reduce Plugin", Baked-weight inputs).
"""
from concurrent.futures import ThreadPoolExecutor
import ctypes

import numpy as np
import pytest
import torch

import synth_inputs as si
from gemm_checks import TOL, offset_view, refs, row_checks

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import nvfp4_block_scaled_quantize_amd as nv
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return nv


def _quantize_groups(oracle, x, group_rows, act=0, want_scale=True):
    """oracle.quantize on independent row groups in parallel threads (the
    oracle call releases the GIL); the same result as one call."""
    rows = x.shape[0]
    n = max(1, min(16, rows // group_rows))
    per = (rows // group_rows + n - 1) // n * group_rows
    parts = [(r, min(r + per, rows)) for r in range(0, rows, per)]
    with ThreadPoolExecutor(len(parts)) as ex:
        res = list(ex.map(lambda p: oracle.quantize(x[p[0]:p[1]], act=act, group_rows=group_rows,
                                                    want_scale=want_scale), parts))
    out = {k: np.concatenate([r[k] for r in res]) for k in ("codes", "sf", "g_dec")}
    out["scale"] = np.concatenate([r["scale"] for r in res]) if want_scale else None
    return out


# ---------------------------------------------------------------- full C3

@pytest.fixture(scope="module")
def c3(oracle):
    a, w = si.gemm_inputs("C3")
    qa = _quantize_groups(oracle, a, 1)
    qw = oracle.quantize(w, group_rows=w.shape[0], want_scale=False)
    A = oracle.dequant_act(qa["codes"], qa["scale"])
    W = oracle.dequant_weight(qw["codes"], qw["sf"], qw["g_dec"][0])
    ref, absref = refs(A, W)
    del A, W
    return dict(a=a, w=w, qa=qa, qw=qw, ref=ref, absref=absref)


def test_c3_weight_and_activation_quantize_bit_exact(nv, c3):
    dev = "cuda"
    N = c3["w"].shape[0]
    gw = nv.quantize(c3["w"].to(dev), group_rows=N, want_scale=False)      # 1024 partial maxima
    ga = nv.act_quant(c3["a"].to(dev), "none")
    torch.cuda.synchronize()
    for k in ("codes", "sf"):
        assert np.array_equal(gw[k].cpu().numpy(), c3["qw"][k]), k
        assert np.array_equal(ga[k].cpu().numpy(), c3["qa"][k]), k
    assert np.array_equal(gw["g_dec"].cpu().numpy().view(np.uint32), c3["qw"]["g_dec"].view(np.uint32))
    for k in ("g_dec", "scale"):
        assert np.array_equal(ga[k].cpu().numpy().view(np.uint32), c3["qa"][k].view(np.uint32)), k


@pytest.mark.parametrize("layout", ["pretiled", "plain"])
def test_c3_gemm_every_row(nv, oracle, c3, layout):
    dev = "cuda"
    qa, qw = c3["qa"], c3["qw"]
    t = lambda v: torch.from_numpy(v).to(dev)
    if layout == "pretiled":
        wt = nv.pretile_weight(t(qw["codes"]), t(qw["sf"]))
        y = nv.gemm_pretiled(t(qa["codes"]), t(qa["scale"]), wt, t(qw["g_dec"][:1]))
    else:
        y = nv.gemm(t(qa["codes"]), t(qa["scale"]), t(qw["codes"]), t(qw["sf"]), t(qw["g_dec"][:1]))
    torch.cuda.synchronize()
    yh = y.cpu().double().numpy()
    assert np.all(np.isfinite(yh))
    row_checks(yh, c3["ref"], c3["absref"], c3["a"].shape[1], 2.0 ** -11)
    assert oracle.rel_fro(yh, c3["ref"]) <= TOL


@pytest.mark.parametrize("K", [128, 192])
def test_tile_order_shape_every_row(nv, oracle, K):
    # B=4096, N=8192: 32 x 16 tiles of 128 x 512, the XCD-aware order; K=192
    # also has a ragged 64-k tail for the 128-k pre-tiled chunks (plain only)
    B, N = 4096, 8192
    d = si.random_nvfp4_operands(B, N, K, seed=K)
    dev = "cuda"
    t = {k: torch.from_numpy(v).to(dev) for k, v in d.items()}
    ref, absref = refs(oracle.dequant_act(d["a_codes"], d["a_scale"]),
                        oracle.dequant_weight(d["w_codes"], d["w_sf"], d["w_g"][0]))
    y = nv.gemm(t["a_codes"], t["a_scale"], t["w_codes"], t["w_sf"], t["w_g"])
    torch.cuda.synchronize()
    row_checks(y.cpu().double().numpy(), ref, absref, K, 2.0 ** -11)
    if K % 128 == 0:
        wt = nv.pretile_weight(t["w_codes"], t["w_sf"])
        y2 = nv.gemm_pretiled(t["a_codes"], t["a_scale"], wt, t["w_g"])
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_mx_tile_order_shape_every_row(nv, oracle):
    # 256 x 256 tiles: 16 x 32 = 512 tiles, the XCD-aware chunk order
    B, N, K = 4096, 8192, 128
    d = si.random_mx_operands(B, N, K, seed=3)
    dev = "cuda"
    t = lambda v: torch.from_numpy(v).to(dev)
    a = nv.mx_tile(t(d["a_codes"]), t(d["a_sf"]))
    w = nv.mx_tile(t(d["w_codes"]), t(d["w_sf"]))
    y = nv.mx_gemm(a, t(d["a_g"]), w, t(d["w_g"]))
    torch.cuda.synchronize()
    ref, absref = refs(oracle.dequant_mx(d["a_codes"], d["a_sf"], d["a_g"]),
                        oracle.dequant_mx(d["w_codes"], d["w_sf"], np.float32(d["w_g"][0])))
    row_checks(y.cpu().double().numpy(), ref, absref, K, 0.0)


# ---------------------------------------------------------------- weights as benchmarked

def test_c2_weight_quantize_bit_exact(nv, oracle):
    _, w = si.gemm_inputs("C2", B=1)
    q = oracle.quantize(w, group_rows=w.shape[0], want_scale=False)
    g = nv.quantize(w.cuda(), group_rows=w.shape[0], want_scale=False)
    torch.cuda.synchronize()
    for k in ("codes", "sf"):
        assert np.array_equal(g[k].cpu().numpy(), q[k]), k
    assert np.array_equal(g["g_dec"].cpu().numpy().view(np.uint32), q["g_dec"].view(np.uint32))


@pytest.mark.parametrize("which", ["w1", "w2"])
def test_c5_expert_weights_quantize_bit_exact(nv, oracle, which):
    d = si.moe_inputs()
    rows_per_expert = d["inter"] if which == "w1" else d["hidden"]
    w = d[which]
    q = _quantize_groups(oracle, w, rows_per_expert, want_scale=False)
    g = nv.quantize(w.cuda(), group_rows=rows_per_expert, want_scale=False)
    torch.cuda.synchronize()
    for k in ("codes", "sf"):
        assert np.array_equal(g[k].cpu().numpy(), q[k]), k
    assert np.array_equal(g["g_dec"].cpu().numpy().view(np.uint32), q["g_dec"].view(np.uint32))
    assert q["g_dec"].shape == (d["E"],)


# ---------------------------------------------------------------- boundary paths

# decode shapes, and prefill shapes whose FP16 prologue keeps a row in
# registers (K <= 16384) or takes two passes over it (K = 16640)
@pytest.mark.parametrize("B,N,K", [(1, 96, 256), (8, 8192, 4096), (13, 64, 528), (40, 64, 1024),
                                   (24, 64, 16384 + 256)])
def test_activation_codes_at_2_byte_offset(nv, oracle, B, N, K):
    d = si.random_nvfp4_operands(B, N, K, seed=B + K)
    t = {k: torch.from_numpy(v).cuda() for k, v in d.items()}
    y0 = nv.gemm(t["a_codes"], t["a_scale"], t["w_codes"], t["w_sf"], t["w_g"])
    a2 = offset_view(t["a_codes"], 2)
    assert a2.data_ptr() % 4 == 2
    y1 = nv.gemm(a2, t["a_scale"], t["w_codes"], t["w_sf"], t["w_g"])
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    ref = oracle.gemm_ref(d["a_codes"], d["a_scale"], d["w_codes"], d["w_sf"], d["w_g"][0])
    assert oracle.rel_fro(y1.cpu().double().numpy(), ref) <= TOL


@pytest.mark.parametrize("B,N,K", [(1, 100, 256), (7, 64, 4096), (16, 48, 96), (40, 80, 640), (300, 144, 544),
                                   (64, 512, 1024)])
def test_misaligned_weights_bit_identical(nv, oracle, B, N, K):
    # weight codes at offset 1 and E4M3 bytes at offset 3: the byte-load path
    d = si.random_nvfp4_operands(B, N, K, seed=N + K)
    t = {k: torch.from_numpy(v).cuda() for k, v in d.items()}
    y0 = nv.gemm(t["a_codes"], t["a_scale"], t["w_codes"], t["w_sf"], t["w_g"])
    w1, s1 = offset_view(t["w_codes"], 1), offset_view(t["w_sf"], 3)
    y1 = nv.gemm(t["a_codes"], t["a_scale"], w1, s1, t["w_g"])
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    ref = oracle.gemm_ref(d["a_codes"], d["a_scale"], d["w_codes"], d["w_sf"], d["w_g"][0])
    assert oracle.rel_fro(y1.cpu().double().numpy(), ref) <= TOL


@pytest.mark.parametrize("B,N,K", [(1, 64, 16), (3, 40, 48), (16, 96, 4112), (17, 72, 80), (200, 300, 1040)])
@pytest.mark.parametrize("offset", [0, 1])
def test_k_multiple_of_16_only(nv, oracle, B, N, K, offset):
    # K % 32 == 16: the [N, K/16] block scales of the plugin contract with an
    # odd number of 16-blocks per row; quantized operands from the oracle
    a = si.bf16_normal((B, K), 1.0, 83, 0, seed=K)
    w = si.bf16_normal((N, K), 0.02, 83, 1, seed=K)
    qa = oracle.quantize(a)
    qw = oracle.quantize(w, group_rows=N, want_scale=False)
    t = lambda v: torch.from_numpy(v).cuda()
    wc, ws = t(qw["codes"]), t(qw["sf"])
    if offset:
        wc, ws = offset_view(wc, offset), offset_view(ws, offset)
    y = nv.gemm(t(qa["codes"]), t(qa["scale"]), wc, ws, t(qw["g_dec"]))
    torch.cuda.synchronize()
    ref = oracle.gemm_ref(qa["codes"], qa["scale"], qw["codes"], qw["sf"], qw["g_dec"][0])
    assert oracle.rel_fro(y.cpu().double().numpy(), ref) <= TOL


def test_external_weight_matches_oracle_k_multiple_of_16(nv, oracle):
    # external-weight mode ("Fused Nvfp4 GEMM All Reduce Plugin", External-weight
    # inputs) against the fp64 oracle, with K % 32 == 16 and unaligned weights
    B, N, K = 24, 80, 208
    a = si.bf16_normal((B, K), 1.0, 84, 0)
    w = si.bf16_normal((N, K), 0.02, 84, 1)
    qa = oracle.quantize(a)
    qw = oracle.quantize(w, group_rows=N, want_scale=False)
    t = lambda v: torch.from_numpy(v).cuda()
    wc, ws = offset_view(t(qw["codes"]), 5), offset_view(t(qw["sf"]), 1)
    nv.register_weight(77, wc, ws)
    try:
        y = nv.gemm_external(t(qa["codes"]), t(qa["scale"]), 77, N, t(qw["g_dec"]))
        torch.cuda.synchronize()
    finally:
        nv.unregister_weight(77, torch.cuda.current_device())
    ref = oracle.gemm_ref(qa["codes"], qa["scale"], qw["codes"], qw["sf"], qw["g_dec"][0])
    assert oracle.rel_fro(y.cpu().double().numpy(), ref) <= TOL


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_per_tensor_quantize_at_2_byte_offset(nv, oracle, dtype):
    # not 16-byte aligned: the scalar row kernel, fed the group's partial maxima
    rows, k = 96, 272
    x = si.normal_f32((rows, k), 0.5, 85, 0)
    x = torch.from_numpy(x).to(dtype)
    q = oracle.quantize(x, group_rows=rows)
    xg = offset_view(x.cuda(), 2)
    assert xg.data_ptr() % 16 == 2
    g = nv.quantize(xg, group_rows=rows)
    q2 = oracle.quantize(x, group_rows=rows // 4)
    g2 = nv.quantize(xg, group_rows=rows // 4)
    torch.cuda.synchronize()
    for want, got in ((q, g), (q2, g2)):
        for k_ in ("codes", "sf"):
            assert np.array_equal(got[k_].cpu().numpy(), want[k_]), k_
        for k_ in ("g_dec", "scale"):
            assert np.array_equal(got[k_].cpu().numpy().view(np.uint32), want[k_].view(np.uint32)), k_


# ---------------------------------------------------------------- MoE sizes

def _moe_case(oracle, T, E, hidden, inter, seed):
    logits = si.normal_f32((T, E), 1.0, 86, 3, seed)
    bias = si.normal_f32((E,), 0.1, 86, 4, seed)
    x = si.fp16_normal((T, hidden), 1.0, 86, 0, seed)
    w1 = si.bf16_normal((E * inter, hidden), 0.02, 86, 1, seed)
    w2 = si.bf16_normal((E * hidden, inter), 0.02, 86, 2, seed)
    q1 = oracle.quantize(w1, group_rows=inter, want_scale=False)
    q2 = oracle.quantize(w2, group_rows=hidden, want_scale=False)
    return dict(logits=logits, bias=bias, x=x,
                w1=(q1["codes"].reshape(E, inter, hidden // 2), q1["sf"].reshape(E, inter, hidden // 16), q1["g_dec"]),
                w2=(q2["codes"].reshape(E, hidden, inter // 2), q2["sf"].reshape(E, hidden, inter // 16), q2["g_dec"]))


def _moe_check(nv, oracle, c, top_k, n_group, topk_group, tokens):
    t = lambda v: torch.from_numpy(np.ascontiguousarray(v)).cuda()
    out, ids, wts = nv.moe_w4a16(t(c["logits"]), t(c["bias"]), c["x"].cuda(), *map(t, c["w1"]), *map(t, c["w2"]),
                                 top_k=top_k, n_group=n_group, topk_group=topk_group, want_routing=True)
    torch.cuda.synchronize()
    rid, rw = oracle.route(c["logits"], c["bias"], top_k, n_group, topk_group, True, 1.0)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.array_equal(wts.cpu().numpy().view(np.uint32), rw.view(np.uint32))
    o = out.cpu().double().numpy()
    assert np.all(np.isfinite(o))
    ref = oracle.moe_ref(c["x"].numpy(), rid, rw, *c["w1"], *c["w2"], tokens=tokens)
    assert oracle.rel_fro(o[tokens], ref) <= TOL


@pytest.mark.parametrize("T", [512, 520, 1024])
def test_moe_more_than_4096_pairs(nv, oracle, T):
    # T * top_k = 4096, 4160, 8192 (token, expert) pairs: both branches of the
    # routing-list kernel, and the share per wave above its register cache
    c = _moe_case(oracle, T, 64, 128, 128, seed=T)
    _moe_check(nv, oracle, c, 8, 8, 4, tokens=list(range(0, T, 7)) + [T - 1])


def test_moe_one_expert_above_65536_tokens(nv, oracle):
    T = 66000
    c = _moe_case(oracle, T, 2, 64, 64, seed=1)
    c["logits"][:, 0] = 30.0           # every token picks expert 0 (top-1): score ~1 vs ~0
    c["logits"][:, 1] = -30.0
    _moe_check(nv, oracle, c, 1, 1, 1, tokens=[0, 1, 4095, 40000, 65535, 65536, T - 1])


# ---------------------------------------------------------------- canaries

GUARD = 4096
PAT = 0xA5


class Guarded:
    """Output buffers with GUARD canary bytes on both sides."""

    def __init__(self):
        self.bufs = []

    def __call__(self, shape, dtype):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        buf = torch.full((n + 2 * GUARD,), PAT, dtype=torch.uint8, device="cuda")
        self.bufs.append((buf, n))
        return buf[GUARD:GUARD + n].view(dtype).view(shape)

    def check(self):
        torch.cuda.synchronize()
        for i, (buf, n) in enumerate(self.bufs):
            h = buf.cpu().numpy()
            assert np.all(h[:GUARD] == PAT) and np.all(h[GUARD + n:] == PAT), "buffer %d overrun" % i


def test_no_writes_outside_any_output(nv, oracle):
    g = Guarded()
    dev = "cuda"
    # quantize per token / per tensor, act_quant SwiGLU (ragged shapes)
    x = si.bf16_normal((37, 208), 1.0, 87, 0).to(dev)
    for grp in (1, 37):
        o = {"codes": g((37, 104), torch.uint8), "sf": g((37, 13), torch.uint8),
             "g_dec": g((37 // grp,), torch.float32), "scale": g((37, 13), torch.float32)}
        ws = g((max(nv.quantize_workspace_size(37, 208, grp), 1),), torch.uint8)
        nv.quantize(x, group_rows=grp, out=o, workspace=ws)
    xs = si.swiglu_input(rows=5, H=272).to(dev)
    nv.act_quant(xs, "swiglu", out={"codes": g((5, 136), torch.uint8), "sf": g((5, 17), torch.uint8),
                                    "g_dec": g((5,), torch.float32), "scale": g((5, 17), torch.float32)})
    # GEMM: decode, prefill, register-staged (K % 64 != 0), byte-load paths
    for B, N, K in [(5, 96, 256), (300, 528, 640), (70, 72, 96), (9, 40, 48), (130, 40, 80)]:
        d = si.random_nvfp4_operands(B, N, K, seed=B)
        t = {k: torch.from_numpy(v).to(dev) for k, v in d.items()}
        y = g((B, N), torch.float16)
        ws = g((max(nv.gemm_workspace_size(B, N, K), 1),), torch.uint8)
        nv.gemm(t["a_codes"], t["a_scale"], t["w_codes"], t["w_sf"], t["w_g"], out=y, workspace=ws)
        if N % 16 == 0 and K % 128 == 0:
            wt = nv.pretile_weight(t["w_codes"], t["w_sf"])
            wt2 = {"codes": g((N * K // 2,), torch.uint8), "sf": g((N * K // 16,), torch.uint8), "N": N, "K": K}
            assert nv.lib().nvfp4_pretile_weight(ctypes.c_void_p(t["w_codes"].data_ptr()),
                                          ctypes.c_void_p(t["w_sf"].data_ptr()), N, K,
                                          ctypes.c_void_p(wt2["codes"].data_ptr()),
                                          ctypes.c_void_p(wt2["sf"].data_ptr()),
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
            nv.gemm_pretiled(t["a_codes"], t["a_scale"], wt, t["w_g"], out=g((B, N), torch.float16), workspace=ws)
        nv.register_weight(91, t["w_codes"], t["w_sf"])
        try:
            nv.gemm_external(t["a_codes"], t["a_scale"], 91, N, t["w_g"], out=g((B, N), torch.float16), workspace=ws)
        finally:
            torch.cuda.synchronize()
            nv.unregister_weight(91, torch.cuda.current_device())
    # MoE
    T, E, H, I = 40, 16, 128, 192
    c = _moe_case(oracle, T, E, H, I, seed=2)
    tt = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev)
    L = nv.lib()
    out, ids, wts = g((T, H), torch.float16), g((T, 4), torch.int32), g((T, 4), torch.float32)
    wsb = nv.moe_workspace_size(T, E, 4, H, I)
    ws = g((wsb,), torch.uint8)
    args = [tt(c["logits"]), tt(c["bias"]), c["x"].to(dev), *map(tt, c["w1"]), *map(tt, c["w2"])]
    rc = L.nvfp4_moe_w4a16(*[ctypes.c_void_p(a.data_ptr()) for a in args], ctypes.c_void_p(out.data_ptr()),
                           ctypes.c_void_p(ids.data_ptr()), ctypes.c_void_p(wts.data_ptr()), T, E, 4, H, I, 4, 2,
                           1, 1.0, ctypes.c_void_p(ws.data_ptr()), wsb,
                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == nv.NVFP4_OK
    # MXFP4: row and tile layouts (ragged rows), tile permutation, GEMM
    xm = si.bf16_normal((45, 256), 1.0, 88, 0).to(dev)
    nv.mx_quantize(xm, out={"codes": g((45, 128), torch.uint8), "sf": g((45, 8), torch.uint8),
                            "g_dec": g((45,), torch.float32)})
    nc, ns = nv.mx_tiled_sizes(45, 256)
    qa = nv.mx_quantize(xm, tiled=True, out={"codes": g((nc,), torch.uint8), "sf": g((ns,), torch.uint8),
                                             "g_dec": g((45,), torch.float32)})
    dm = si.random_mx_operands(45, 64, 256, seed=4)
    wq = nv.mx_tile(torch.from_numpy(dm["w_codes"]).to(dev), torch.from_numpy(dm["w_sf"]).to(dev))
    ct, st = g((64 * 128,), torch.uint8), g((64 * 8,), torch.uint8)
    wrow = (torch.from_numpy(dm["w_codes"]).to(dev), torch.from_numpy(dm["w_sf"]).to(dev))
    assert L.nvfp4_mx_tile(ctypes.c_void_p(wrow[0].data_ptr()), ctypes.c_void_p(wrow[1].data_ptr()), 64, 256,
                           ctypes.c_void_p(ct.data_ptr()), ctypes.c_void_p(st.data_ptr()),
                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    for B in (45, 20):   # wide and skinny MX kernels
        nv.mx_gemm(dict(qa, rows=B) if B == 45 else nv.mx_quantize(xm[:B], tiled=True), qa["g_dec"][:B], wq,
                   torch.from_numpy(dm["w_g"]).to(dev), out=g((B, 64), torch.float16))
    g.check()


# ---------------------------------------------------------------- launches per call

def _hip():
    # the HIP runtime torch and the library already share (one soname)
    return ctypes.CDLL("libamdhip64.so.7")


def _captured_node_types(fn):
    """Runs fn(stream) once to warm up, then captures it into a HIP graph and
    returns the types of the graph's nodes (0 = kernel)."""
    hip = _hip()
    s = torch.cuda.Stream()
    fn(s)
    torch.cuda.synchronize()
    h = ctypes.c_void_p(s.cuda_stream)
    assert hip.hipStreamBeginCapture(h, 2) == 0          # relaxed capture mode
    fn(s)
    graph = ctypes.c_void_p()
    assert hip.hipStreamEndCapture(h, ctypes.byref(graph)) == 0
    n = ctypes.c_size_t(0)
    assert hip.hipGraphGetNodes(graph, None, ctypes.byref(n)) == 0
    nodes = (ctypes.c_void_p * max(n.value, 1))()
    assert hip.hipGraphGetNodes(graph, nodes, ctypes.byref(n)) == 0
    types = []
    for i in range(n.value):
        ty = ctypes.c_int(-1)
        assert hip.hipGraphNodeGetType(ctypes.c_void_p(nodes[i]), ctypes.byref(ty)) == 0
        types.append(ty.value)
    hip.hipGraphDestroy(graph)
    torch.cuda.synchronize()
    return types


def test_kernel_launches_per_call(nv, oracle):
    dev = "cuda"
    x = si.bf16_normal((64, 256), 1.0, 89, 0).to(dev)
    xs = si.swiglu_input(rows=8, H=256).to(dev)
    qa = nv.act_quant(x, "none")
    d8 = {k: torch.from_numpy(v).to(dev) for k, v in si.random_nvfp4_operands(8, 128, 256, seed=1).items()}
    d256 = {k: torch.from_numpy(v).to(dev) for k, v in si.random_nvfp4_operands(256, 512, 256, seed=2).items()}
    wt = nv.pretile_weight(d256["w_codes"], d256["w_sf"])
    ws = torch.empty(max(nv.gemm_workspace_size(256, 512, 256), nv.quantize_workspace_size(64, 256, 64)),
                     dtype=torch.uint8, device=dev)
    y8 = torch.empty((8, 128), dtype=torch.float16, device=dev)
    y256 = torch.empty((256, 512), dtype=torch.float16, device=dev)
    c = _moe_case(oracle, 16, 8, 64, 64, seed=3)
    tt = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev)
    margs = [tt(c["logits"]), tt(c["bias"]), c["x"].to(dev), *map(tt, c["w1"]), *map(tt, c["w2"])]
    mout = torch.empty((16, 64), dtype=torch.float16, device=dev)
    mws = torch.empty(nv.moe_workspace_size(16, 8, 2, 64, 64), dtype=torch.uint8, device=dev)
    c2 = _moe_case(oracle, 16, 8, 128, 128, seed=4)
    w1t = nv.moe_pretile_weights(tt(c2["w1"][0]), tt(c2["w1"][1]))
    w2t = nv.moe_pretile_weights(tt(c2["w2"][0]), tt(c2["w2"][1]))
    margs_t = [tt(c2["logits"]), tt(c2["bias"]), c2["x"].to(dev), *w1t, tt(c2["w1"][2]), *w2t, tt(c2["w2"][2])]
    mout_t = torch.empty((16, 128), dtype=torch.float16, device=dev)
    mws_t = torch.empty(nv.moe_workspace_size(16, 8, 2, 128, 128), dtype=torch.uint8, device=dev)
    qo = {"codes": torch.empty((64, 128), dtype=torch.uint8, device=dev),
          "sf": torch.empty((64, 16), dtype=torch.uint8, device=dev),
          "g_dec": torch.empty((64,), dtype=torch.float32, device=dev),
          "scale": torch.empty((64, 16), dtype=torch.float32, device=dev)}
    mq = nv.mx_quantize(x, tiled=True)
    mw = nv.mx_quantize(si.bf16_normal((128, 256), 0.02, 89, 1).to(dev), group_rows=128, tiled=True)
    my = torch.empty((64, 128), dtype=torch.float16, device=dev)
    mrow = nv.mx_quantize(x)
    # expected kernels per call
    cases = {
        "act_quant": (1, lambda s: nv.act_quant(x, "none", out=qo, stream=s)),
        "act_quant_swiglu": (1, lambda s: nv.act_quant(xs, "swiglu", out=dict(
            qo, codes=qo["codes"][:8], sf=qo["sf"][:8], g_dec=qo["g_dec"][:8], scale=qo["scale"][:8]), stream=s)),
        "quantize_per_tensor": (3, lambda s: nv.quantize(x, group_rows=64, out=qo, workspace=ws, stream=s)),
        "gemm_decode": (1, lambda s: nv.gemm(d8["a_codes"], d8["a_scale"], d8["w_codes"], d8["w_sf"], d8["w_g"],
                                             out=y8, stream=s)),
        "gemm_prefill": (2, lambda s: nv.gemm(d256["a_codes"], d256["a_scale"], d256["w_codes"], d256["w_sf"],
                                              d256["w_g"], out=y256, workspace=ws, stream=s)),
        "gemm_pretiled": (2, lambda s: nv.gemm_pretiled(d256["a_codes"], d256["a_scale"], wt, d256["w_g"],
                                                        out=y256, workspace=ws, stream=s)),
        "pretile_weight": (1, lambda s: nv.pretile_weight(d256["w_codes"], d256["w_sf"], stream=s)),
        "moe": (5, lambda s: nv.moe_w4a16(*margs, top_k=2, n_group=2, topk_group=1, out=mout, workspace=mws,
                                          stream=s)),
        "moe_pretiled": (5, lambda s: nv.moe_w4a16_pretiled(*margs_t, top_k=2, n_group=2, topk_group=1, out=mout_t,
                                                            workspace=mws_t, stream=s)),
        "mx_quantize_tiled": (1, lambda s: nv.mx_quantize(x, tiled=True, out=mq, stream=s)),
        "mx_tile": (1, lambda s: nv.mx_tile(mrow["codes"], mrow["sf"], stream=s)),
        "mx_gemm": (1, lambda s: nv.mx_gemm(mq, mq["g_dec"], mw, mw["g_dec"], out=my, stream=s)),
    }
    for name, (want, fn) in cases.items():
        types = _captured_node_types(fn)
        assert types == [0] * want, (name, types)

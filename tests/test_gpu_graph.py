"""HIP-graph replays of the hot path reproduce the eager results bit for bit.

The secondary workloads of bench.py are timed by replaying HIP graphs of
library calls.  This test captures one call of every entry point on the path
(per-tensor and per-token NVFP4 quantization, fused SwiGLU quantization on the
tabulated kernel, decode and prefill GEMM, the pre-tiled GEMM, the MoE layer,
MX quantization into the tile layout and the MX GEMM) in one graph, replays it
several times with eager work and synchronizations between the replays, and
compares every replay with the eager outputs.  The kernels are deterministic
(fixed reduction orders, integer-max atomics only), so the comparison is exact.
The library itself issues no memsets and no allocations; every buffer the
captured calls write is allocated before the capture.
"""
import numpy as np
import pytest
import torch

import synth_inputs as si

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import nvfp4_block_scaled_quantize_amd as nv
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return nv


def _flat(obj):
    """Every tensor of a result (tensor, dict or tuple) in a fixed order."""
    if isinstance(obj, torch.Tensor):
        return [obj]
    if isinstance(obj, dict):
        return [t for k in sorted(obj) for t in _flat(obj[k])]
    if isinstance(obj, (tuple, list)):
        return [t for o in obj for t in _flat(o)]
    return []


def test_graph_replays_match_eager(nv):
    dev = torch.device("cuda:0")
    torch.manual_seed(0)
    # operands: NVFP4 weights [512, 512] per tensor, activations for decode
    # (B = 4) and prefill (B = 256), SwiGLU rows for the tabulated kernel
    a_pre, w = si.gemm_inputs("C1", B=256, K=512, N=512)
    a_dec = a_pre[:4].contiguous()
    x_sw = si.swiglu_input(rows=1024, H=512).to(dev)
    w_d, a_pre_d, a_dec_d = w.to(dev), a_pre.to(dev), a_dec.to(dev)
    md = si.moe_inputs(T=32, E=16, hidden=256, inter=128)
    E, T, Hd, I, topk = 16, 32, 256, 128, 4

    def q_out(rows, k, groups, scale=True):
        return {"codes": torch.empty((rows, k // 2), dtype=torch.uint8, device=dev),
                "sf": torch.empty((rows, k // 16), dtype=torch.uint8, device=dev),
                "g_dec": torch.empty((groups,), dtype=torch.float32, device=dev),
                "scale": torch.empty((rows, k // 16), dtype=torch.float32, device=dev) if scale else None}

    outs = {
        "wq": q_out(512, 512, 1, scale=False),
        "qdec": q_out(4, 512, 4),
        "qpre": q_out(256, 512, 256),
        "qsw": q_out(1024, 512, 1024),
        "ydec": torch.empty((4, 512), dtype=torch.float16, device=dev),
        "ypre": torch.empty((256, 512), dtype=torch.float16, device=dev),
        "ytl": torch.empty((256, 512), dtype=torch.float16, device=dev),
        "moe": torch.empty((T, Hd), dtype=torch.float16, device=dev),
        "ymx": torch.empty((256, 512), dtype=torch.float16, device=dev),
    }
    nc, ns = nv.mx_tiled_sizes(256, 512)
    outs["mxa"] = {"codes": torch.empty(nc, dtype=torch.uint8, device=dev),
                   "sf": torch.empty(ns, dtype=torch.uint8, device=dev),
                   "g_dec": torch.empty((256,), dtype=torch.float32, device=dev)}
    wsq = torch.empty(max(nv.quantize_workspace_size(512, 512, 512), 256), dtype=torch.uint8,
                      device=dev)
    wsg = torch.empty(max(nv.gemm_workspace_size(256, 512, 512), 256), dtype=torch.uint8, device=dev)
    wsm = torch.empty(nv.moe_workspace_size(T, E, topk, Hd, I), dtype=torch.uint8, device=dev)
    # MoE and MX weights are prepared once, outside the graph
    w1 = nv.quantize(md["w1"].to(dev), group_rows=I, want_scale=False)
    w2 = nv.quantize(md["w2"].to(dev), group_rows=Hd, want_scale=False)
    margs = [torch.from_numpy(md["logits"]).to(dev), torch.from_numpy(md["bias"]).to(dev), md["x"].to(dev),
             w1["codes"].view(E, I, Hd // 2), w1["sf"].view(E, I, Hd // 16), w1["g_dec"],
             w2["codes"].view(E, Hd, I // 2), w2["sf"].view(E, Hd, I // 16), w2["g_dec"]]
    mkw = dict(top_k=topk, n_group=4, topk_group=2, norm_topk_prob=True, routed_scaling=1.0,
               out=outs["moe"], workspace=wsm)
    mxw = nv.mx_quantize(w_d, group_rows=512, tiled=True)

    def run():
        wq = nv.quantize(w_d, group_rows=512, want_scale=False, out=outs["wq"], workspace=wsq)
        wt = nv.pretile_weight(wq["codes"], wq["sf"]) if "wt" not in outs else outs["wt"]
        outs["wt"] = wt
        qd = nv.act_quant(a_dec_d, "none", out=outs["qdec"])
        qp = nv.act_quant(a_pre_d, "none", out=outs["qpre"])
        nv.act_quant(x_sw, "swiglu", out=outs["qsw"])
        nv.gemm(qd["codes"], qd["scale"], wq["codes"], wq["sf"], wq["g_dec"], out=outs["ydec"], workspace=wsg)
        nv.gemm(qp["codes"], qp["scale"], wq["codes"], wq["sf"], wq["g_dec"], out=outs["ypre"], workspace=wsg)
        nv.gemm_pretiled(qp["codes"], qp["scale"], wt, wq["g_dec"], out=outs["ytl"], workspace=wsg)
        nv.moe_w4a16(*margs, **mkw)
        qa = nv.mx_quantize(a_pre_d, tiled=True, out=outs["mxa"])
        nv.mx_gemm(qa, qa["g_dec"], mxw, mxw["g_dec"], out=outs["ymx"])

    # eager pass (also pre-tiles the weight once, outside the graph)
    run()
    torch.cuda.synchronize()
    keys = [k for k in sorted(outs) if k != "wt"]
    ref = [t.clone() for k in keys for t in _flat(outs[k])]
    assert all(t.numel() > 0 for t in ref)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        # clear every output and do unrelated eager work between the replays
        for k in keys:
            for t in _flat(outs[k]):
                t.zero_()
        junk = torch.randn(1 << 20, device=dev).cumsum(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t for k in keys for t in _flat(outs[k])]
        assert len(got) == len(ref)
        for i, (x, y) in enumerate(zip(got, ref)):
            assert torch.equal(x.view(torch.uint8) if x.dtype != torch.uint8 else x,
                               y.view(torch.uint8) if y.dtype != torch.uint8 else y), (rep, i)
        del junk
    # the replayed outputs are non-trivial
    assert float(outs["ypre"].float().abs().sum()) > 0 and float(outs["moe"].float().abs().sum()) > 0
    assert np.isfinite(outs["ymx"].float().cpu().numpy()).all()

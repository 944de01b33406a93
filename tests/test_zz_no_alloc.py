"""The no-allocation MoE entry point, nvfp4_moe_w4a16_noalloc, against the
workspace entry point nvfp4_moe_w4a16 through the C ABI.

Two calls in a row on the library's fixed device scratch -- the C5 layer
(256 tokens, 64 experts, top-8, hidden 2048, inter 1024), then a smaller
layer that finds the first call's contents in the scratch -- each
bit-identical to the workspace entry point on the same inputs, and within
1e-3 of the fp64 oracle on sampled tokens with the oracle's routing ids and
weights exactly.  Inputs are drawn directly in the stored NVFP4 formats by
the seeded generators.
"""
import ctypes

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


def _layer(T, E, hidden, inter, seed):
    f1 = si.random_nvfp4_operands(1, E * inter, hidden, seed=seed, config=62)
    f2 = si.random_nvfp4_operands(1, E * hidden, inter, seed=seed, config=63)
    # a different global per expert, small enough that the FP16 output stays
    # far from overflow with these full-range random scale bytes
    g1 = (f1["w_g"][0] * np.exp2(-(np.arange(E) % 3))).astype(np.float32)
    g2 = (f2["w_g"][0] * np.exp2(-2 - (np.arange(E) % 2))).astype(np.float32)
    return dict(T=T, E=E, hidden=hidden, inter=inter,
                logits=si.normal_f32((T, E), 1.0, 90, 3, seed), bias=si.normal_f32((E,), 0.1, 90, 4, seed),
                x=si.fp16_normal((T, hidden), 1.0, 90, 0, seed),
                w1=(f1["w_codes"].reshape(E, inter, hidden // 2), f1["w_sf"].reshape(E, inter, hidden // 16), g1),
                w2=(f2["w_codes"].reshape(E, hidden, inter // 2), f2["w_sf"].reshape(E, hidden, inter // 16), g2))


def _run(nv, c, top_k, n_group, topk_group, noalloc):
    dev = "cuda"
    t = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev)
    ins = [t(c["logits"]), t(c["bias"]), c["x"].to(dev), *map(t, c["w1"]), *map(t, c["w2"])]
    T, E, H, I = c["T"], c["E"], c["hidden"], c["inter"]
    out = torch.empty((T, H), dtype=torch.float16, device=dev)
    ids = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    for buf in (out, ids, wts):
        buf.view(torch.uint8).fill_(0x5A)
    p = [ctypes.c_void_p(a.data_ptr()) for a in ins + [out, ids, wts]]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    L = nv.lib()
    if noalloc:
        rc = L.nvfp4_moe_w4a16_noalloc(*p, T, E, top_k, H, I, n_group, topk_group, 1, 1.0, stream)
    else:
        nb = L.nvfp4_moe_w4a16_workspace_size(T, E, top_k, H, I)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        rc = L.nvfp4_moe_w4a16(*p, T, E, top_k, H, I, n_group, topk_group, 1, 1.0,
                               ctypes.c_void_p(ws.data_ptr()), nb, stream)
    assert rc == nv.NVFP4_OK, rc
    torch.cuda.synchronize()
    return out.cpu(), ids.cpu().numpy(), wts.cpu().numpy()


def _check_pair(nv, oracle, c, top_k, n_group, topk_group, tokens):
    got = _run(nv, c, top_k, n_group, topk_group, noalloc=True)
    want = _run(nv, c, top_k, n_group, topk_group, noalloc=False)
    assert torch.equal(got[0].view(torch.int16), want[0].view(torch.int16))
    assert np.array_equal(got[1], want[1])
    assert np.array_equal(got[2].view(np.uint32), want[2].view(np.uint32))
    rid, rw = oracle.route(c["logits"], c["bias"], top_k, n_group, topk_group, True, 1.0)
    assert np.array_equal(got[1], rid)
    assert np.array_equal(got[2].view(np.uint32), rw.view(np.uint32))
    ref = oracle.moe_ref(c["x"].numpy(), rid, rw, *c["w1"], *c["w2"], tokens=tokens)
    o = got[0].double().numpy()
    assert np.all(np.isfinite(o))
    assert oracle.rel_fro(o[tokens], ref) <= TOL
    return got


def test_noalloc_matches_workspace_entry_point_twice(nv, oracle):
    # first call: the C5 layer (about 20 MiB of the 32 MiB scratch)
    big = _layer(256, 64, 2048, 1024, seed=5)
    assert nv.moe_workspace_size(256, 64, 8, 2048, 1024) <= nv.NOALLOC_SCRATCH_BYTES
    first = _check_pair(nv, oracle, big, 8, 8, 4, tokens=[0, 1, 77, 128, 200, 255])
    # second call: a smaller layer on the same scratch, which still holds the
    # first call's contents
    small = _layer(37, 16, 256, 128, seed=6)
    _check_pair(nv, oracle, small, 4, 4, 2, tokens=list(range(37)))
    # and the first layer again: the same bytes as before
    again = _run(nv, big, 8, 8, 4, noalloc=True)
    assert torch.equal(again[0].view(torch.int16), first[0].view(torch.int16))


def test_noalloc_refuses_a_problem_beyond_its_scratch(nv):
    c = _layer(8, 64, 2048, 1024, seed=7)
    T = 4096   # workspace of 4096 tokens exceeds the fixed scratch
    assert nv.moe_workspace_size(T, 64, 8, 2048, 1024) > nv.NOALLOC_SCRATCH_BYTES
    dev = "cuda"
    t = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev)
    ins = [t(np.zeros((T, 64), np.float32)), t(c["bias"]), torch.zeros((T, 2048), dtype=torch.float16, device=dev),
           *map(t, c["w1"]), *map(t, c["w2"])]
    out = torch.zeros((T, 2048), dtype=torch.float16, device=dev)
    rc = nv.lib().nvfp4_moe_w4a16_noalloc(*[ctypes.c_void_p(a.data_ptr()) for a in ins + [out]], None, None,
                                          T, 64, 8, 2048, 1024, 8, 4, 1, 1.0, None)
    assert rc == nv.NVFP4_ESCRATCH
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0   # nothing launched

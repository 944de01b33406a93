"""GPU parity of nvfp4_moe_w4a16 against the oracle.

Routing ("Nvfp4 A16 Blackwell Moe Runner", Nvfp4A16BlackwellMoeParams:
sigmoid group-top-k with correction bias, normTopkProb, routedScalingFactor):
expert ids must equal the oracle's exactly and the weights bit-for-bit (both
sides evaluate the same binary32 operations).  Layer output: relative
Frobenius error <= 1e-3 against the fp64 oracle on the same NVFP4 weights
(quantized per expert by the oracle) and the oracle's routing.
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


def _case(oracle, T, E, hidden, inter, seed, w_std=0.02):
    logits = si.normal_f32((T, E), 1.0, 70, 3, seed)
    bias = si.normal_f32((E,), 0.1, 70, 4, seed)
    x = si.fp16_normal((T, hidden), 1.0, 70, 0, seed)
    w1 = si.bf16_normal((E * inter, hidden), w_std, 70, 1, seed)
    w2 = si.bf16_normal((E * hidden, inter), w_std, 70, 2, seed)
    q1 = oracle.quantize(w1, group_rows=inter, want_scale=False)
    q2 = oracle.quantize(w2, group_rows=hidden, want_scale=False)
    return dict(logits=logits, bias=bias, x=x,
                w1=(q1["codes"].reshape(E, inter, hidden // 2), q1["sf"].reshape(E, inter, hidden // 16), q1["g_dec"]),
                w2=(q2["codes"].reshape(E, hidden, inter // 2), q2["sf"].reshape(E, hidden, inter // 16), q2["g_dec"]))


def _run(nv, c, top_k, n_group, topk_group, norm=True, scaling=1.0):
    dev = "cuda"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    out, ids, wts = nv.moe_w4a16(t(c["logits"]), t(c["bias"]), c["x"].to(dev), t(c["w1"][0]), t(c["w1"][1]),
                                 t(c["w1"][2]), t(c["w2"][0]), t(c["w2"][1]), t(c["w2"][2]), top_k=top_k,
                                 n_group=n_group, topk_group=topk_group, norm_topk_prob=norm,
                                 routed_scaling=scaling, want_routing=True)
    torch.cuda.synchronize()
    return out.cpu().double().numpy(), ids.cpu().numpy(), wts.cpu().numpy()


def _check(oracle, nv, c, top_k, n_group, topk_group, norm=True, scaling=1.0, tokens=None):
    out, ids, wts = _run(nv, c, top_k, n_group, topk_group, norm, scaling)
    rid, rw = oracle.route(c["logits"], c["bias"], top_k, n_group, topk_group, norm, scaling)
    assert np.array_equal(ids, rid)
    assert np.array_equal(wts.view(np.uint32), rw.view(np.uint32))
    ref = oracle.moe_ref(c["x"].numpy(), rid, rw, *c["w1"], *c["w2"], tokens=tokens)
    got = out if tokens is None else out[tokens]
    err = oracle.rel_fro(got, ref)
    assert err <= TOL, err
    assert np.all(np.isfinite(out))


@pytest.mark.parametrize("T,E,top_k,n_group,topk_group,hidden,inter",
                         [(5, 8, 2, 2, 1, 64, 128), (32, 16, 4, 4, 2, 256, 128), (70, 64, 8, 8, 4, 128, 64),
                          (300, 32, 6, 4, 3, 192, 320), (3, 256, 16, 16, 4, 64, 64),
                          (600, 8, 4, 2, 2, 64, 64), (200, 8, 2, 2, 2, 448, 320),
                          (1500, 4, 1, 1, 1, 576, 128), (1, 8, 2, 2, 1, 64, 64), (8, 4, 2, 1, 1, 64, 8192),
                          (2048, 8, 2, 2, 2, 64, 64), (2049, 8, 2, 2, 2, 64, 64)])
def test_small_layers(nv, oracle, T, E, top_k, n_group, topk_group, hidden, inter):
    c = _case(oracle, T, E, hidden, inter, seed=T + E)
    _check(oracle, nv, c, top_k, n_group, topk_group)


def test_nan_router_logits_rank_last(nv, oracle):
    # a NaN score ranks below every number (the reading both sides implement)
    c = _case(oracle, 64, 32, 128, 64, seed=21)
    rng = np.random.default_rng(21)
    lg = c["logits"].copy()
    lg[rng.random(lg.shape) < 0.05] = np.nan
    c["logits"] = lg
    _check(oracle, nv, c, 4, 4, 2)


@pytest.mark.parametrize("T,E,top_k,n_group,topk_group,levels",
                         [(96, 64, 8, 8, 4, 5), (96, 64, 8, 8, 4, 1), (40, 256, 16, 16, 4, 3),
                          (64, 32, 6, 4, 3, 2), (48, 16, 4, 16, 4, 2)])
def test_routing_ties_resolved_by_lower_index(nv, oracle, T, E, top_k, n_group, topk_group, levels):
    # router logits and bias drawn from a few values (levels = 1: every score
    # equal), so biased scores, group scores and candidates tie often; both
    # sides take the higher score first and the lower index on ties (the
    # oracle by repeated selection, the kernel by rank counts)
    c = _case(oracle, T, E, 64, 64, seed=T + E + levels)
    rng = np.random.default_rng(T + E + levels)
    c["logits"] = (rng.integers(0, levels, size=(T, E)) * 0.5).astype(np.float32)
    c["bias"] = (rng.integers(0, levels, size=(E,)) * 0.25).astype(np.float32)
    _check(oracle, nv, c, top_k, n_group, topk_group)


def test_infinite_bias_matches_oracle(nv, oracle):
    # +inf / -inf correction biases and NaN logits: infinite biased scores,
    # and groups whose two best sum to NaN (ranked below every number on both
    # sides); ids exact, weights bit for bit
    c = _case(oracle, 64, 32, 64, 64, seed=33)
    rng = np.random.default_rng(33)
    bias = c["bias"].copy()
    bias[[0, 5, 9, 20]] = np.inf
    bias[[1, 4, 8, 21, 30]] = -np.inf
    lg = c["logits"].copy()
    lg[rng.random(lg.shape) < 0.05] = np.nan
    c["bias"], c["logits"] = bias, lg
    # two experts per group: groups {0, 1}, {4, 5}, {8, 9}, {20, 21} sum +inf and -inf
    _check(oracle, nv, c, 4, 16, 4)


def test_no_normalisation_and_scaling(nv, oracle):
    c = _case(oracle, 24, 16, 64, 64, seed=9)
    _check(oracle, nv, c, 4, 4, 2, norm=False, scaling=2.5)


def test_full_size_sampled_tokens(nv, oracle):
    cf = si.CONFIGS["C5"]
    d = si.moe_inputs()
    E, H, I = d["E"], d["hidden"], d["inter"]
    q1 = oracle.quantize(d["w1"], group_rows=I, want_scale=False)
    q2 = oracle.quantize(d["w2"], group_rows=H, want_scale=False)
    c = dict(logits=d["logits"], bias=d["bias"], x=d["x"],
             w1=(q1["codes"].reshape(E, I, H // 2), q1["sf"].reshape(E, I, H // 16), q1["g_dec"]),
             w2=(q2["codes"].reshape(E, H, I // 2), q2["sf"].reshape(E, H, I // 16), q2["g_dec"]))
    _check(oracle, nv, c, cf["top_k"], cf["n_group"], cf["topk_group"], cf["norm_topk_prob"],
           cf["routed_scaling"], tokens=[0, 1, 2, 100, 200, 255])


def test_deterministic(nv, oracle):
    c = _case(oracle, 40, 16, 128, 64, seed=11)
    a = _run(nv, c, 4, 4, 2)[0]
    b = _run(nv, c, 4, 4, 2)[0]
    assert np.array_equal(a, b)


@pytest.mark.parametrize("T,E,top_k,n_group,topk_group,hidden,inter",
                         [(32, 16, 4, 4, 2, 256, 128), (300, 32, 6, 4, 3, 384, 256),
                          (200, 8, 2, 2, 2, 640, 384),     # 640 rows: the last fc2 tile past N
                          (8, 4, 2, 1, 1, 128, 8192),      # inter at its maximum (64 fc1 row tiles)
                          (1, 8, 2, 2, 1, 128, 128)])
def test_pretiled_weights_bit_identical(nv, oracle, T, E, top_k, n_group, topk_group, hidden, inter):
    # nvfp4_moe_w4a16_pretiled on moe_pretile_weights() of the same weights:
    # the same values through the same arithmetic, only the copy layout differs
    c = _case(oracle, T, E, hidden, inter, seed=T + E + 1)
    dev = "cuda"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    w1, s1, w2, s2 = t(c["w1"][0]), t(c["w1"][1]), t(c["w2"][0]), t(c["w2"][1])
    args = (t(c["logits"]), t(c["bias"]), c["x"].to(dev))
    kw = dict(top_k=top_k, n_group=n_group, topk_group=topk_group, want_routing=True)
    y0, i0, w0 = nv.moe_w4a16(*args, w1, s1, t(c["w1"][2]), w2, s2, t(c["w2"][2]), **kw)
    w1t, s1t = nv.moe_pretile_weights(w1, s1)
    w2t, s2t = nv.moe_pretile_weights(w2, s2)
    y1, i1, w1w = nv.moe_w4a16_pretiled(*args, w1t, s1t, t(c["w1"][2]), w2t, s2t, t(c["w2"][2]), **kw)
    torch.cuda.synchronize()
    assert torch.equal(i0, i1) and torch.equal(w0.view(torch.int32), w1w.view(torch.int32))
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    rid, rw = oracle.route(c["logits"], c["bias"], top_k, n_group, topk_group, True, 1.0)
    ref = oracle.moe_ref(c["x"].numpy(), rid, rw, *c["w1"], *c["w2"])
    assert oracle.rel_fro(y1.cpu().double().numpy(), ref) <= TOL


def test_pretiled_weights_full_size(nv, oracle):
    # the benchmarked layer: pre-tiled and plain weights give the same output
    cf = si.CONFIGS["C5"]
    d = si.moe_inputs()
    E, H, I = d["E"], d["hidden"], d["inter"]
    q1 = oracle.quantize(d["w1"], group_rows=I, want_scale=False)
    q2 = oracle.quantize(d["w2"], group_rows=H, want_scale=False)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    w1, s1 = t(q1["codes"].reshape(E, I, H // 2)), t(q1["sf"].reshape(E, I, H // 16))
    w2, s2 = t(q2["codes"].reshape(E, H, I // 2)), t(q2["sf"].reshape(E, H, I // 16))
    g1, g2 = t(q1["g_dec"]), t(q2["g_dec"])
    args = (t(d["logits"]), t(d["bias"]), d["x"].cuda())
    kw = dict(top_k=cf["top_k"], n_group=cf["n_group"], topk_group=cf["topk_group"],
              norm_topk_prob=cf["norm_topk_prob"], routed_scaling=cf["routed_scaling"])
    y0 = nv.moe_w4a16(*args, w1, s1, g1, w2, s2, g2, **kw)
    y1 = nv.moe_w4a16_pretiled(*args, *nv.moe_pretile_weights(w1, s1), g1, *nv.moe_pretile_weights(w2, s2), g2, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))

"""Pins of the fp64 GEMM / MoE references and of the oracle router.

GEMM: y[B,N] = deq(a)[B,K] . deq(w)[N,K]^T ("Fused Nvfp4 GEMM All Reduce
Plugin", Baked-weight inputs and Output).  Pinned by a plain triple loop on
tiny operands and by closed forms (identity, permutation and all-ones weights).

Router: sigmoid group-top-k with a correction bias ("Nvfp4 A16 Blackwell Moe
Runner", Nvfp4A16BlackwellMoeParams).  Pinned by exhaustive enumeration of all
group and expert subsets on small cases, by the tie rule, and by invariants.
"""
import itertools

import numpy as np
import pytest
import torch

import synth_inputs as si


def _quant_pair(oracle, B, N, K, seed):
    a = si.bf16_normal((B, K), 1.0, 98, 0, seed)
    w = si.bf16_normal((N, K), 0.02, 98, 1, seed)
    qa = oracle.quantize(a)
    qw = oracle.quantize(w, group_rows=N)
    return qa, qw


def test_gemm_matmul_equals_triple_loop(oracle):
    qa, qw = _quant_pair(oracle, 3, 5, 48, 0)
    A = oracle.dequant_act(qa["codes"], qa["scale"])
    W = oracle.dequant_weight(qw["codes"], qw["sf"], qw["g_dec"][0])
    y = oracle.gemm_ref(qa["codes"], qa["scale"], qw["codes"], qw["sf"], qw["g_dec"][0])
    y2 = oracle.gemm_ref_loops(A, W)
    assert np.allclose(y, y2, rtol=1e-12, atol=1e-15)


def _unit_weight(N, K, pattern):
    """Weights whose dequantized value is exactly `pattern` (entries 0/1):
    code 2 (=1.0) where pattern is 1, E4M3 scale 0x38 (=1.0), global 1.0."""
    nib = np.where(pattern > 0, 2, 0).astype(np.uint8)
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    sf = np.full((N, K // 16), 0x38, np.uint8)
    return codes, sf, np.float32(1.0)


def test_gemm_closed_forms(oracle):
    B, K = 4, 64
    qa, _ = _quant_pair(oracle, B, 8, K, 1)
    A = oracle.dequant_act(qa["codes"], qa["scale"])
    # identity
    wc, ws, wg = _unit_weight(K, K, np.eye(K))
    y = oracle.gemm_ref(qa["codes"], qa["scale"], wc, ws, wg)
    assert np.array_equal(y, A)
    # permutation: output column n reads weight row n
    perm = np.random.default_rng(0).permutation(K)
    P = np.zeros((K, K)); P[np.arange(K), perm] = 1
    wc, ws, wg = _unit_weight(K, K, P)
    y = oracle.gemm_ref(qa["codes"], qa["scale"], wc, ws, wg)
    assert np.array_equal(y, A[:, perm])
    # all ones: row sums
    wc, ws, wg = _unit_weight(3, K, np.ones((3, K)))
    y = oracle.gemm_ref(qa["codes"], qa["scale"], wc, ws, wg)
    assert np.allclose(y, np.repeat(A.sum(axis=1, keepdims=True), 3, axis=1), rtol=1e-14)
    # the global weight scale multiplies every output
    y2 = oracle.gemm_ref(qa["codes"], qa["scale"], wc, ws, np.float32(0.25))
    assert np.array_equal(y2, y * 0.25)


def test_dequant_weight_uses_block_scale_per_16(oracle):
    wc, ws, wg = _unit_weight(2, 64, np.ones((2, 64)))
    ws = ws.copy(); ws[1, 2] = 0x40                      # 2.0 on row 1, block 2
    W = oracle.dequant_weight(wc, ws, wg)
    assert np.all(W[0] == 1.0)
    assert np.all(W[1, 32:48] == 2.0) and np.all(W[1, :32] == 1.0) and np.all(W[1, 48:] == 1.0)


# ---------------------------------------------------------------- router

def _brute_route(s, b, top_k, n_group, topk_group):
    """Exhaustive: the kept groups are the group subset whose sorted score
    vector is largest; the chosen experts the subset (inside kept groups) whose
    sorted biased-score vector is largest; output in decreasing score order."""
    E = len(b)
    gsz = E // n_group
    gscore = []
    for g in range(n_group):
        v = sorted(b[g * gsz:(g + 1) * gsz], reverse=True)
        gscore.append(np.float32(v[0]) + np.float32(v[1]) if gsz > 1 else np.float32(v[0]))
    best_groups = max(itertools.combinations(range(n_group), topk_group),
                      key=lambda gs: sorted((gscore[g] for g in gs), reverse=True))
    cand = [e for e in range(E) if e // gsz in best_groups]
    best = max(itertools.combinations(cand, top_k),
               key=lambda es: sorted((b[e] for e in es), reverse=True))
    return sorted(best, key=lambda e: -b[e])


@pytest.mark.parametrize("E,n_group,topk_group,top_k", [(8, 2, 1, 3), (12, 4, 2, 4), (16, 4, 3, 5)])
def test_route_exhaustive_small(oracle, E, n_group, topk_group, top_k):
    rng = np.random.default_rng(E)
    T = 40
    logits = rng.standard_normal((T, E)).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.1).astype(np.float32)
    ids, w = oracle.route(logits, bias, top_k, n_group, topk_group, True, 1.0)
    for t in range(T):
        s = [oracle.sigmoid_f32(float(v)) for v in logits[t]]
        b = [np.float32(np.float32(si_) + bias[e]) for e, si_ in enumerate(s)]
        want = _brute_route(s, b, top_k, n_group, topk_group)
        assert list(ids[t]) == want, t
        ws = np.array([s[e] for e in want], np.float32)
        assert np.allclose(w[t], ws / ws.sum(), rtol=1e-6)


def test_route_nan_scores_rank_last(oracle):
    # NaN is given no order by the pages; the reading taken is that a NaN
    # score ranks below every number (ties among them to the lower index)
    logits = np.zeros((3, 8), np.float32)
    logits[0, 0] = np.nan                 # would otherwise win the tie at index 0
    logits[1, :] = np.nan                 # every score NaN: lowest indices of the kept group
    logits[2, 5] = 4.0
    logits[2, 4] = np.nan
    bias = np.zeros(8, np.float32)
    ids, w = oracle.route(logits, bias, 2, 2, 1, True, 1.0)
    assert ids[0].tolist() == [1, 2]
    assert ids[1].tolist() == [0, 1]
    assert ids[2].tolist() == [5, 6]
    assert np.all(np.isfinite(w[[0, 2]]))


def test_route_nan_group_score_ranks_last(oracle):
    # a group whose two best biased scores are +inf and -inf (an infinite
    # correction bias) sums to NaN; the reading: like a NaN expert score, it
    # ranks below every number.  Worked by hand: s = 0.5 for every expert;
    # group scores g0 = inf + -inf -> NaN (ranks last), g1 = 0.6 + 0.5 = 1.1,
    # g2 = 1.0, g3 = 0.7 + 0.7 = 1.4; the two kept groups are g3, g1; the
    # best two candidates 6 and 7 (0.7, a tie: lower index first).
    logits = np.zeros((2, 8), np.float32)
    bias = np.array([np.inf, -np.inf, 0.1, 0.0, 0.0, 0.0, 0.2, 0.2], np.float32)
    bias2 = bias.copy()
    bias2[[0, 1]] = bias[[1, 0]]          # the same group with its experts swapped
    ids, w = oracle.route(logits[:1], bias, 2, 4, 2, True, 1.0)
    assert ids.tolist() == [[6, 7]]
    assert np.array_equal(w, np.array([[0.5, 0.5]], np.float32))
    ids2, _ = oracle.route(logits[:1], bias2, 2, 4, 2, True, 1.0)
    assert ids2.tolist() == [[6, 7]]
    # every group NaN or -inf: the lowest-index groups are kept, and the
    # +inf experts (biased score +inf) rank first within them
    b3 = np.array([np.inf, -np.inf, -np.inf, np.inf, np.inf, -np.inf, -np.inf, -np.inf], np.float32)
    ids3, _ = oracle.route(logits[:1], b3, 2, 4, 2, True, 1.0)
    assert ids3.tolist() == [[0, 3]]


def test_route_ties_go_to_lower_index(oracle):
    logits = np.zeros((2, 16), np.float32)
    bias = np.zeros(16, np.float32)
    ids, w = oracle.route(logits, bias, 3, 4, 2, True, 2.5)
    assert ids.tolist() == [[0, 1, 2], [0, 1, 2]]
    assert np.allclose(w, 2.5 / 3, rtol=1e-6)


def test_route_invariants_c5_shape(oracle):
    d = si.moe_inputs(weights=False)
    c = si.CONFIGS["C5"]
    ids, w = oracle.route(d["logits"], d["bias"], c["top_k"], c["n_group"], c["topk_group"],
                          c["norm_topk_prob"], c["routed_scaling"])
    gsz = c["E"] // c["n_group"]
    for t in range(c["T"]):
        assert len(set(ids[t].tolist())) == c["top_k"]
        assert len({int(e) // gsz for e in ids[t]}) <= c["topk_group"]
        assert abs(float(w[t].sum()) - c["routed_scaling"]) < 1e-5
        b = [np.float32(oracle.sigmoid_f32(float(v))) + d["bias"][e] for e, v in enumerate(d["logits"][t])]
        assert all(b[ids[t][j]] >= b[ids[t][j + 1]] for j in range(c["top_k"] - 1))


def test_route_without_normalisation_returns_sigmoid(oracle):
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((5, 16)).astype(np.float32)
    bias = np.zeros(16, np.float32)
    ids, w = oracle.route(logits, bias, 4, 4, 2, False, 1.5)
    for t in range(5):
        for j in range(4):
            assert w[t, j] == np.float32(np.float32(oracle.sigmoid_f32(float(logits[t, ids[t, j]]))) * np.float32(1.5))


def test_moe_ref_closed_form(oracle):
    # fc1 and fc2 equal to identity: out_t = sum_j w_tj * relu(x_t)^2
    H = 32
    T, E, top_k = 6, 4, 2
    x = torch.from_numpy(np.random.default_rng(4).standard_normal((T, H)).astype(np.float32)).half()
    wc, ws, _ = _unit_weight(H, H, np.eye(H))
    w1c = np.stack([wc] * E); w1s = np.stack([ws] * E); g = np.ones(E, np.float32)
    ids = np.array([[t % E, (t + 1) % E] for t in range(T)], np.int32)
    wts = np.full((T, top_k), 0.5, np.float32)
    out = oracle.moe_ref(x.numpy(), ids, wts, w1c, w1s, g, w1c, w1s, g)
    xr = np.maximum(x.double().numpy(), 0) ** 2
    assert np.allclose(out, xr, rtol=1e-14)
    # expert global scales multiply fc1 (squared by ReLU^2) and fc2 outputs
    g1 = np.full(E, 2.0, np.float32); g2 = np.full(E, 3.0, np.float32)
    out2 = oracle.moe_ref(x.numpy(), ids, wts, w1c, w1s, g1, w1c, w1s, g2)
    assert np.allclose(out2, xr * 4.0 * 3.0, rtol=1e-14)


def _select_weight(N, K, src, sf_byte):
    """Weights [N, K] whose row n holds code 2 (= 1.0) at column src[n] and
    zeros elsewhere, every block scale the E4M3 byte sf_byte."""
    nib = np.zeros((N, K), np.uint8)
    nib[np.arange(N), src] = 2
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return codes, np.full((N, K // 16), sf_byte, np.uint8)


def test_moe_ref_distinct_experts_closed_form(oracle):
    # Every expert is a different selection: fc1_e row i picks x[p_e(i)]
    # (inter != hidden, so a transposed operand cannot even be formed), fc2_e
    # row n picks h[q_e(n)]; expert e has its own power-of-two globals g1[e],
    # g2[e] and its own E4M3 block scale s1[e], s2[e]; routing weights differ
    # per token and rank, and x has negative entries.  Then exactly
    #   out_t[n] = sum_j w_tj * g2[e] s2[e] * (g1[e] s1[e])^2 * relu(x_t[p_e(q_e(n))])^2
    # with e = ids[t, j] ("Nvfp4 A16 Blackwell Moe Runner": per-expert
    # globalScales, ReLU2, normalised top-k weights applied per rank).
    rng = np.random.default_rng(44)
    T, E, top_k, H, I = 7, 5, 3, 32, 48
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).half()
    p = [rng.integers(0, H, I) for _ in range(E)]          # fc1 row i <- x[p_e(i)]
    q = [rng.permutation(I)[:H] for _ in range(E)]         # fc2 row n <- h[q_e(n)]
    e4m3 = {0x30: 0.5, 0x38: 1.0, 0x40: 2.0, 0x48: 4.0}
    s1b = [0x38, 0x40, 0x30, 0x48, 0x38]
    s2b = [0x40, 0x38, 0x48, 0x30, 0x30]
    g1 = np.array([1.0, 0.5, 2.0, 0.25, 4.0], np.float32)
    g2 = np.array([2.0, 0.125, 1.0, 8.0, 0.5], np.float32)
    w1 = [_select_weight(I, H, p[e], s1b[e]) for e in range(E)]
    w2 = [_select_weight(H, I, q[e], s2b[e]) for e in range(E)]
    w1c = np.stack([c for c, _ in w1]); w1s = np.stack([s for _, s in w1])
    w2c = np.stack([c for c, _ in w2]); w2s = np.stack([s for _, s in w2])
    ids = np.stack([rng.permutation(E)[:top_k] for _ in range(T)]).astype(np.int32)
    wts = rng.uniform(0.1, 1.0, (T, top_k)).astype(np.float32)
    out = oracle.moe_ref(x.numpy(), ids, wts, w1c, w1s, g1, w2c, w2s, g2)
    xd = x.double().numpy()
    want = np.zeros((T, H))
    for t in range(T):
        for j in range(top_k):
            e = int(ids[t, j])
            f = float(g2[e]) * e4m3[s2b[e]] * (float(g1[e]) * e4m3[s1b[e]]) ** 2
            want[t] += float(wts[t, j]) * f * np.maximum(xd[t, p[e][q[e]]], 0.0) ** 2
    assert np.allclose(out, want, rtol=1e-13, atol=0.0)
    # `tokens` selects rows of the same result
    sub = oracle.moe_ref(x.numpy(), ids, wts, w1c, w1s, g1, w2c, w2s, g2, tokens=[5, 0, 3])
    assert np.array_equal(sub, out[[5, 0, 3]])


# ---------------------------------------------------------------- pre-tiled weights

def test_pretile_worked_positions(oracle):
    # distinct byte values make each position unambiguous: code byte j of
    # row r is (r * 64 + j) % 251, scale byte j of row r is (r * 8 + j) % 127
    N, K = 32, 256
    w = np.fromfunction(lambda r, j: (r * 64 + j) % 251, (N, K // 2)).astype(np.uint8)
    s = np.fromfunction(lambda r, j: (r * 8 + j) % 127, (N, K // 16)).astype(np.uint8)
    wt, st = oracle.pretile_weight(w, s)
    tile = lambda G, c, lane: (G * (K // 128) + c) * 64 + lane
    # group 0, chunk 0, lane 17 = row 1, k 32..63 -> code bytes 16..31, scale bytes 2, 3
    assert wt[16 * 17:16 * 18].tolist() == w[1, 16:32].tolist()
    assert st[2 * 17:2 * 18].tolist() == s[1, 2:4].tolist()
    # group 1, chunk 1, lane 63 = row 31, k = 128 + 96 .. 255 -> code bytes 112..127, scale 14, 15
    t = tile(1, 1, 63)
    assert wt[16 * t:16 * t + 16].tolist() == w[31, 112:128].tolist()
    assert st[2 * t:2 * t + 2].tolist() == s[31, 14:16].tolist()
    # a row group is contiguous: group 1 starts at 16 rows * K/2 bytes
    assert wt[16 * tile(1, 0, 0):16 * tile(1, 0, 0) + 16].tolist() == w[16, 0:16].tolist()


def test_pretile_reshape_matches_loops_and_is_a_permutation(oracle):
    rng = np.random.default_rng(12)
    for N, K in [(16, 128), (48, 384), (32, 1024)]:
        w = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
        s = rng.integers(0, 127, (N, K // 16), dtype=np.uint8)
        wt, st = oracle.pretile_weight(w, s)
        wl, sl = oracle.pretile_weight_loops(w, s)
        assert np.array_equal(wt, wl) and np.array_equal(st, sl)
        assert np.array_equal(np.sort(wt), np.sort(w.reshape(-1)))
        assert np.array_equal(np.sort(st), np.sort(s.reshape(-1)))

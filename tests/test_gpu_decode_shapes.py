"""Decode GEMM (B <= 16: gemm_skinny4 on the FP4 matrix cores for B <= 4,
gemm_skinny16 on dequantized FP16 weights above) over the shapes that
exercise their work split: each wave owns every eighth 128-k chunk of K and
processes them in rounds of four, with two activation groups of two chunks
per round.  Shapes cover waves without chunks (K < 1024), a partial last
chunk (K % 128 != 0, with K % 64 == 0 on the FP4 kernel's 16-byte activation
loads and K % 64 == 32 on its byte loads), K % 32 == 16 (weights on the
byte-load path), full and partial rounds, several rounds per wave
(K = 16384), ragged N, one and two token pairs of the FP4 kernel, and both
activation-item widths of the FP16 kernel (B <= 8, <= 16).  Operands are oracle-quantized
from seeded bf16 data ("Fused Nvfp4 GEMM All Reduce Plugin", Baked-weight
inputs); every element is checked against the fp64 oracle within the bound of
the arithmetic, and the weight layouts (plain rows, byte loads at an odd
offset, pre-tiled) and the activation-code alignments give bit-identical
outputs.
"""
import numpy as np
import pytest
import torch

import synth_inputs as si
from gemm_checks import offset_view, refs, row_checks

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import nvfp4_block_scaled_quantize_amd as nv
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return nv


SHAPES = [(1, 32, 16),          # one partial chunk; seven waves without chunks
          (2, 40, 48),          # K % 32 == 16: byte-load weights
          (4, 96, 640),         # five chunks: one partial round per wave
          (3, 17, 1024),        # ragged N, one chunk per wave
          (2, 96, 4096 + 64),   # FP4 kernel: partial last chunk, 16-byte activation loads
          (4, 256, 4224),       # FP4 kernel, two pairs: a full and a partial round on wave 0
          (1, 64, 2048 + 32),   # FP4 kernel: partial last chunk, byte activation loads
          (5, 64, 4096),        # FP16 kernel: one full round per wave
          (8, 256, 4224),       # 33 chunks: a full and a partial round on wave 0
          (13, 48, 8192 + 32),  # widest items, partial last chunk
          (16, 1040, 16384)]    # four rounds per wave, N not a multiple of 32


@pytest.mark.parametrize("B,N,K", SHAPES)
def test_decode_shapes(nv, oracle, B, N, K):
    a = si.bf16_normal((B, K), 1.0, 91, 0, seed=B * 7 + K)
    w = si.bf16_normal((N, K), 0.02, 91, 1, seed=N + K)
    qa = oracle.quantize(a)
    qw = oracle.quantize(w, group_rows=N, want_scale=False)
    t = lambda v: torch.from_numpy(np.ascontiguousarray(v)).cuda()
    ac, asc, wc, ws, wg = t(qa["codes"]), t(qa["scale"]), t(qw["codes"]), t(qw["sf"]), t(qw["g_dec"][:1])
    ys = {}
    if K % 32 == 0:
        ys["plain"] = nv.gemm(ac, asc, wc, ws, wg)
        ys["act codes at offset 2"] = nv.gemm(offset_view(ac, 2), asc, wc, ws, wg)
    ys["weights at odd offsets"] = nv.gemm(ac, asc, offset_view(wc, 1), offset_view(ws, 3), wg)
    if K % 128 == 0 and N % 16 == 0:
        ys["pre-tiled"] = nv.gemm_pretiled(ac, asc, nv.pretile_weight(wc, ws), wg)
    torch.cuda.synchronize()
    A = oracle.dequant_act(qa["codes"], qa["scale"])
    W = oracle.dequant_weight(qw["codes"], qw["sf"], qw["g_dec"][0])
    ref, absref = refs(A, W)
    first = None
    for name, y in ys.items():
        row_checks(y.cpu().double().numpy(), ref, absref, K, 2.0 ** -11)
        if first is None:
            first = (name, y)
        else:
            assert torch.equal(y.view(torch.int16), first[1].view(torch.int16)), (name, first[0])

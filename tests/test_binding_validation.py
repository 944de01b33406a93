"""The Python binding rejects operands the C ABI cannot check (dtype, shape,
element count of operands and caller-supplied outputs) before any call; on
the CPU every well-formed call then stops at the device check.  No GPU."""
import pytest
import torch


@pytest.fixture(scope="module")
def nv():
    import nvfp4_block_scaled_quantize_amd as nv
    return nv


def u8(*s):
    return torch.zeros(s, dtype=torch.uint8)


def f32(*s):
    return torch.zeros(s, dtype=torch.float32)


def test_quantize_and_act_quant(nv):
    x = torch.zeros((4, 64), dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="bfloat16 or float16"):
        nv.quantize(x.float())
    with pytest.raises(ValueError, match="2-D"):
        nv.quantize(torch.zeros(64, dtype=torch.bfloat16))
    good = {"codes": u8(4, 32), "sf": u8(4, 4), "g_dec": f32(4), "scale": f32(4, 4)}
    for key, bad in [("codes", u8(4, 16)), ("sf", u8(4, 3)), ("g_dec", f32(3)), ("scale", f32(4, 5)),
                     ("codes", torch.zeros((4, 32), dtype=torch.int8))]:
        o = dict(good, **{key: bad})
        with pytest.raises((TypeError, ValueError), match=key):
            nv.quantize(x, out=o)
    with pytest.raises(ValueError, match="codes"):
        nv.act_quant(torch.zeros((4, 128), dtype=torch.bfloat16), "swiglu", out=dict(good, codes=u8(4, 64)))
    with pytest.raises(ValueError, match="GPU"):
        nv.quantize(x, out=good)


def test_gemm_operands(nv):
    B, N, K = 4, 32, 64
    ok = dict(a_codes=u8(B, K // 2), a_scale=f32(B, K // 16), w_codes=u8(N, K // 2), w_sf=u8(N, K // 16),
              w_g=f32(1))
    for key, bad, exc in [("a_scale", f32(B, K // 32), ValueError), ("a_scale", u8(B, K // 16), TypeError),
                          ("w_codes", u8(N, K // 4), ValueError), ("w_sf", u8(N, 3), ValueError),
                          ("w_g", f32(0), ValueError), ("w_g", torch.zeros(1, dtype=torch.float64), TypeError),
                          ("a_codes", torch.zeros((B, K // 2), dtype=torch.int16), TypeError)]:
        with pytest.raises(exc, match=key):
            nv.gemm(**dict(ok, **{key: bad}))
    with pytest.raises(ValueError, match="out"):
        nv.gemm(**ok, out=torch.zeros((B, N + 1), dtype=torch.float16))
    with pytest.raises(TypeError, match="out"):
        nv.gemm(**ok, out=torch.zeros((B, N), dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU"):
        nv.gemm(**ok)
    wt = {"codes": u8(N * K // 2 - 1), "sf": u8(N * K // 16), "N": N, "K": K}
    with pytest.raises(ValueError, match="codes"):
        nv.gemm_pretiled(ok["a_codes"], ok["a_scale"], wt, ok["w_g"])
    with pytest.raises(ValueError, match="K"):
        nv.gemm_pretiled(ok["a_codes"], ok["a_scale"], dict(wt, K=2 * K), ok["w_g"])
    with pytest.raises(ValueError, match="out"):
        nv.gemm_external(ok["a_codes"], ok["a_scale"], 3, N, ok["w_g"], out=torch.zeros((B, 2 * N), dtype=torch.float16))
    with pytest.raises(ValueError, match="w_sf"):
        nv.register_weight(5, ok["w_codes"], u8(N, 5))
    with pytest.raises(ValueError, match="w_sf"):
        nv.pretile_weight(ok["w_codes"], u8(N + 1, K // 16))


def test_moe_operands(nv):
    T, E, H, I = 6, 8, 64, 128
    ok = [f32(T, E), f32(E), torch.zeros((T, H), dtype=torch.float16), u8(E, I, H // 2), u8(E, I, H // 16),
          f32(E), u8(E, H, I // 2), u8(E, H, I // 16), f32(E)]
    names = ["logits", "bias", "x", "w1", "w1_sf", "w1_g", "w2", "w2_sf", "w2_g"]
    bads = {"logits": torch.zeros((T, E), dtype=torch.bfloat16), "bias": f32(E - 1),
            "x": torch.zeros((T, H), dtype=torch.bfloat16), "w1_sf": u8(E, I, H // 8), "w1_g": f32(E - 1),
            "w2": u8(E, H, I), "w2_sf": u8(E, H + 1, I // 16), "w2_g": f32(2)}
    kw = dict(top_k=2, n_group=2, topk_group=1)
    for name, bad in bads.items():
        args = list(ok)
        args[names.index(name)] = bad
        with pytest.raises((TypeError, ValueError), match=name):
            nv.moe_w4a16(*args, **kw)
    with pytest.raises(ValueError, match="out"):
        nv.moe_w4a16(*ok, **kw, out=torch.zeros((T, H + 64), dtype=torch.float16))
    with pytest.raises(ValueError, match="GPU"):
        nv.moe_w4a16(*ok, **kw)


def test_mx_operands(nv):
    x = torch.zeros((40, 256), dtype=torch.float16)
    nc, ns = nv.mx_tiled_sizes(40, 256)
    with pytest.raises(ValueError, match="codes"):
        nv.mx_quantize(x, tiled=True, out={"codes": u8(nc - 1), "sf": u8(ns), "g_dec": f32(40)})
    with pytest.raises(ValueError, match="sf"):
        nv.mx_quantize(x, out={"codes": u8(40, 128), "sf": u8(40, 4), "g_dec": f32(40)})
    with pytest.raises(ValueError, match="sf"):
        nv.mx_tile(u8(40, 128), u8(40, 9))
    a = {"codes": u8(nc), "sf": u8(ns), "rows": 40, "K": 256, "tiled": True}
    w = {"codes": u8(64 * 128), "sf": u8(64 * 8), "rows": 64, "K": 256, "tiled": True}
    with pytest.raises(ValueError, match="a_g"):
        nv.mx_gemm(a, f32(39), w, f32(1))
    with pytest.raises(TypeError, match="w_g"):
        nv.mx_gemm(a, f32(40), w, torch.zeros(1, dtype=torch.float16))
    with pytest.raises(ValueError, match="GPU"):
        nv.mx_gemm(a, f32(40), w, f32(1))

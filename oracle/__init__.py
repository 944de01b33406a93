"""CPU oracle for the NVFP4 hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never imports,
links or calls it, and it shares no code with the HIP kernels.

Two parts:

* ``nvfp4_oracle.c`` (plain C, binary32, no contraction) -- the quantizer, the
  activations, the exp it uses, and the MoE router.  Quantized codes and scale
  bytes are integer results decided by binary32 arithmetic, so both sides take
  those decisions in binary32; this file fixes every operation.
* this module (numpy float64) -- dequantization and the GEMM / MoE references.
  The GEMM reference is the definition itself: y = deq(a) . deq(w)^T in fp64
  ("Fused Nvfp4 GEMM All Reduce Plugin", Baked-weight inputs and Output).

The readings the pages leave open are listed at the top of ``nvfp4_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_nvfp4.so")

ACT_NONE, ACT_SWIGLU, ACT_RELU2 = 0, 1, 2
DTYPE_BF16, DTYPE_FP16 = 0, 1

# gcc flags: IEEE binary32 on SSE, one rounding per operation, no contraction.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fno-builtin",
          "-fPIC", "-shared"]


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (building the checker, not using it)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        c_f, c_d, c_u8, c_i, c_i64, c_p = (ctypes.c_float, ctypes.c_double, ctypes.c_uint8,
                                           ctypes.c_int, ctypes.c_int64, ctypes.c_void_p)
        L.oracle_e4m3_decode.argtypes = [c_u8]; L.oracle_e4m3_decode.restype = c_d
        L.oracle_e4m3_encode.argtypes = [c_f]; L.oracle_e4m3_encode.restype = c_u8
        L.oracle_e2m1_decode.argtypes = [c_u8]; L.oracle_e2m1_decode.restype = c_d
        L.oracle_e2m1_encode.argtypes = [c_f]; L.oracle_e2m1_encode.restype = c_u8
        L.oracle_exp.argtypes = [c_f]; L.oracle_exp.restype = c_f
        L.oracle_swiglu.argtypes = [c_f, c_f]; L.oracle_swiglu.restype = c_f
        L.oracle_relu2.argtypes = [c_f]; L.oracle_relu2.restype = c_f
        L.oracle_sigmoid.argtypes = [c_f]; L.oracle_sigmoid.restype = c_f
        L.oracle_input_to_float.argtypes = [ctypes.c_uint16, c_i]
        L.oracle_input_to_float.restype = c_f
        L.oracle_global_scale.argtypes = [c_f, c_p, c_p]; L.oracle_global_scale.restype = None
        L.oracle_quantize_block.argtypes = [c_p, c_f, c_f, c_p, c_p, c_p]
        L.oracle_quantize_block.restype = None
        L.oracle_quantize.argtypes = [c_p, c_i, c_i64, c_i64, c_i, c_i64, c_p, c_p, c_p, c_p]
        L.oracle_quantize.restype = c_i
        L.oracle_activation.argtypes = [c_p, c_i, c_i64, c_i64, c_i, c_p]
        L.oracle_activation.restype = c_i
        L.oracle_route.argtypes = [c_p, c_p, c_i, c_i, c_i, c_i, c_i, c_i, c_f, c_p, c_p]
        L.oracle_route.restype = c_i
        L.oracle_e8m0_decode.argtypes = [c_u8]; L.oracle_e8m0_decode.restype = c_d
        L.oracle_e8m0_encode_up.argtypes = [c_f]; L.oracle_e8m0_encode_up.restype = c_u8
        L.oracle_mx_quantize_block.argtypes = [c_p, c_f, c_f, c_p, c_p, c_p]
        L.oracle_mx_quantize_block.restype = None
        L.oracle_mx_quantize.argtypes = [c_p, c_i, c_i64, c_i64, c_i, c_i64, c_p, c_p, c_p]
        L.oracle_mx_quantize.restype = c_i
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------
# scalar formats
# --------------------------------------------------------------------------

def e4m3_decode(b: int) -> float:
    return lib().oracle_e4m3_decode(int(b))


def e4m3_encode(x: float) -> int:
    return lib().oracle_e4m3_encode(float(x))


def e2m1_decode(n: int) -> float:
    return lib().oracle_e2m1_decode(int(n))


def e2m1_encode(v: float) -> int:
    return lib().oracle_e2m1_encode(float(v))


def exp_f32(x: float) -> float:
    return lib().oracle_exp(float(x))


def sigmoid_f32(x: float) -> float:
    return lib().oracle_sigmoid(float(x))


def swiglu_f32(g: float, u: float) -> float:
    return lib().oracle_swiglu(float(g), float(u))


def relu2_f32(x: float) -> float:
    return lib().oracle_relu2(float(x))


def global_scale(amax: float):
    ge = ctypes.c_float(); gd = ctypes.c_float()
    lib().oracle_global_scale(float(amax), ctypes.byref(ge), ctypes.byref(gd))
    return ge.value, gd.value


def quantize_block(y16: np.ndarray, g_enc: float, g_dec: float):
    """One 16-element block -> (sf byte, combined fp32 scale, 8 code bytes)."""
    y = np.ascontiguousarray(y16, dtype=np.float32)
    assert y.shape == (16,)
    sf = ctypes.c_uint8(); c = ctypes.c_float(); codes = np.zeros(8, np.uint8)
    lib().oracle_quantize_block(_ptr(y), float(g_enc), float(g_dec), ctypes.byref(sf),
                                ctypes.byref(c), _ptr(codes))
    return sf.value, c.value, codes


# --------------------------------------------------------------------------
# quantizer
# --------------------------------------------------------------------------

def _as_u16(x) -> tuple[np.ndarray, int]:
    """Accept a torch bf16/fp16 CPU tensor or a uint16 numpy array (+dtype)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            dt = {torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_FP16}[x.dtype]
            return np.ascontiguousarray(x.contiguous().view(torch.int16).numpy().view(np.uint16)), dt
    except ImportError:  # pragma: no cover
        pass
    raise TypeError("pass a torch bfloat16/float16 CPU tensor")


def quantize(x, act: int = ACT_NONE, group_rows: int = 1, want_scale: bool = True):
    """NVFP4-quantize a 2-D bf16/fp16 tensor.

    Returns dict(codes [rows, k/2] u8, sf [rows, k/16] u8, g_dec [rows/group_rows] f32,
    scale [rows, k/16] f32 or None).
    """
    u16, dt = _as_u16(x)
    rows, k_in = u16.shape
    k_out = k_in // 2 if act == ACT_SWIGLU else k_in
    codes = np.zeros((rows, k_out // 2), np.uint8)
    sf = np.zeros((rows, k_out // 16), np.uint8)
    g = np.zeros((rows // group_rows if rows else 0,), np.float32)
    c = np.zeros((rows, k_out // 16), np.float32) if want_scale else None
    rc = lib().oracle_quantize(_ptr(u16), dt, rows, k_in, act, group_rows, _ptr(codes), _ptr(sf),
                               _ptr(g), _ptr(c) if c is not None else None)
    if rc != 0:
        raise ValueError("oracle_quantize rejected the arguments")
    return {"codes": codes, "sf": sf, "g_dec": g, "scale": c}


def activation(x, act: int) -> np.ndarray:
    u16, dt = _as_u16(x)
    rows, k_in = u16.shape
    k_out = k_in // 2 if act == ACT_SWIGLU else k_in
    y = np.zeros((rows, k_out), np.float32)
    lib().oracle_activation(_ptr(u16), dt, rows, k_in, act, _ptr(y))
    return y


# --------------------------------------------------------------------------
# dequantization and the fp64 GEMM reference
# --------------------------------------------------------------------------

_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                  -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0], np.float64)


def e4m3_table() -> np.ndarray:
    return np.array([e4m3_decode(b) for b in range(256)], np.float64)


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """[rows, k/2] packed bytes -> [rows, k] nibbles (low nibble = even k)."""
    lo = codes & 0xF
    hi = codes >> 4
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def dequant_act(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Activation operand: e2m1(code) * combined fp32 scale of its 16-block."""
    q = _E2M1[unpack_codes(codes)]
    return q * np.repeat(scale.astype(np.float64), 16, axis=-1)


def dequant_weight(codes: np.ndarray, sf: np.ndarray, g_dec) -> np.ndarray:
    """Weight operand: e2m1(code) * e4m3(block scale) * fp32 global scale."""
    tab = e4m3_table()
    q = _E2M1[unpack_codes(codes)]
    return q * np.repeat(tab[sf], 16, axis=-1) * np.float64(np.float32(g_dec))


def gemm_ref(a_codes, a_scale, w_codes, w_sf, w_g, rows=None) -> np.ndarray:
    """y[B, N] = deq(a) . deq(w)^T in float64 (optionally only for `rows` of a)."""
    if rows is not None:
        a_codes = a_codes[rows]
        a_scale = a_scale[rows]
    A = dequant_act(a_codes, a_scale)
    W = dequant_weight(w_codes, w_sf, w_g)
    return A @ W.T


def gemm_ref_loops(A: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Triple loop in float64 (tiny sizes only) -- pins the library matmul."""
    B, K = A.shape
    N = W.shape[0]
    y = np.zeros((B, N), np.float64)
    for b in range(B):
        for n in range(N):
            s = 0.0
            for k in range(K):
                s += float(A[b, k]) * float(W[n, k])
            y[b, n] = s
    return y


def rel_fro(y, ref) -> float:
    y = np.asarray(y, np.float64); ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(y - ref) / den) if den > 0 else float(np.linalg.norm(y))


# --------------------------------------------------------------------------
# MoE
# --------------------------------------------------------------------------

def route(logits: np.ndarray, bias: np.ndarray, top_k: int, n_group: int, topk_group: int,
          norm_topk_prob: bool = True, routed_scaling: float = 1.0):
    lg = np.ascontiguousarray(logits, np.float32)
    bs = np.ascontiguousarray(bias, np.float32)
    T, E = lg.shape
    ids = np.zeros((T, top_k), np.int32)
    w = np.zeros((T, top_k), np.float32)
    rc = lib().oracle_route(_ptr(lg), _ptr(bs), T, E, top_k, n_group, topk_group,
                            int(bool(norm_topk_prob)), float(routed_scaling), _ptr(ids), _ptr(w))
    if rc != 0:
        raise ValueError("oracle_route rejected the arguments")
    return ids, w


def moe_ref(x_fp16: np.ndarray, ids: np.ndarray, weights: np.ndarray,
            w1_codes, w1_sf, w1_g, w2_codes, w2_sf, w2_g, tokens=None) -> np.ndarray:
    """out[t] = sum_j w[t,j] * (relu(x_t . W1_e^T)^2) . W2_e^T, all in float64.

    ("Nvfp4 A16 Blackwell Moe Runner": FP16 activations, NVFP4 fc1/fc2 weights
    with per-expert FP32 global scales, ReLU2.)  `tokens` restricts the rows.
    Each expert's weights are dequantized once; the per-pair results are summed
    per token in rank order j = 0..top_k-1.
    """
    x = np.asarray(x_fp16).astype(np.float64)
    tok = list(range(x.shape[0])) if tokens is None else list(tokens)
    top_k = ids.shape[1]
    o = {}
    experts = sorted({int(ids[t, j]) for t in tok for j in range(top_k)})
    for e in experts:
        W1 = dequant_weight(w1_codes[e], w1_sf[e], w1_g[e])
        W2 = dequant_weight(w2_codes[e], w2_sf[e], w2_g[e])
        for t in tok:
            for j in range(top_k):
                if int(ids[t, j]) == e:
                    h = np.maximum(W1 @ x[t], 0.0) ** 2
                    o[(t, j)] = W2 @ h
    out = np.zeros((len(tok), x.shape[1]), np.float64)
    for oi, t in enumerate(tok):
        for j in range(top_k):
            out[oi] += float(weights[t, j]) * o[(t, j)]
    return out


# ---------------------------------------------------------------- pre-tiled weights
# The layout is a pure reordering defined in include/nvfp4_mi355x.h (the role
# of the baked N128_K64 weight tiling of "Nvfp4 A16 Blackwell Moe Runner" and
# of the weight shuffles of "feature: add fp4 mm using trtllm backend"):
# row group G = rows 16G..16G+15, 128-k chunk c, 16-byte lane l = r + 16q
# holds the 32 codes of row 16G + r at k = 128c + 32q .. +31; the 2-byte
# scale lane l holds that row's two E4M3 bytes for the same k.

def pretile_weight_loops(w_codes: np.ndarray, w_sf: np.ndarray):
    """The layout written out element by element (small sizes only)."""
    N, K = w_codes.shape[0], w_codes.shape[1] * 2
    nch = K // 128
    wt = np.zeros(N * K // 2, np.uint8)
    st = np.zeros(N * K // 16, np.uint8)
    for G in range(N // 16):
        for c in range(nch):
            for lane in range(64):
                r, q = 16 * G + lane % 16, lane // 16
                k = 128 * c + 32 * q
                t = (G * nch + c) * 64 + lane
                wt[16 * t:16 * t + 16] = w_codes[r, k // 2:k // 2 + 16]
                st[2 * t:2 * t + 2] = w_sf[r, k // 16:k // 16 + 2]
    return wt, st


def pretile_weight(w_codes: np.ndarray, w_sf: np.ndarray):
    """Same layout by reshaping: codes [G, r, c, q, 16 B] -> [G, c, q, r, 16 B],
    E4M3 bytes [G, r, c, q, 2 B] -> [G, c, q, r, 2 B]."""
    N, K = w_codes.shape[0], w_codes.shape[1] * 2
    nch = K // 128
    wt = w_codes.reshape(N // 16, 16, nch, 4, 16).transpose(0, 2, 3, 1, 4).reshape(-1)
    st = w_sf.reshape(N // 16, 16, nch, 4, 2).transpose(0, 2, 3, 1, 4).reshape(-1)
    return np.ascontiguousarray(wt), np.ascontiguousarray(st)


# ---------------------------------------------------------------- MXFP4 variant
# The UE8M0_SF switch of the block helper in "perf: optimize per-token nvfp4
# quantization kernel" (review): E8M0 block scales over 32 elements.  The
# readings are listed at the top of nvfp4_oracle.c.

def e8m0_decode(b: int) -> float:
    return lib().oracle_e8m0_decode(int(b))


def e8m0_encode_up(x: float) -> int:
    return lib().oracle_e8m0_encode_up(float(x))


def mx_quantize_block(y32: np.ndarray, g_enc: float, g_dec: float):
    """One 32-element block -> (E8M0 byte, combined fp32 scale, 16 code bytes)."""
    y = np.ascontiguousarray(y32, dtype=np.float32)
    assert y.shape == (32,)
    sf = ctypes.c_uint8(); c = ctypes.c_float(); codes = np.zeros(16, np.uint8)
    lib().oracle_mx_quantize_block(_ptr(y), float(g_enc), float(g_dec), ctypes.byref(sf),
                                   ctypes.byref(c), _ptr(codes))
    return sf.value, c.value, codes


def mx_quantize(x, act: int = ACT_NONE, group_rows: int = 1):
    """MXFP4-quantize a 2-D bf16/fp16 tensor.

    Returns dict(codes [rows, k/2] u8, sf [rows, k/32] u8 E8M0, g_dec [rows/group_rows] f32).
    """
    u16, dt = _as_u16(x)
    rows, k_in = u16.shape
    k_out = k_in // 2 if act == ACT_SWIGLU else k_in
    codes = np.zeros((rows, k_out // 2), np.uint8)
    sf = np.zeros((rows, k_out // 32), np.uint8)
    g = np.zeros((rows // group_rows if rows else 0,), np.float32)
    rc = lib().oracle_mx_quantize(_ptr(u16), dt, rows, k_in, act, group_rows, _ptr(codes),
                                  _ptr(sf), _ptr(g))
    if rc != 0:
        raise ValueError("oracle_mx_quantize rejected the arguments")
    return {"codes": codes, "sf": sf, "g_dec": g}


def e8m0_table() -> np.ndarray:
    return np.array([e8m0_decode(b) for b in range(256)], np.float64)


def dequant_mx(codes: np.ndarray, sf: np.ndarray, g_dec) -> np.ndarray:
    """e2m1(code) * e8m0(block scale) * fp32 global scale (one per row, or a scalar)."""
    q = _E2M1[unpack_codes(codes)]
    g = np.asarray(g_dec, np.float32).astype(np.float64)
    if g.ndim == 1:
        g = g[:, None]
    return q * np.repeat(e8m0_table()[sf], 32, axis=-1) * g


def mx_gemm_ref(a_codes, a_sf, a_g, w_codes, w_sf, w_g, rows=None) -> np.ndarray:
    """y[B, N] = deq(a) . deq(w)^T in float64; a_g one global per row, w_g a scalar."""
    if rows is not None:
        a_codes, a_sf, a_g = a_codes[rows], a_sf[rows], np.asarray(a_g)[rows]
    A = dequant_mx(a_codes, a_sf, a_g)
    W = dequant_mx(w_codes, w_sf, np.float32(w_g))
    return A @ W.T


# The MX tile layout (defined in include/nvfp4_mi355x.h): rows padded to a
# multiple of 32 with zero codes and zero scale bytes; row group G = rows
# 32G..32G+31; per 64-k chunk a 1 KiB code tile whose 16-byte lane
# l = r + 32h holds the codes of row 32G + r at k = 64c + 32h .. +31; per
# 128-k chunk a 128 B scale tile whose 2-byte lane l = r + 32h holds, in byte j,
# the E8M0 byte of block 4c + 2j + h of row 32G + r.  Tiles are stored
# (G, chunk) row-major.

def mx_tile_loops(codes: np.ndarray, sf: np.ndarray):
    """The layout written out element by element (small sizes only)."""
    R, K = codes.shape[0], codes.shape[1] * 2
    G = (R + 31) // 32
    ct = np.zeros(G * 32 * K // 2, np.uint8)
    st = np.zeros(G * 32 * K // 32, np.uint8)
    for g in range(G):
        for c in range(K // 64):
            for lane in range(64):
                r, h = 32 * g + lane % 32, lane // 32
                if r >= R:
                    continue
                k = 64 * c + 32 * h
                t = (g * (K // 64) + c) * 64 + lane
                ct[16 * t:16 * t + 16] = codes[r, k // 2:k // 2 + 16]
        for c in range(K // 128):
            for lane in range(64):
                r, h = 32 * g + lane % 32, lane // 32
                if r >= R:
                    continue
                t = (g * (K // 128) + c) * 64 + lane
                for j in range(2):
                    st[2 * t + j] = sf[r, 4 * c + 2 * j + h]
    return ct, st


def mx_tile(codes: np.ndarray, sf: np.ndarray):
    """Same layout by reshaping: codes [G, r, c, h, 16 B] -> [G, c, h, r, 16 B];
    scale bytes [G, r, c, j, h] -> [G, c, h, r, j]."""
    R, K = codes.shape[0], codes.shape[1] * 2
    G = (R + 31) // 32
    cp = np.zeros((G * 32, K // 2), np.uint8); cp[:R] = codes
    sp = np.zeros((G * 32, K // 32), np.uint8); sp[:R] = sf
    ct = cp.reshape(G, 32, K // 64, 2, 16).transpose(0, 2, 3, 1, 4).reshape(-1)
    st = sp.reshape(G, 32, K // 128, 2, 2).transpose(0, 2, 4, 1, 3).reshape(-1)
    return np.ascontiguousarray(ct), np.ascontiguousarray(st)

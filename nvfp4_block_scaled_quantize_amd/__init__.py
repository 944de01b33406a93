"""Python binding of libnvfp4_mi355x.so (the C ABI in include/nvfp4_mi355x.h).

Argument marshalling only: every step of the NVFP4 path runs in the HIP
kernels of the shared library.  torch supplies device memory and the current
HIP stream.  There is no CPU fallback: if the library is missing the import
fails, and every call checks the library's status code.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4_mi355x.so")

NVFP4_OK, NVFP4_EINVAL, NVFP4_EUNSUPPORTED, NVFP4_EWORKSPACE, NVFP4_EHIP, NVFP4_ESCRATCH = range(6)
NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024   # NVFP4_NOALLOC_SCRATCH_BYTES
NVFP4_BF16, NVFP4_FP16 = 0, 1
ACT = {"none": 0, "swiglu": 1, "relu2": 2}

EXPORTS = [
    "nvfp4_status_string", "nvfp4_quantize", "nvfp4_quantize_workspace_size", "nvfp4_act_quant",
    "nvfp4_gemm", "nvfp4_gemm_workspace_size", "nvfp4_moe_w4a16", "nvfp4_moe_w4a16_workspace_size",
    "nvfp4_register_weight", "nvfp4_unregister_weight", "nvfp4_gemm_external",
    "nvfp4_pretile_weight", "nvfp4_gemm_pretiled", "nvfp4_mx_quantize", "nvfp4_mx_tile",
    "nvfp4_mx_gemm", "nvfp4_moe_w4a16_noalloc", "nvfp4_moe_w4a16_pretiled",
]
MX_ROWS, MX_TILED = 0, 1


class Nvfp4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (what, _lib.nvfp4_status_string(status).decode(), status))


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError("libnvfp4_mi355x.so is not built; run nvfp4_block_scaled_quantize_amd/build.py "
                          "(hipcc, gfx950) first -- there is no fallback implementation")
    L = ctypes.CDLL(LIB_PATH)
    p, i32, i64, sz, f32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                            ctypes.c_float)
    L.nvfp4_status_string.argtypes = [i32]; L.nvfp4_status_string.restype = ctypes.c_char_p
    L.nvfp4_quantize.argtypes = [p, i32, i64, i64, i64, p, p, p, p, p, sz, p]
    L.nvfp4_quantize.restype = i32
    L.nvfp4_quantize_workspace_size.argtypes = [i64, i64, i64]
    L.nvfp4_quantize_workspace_size.restype = sz
    L.nvfp4_act_quant.argtypes = [p, i32, i64, i64, i32, p, p, p, p, p]
    L.nvfp4_act_quant.restype = i32
    L.nvfp4_gemm.argtypes = [p, p, p, p, p, p, i64, i64, i64, p, sz, p]
    L.nvfp4_gemm.restype = i32
    L.nvfp4_gemm_workspace_size.argtypes = [i64, i64, i64]
    L.nvfp4_gemm_workspace_size.restype = sz
    L.nvfp4_moe_w4a16.argtypes = [p, p, p, p, p, p, p, p, p, p, p, p,
                                  i32, i32, i32, i32, i32, i32, i32, i32, f32, p, sz, p]
    L.nvfp4_moe_w4a16.restype = i32
    L.nvfp4_moe_w4a16_pretiled.argtypes = [p, p, p, p, p, p, p, p, p, p, p, p,
                                           i32, i32, i32, i32, i32, i32, i32, i32, f32, p, sz, p]
    L.nvfp4_moe_w4a16_pretiled.restype = i32
    L.nvfp4_moe_w4a16_noalloc.argtypes = [p, p, p, p, p, p, p, p, p, p, p, p,
                                          i32, i32, i32, i32, i32, i32, i32, i32, f32, p]
    L.nvfp4_moe_w4a16_noalloc.restype = i32
    L.nvfp4_moe_w4a16_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    L.nvfp4_moe_w4a16_workspace_size.restype = sz
    L.nvfp4_register_weight.argtypes = [i32, i32, p, p, i32, i32, i32]
    L.nvfp4_register_weight.restype = i32
    L.nvfp4_unregister_weight.argtypes = [i32, i32]
    L.nvfp4_unregister_weight.restype = i32
    L.nvfp4_gemm_external.argtypes = [p, p, i32, p, p, i64, i64, i64, p, sz, p]
    L.nvfp4_gemm_external.restype = i32
    L.nvfp4_pretile_weight.argtypes = [p, p, i64, i64, p, p, p]
    L.nvfp4_pretile_weight.restype = i32
    L.nvfp4_gemm_pretiled.argtypes = [p, p, p, p, p, p, i64, i64, i64, p, sz, p]
    L.nvfp4_gemm_pretiled.restype = i32
    L.nvfp4_mx_quantize.argtypes = [p, i32, i64, i64, i32, i64, i32, p, p, p, p, sz, p]
    L.nvfp4_mx_quantize.restype = i32
    L.nvfp4_mx_tile.argtypes = [p, p, i64, i64, p, p, p]
    L.nvfp4_mx_tile.restype = i32
    L.nvfp4_mx_gemm.argtypes = [p, p, p, i64, p, p, p, p, i64, i64, i64, p]
    L.nvfp4_mx_gemm.restype = i32
    return L


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_dev(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")


def _need(t, name: str, dtype, shape=None, min_numel=None):
    """Checks what the C ABI cannot: the dtype and the shape (or, for flat
    buffers, the element count) of an operand or a caller-supplied output.  A
    wrong one would be an out-of-bounds device access, so it is an error here."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError("%s must hold at least %d elements, got %d" % (name, min_numel, t.numel()))


def _need_2d(x, name: str):
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("%s must be a 2-D tensor" % name)


def _dtype_code(x: torch.Tensor) -> int:
    if x.dtype == torch.bfloat16:
        return NVFP4_BF16
    if x.dtype == torch.float16:
        return NVFP4_FP16
    raise TypeError("input must be bfloat16 or float16")


def _workspace(nbytes: int, device, workspace: torch.Tensor | None):
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor")
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small: need %d bytes" % nbytes)
        return workspace, workspace.numel() * workspace.element_size()
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def _quant_out(o: dict, rows: int, k: int, ngroups: int):
    """Checks a caller-supplied output dict of quantize() / act_quant()."""
    _need(o.get("codes"), "out['codes']", torch.uint8, (rows, k // 2))
    _need(o.get("sf"), "out['sf']", torch.uint8, (rows, k // 16))
    _need(o.get("g_dec"), "out['g_dec']", torch.float32, min_numel=ngroups)
    if o.get("scale") is not None:
        _need(o["scale"], "out['scale']", torch.float32, (rows, k // 16))


def quantize_workspace_size(rows: int, k: int, group_rows: int) -> int:
    """Bytes of caller workspace that quantize() / mx_quantize() need for one
    global per `group_rows` rows (0 for per-token globals)."""
    return int(_lib.nvfp4_quantize_workspace_size(rows, k, group_rows))


def quantize(x: torch.Tensor, group_rows: int = 1, want_scale: bool = True, out: dict | None = None,
             workspace: torch.Tensor | None = None, stream=None) -> dict:
    """NVFP4-quantize x [rows, k] with one global scale per `group_rows` rows."""
    _need_2d(x, "x")
    _dtype_code(x)
    rows, k = x.shape
    if out is not None:
        _quant_out(out, rows, k, rows // max(group_rows, 1))
    _check_dev(x)
    dev = x.device
    o = out or {
        "codes": torch.empty((rows, k // 2), dtype=torch.uint8, device=dev),
        "sf": torch.empty((rows, k // 16), dtype=torch.uint8, device=dev),
        "g_dec": torch.empty((rows // max(group_rows, 1),), dtype=torch.float32, device=dev),
        "scale": torch.empty((rows, k // 16), dtype=torch.float32, device=dev) if want_scale else None,
    }
    ws, wsb = _workspace(_lib.nvfp4_quantize_workspace_size(rows, k, group_rows), dev, workspace)
    st = _lib.nvfp4_quantize(_ptr(x), _dtype_code(x), rows, k, group_rows, _ptr(o["codes"]), _ptr(o["sf"]),
                             _ptr(o["g_dec"]), _ptr(o.get("scale")), _ptr(ws), wsb, _stream(stream))
    if st != NVFP4_OK:
        raise Nvfp4Error(st, "nvfp4_quantize")
    return o


def act_quant(x: torch.Tensor, act: str = "none", want_scale: bool = True, out: dict | None = None,
              stream=None) -> dict:
    """Fused activation (none / swiglu / relu2) + per-token NVFP4 quantization."""
    _need_2d(x, "x")
    _dtype_code(x)
    rows, k_in = x.shape
    a = ACT[act] if isinstance(act, str) else int(act)
    k_out = k_in // 2 if a == ACT["swiglu"] else k_in
    if out is not None:
        _quant_out(out, rows, k_out, rows)
    _check_dev(x)
    dev = x.device
    o = out or {
        "codes": torch.empty((rows, k_out // 2), dtype=torch.uint8, device=dev),
        "sf": torch.empty((rows, k_out // 16), dtype=torch.uint8, device=dev),
        "g_dec": torch.empty((rows,), dtype=torch.float32, device=dev),
        "scale": torch.empty((rows, k_out // 16), dtype=torch.float32, device=dev) if want_scale else None,
    }
    st = _lib.nvfp4_act_quant(_ptr(x), _dtype_code(x), rows, k_out, a, _ptr(o["codes"]), _ptr(o["sf"]),
                              _ptr(o["g_dec"]), _ptr(o.get("scale")), _stream(stream))
    if st != NVFP4_OK:
        raise Nvfp4Error(st, "nvfp4_act_quant")
    return o


def gemm_workspace_size(B: int, N: int, K: int) -> int:
    return int(_lib.nvfp4_gemm_workspace_size(B, N, K))


def gemm(a_codes: torch.Tensor, a_scale: torch.Tensor, w_codes: torch.Tensor, w_sf: torch.Tensor,
         w_g: torch.Tensor, out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
         stream=None) -> torch.Tensor:
    """y[B, N] fp16 = deq(a) . deq(w)^T."""
    _need_2d(a_codes, "a_codes")
    _need_2d(w_codes, "w_codes")
    B, K = a_codes.shape[0], a_codes.shape[1] * 2
    N = w_codes.shape[0]
    _need(a_codes, "a_codes", torch.uint8)
    _need(a_scale, "a_scale", torch.float32, (B, K // 16))
    _need(w_codes, "w_codes", torch.uint8, (N, K // 2))
    _need(w_sf, "w_sf", torch.uint8, (N, K // 16))
    _need(w_g, "w_g", torch.float32, min_numel=1)
    if out is not None:
        _need(out, "out", torch.float16, (B, N))
    _check_dev(a_codes, a_scale, w_codes, w_sf, w_g, out)
    y = out if out is not None else torch.empty((B, N), dtype=torch.float16, device=a_codes.device)
    ws, wsb = _workspace(gemm_workspace_size(B, N, K), a_codes.device, workspace)
    st = _lib.nvfp4_gemm(_ptr(a_codes), _ptr(a_scale), _ptr(w_codes), _ptr(w_sf), _ptr(w_g), _ptr(y),
                         B, N, K, _ptr(ws), wsb, _stream(stream))
    if st != NVFP4_OK:
        raise Nvfp4Error(st, "nvfp4_gemm")
    return y


def pretile_weight(w_codes: torch.Tensor, w_sf: torch.Tensor, stream=None) -> dict:
    """The pre-tiled layout of [N, K/2] codes and [N, K/16] E4M3 bytes (flat
    uint8 tensors of N*K/2 and N*K/16 bytes)."""
    _need_2d(w_codes, "w_codes")
    N, K = w_codes.shape[0], w_codes.shape[1] * 2
    _need(w_codes, "w_codes", torch.uint8)
    _need(w_sf, "w_sf", torch.uint8, (N, K // 16))
    _check_dev(w_codes, w_sf)
    wt = torch.empty(N * K // 2, dtype=torch.uint8, device=w_codes.device)
    st = torch.empty(N * K // 16, dtype=torch.uint8, device=w_codes.device)
    rc = _lib.nvfp4_pretile_weight(_ptr(w_codes), _ptr(w_sf), N, K, _ptr(wt), _ptr(st), _stream(stream))
    if rc != NVFP4_OK:
        raise Nvfp4Error(rc, "nvfp4_pretile_weight")
    return {"codes": wt, "sf": st, "N": N, "K": K}


def gemm_pretiled(a_codes: torch.Tensor, a_scale: torch.Tensor, wt: dict, w_g: torch.Tensor,
                  out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                  stream=None) -> torch.Tensor:
    """gemm() with weights from pretile_weight()."""
    _need_2d(a_codes, "a_codes")
    B, K = a_codes.shape[0], a_codes.shape[1] * 2
    N = wt["N"]
    if K != wt["K"]:
        raise ValueError("activation K %d differs from the pre-tiled weight's K %d" % (K, wt["K"]))
    _need(a_codes, "a_codes", torch.uint8)
    _need(a_scale, "a_scale", torch.float32, (B, K // 16))
    _need(wt["codes"], "wt['codes']", torch.uint8, min_numel=N * K // 2)
    _need(wt["sf"], "wt['sf']", torch.uint8, min_numel=N * K // 16)
    _need(w_g, "w_g", torch.float32, min_numel=1)
    if out is not None:
        _need(out, "out", torch.float16, (B, N))
    _check_dev(a_codes, a_scale, w_g, wt["codes"], wt["sf"], out)
    y = out if out is not None else torch.empty((B, N), dtype=torch.float16, device=a_codes.device)
    ws, wsb = _workspace(gemm_workspace_size(B, N, K), a_codes.device, workspace)
    rc = _lib.nvfp4_gemm_pretiled(_ptr(a_codes), _ptr(a_scale), _ptr(wt["codes"]), _ptr(wt["sf"]), _ptr(w_g),
                                  _ptr(y), B, N, K, _ptr(ws), wsb, _stream(stream))
    if rc != NVFP4_OK:
        raise Nvfp4Error(rc, "nvfp4_gemm_pretiled")
    return y


def register_weight(resource_id: int, w_codes: torch.Tensor, w_sf: torch.Tensor) -> None:
    """Registers an external weight ([N, K/2] codes, [N, K/16] E4M3 bytes) for
    (the tensors' device, resource_id).  The tensors must outlive the
    registration: unregister before freeing them."""
    _need_2d(w_codes, "w_codes")
    N, K = w_codes.shape[0], w_codes.shape[1] * 2
    _need(w_codes, "w_codes", torch.uint8)
    _need(w_sf, "w_sf", torch.uint8, (N, K // 16))
    _check_dev(w_codes, w_sf)
    st = _lib.nvfp4_register_weight(w_codes.device.index or 0, resource_id, _ptr(w_codes), _ptr(w_sf),
                                    N, K, K // 16)
    if st != NVFP4_OK:
        raise Nvfp4Error(st, "nvfp4_register_weight")


def unregister_weight(resource_id: int, device: int = 0) -> None:
    st = _lib.nvfp4_unregister_weight(device, resource_id)
    if st != NVFP4_OK:
        raise Nvfp4Error(st, "nvfp4_unregister_weight")


def gemm_external(a_codes: torch.Tensor, a_scale: torch.Tensor, resource_id: int, N: int,
                  w_g: torch.Tensor, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """gemm() with the weight registered under resource_id on the current device."""
    _need_2d(a_codes, "a_codes")
    B, K = a_codes.shape[0], a_codes.shape[1] * 2
    _need(a_codes, "a_codes", torch.uint8)
    _need(a_scale, "a_scale", torch.float32, (B, K // 16))
    _need(w_g, "w_g", torch.float32, min_numel=1)
    if out is not None:
        _need(out, "out", torch.float16, (B, N))
    _check_dev(a_codes, a_scale, w_g, out)
    y = out if out is not None else torch.empty((B, N), dtype=torch.float16, device=a_codes.device)
    ws, wsb = _workspace(gemm_workspace_size(B, N, K), a_codes.device, workspace)
    st = _lib.nvfp4_gemm_external(_ptr(a_codes), _ptr(a_scale), resource_id, _ptr(w_g), _ptr(y),
                                  B, N, K, _ptr(ws), wsb, _stream(stream))
    if st != NVFP4_OK:
        raise Nvfp4Error(st, "nvfp4_gemm_external")
    return y


def moe_workspace_size(tokens, experts, top_k, hidden, inter) -> int:
    return int(_lib.nvfp4_moe_w4a16_workspace_size(tokens, experts, top_k, hidden, inter))


def moe_w4a16(logits, bias, x, w1, w1_sf, w1_g, w2, w2_sf, w2_g, top_k, n_group, topk_group,
              norm_topk_prob=True, routed_scaling=1.0, out=None, want_routing=False,
              workspace=None, stream=None):
    """Routed W4A16 MoE layer; returns out (and (ids, weights) if want_routing)."""
    return _moe(_lib.nvfp4_moe_w4a16, "nvfp4_moe_w4a16", logits, bias, x, w1, w1_sf, w1_g, w2, w2_sf,
                w2_g, top_k, n_group, topk_group, norm_topk_prob, routed_scaling, out, want_routing,
                workspace, stream)


def moe_pretile_weights(w: torch.Tensor, w_sf: torch.Tensor, stream=None) -> tuple:
    """The pre-tiled layout of stacked expert weights [E, N, K/2] codes and
    [E, N, K/16] E4M3 bytes (nvfp4_pretile_weight of the [E*N, K] matrix),
    returned with the same shapes."""
    if not isinstance(w, torch.Tensor) or w.dim() != 3:
        raise ValueError("w must be a 3-D tensor [experts, rows, K/2]")
    E, N, K2 = w.shape
    _need(w, "w", torch.uint8)
    _need(w_sf, "w_sf", torch.uint8, (E, N, K2 // 8))
    t = pretile_weight(w.reshape(E * N, K2), w_sf.reshape(E * N, K2 // 8), stream=stream)
    return t["codes"].view(E, N, K2), t["sf"].view(E, N, K2 // 8)


def moe_w4a16_pretiled(logits, bias, x, w1, w1_sf, w1_g, w2, w2_sf, w2_g, top_k, n_group, topk_group,
                       norm_topk_prob=True, routed_scaling=1.0, out=None, want_routing=False,
                       workspace=None, stream=None):
    """moe_w4a16() with w1/w1_sf and w2/w2_sf from moe_pretile_weights()
    (same shapes and results)."""
    return _moe(_lib.nvfp4_moe_w4a16_pretiled, "nvfp4_moe_w4a16_pretiled", logits, bias, x, w1, w1_sf,
                w1_g, w2, w2_sf, w2_g, top_k, n_group, topk_group, norm_topk_prob, routed_scaling, out,
                want_routing, workspace, stream)


def _moe(fn, name, logits, bias, x, w1, w1_sf, w1_g, w2, w2_sf, w2_g, top_k, n_group, topk_group,
         norm_topk_prob, routed_scaling, out, want_routing, workspace, stream):
    _need_2d(logits, "logits")
    _need_2d(x, "x")
    T, E = logits.shape
    hidden = x.shape[1]
    if not isinstance(w1, torch.Tensor) or w1.dim() != 3:
        raise ValueError("w1 must be a 3-D tensor [experts, inter, hidden/2]")
    inter = w1.shape[1]
    _need(logits, "logits", torch.float32)
    _need(bias, "bias", torch.float32, (E,))
    _need(x, "x", torch.float16, (T, hidden))
    _need(w1, "w1", torch.uint8, (E, inter, hidden // 2))
    _need(w1_sf, "w1_sf", torch.uint8, (E, inter, hidden // 16))
    _need(w1_g, "w1_g", torch.float32, min_numel=E)
    _need(w2, "w2", torch.uint8, (E, hidden, inter // 2))
    _need(w2_sf, "w2_sf", torch.uint8, (E, hidden, inter // 16))
    _need(w2_g, "w2_g", torch.float32, min_numel=E)
    if out is not None:
        _need(out, "out", torch.float16, (T, hidden))
    _check_dev(logits, bias, x, w1, w1_sf, w1_g, w2, w2_sf, w2_g, out)
    o = out if out is not None else torch.empty((T, hidden), dtype=torch.float16, device=x.device)
    ids = torch.empty((T, top_k), dtype=torch.int32, device=x.device) if want_routing else None
    wts = torch.empty((T, top_k), dtype=torch.float32, device=x.device) if want_routing else None
    ws, wsb = _workspace(moe_workspace_size(T, E, top_k, hidden, inter), x.device, workspace)
    st = fn(_ptr(logits), _ptr(bias), _ptr(x), _ptr(w1), _ptr(w1_sf), _ptr(w1_g),
            _ptr(w2), _ptr(w2_sf), _ptr(w2_g), _ptr(o), _ptr(ids), _ptr(wts),
            T, E, top_k, hidden, inter, n_group, topk_group, int(bool(norm_topk_prob)),
            float(routed_scaling), _ptr(ws), wsb, _stream(stream))
    if st != NVFP4_OK:
        raise Nvfp4Error(st, name)
    return (o, ids, wts) if want_routing else o


def moe_w4a16_noalloc(logits, bias, x, w1, w1_sf, w1_g, w2, w2_sf, w2_g, top_k, n_group, topk_group,
                      norm_topk_prob=True, routed_scaling=1.0, out=None, ids_out=None, w_out=None, stream=None):
    """moe_w4a16() on the library's fixed device scratch: no workspace, nothing
    allocated by the library (pass `out` to allocate nothing here either).
    Calls that overlap in time on one GPU race."""
    _need_2d(logits, "logits")
    _need_2d(x, "x")
    T, E = logits.shape
    hidden = x.shape[1]
    if not isinstance(w1, torch.Tensor) or w1.dim() != 3:
        raise ValueError("w1 must be a 3-D tensor [experts, inter, hidden/2]")
    inter = w1.shape[1]
    _need(logits, "logits", torch.float32)
    _need(bias, "bias", torch.float32, (E,))
    _need(x, "x", torch.float16, (T, hidden))
    _need(w1, "w1", torch.uint8, (E, inter, hidden // 2))
    _need(w1_sf, "w1_sf", torch.uint8, (E, inter, hidden // 16))
    _need(w1_g, "w1_g", torch.float32, min_numel=E)
    _need(w2, "w2", torch.uint8, (E, hidden, inter // 2))
    _need(w2_sf, "w2_sf", torch.uint8, (E, hidden, inter // 16))
    _need(w2_g, "w2_g", torch.float32, min_numel=E)
    for t, name, dt in ((out, "out", torch.float16), (ids_out, "ids_out", torch.int32), (w_out, "w_out", torch.float32)):
        if t is not None:
            _need(t, name, dt, (T, hidden) if name == "out" else (T, top_k))
    _check_dev(logits, bias, x, w1, w1_sf, w1_g, w2, w2_sf, w2_g, out, ids_out, w_out)
    o = out if out is not None else torch.empty((T, hidden), dtype=torch.float16, device=x.device)
    st = _lib.nvfp4_moe_w4a16_noalloc(_ptr(logits), _ptr(bias), _ptr(x), _ptr(w1), _ptr(w1_sf), _ptr(w1_g),
                                      _ptr(w2), _ptr(w2_sf), _ptr(w2_g), _ptr(o), _ptr(ids_out), _ptr(w_out),
                                      T, E, top_k, hidden, inter, n_group, topk_group, int(bool(norm_topk_prob)),
                                      float(routed_scaling), _stream(stream))
    if st != NVFP4_OK:
        raise Nvfp4Error(st, "nvfp4_moe_w4a16_noalloc")
    return o


# ---------------------------------------------------------------- MXFP4 variant

def mx_tiled_sizes(rows: int, k: int) -> tuple[int, int]:
    """Bytes of the MX tile layout of a [rows, k] operand: (codes, scale bytes)."""
    r32 = (rows + 31) // 32 * 32
    return r32 * k // 2, r32 * k // 32


def mx_quantize(x: torch.Tensor, act: str = "none", group_rows: int = 1, tiled: bool = False,
                out: dict | None = None, workspace: torch.Tensor | None = None, stream=None) -> dict:
    """MXFP4 quantization (E8M0 scale per 32 elements) of x [rows, k_in], with the
    optional activation in front.  Returns dict(codes, sf, g_dec, rows, K, tiled):
    [rows, k/2] and [rows, k/32] uint8 in the row layout, flat uint8 tensors in
    the MX tile layout."""
    _need_2d(x, "x")
    _dtype_code(x)
    rows, k_in = x.shape
    a = ACT[act] if isinstance(act, str) else int(act)
    k = k_in // 2 if a == ACT["swiglu"] else k_in
    if out is not None:
        if tiled:
            nc, ns = mx_tiled_sizes(rows, k)
            _need(out.get("codes"), "out['codes']", torch.uint8, min_numel=nc)
            _need(out.get("sf"), "out['sf']", torch.uint8, min_numel=ns)
        else:
            _need(out.get("codes"), "out['codes']", torch.uint8, (rows, k // 2))
            _need(out.get("sf"), "out['sf']", torch.uint8, (rows, k // 32))
        _need(out.get("g_dec"), "out['g_dec']", torch.float32, min_numel=rows // max(group_rows, 1))
    _check_dev(x)
    dev = x.device
    if out is None:
        if tiled:
            nc, ns = mx_tiled_sizes(rows, k)
            codes = torch.empty(nc, dtype=torch.uint8, device=dev)
            sf = torch.empty(ns, dtype=torch.uint8, device=dev)
        else:
            codes = torch.empty((rows, k // 2), dtype=torch.uint8, device=dev)
            sf = torch.empty((rows, k // 32), dtype=torch.uint8, device=dev)
        out = {"codes": codes, "sf": sf,
               "g_dec": torch.empty((rows // max(group_rows, 1),), dtype=torch.float32, device=dev)}
    out.update(rows=rows, K=k, tiled=bool(tiled))
    ws, wsb = _workspace(_lib.nvfp4_quantize_workspace_size(rows, k, group_rows), dev, workspace)
    st = _lib.nvfp4_mx_quantize(_ptr(x), _dtype_code(x), rows, k, a, group_rows,
                                MX_TILED if tiled else MX_ROWS, _ptr(out["codes"]), _ptr(out["sf"]),
                                _ptr(out["g_dec"]), _ptr(ws), wsb, _stream(stream))
    if st != NVFP4_OK:
        raise Nvfp4Error(st, "nvfp4_mx_quantize")
    return out


def mx_tile(codes: torch.Tensor, sf: torch.Tensor, stream=None) -> dict:
    """The MX tile layout of [rows, k/2] codes and [rows, k/32] E8M0 bytes."""
    _need_2d(codes, "codes")
    rows, k = codes.shape[0], codes.shape[1] * 2
    _need(codes, "codes", torch.uint8)
    _need(sf, "sf", torch.uint8, (rows, k // 32))
    _check_dev(codes, sf)
    nc, ns = mx_tiled_sizes(rows, k)
    ct = torch.empty(nc, dtype=torch.uint8, device=codes.device)
    stt = torch.empty(ns, dtype=torch.uint8, device=codes.device)
    rc = _lib.nvfp4_mx_tile(_ptr(codes), _ptr(sf), rows, k, _ptr(ct), _ptr(stt), _stream(stream))
    if rc != NVFP4_OK:
        raise Nvfp4Error(rc, "nvfp4_mx_tile")
    return {"codes": ct, "sf": stt, "rows": rows, "K": k, "tiled": True}


def mx_gemm(a: dict, a_g: torch.Tensor, w: dict, w_g: torch.Tensor, a_group_rows: int = 1,
            out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y[B, N] fp16 = deq(a) . deq(w)^T for MXFP4 operands in the MX tile layout
    (dicts from mx_quantize(tiled=True) or mx_tile)."""
    if not (a.get("tiled") and w.get("tiled")):
        raise ValueError("mx_gemm takes operands in the MX tile layout")
    B, N, K = a["rows"], w["rows"], a["K"]
    if w["K"] != K:
        raise ValueError("operand K differs")
    for op, r in ((a, B), (w, N)):
        nc, ns = mx_tiled_sizes(r, K)
        if op["codes"].dtype != torch.uint8 or op["sf"].dtype != torch.uint8 or \
                op["codes"].numel() < nc or op["sf"].numel() < ns:
            raise ValueError("tile buffers smaller than the MX tile layout of %d x %d" % (r, K))
    _need(a_g, "a_g", torch.float32, min_numel=B // max(a_group_rows, 1))
    _need(w_g, "w_g", torch.float32, min_numel=1)
    if out is not None:
        _need(out, "out", torch.float16, (B, N))
    _check_dev(a["codes"], a["sf"], a_g, w["codes"], w["sf"], w_g, out)
    y = out if out is not None else torch.empty((B, N), dtype=torch.float16, device=a["codes"].device)
    rc = _lib.nvfp4_mx_gemm(_ptr(a["codes"]), _ptr(a["sf"]), _ptr(a_g), a_group_rows, _ptr(w["codes"]),
                            _ptr(w["sf"]), _ptr(w_g), _ptr(y), B, N, K, _stream(stream))
    if rc != NVFP4_OK:
        raise Nvfp4Error(rc, "nvfp4_mx_gemm")
    return y

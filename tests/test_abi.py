"""The C-ABI library loads and exports every function include/nvfp4_mi355x.h
declares; host-side validation rejects bad arguments before touching a GPU.

Runs without a GPU: only calls whose arguments fail validation are made (they
return before any HIP call).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4_mi355x.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def nv():
    import nvfp4_block_scaled_quantize_amd as nv
    return nv


def test_every_declared_symbol_is_exported(nv):
    names = _declared()
    assert len(names) >= 8
    for n in names:
        assert hasattr(nv.lib(), n), n
    assert sorted(nv.EXPORTS) == names


def test_status_strings(nv):
    for s in range(5):
        assert nv.lib().nvfp4_status_string(s)
    assert nv.lib().nvfp4_status_string(99) == b"unknown status"


def test_quantize_validation_without_gpu(nv):
    L = nv.lib()
    p = ctypes.c_void_p(256)   # never dereferenced: validation fails first
    # K not a multiple of 16
    assert L.nvfp4_quantize(p, 0, 4, 24, 1, p, p, p, None, None, 0, None) == nv.NVFP4_EINVAL
    # bad dtype, bad group
    assert L.nvfp4_quantize(p, 7, 4, 32, 1, p, p, p, None, None, 0, None) == nv.NVFP4_EINVAL
    assert L.nvfp4_quantize(p, 0, 6, 32, 4, p, p, p, None, None, 0, None) == nv.NVFP4_EINVAL
    # null pointer
    assert L.nvfp4_quantize(None, 0, 4, 32, 1, p, p, p, None, None, 0, None) == nv.NVFP4_EINVAL
    # per-tensor without workspace
    assert L.nvfp4_quantize(p, 0, 4, 32, 4, p, p, p, None, None, 0, None) == nv.NVFP4_EWORKSPACE
    # rows == 0 is a no-op
    assert L.nvfp4_quantize(p, 0, 0, 32, 1, p, p, p, None, None, 0, None) == nv.NVFP4_OK
    # bad activation
    assert L.nvfp4_act_quant(p, 0, 4, 32, 9, p, p, p, None, None) == nv.NVFP4_EINVAL
    assert nv.lib().nvfp4_quantize_workspace_size(8, 64, 1) == 0
    assert nv.lib().nvfp4_quantize_workspace_size(8, 64, 8) > 0


def test_gemm_validation_without_gpu(nv):
    L = nv.lib()
    p = ctypes.c_void_p(256)
    assert L.nvfp4_gemm(p, p, p, p, p, p, 4, 8, 40, None, 0, None) == nv.NVFP4_EINVAL   # K % 16
    assert L.nvfp4_gemm(None, p, p, p, p, p, 4, 8, 64, None, 0, None) == nv.NVFP4_EINVAL
    assert L.nvfp4_gemm(p, ctypes.c_void_p(258), p, p, p, p, 4, 8, 64, None, 0, None) == nv.NVFP4_EINVAL
    assert L.nvfp4_gemm(p, p, p, p, p, ctypes.c_void_p(257), 4, 8, 64, None, 0, None) == nv.NVFP4_EINVAL
    assert L.nvfp4_gemm(p, p, p, p, p, p, 0, 8, 64, None, 0, None) == nv.NVFP4_OK
    # large batches need a workspace, 256-byte aligned
    need = nv.gemm_workspace_size(4096, 8192, 8192)
    assert need > 0
    assert L.nvfp4_gemm(p, p, p, p, p, p, 4096, 8192, 8192, None, 0, None) == nv.NVFP4_EWORKSPACE
    assert L.nvfp4_gemm(p, p, p, p, p, p, 4096, 8192, 8192, ctypes.c_void_p(4096 + 16), need,
                        None) == nv.NVFP4_EWORKSPACE
    assert L.nvfp4_gemm(p, p, p, p, p, p, 4096, 8192, 8192, ctypes.c_void_p(4096), need - 1,
                        None) == nv.NVFP4_EWORKSPACE
    assert L.nvfp4_gemm_pretiled(p, p, p, p, p, p, 4096, 8192, 8192, ctypes.c_void_p(4096 + 16), need,
                                 None) == nv.NVFP4_EWORKSPACE


def test_moe_validation_without_gpu(nv):
    L = nv.lib()
    p = ctypes.c_void_p(256)
    args = [p] * 10 + [None, None]
    # experts not divisible by n_group
    assert L.nvfp4_moe_w4a16(*args, 4, 10, 2, 64, 64, 3, 1, 1, 1.0, None, 0, None) == nv.NVFP4_EINVAL
    # top_k larger than the kept experts
    assert L.nvfp4_moe_w4a16(*args, 4, 8, 5, 64, 64, 4, 2, 1, 1.0, None, 0, None) == nv.NVFP4_EINVAL
    # hidden / inter not multiples of 64
    assert L.nvfp4_moe_w4a16(*args, 4, 8, 2, 96, 64, 4, 2, 1, 1.0, None, 0, None) == nv.NVFP4_EINVAL
    assert L.nvfp4_moe_w4a16(*args, 4, 8, 2, 64, 32, 4, 2, 1, 1.0, None, 0, None) == nv.NVFP4_EINVAL
    # missing workspace
    assert L.nvfp4_moe_w4a16(*args, 4, 8, 2, 64, 64, 4, 2, 1, 1.0, None, 0, None) == nv.NVFP4_EWORKSPACE
    # the no-allocation variant: same argument checks; a problem whose
    # workspace exceeds its fixed scratch is refused before any launch
    assert L.nvfp4_moe_w4a16_noalloc(*args, 4, 10, 2, 64, 64, 3, 1, 1, 1.0, None) == nv.NVFP4_EINVAL
    assert L.nvfp4_moe_w4a16_noalloc(*args, 0, 8, 2, 64, 64, 4, 2, 1, 1.0, None) == nv.NVFP4_OK
    big = (4096, 64, 8, 2048, 1024)
    assert nv.moe_workspace_size(*big) > nv.NOALLOC_SCRATCH_BYTES
    assert L.nvfp4_moe_w4a16_noalloc(*args, *big[:3], 2048, 1024, 8, 4, 1, 1.0, None) == nv.NVFP4_ESCRATCH
    assert nv.moe_workspace_size(256, 64, 8, 2048, 1024) <= nv.NOALLOC_SCRATCH_BYTES   # the C5 layer fits
    assert L.nvfp4_status_string(nv.NVFP4_ESCRATCH).startswith(b"problem larger")
    # the pre-tiled-weight variant: the same checks, and whole 128-k chunks
    assert L.nvfp4_moe_w4a16_pretiled(*args, 4, 10, 2, 128, 128, 3, 1, 1, 1.0, None, 0, None) == nv.NVFP4_EINVAL
    assert L.nvfp4_moe_w4a16_pretiled(*args, 4, 8, 2, 192, 128, 4, 2, 1, 1.0, None, 0, None) == nv.NVFP4_EINVAL
    assert L.nvfp4_moe_w4a16_pretiled(*args, 4, 8, 2, 128, 64, 4, 2, 1, 1.0, None, 0, None) == nv.NVFP4_EINVAL
    assert L.nvfp4_moe_w4a16_pretiled(*args, 0, 8, 2, 128, 128, 4, 2, 1, 1.0, None, 0, None) == nv.NVFP4_OK
    assert L.nvfp4_moe_w4a16_pretiled(*args, 4, 8, 2, 128, 128, 4, 2, 1, 1.0, None, 0, None) == nv.NVFP4_EWORKSPACE


def test_external_weight_registry_without_gpu(nv):
    # "Fused Nvfp4 GEMM All Reduce Plugin", external-weight mode: the registry
    # is host-only, so it works (and validates) without a GPU
    L = nv.lib()
    w, s = ctypes.c_void_p(4096), ctypes.c_void_p(8192)
    assert L.nvfp4_register_weight(0, 7, w, s, 64, 128, 8) == nv.NVFP4_OK
    assert L.nvfp4_register_weight(0, 7, w, s, 64, 128, 8) == nv.NVFP4_EINVAL      # already registered
    assert L.nvfp4_register_weight(1, 7, w, s, 64, 128, 8) == nv.NVFP4_OK          # other device
    assert L.nvfp4_register_weight(0, -1, w, s, 64, 128, 8) == nv.NVFP4_EINVAL     # baked-weight id
    assert L.nvfp4_register_weight(0, 8, w, s, 64, 128, 4) == nv.NVFP4_EINVAL      # scale_cols != K/16
    assert L.nvfp4_register_weight(0, 8, w, s, 64, 40, 2) == nv.NVFP4_EINVAL       # K % 16 != 0
    assert L.nvfp4_register_weight(0, 8, None, s, 64, 128, 8) == nv.NVFP4_EINVAL
    # K % 32 == 16 and unaligned pointers are accepted (the GEMM's byte-load path)
    assert L.nvfp4_register_weight(0, 9, ctypes.c_void_p(4104), ctypes.c_void_p(8193), 64, 48, 3) == nv.NVFP4_OK
    assert L.nvfp4_unregister_weight(0, 9) == nv.NVFP4_OK
    assert L.nvfp4_unregister_weight(0, 7) == nv.NVFP4_OK
    assert L.nvfp4_unregister_weight(0, 7) == nv.NVFP4_EINVAL
    assert L.nvfp4_unregister_weight(1, 7) == nv.NVFP4_OK
    assert L.nvfp4_unregister_weight(0, 8) == nv.NVFP4_EINVAL
    p = ctypes.c_void_p(256)
    assert L.nvfp4_gemm_external(p, p, -3, p, p, 4, 64, 128, None, 0, None) == nv.NVFP4_EINVAL


def test_pretiled_validation_without_gpu(nv):
    L = nv.lib()
    p, p4 = ctypes.c_void_p(4096), ctypes.c_void_p(4100)
    # N % 16, K % 128, alignment of the tiled scale buffer
    assert L.nvfp4_pretile_weight(p, p, 40, 256, p, p, None) == nv.NVFP4_EINVAL
    assert L.nvfp4_pretile_weight(p, p, 48, 320, p, p, None) == nv.NVFP4_EINVAL
    assert L.nvfp4_pretile_weight(p, p, 48, 256, p, ctypes.c_void_p(4098), None) == nv.NVFP4_EINVAL
    assert L.nvfp4_gemm_pretiled(p, p, p, p, p, p, 4, 40, 256, None, 0, None) == nv.NVFP4_EINVAL
    assert L.nvfp4_gemm_pretiled(p, p, p, p, p, p, 4, 48, 192, None, 0, None) == nv.NVFP4_EINVAL
    assert L.nvfp4_gemm_pretiled(p, p, ctypes.c_void_p(4104), p, p, p, 4, 48, 256, None, 0, None) == nv.NVFP4_EINVAL
    assert L.nvfp4_gemm_pretiled(p, p4, p, p, p, p, 0, 48, 256, None, 0, None) == nv.NVFP4_OK   # B == 0


def test_mx_validation_without_gpu(nv):
    L = nv.lib()
    p = ctypes.c_void_p(4096)
    # quantizer: k % 32 (rows) / % 128 (tiled), activation only per token,
    # unaligned input, bad layout, k beyond the register cache
    assert L.nvfp4_mx_quantize(p, 0, 4, 48, 0, 1, nv.MX_ROWS, p, p, p, None, 0, None) == nv.NVFP4_EINVAL
    assert L.nvfp4_mx_quantize(p, 0, 4, 96, 0, 1, nv.MX_TILED, p, p, p, None, 0, None) == nv.NVFP4_EINVAL
    assert L.nvfp4_mx_quantize(p, 0, 4, 128, 1, 2, nv.MX_ROWS, p, p, p, None, 0, None) == nv.NVFP4_EINVAL
    assert L.nvfp4_mx_quantize(ctypes.c_void_p(4104), 0, 4, 128, 0, 1, nv.MX_ROWS, p, p, p, None, 0,
                               None) == nv.NVFP4_EINVAL
    assert L.nvfp4_mx_quantize(p, 0, 4, 128, 0, 1, 2, p, p, p, None, 0, None) == nv.NVFP4_EINVAL
    assert L.nvfp4_mx_quantize(p, 0, 4, 65536, 0, 1, nv.MX_ROWS, p, p, p, None, 0, None) == nv.NVFP4_EUNSUPPORTED
    assert L.nvfp4_mx_quantize(p, 0, 4, 128, 0, 4, nv.MX_ROWS, p, p, p, None, 0, None) == nv.NVFP4_EWORKSPACE
    assert L.nvfp4_mx_quantize(p, 0, 0, 128, 0, 1, nv.MX_ROWS, p, p, p, None, 0, None) == nv.NVFP4_OK
    # tile permutation: k % 128, alignment
    assert L.nvfp4_mx_tile(p, p, 40, 192, p, p, None) == nv.NVFP4_EINVAL
    assert L.nvfp4_mx_tile(ctypes.c_void_p(4100), p, 40, 256, p, p, None) == nv.NVFP4_EINVAL
    assert L.nvfp4_mx_tile(p, p, 0, 256, p, p, None) == nv.NVFP4_OK
    # GEMM: N % 32, K % 128, B % a_group_rows, alignment, B == 0
    assert L.nvfp4_mx_gemm(p, p, p, 1, p, p, p, p, 4, 48, 256, None) == nv.NVFP4_EINVAL
    assert L.nvfp4_mx_gemm(p, p, p, 1, p, p, p, p, 4, 64, 192, None) == nv.NVFP4_EINVAL
    assert L.nvfp4_mx_gemm(p, p, p, 3, p, p, p, p, 4, 64, 256, None) == nv.NVFP4_EINVAL
    assert L.nvfp4_mx_gemm(p, p, p, 1, p, p, p, ctypes.c_void_p(4100), 4, 64, 256, None) == nv.NVFP4_EINVAL
    assert L.nvfp4_mx_gemm(p, p, p, 1, p, p, p, p, 0, 64, 256, None) == nv.NVFP4_OK

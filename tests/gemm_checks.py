"""Element-wise GEMM checks and operand views shared by the GPU tests (test helper)."""
import numpy as np
import torch

TOL = 1e-3


def row_checks(y, ref, absref, K, act_rounding):
    """Relative Frobenius error <= TOL in every row, and every element within
    the bound the arithmetic allows:
        |y - ref| <= 2^-10 |ref| + 2^-25 + (act_rounding + K 2^-24) (|A| |W|^T)
    -- the FP16 output rounding (relative 2^-11, with slack for the fp32
    epilogue; absolute 2^-25 for outputs in FP16's subnormal range), the one
    rounding of each activation operand (2^-11 relative for the NVFP4 path's
    FP16 operand, 0 for MXFP4's exact FP4 operand) and the worst-case error
    of an fp32 sum of K products.  A wrong element or tile breaks it."""
    y = np.asarray(y, np.float64)
    num = np.linalg.norm(y - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    rel = num / np.where(den > 0, den, 1.0)
    assert rel.max() <= TOL, (int(rel.argmax()), float(rel.max()))
    err = np.abs(y - ref)
    out_round = 2.0 ** -10 * np.abs(ref) + 2.0 ** -25
    bound = out_round + (act_rounding + K * 2.0 ** -24) * absref
    bad = err > bound
    if bad.any():
        # what the failing elements needed beyond the output rounding, per |A| |W|^T
        need = (err - out_round) / np.where(absref > 0, absref, 1.0)
        i = np.unravel_index(np.argmax(need), need.shape)
        raise AssertionError("%d elements beyond the bound; first %s; largest (err - output rounding)/absref = %.3e "
                             "at %s (err %.3e, ref %.3e, absref %.3e); bound factor %.3e"
                             % (int(bad.sum()), np.argwhere(bad)[:3].tolist(), float(need[i]), i,
                                float(err[i]), float(ref[i]), float(absref[i]), act_rounding + K * 2.0 ** -24))
    return float(rel.max())


def refs(A, W):
    """fp64 A . W^T and |A| . |W|^T."""
    return A @ W.T, np.abs(A) @ np.abs(W).T


def offset_view(t: torch.Tensor, offset: int) -> torch.Tensor:
    """The same values at `offset` bytes past a fresh allocation."""
    nbytes = t.numel() * t.element_size()
    buf = torch.empty(nbytes + 64, dtype=torch.uint8, device=t.device)
    v = buf[offset:offset + nbytes]
    v.copy_(t.contiguous().view(torch.uint8).reshape(-1))
    return v.view(t.dtype).view(t.shape)

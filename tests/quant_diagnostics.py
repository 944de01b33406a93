"""Saturation and zero-code diagnostics of NVFP4 quantizer outputs (test helper).

The failure modes a quantizer shows in production are outputs stuck at the
format maximum or collapsing to zero ("Building Custom TensorRT-LLM Plugins for
Low-Latency FP8 Inference at Scale", "Production Pitfalls & Hard Lessons",
item 2, checked there with a profiler).  These helpers count them on packed
outputs -- codes [rows, k/2] (low nibble = even k) and E4M3 scale bytes
[rows, k/16] -- and check two properties of the two-level NVFP4 scale chain
that hold at any size:

* a block whose scale byte is a normal E4M3 value holds a code of magnitude 6:
  its largest element, divided by the decoded block scale, lies within one
  E4M3 rounding step (6.25 %) of 6, above the 5.0 midpoint to the next grid
  point down;
* with a per-row global scale, the block holding a nonzero row's maximum gets
  the largest E4M3 scale, 448 (byte 0x7E).
"""
import numpy as np

E2M1_MAX_MAG = 7        # magnitude index of 6.0
E4M3_448 = 0x7E


def element_codes(codes: np.ndarray) -> np.ndarray:
    """[rows, k/2] packed bytes -> [rows, k] 4-bit codes."""
    c = np.asarray(codes)
    return np.stack([c & 15, c >> 4], axis=-1).reshape(c.shape[0], -1)


def stats(codes: np.ndarray, sf: np.ndarray) -> dict:
    n = element_codes(codes)
    sf = np.asarray(sf)
    mag = n & 7
    hist = np.bincount(n.ravel(), minlength=16)
    total = max(n.size, 1)
    blocks = max(sf.size, 1)
    exp_field = (sf >> 3) & 15
    normal = (exp_field >= 1) & ((sf & 0x7F) != 0x7F)
    blk_max = mag.reshape(n.shape[0], -1, 16).max(axis=-1)
    return {
        "code_hist": hist.tolist(),
        "zero_code_share": float((hist[0] + hist[8]) / total),
        "max_code_share": float((hist[7] + hist[15]) / total),
        "zero_scale_share": float(np.count_nonzero(sf == 0) / blocks),
        "subnormal_scale_share": float(np.count_nonzero((exp_field == 0) & (sf != 0)) / blocks),
        "scale_448_share": float(np.count_nonzero(sf == E4M3_448) / blocks),
        "normal_blocks_without_max_code": int(np.count_nonzero(normal & (blk_max != E2M1_MAX_MAG))),
        "nonzero_rows_without_448": int(np.count_nonzero((sf.max(axis=1) != 0) & ~np.any(sf == E4M3_448, axis=1))),
    }


def report(name: str, s: dict) -> str:
    line = ("%s: zero codes %.1f %%, +-6 codes %.2f %%, zero scales %.2f %%, subnormal scales %.2f %%, "
            "448 scales %.3f %%, normal blocks without +-6: %d, rows without 448: %d"
            % (name, 100 * s["zero_code_share"], 100 * s["max_code_share"], 100 * s["zero_scale_share"],
               100 * s["subnormal_scale_share"], 100 * s["scale_448_share"],
               s["normal_blocks_without_max_code"], s["nonzero_rows_without_448"]))
    print(line)
    return line

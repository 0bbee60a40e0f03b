"""q8_row weights, float64 oracle (test infrastructure: only tests/, the
smoke check and the benchmark's CPU baseline may import it).

The SAM3 page (cortiq-engine sam3.rs, ``bad_scales``) describes the q8_row
tensor type by its bytes: a 2-D tensor of shape [rows, cols] stores
rows * cols one-byte payload elements, row-major, followed by one float16
scale per row (little-endian, two bytes each). The dequantized matrix is
read here as payload (signed 8-bit) times its row's scale.

Pins (tests/test_oracle.py): a hand-built byte buffer in that layout with
hand-computed values; dequantizing the synthetic quantizer's output lands
within half a scale step of the original matrix.
"""
import numpy as np


def q8_row_from_bytes(buf, rows, cols):
    """Split a q8_row tensor's bytes into (int8 payload [rows, cols],
    float16 scales [rows])."""
    b = np.frombuffer(bytes(buf), dtype=np.uint8)
    if b.size < rows * cols + 2 * rows:
        raise ValueError("q8_row tensor too short")
    q = b[:rows * cols].view(np.int8).reshape(rows, cols)
    s = b[rows * cols:rows * cols + 2 * rows].view("<f2")
    return q.copy(), s.copy()


def dequant_q8_row(q, scale):
    """W[r, c] = q[r, c] * scale[r], in float64."""
    return np.asarray(q, dtype=np.float64) * np.asarray(scale, dtype=np.float64)[:, None]


def dequant_block(inputs):
    """A block's input dict with every (<name>_w int8, <name>_s float16)
    pair replaced by the dequantized float64 matrix."""
    out = {k: v for k, v in inputs.items() if not k.endswith("_s")}
    for k in [k for k in inputs if k.endswith("_w")]:
        out[k] = dequant_q8_row(inputs[k], inputs[k[:-2] + "_s"])
    return out

"""bfloat16 decode (bits -> value), exact.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

bfloat16 is the top half of an IEEE binary32: value = float32(bits << 16).
Used for the small w16a16 operands of the fused add in CUTLASS issue #2058
("[QST] How to implement a fused mixed precision matrix multiplication such as
w4a4 + w16a16?", hyx1999's statement of the inputs) and for reading the GEMMs'
bf16 outputs.
"""

import numpy as np


def bf16_decode(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

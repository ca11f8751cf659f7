"""Exact decoding of the logit bytes the GPU reads (oracle; test infrastructure).

bf16 is the top half of an IEEE float32, so widening its 16 bits into the
high half of a 32-bit word and reading that word as float32 is exact, and so
is the further widening to float64.
"""

import numpy as np

DTYPE_F32 = 0
DTYPE_BF16 = 1


def bf16_bits_to_f64(bits):
    """uint16 bf16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def decode_logits(arr, dtype):
    """Logit array as stored (uint16 bf16 bits or float32) -> float64."""
    if dtype == DTYPE_BF16:
        return bf16_bits_to_f64(arr)
    if dtype == DTYPE_F32:
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    raise ValueError("unknown dtype %r" % (dtype,))

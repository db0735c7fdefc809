"""Exact widening of stored KV/query values to float64 (oracle, test infrastructure).

The pages store the cache in half precision: FP16 in [PA-explainer]
"背景：KV Cache的显存困境" and [vLLM-what] "1）KV cache 显存估算", BF16 in
[PA-notes] §12 题1.  The tiny parity case uses float32.  Every one of these
formats widens to float64 without rounding, so the oracle sees exactly the
values the GPU reads.

bfloat16 has no numpy type: such arrays are carried as their raw uint16 bit
patterns.  A bfloat16 value is the upper half of the float32 with the same
sign, exponent and leading seven mantissa bits, so widening is a 16-bit left
shift followed by a float32 reinterpretation.
"""

import numpy as np

DTYPES = ("f32", "f16", "bf16")

_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}


def storage_type(dtype):
    """numpy type that carries values of ``dtype`` (bf16 -> uint16 bits)."""
    if dtype not in _STORAGE:
        raise ValueError(f"unknown dtype {dtype!r}")
    return _STORAGE[dtype]


def to_f64(a, dtype):
    """Widen an array stored as ``dtype`` to float64, exactly."""
    a = np.asarray(a)
    want = storage_type(dtype)
    if a.dtype != want:
        raise TypeError(f"{dtype} data must be carried as {np.dtype(want)}, got {a.dtype}")
    if dtype == "bf16":
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def from_f32_bits(bits):
    """float32 values from their uint32 bit patterns (used by golden fixtures)."""
    return np.asarray(bits, dtype=np.uint32).view(np.float32)

"""Seeded synthetic inputs for the weight-quantized GEMM workloads.

This module only draws random numbers and fills the page's deterministic
float-weight pattern. It holds none of the method's arithmetic (no
quantisation, no dequantisation, no product): both the CPU oracle's tests
and the HIP path's bench consume what it returns.

Workload shapes follow the MNN GemmSpeed benchmark page (section "Why Conv1x1
is used to measure GEMM": C = A[M,K] x B[K,N] for LLM linear layers; section
"Default test sizes and the meaning of M": M=8 is near single-request decode,
M=512 a long prefill). Distributions follow the workload recipe of this
library: A ~ N(0,1), float weights W ~ N(0, 0.02) laid out [N][K] (one row
per output channel), and for the float path the page's filler
((i % 127) - 63) / 1000 over the flat index i = k*N + n of the {K, N}
weight.

Generator: numpy PCG64 via ``default_rng(seed)``; A is drawn first, then W.
"""
from __future__ import annotations

import numpy as np

__all__ = ["CONFIGS", "activations", "normal_weights", "float_pattern_weights",
           "make_inputs"]

# name -> (format, M, K, N, seed). The formats are the library's format names.
CONFIGS = {
    "f32":             ("f32",     16,   256,   256, 101),
    "f32_tail":        ("f32",      3,   137,    70, 102),
    "int8b0_decode":   ("int8b0",   1,  4096,  4096, 201),
    "int4b64_decode":  ("int4b64",  1,  4096, 11008, 301),
    "int4b64_prefill": ("int4b64", 512, 4096,  4096, 401),
    "w4a8_prefill":    ("w4a8",  1024,  3072,  8192, 501),
}


def activations(rng: np.random.Generator, M: int, K: int, fp16: bool) -> np.ndarray:
    """A ~ N(0,1), drawn in float32, optionally cast (round-to-nearest-even) to fp16."""
    a = rng.standard_normal((M, K), dtype=np.float32)
    return a.astype(np.float16) if fp16 else a


def normal_weights(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    """Float weights W ~ N(0, 0.02) as float32, laid out [N][K]."""
    w = rng.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(0.02)
    return w


def float_pattern_weights(K: int, N: int) -> np.ndarray:
    """The page's float-weight filler ((i % 127) - 63) / 1000 with i = k*N + n.

    Returned as B float32 [K][N]. The division is a real division (an integer
    division would make every weight zero), done in float64 and rounded once
    to float32.
    """
    i = np.arange(K * N, dtype=np.int64).reshape(K, N)
    return (((i % 127) - 63).astype(np.float64) / 1000.0).astype(np.float32)


def half_pattern_weights(K: int, N: int) -> np.ndarray:
    """fp16 weights for the float mode at FP16 precision: the page's float
    filler rounded to fp16, B float16 [K][N]."""
    return float_pattern_weights(K, N).astype(np.float16)


def make_inputs(name: str):
    """Inputs of a named workload: dict(format, M, K, N, seed, A, and W or B)."""
    fmt, M, K, N, seed = CONFIGS[name]
    rng = np.random.default_rng(seed)
    out = {"format": fmt, "M": M, "K": K, "N": N, "seed": seed}
    if fmt == "f32":
        out["A"] = activations(rng, M, K, fp16=False)
        out["B"] = float_pattern_weights(K, N)
    else:
        out["A"] = activations(rng, M, K, fp16=True)
        out["W"] = normal_weights(rng, N, K)
    return out


# The benchmark page's default test sizes ("Default test sizes and the meaning
# of M"): LLM linear layers (K, N) run at M in {8, 32, 128, 512}.
PAGE_KN = [(2560, 4096), (2560, 1024), (4096, 2560), (2560, 9728), (9728, 2560)]
PAGE_M = [8, 32, 128, 512]

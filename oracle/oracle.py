"""Python face of the CPU oracle (oracle.c) for the weight-quantized GEMM.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
bench's CPU-baseline leg, never by the product path. It shares nothing with
the HIP library: it loads its own C library, built from ``oracle.c`` with gcc
(no -ffast-math, no contraction), and turns numpy arrays into its plain
pointer arguments. All arithmetic happens in ``oracle.c``.

Formats and layouts are the canonical ones of the MNN GemmSpeed benchmark page
(section "Why Conv1x1 is used to measure GEMM"): A [M][K] (fp32 for the
float mode, fp16 otherwise), float B [K][N], quantised codes [N][K] (Int8) or
[N][K/2] nibble-packed low nibble first (Int4), and [offset, scale] pairs
[N][K/block][2].
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11",
          "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
          "-Wall", "-Wextra"]


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile oracle.c into a shared library with gcc; returns its path."""
    cmd = ["gcc", *CFLAGS, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load (building first if needed) the oracle library."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        if (not os.path.exists(_LIB) or
                os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build()
        _lib = _declare(ctypes.CDLL(_LIB))
    return _lib


def _declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.orc_half_to_double.argtypes = [ctypes.c_uint16]
    lib.orc_half_to_double.restype = ctypes.c_double
    lib.orc_quantize.argtypes = [I, I, I, I, P, P, P]
    lib.orc_gemm_f32.argtypes = [I, I, I, P, P, P]
    lib.orc_gemm_blockq.argtypes = [I, I, I, I, I, P, P, P, P]
    lib.orc_w4a8_actquant.argtypes = [I, I, P, P, P, P]
    lib.orc_w4a8_dot.argtypes = [I, I, I, P, P, P]
    lib.orc_w4a8_rescale.argtypes = [I, I, P, P, P, P, P]
    lib.orc_w4a8_dequant_product.argtypes = [I, I, I, P, P, P, P, P]
    lib.orc_epilogue.argtypes = [I, I, P, P, P, P, I, P]
    lib.orc_round_half.argtypes = [ctypes.c_double]
    lib.orc_round_half.restype = ctypes.c_double
    for f in ("orc_quantize", "orc_gemm_f32", "orc_gemm_blockq",
              "orc_w4a8_actquant", "orc_w4a8_dot", "orc_w4a8_rescale",
              "orc_w4a8_dequant_product", "orc_epilogue"):
        getattr(lib, f).restype = I
    return lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle: {what} rejected its arguments")


# Format table: name -> (bits, block) ; block None means "all of K". Int4 or
# Int8 with any other block size b (the page's blockSize parameter) is named
# "int4b<b>" or "int8b<b>".
FORMATS = {"int4b64": (4, 64), "int8b0": (8, None), "w4a8": (4, None), "int4b0": (4, None)}


def _bits_block(fmt: str, K: int):
    if fmt in FORMATS:
        bits, block = FORMATS[fmt]
    elif fmt.startswith("int4b") and fmt[5:].isdigit():
        bits, block = 4, int(fmt[5:])
    elif fmt.startswith("int8b") and fmt[5:].isdigit():
        bits, block = 8, int(fmt[5:])
    else:
        raise ValueError(f"unknown format {fmt}")
    return bits, (K if block is None else block)


def half_to_double(h: int, lib=None) -> float:
    return (lib or load()).orc_half_to_double(h)


def quantize(W: np.ndarray, fmt: str, lib=None):
    """Float W [N][K] -> (canonical codes, pairs [N][nblk][2] float32)."""
    lib = lib or load()
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    bits, block = _bits_block(fmt, K)
    q = np.zeros((N, K if bits == 8 else K // 2), dtype=np.uint8)
    pairs = np.zeros((N, K // block, 2), dtype=np.float32)
    _check(lib.orc_quantize(N, K, bits, block, _p(W), _p(q), _p(pairs)), "quantize")
    return q, pairs


def gemm_f32(A: np.ndarray, B: np.ndarray, lib=None) -> np.ndarray:
    lib = lib or load()
    A = np.ascontiguousarray(A, dtype=np.float32)
    B = np.ascontiguousarray(B, dtype=np.float32)
    M, K = A.shape
    K2, N = B.shape
    assert K == K2
    C = np.zeros((M, N), dtype=np.float64)
    _check(lib.orc_gemm_f32(M, K, N, _p(A), _p(B), _p(C)), "gemm_f32")
    return C


def gemm_blockq(A: np.ndarray, q: np.ndarray, pairs: np.ndarray, fmt: str,
                lib=None) -> np.ndarray:
    """fp16 A [M][K] x dequantised canonical weights -> C float64 [M][N]."""
    lib = lib or load()
    A = np.ascontiguousarray(A, dtype=np.float16)
    q = np.ascontiguousarray(q, dtype=np.uint8)
    pairs = np.ascontiguousarray(pairs, dtype=np.float32)
    M, K = A.shape
    N = q.shape[0]
    bits, block = _bits_block(fmt, K)
    assert q.shape == (N, K if bits == 8 else K // 2)
    assert pairs.shape == (N, K // block, 2)
    C = np.zeros((M, N), dtype=np.float64)
    _check(lib.orc_gemm_blockq(M, K, N, bits, block, _p(A.view(np.uint16)),
                               _p(q), _p(pairs), _p(C)), "gemm_blockq")
    return C


def w4a8_actquant(A: np.ndarray, lib=None):
    """fp16 A [M][K] -> (qa int8 [M][K], sa float32 [M], S int32 [M])."""
    lib = lib or load()
    A = np.ascontiguousarray(A, dtype=np.float16)
    M, K = A.shape
    qa = np.zeros((M, K), dtype=np.int8)
    sa = np.zeros(M, dtype=np.float32)
    S = np.zeros(M, dtype=np.int32)
    _check(lib.orc_w4a8_actquant(M, K, _p(A.view(np.uint16)), _p(qa), _p(sa), _p(S)),
           "w4a8_actquant")
    return qa, sa, S


def w4a8_dot(qa: np.ndarray, q: np.ndarray, lib=None) -> np.ndarray:
    """Exact integer product D = qa . q^T (int64) with q the int4 codes."""
    lib = lib or load()
    qa = np.ascontiguousarray(qa, dtype=np.int8)
    q = np.ascontiguousarray(q, dtype=np.uint8)
    M, K = qa.shape
    N = q.shape[0]
    assert q.shape == (N, K // 2)
    D = np.zeros((M, N), dtype=np.int64)
    _check(lib.orc_w4a8_dot(M, K, N, _p(qa), _p(q), _p(D)), "w4a8_dot")
    return D


def w4a8_rescale(D, sa, S, pairs, lib=None) -> np.ndarray:
    lib = lib or load()
    D = np.ascontiguousarray(D, dtype=np.int64)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    S = np.ascontiguousarray(S, dtype=np.int32)
    pairs = np.ascontiguousarray(pairs, dtype=np.float32)
    M, N = D.shape
    assert pairs.shape == (N, 1, 2)
    C = np.zeros((M, N), dtype=np.float64)
    _check(lib.orc_w4a8_rescale(M, N, _p(D), _p(sa), _p(S), _p(pairs), _p(C)),
           "w4a8_rescale")
    return C


def w4a8_dequant_product(qa, sa, q, pairs, lib=None) -> np.ndarray:
    lib = lib or load()
    qa = np.ascontiguousarray(qa, dtype=np.int8)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.uint8)
    pairs = np.ascontiguousarray(pairs, dtype=np.float32)
    M, K = qa.shape
    N = q.shape[0]
    C = np.zeros((M, N), dtype=np.float64)
    _check(lib.orc_w4a8_dequant_product(M, K, N, _p(qa), _p(sa), _p(q), _p(pairs), _p(C)),
           "w4a8_dequant_product")
    return C


def w4a8_gemm(A, q, pairs, lib=None):
    """The whole W4A8 path: returns (C float64, qa, sa, S, D)."""
    qa, sa, S = w4a8_actquant(A, lib)
    D = w4a8_dot(qa, q, lib)
    C = w4a8_rescale(D, sa, S, pairs, lib)
    return C, qa, sa, S, D


ACTIVATIONS = {"none": 0, "relu": 1, "silu": 2, "gelu": 3}


def epilogue(P: np.ndarray, bias=None, residual=None, activation="none", out_f16=False,
             lib=None) -> np.ndarray:
    """act(P + bias + residual) in double (the SimdPaddleOCR pull request's
    epilogue order), optionally rounded to fp16 (nearest even). residual is
    float32 or float16 [M][N]; bias float32 [N]."""
    lib = lib or load()
    P = np.ascontiguousarray(P, dtype=np.float64)
    M, N = P.shape
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    r32 = r16 = None
    if residual is not None:
        residual = np.ascontiguousarray(residual)
        if residual.dtype == np.float16:
            r16 = residual.view(np.uint16)
        else:
            r32 = np.ascontiguousarray(residual, dtype=np.float32)
    act = ACTIVATIONS[activation] if isinstance(activation, str) else int(activation)
    out = np.zeros((M, N), dtype=np.float64)
    _check(lib.orc_epilogue(M, N, _p(P), _p(b) if b is not None else None,
                            _p(r32) if r32 is not None else None,
                            _p(r16) if r16 is not None else None, act, _p(out)), "epilogue")
    if out_f16:
        out = np.vectorize(lib.orc_round_half, otypes=[np.float64])(out) if out.size else out
    return out


def round_half(x: float, lib=None) -> float:
    """x rounded to IEEE binary16 (nearest even), as a double."""
    return (lib or load()).orc_round_half(float(x))


def reference(fmt: str, A, B=None, q=None, pairs=None, lib=None) -> np.ndarray:
    """C float64 of one format on canonical inputs."""
    if fmt == "f32":
        return gemm_f32(A, B, lib)
    if fmt == "f16":
        # fp16 weights (the float mode at FP16 precision): the same plain
        # product of the fp16 values, each widened exactly
        return gemm_f32(np.asarray(A, np.float16).astype(np.float32),
                        np.asarray(B, np.float16).astype(np.float32), lib)
    if fmt[:5] in ("int4b", "int8b") and fmt[5:].isdigit():
        return gemm_blockq(A, q, pairs, fmt, lib)
    if fmt == "w4a8":
        return w4a8_gemm(A, q, pairs, lib)[0]
    raise ValueError(fmt)

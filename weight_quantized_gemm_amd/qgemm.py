"""Thin Python binding of libqgemm's C ABI (include/qgemm.h).

Same names as the C entry points; this module only marshals arguments
(numpy arrays for the host-side quantiser and packer, torch tensors for
device buffers, torch's current HIP stream). Every step of the GEMM runs in
the library's HIP kernels. There is no fallback: if libqgemm.so is missing or
a call fails, an exception is raised.

torch is imported before the library is loaded so that the process uses one
HIP runtime (torch's), which the library then binds to by its soname.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

import torch  # noqa: F401  (must be loaded before libqgemm.so; see module doc)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgemm.so")

# Format ids (0-3: the MNN GemmSpeed page's mode numbers; 4: fp16 weights;
# 5: Int4-Block0 with fp16 activations) and names.
QGEMM_F32, QGEMM_INT4_B64, QGEMM_INT8_B0, QGEMM_W4A8, QGEMM_F16, QGEMM_INT4_B0 = 0, 1, 2, 3, 4, 5
FORMATS = {"f32": QGEMM_F32, "int4b64": QGEMM_INT4_B64, "int8b0": QGEMM_INT8_B0,
           "w4a8": QGEMM_W4A8, "f16": QGEMM_F16, "int4b0": QGEMM_INT4_B0}

STATUS = {0: "QGEMM_OK", 1: "QGEMM_ERR_NULL", 2: "QGEMM_ERR_SHAPE", 3: "QGEMM_ERR_FORMAT",
          4: "QGEMM_ERR_ALIGN", 5: "QGEMM_ERR_NOMEM", 6: "QGEMM_ERR_DEVICE",
          7: "QGEMM_ERR_LAUNCH", 8: "QGEMM_ERR_SIZE", 9: "QGEMM_ERR_VALUE"}

# Every symbol include/qgemm.h declares.
EXPORTS = ["qgemm_status_string", "qgemm_abi_version", "qgemm_canonical_size",
           "qgemm_quantize_weights", "qgemm_packed_size", "qgemm_pack_weights",
           "qgemm_unpack_weights", "qgemm_workspace_size", "qgemm_run", "qgemm_run_ws",
           "qgemm_run_ex", "qgemm_run_noalloc", "qgemm_w4a8_debug", "qgemm_set_gemv_max_m",
           "qgemm_quantize_weights_device", "qgemm_quantize_pack_device"]


class QGemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libqgemm.so; raises if it has not been built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m weight_quantized_gemm_amd.build_lib` "
            "(there is no fallback path)")
    lib = ctypes.CDLL(path)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    ZP = ctypes.POINTER(ctypes.c_size_t)
    sig = {
        "qgemm_status_string": ([I], ctypes.c_char_p),
        "qgemm_abi_version": ([], I),
        "qgemm_canonical_size": ([I, I, I, ZP, ZP], I),
        "qgemm_quantize_weights": ([I, I, I, P, P, Z, P, Z], I),
        "qgemm_packed_size": ([I, I, I, ZP, ZP], I),
        "qgemm_pack_weights": ([I, I, I, P, P, P, Z, P, Z], I),
        "qgemm_unpack_weights": ([I, I, I, P, Z, P, Z, P, P], I),
        "qgemm_workspace_size": ([I, I, I, I, ZP], I),
        "qgemm_run": ([I, I, I, I, P, P, P, P, P], I),
        "qgemm_run_ws": ([I, I, I, I, P, P, P, P, P, Z, P], I),
        "qgemm_run_ex": ([I, I, I, I, P, P, P, P, ctypes.POINTER(Epilogue), P, Z, P], I),
        "qgemm_run_noalloc": ([I, I, I, I, P, P, P, P, ctypes.POINTER(Epilogue), P], I),
        "qgemm_w4a8_debug": ([I, I, I, P, P, P, P, P, P, P, P, P, Z, P], I),
        "qgemm_set_gemv_max_m": ([I], I),
        "qgemm_quantize_weights_device": ([I, I, I, P, P, P, P], I),
        "qgemm_quantize_pack_device": ([I, I, I, P, P, P, P], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if path == LIB_PATH:
        _lib = lib
    return lib


ACTIVATIONS = {"none": 0, "relu": 1, "silu": 2, "gelu": 3}
OUT_TYPES = {"f32": 0, "f16": 1}


class Epilogue(ctypes.Structure):
    """Mirror of qgemm_epilogue: C = act(A x B + bias + residual), C fp32 or fp16."""
    _fields_ = [("bias", ctypes.c_void_p), ("residual", ctypes.c_void_p),
                ("activation", ctypes.c_int), ("out_type", ctypes.c_int)]


QGEMM_INT4_BLOCK_BASE = 0x10000
QGEMM_INT8_BLOCK_BASE = 0x2000000


def QGEMM_INT4_BLOCK(b: int) -> int:
    """Format id of Int4 weights with one pair per b K-elements."""
    return QGEMM_INT4_BLOCK_BASE + b


def QGEMM_INT8_BLOCK(b: int) -> int:
    """Format id of Int8 weights with one pair per b K-elements."""
    return QGEMM_INT8_BLOCK_BASE + b


def _fmt(f) -> int:
    """Format id from a name ("int4b64", "int8b0", ..., "int4b<b>" / "int8b<b>"
    for any other Int4 / Int8 block size b) or an id."""
    if not isinstance(f, str):
        return int(f)
    if f in FORMATS:
        return FORMATS[f]
    if f.startswith("int4b") and f[5:].isdigit():
        return QGEMM_INT4_BLOCK(int(f[5:]))
    if f.startswith("int8b") and f[5:].isdigit() and int(f[5:]) > 0:
        return QGEMM_INT8_BLOCK(int(f[5:]))
    raise ValueError(f"unknown format {f}")


def is_int8(fmt) -> bool:
    """Whether a format stores one byte per code (Int8-Block0 and blocked Int8)."""
    f = _fmt(fmt)
    return f == QGEMM_INT8_B0 or f > QGEMM_INT8_BLOCK_BASE


def pairs_per_channel(fmt, K: int) -> int:
    """Canonical pairs per channel of a quantised format."""
    f = _fmt(fmt)
    if f == QGEMM_INT4_B64:
        return K // 64
    if f > QGEMM_INT8_BLOCK_BASE:
        return K // (f - QGEMM_INT8_BLOCK_BASE)
    if f > QGEMM_INT4_BLOCK_BASE:
        return K // (f - QGEMM_INT4_BLOCK_BASE)
    return 1


def _check(st: int, where: str):
    if st != 0:
        raise QGemmError(st, where)


def _np_ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _dev_ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError("device buffers must be contiguous GPU tensors")
    return ctypes.c_void_p(t.data_ptr())


_TORCH_DTYPE_NAMES = {torch.float32: "float32", torch.float16: "float16", torch.uint8: "uint8",
                      torch.int8: "int8", torch.int32: "int32"}


def _need(t, name: str, dtypes, numel: int | None = None, nbytes: int | None = None):
    """Checks a device-buffer argument before anything reaches the library:
    its dtype (one of `dtypes`, or any when None), at least `numel` elements
    and at least `nbytes` bytes. Raw integer addresses and None pass through
    (the C side checks for NULL). Raises ValueError. The kernels would
    otherwise read or write past a buffer that is too small or of the wrong
    element type."""
    if t is None or isinstance(t, int):
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch tensor or a device address, got {type(t).__name__}")
    if t.numel() == 0 and not numel and not nbytes:
        return   # an empty placeholder for an operand the shape never reads
    if dtypes is not None and t.dtype not in dtypes:
        want = " or ".join(_TORCH_DTYPE_NAMES.get(d, str(d)) for d in dtypes)
        raise ValueError(f"{name}: dtype {t.dtype} where {want} is required")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements, at least {numel} required")
    if nbytes is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name}: {t.numel() * t.element_size()} bytes, at least {nbytes} required")


def _check_run_args(M: int, K: int, N: int, fmt, A, Bq, scales, C, out_type=0, bias=None,
                    residual=None, workspace=None, ws_bytes: int = 0):
    """Dtype and size checks shared by the run entry points: A fp32 for the
    fp32 format, fp16 otherwise, [M][K]; C (and the residual) fp32, or fp16
    with the fp16 output; the packed buffers at least the packed sizes of
    (K, N, fmt); the bias [N] fp32; the workspace at least ws_bytes."""
    f = _fmt(fmt)
    if M < 0 or N < 0 or K < 0:
        raise ValueError(f"negative shape M={M} K={K} N={N}")
    if M == 0 or N == 0:
        return
    a_dt = torch.float32 if f == QGEMM_F32 else torch.float16
    _need(A, "A", (a_dt,), numel=M * K)
    c_dt = torch.float16 if out_type in (1, "f16") else torch.float32
    _need(C, "C", (c_dt,), numel=M * N)
    _need(residual, "residual", (c_dt,), numel=M * N)
    _need(bias, "bias", (torch.float32,), numel=N)
    try:
        wb, sb = qgemm_packed_size(K, N, f)
    except QGemmError:
        wb = sb = None   # the library reports the bad shape or format itself
    if f == QGEMM_F32 and wb is not None:
        # the fp32 format's B is the float [K][N] matrix itself, read no
        # further than its K*N elements (the packed size rounds it up to 256)
        wb = K * N * 4
    _need(Bq, "Bq", None, nbytes=wb)
    _need(scales, "scales", None, nbytes=sb)
    if isinstance(workspace, torch.Tensor) and workspace.numel() * workspace.element_size() < ws_bytes:
        raise ValueError(f"workspace: {workspace.numel() * workspace.element_size()} bytes, "
                         f"ws_bytes={ws_bytes} claimed")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


# ---------------------------------------------------------------------------
def qgemm_status_string(status: int) -> str:
    return load().qgemm_status_string(status).decode()


def qgemm_abi_version() -> int:
    return load().qgemm_abi_version()


def qgemm_canonical_size(K: int, N: int, fmt) -> tuple[int, int]:
    q, p = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().qgemm_canonical_size(K, N, _fmt(fmt), ctypes.byref(q), ctypes.byref(p)),
           "qgemm_canonical_size")
    return q.value, p.value


def qgemm_packed_size(K: int, N: int, fmt) -> tuple[int, int]:
    w, s = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().qgemm_packed_size(K, N, _fmt(fmt), ctypes.byref(w), ctypes.byref(s)),
           "qgemm_packed_size")
    return w.value, s.value


def qgemm_workspace_size(M: int, K: int, N: int, fmt) -> int:
    b = ctypes.c_size_t()
    _check(load().qgemm_workspace_size(M, K, N, _fmt(fmt), ctypes.byref(b)),
           "qgemm_workspace_size")
    return b.value


def qgemm_quantize_weights(W: np.ndarray, fmt):
    """Float W [N][K] -> (canonical codes uint8, pairs float32 [N][nblk][2])."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    qb, pf = qgemm_canonical_size(K, N, fmt)
    q = np.empty(qb, dtype=np.uint8)
    pairs = np.empty(pf, dtype=np.float32)
    _check(load().qgemm_quantize_weights(K, N, _fmt(fmt), _np_ptr(W), _np_ptr(q), qb,
                                         _np_ptr(pairs), pf), "qgemm_quantize_weights")
    f = _fmt(fmt)
    qshape = (N, K) if is_int8(f) else (N, K // 2)
    return q.reshape(qshape), pairs.reshape(N, pairs_per_channel(f, K), 2)


def qgemm_pack_weights(K: int, N: int, fmt, w_canonical: np.ndarray,
                       pairs_canonical: np.ndarray | None):
    """Canonical host arrays -> (packed weights uint8, packed pairs uint8), host."""
    wb, sb = qgemm_packed_size(K, N, fmt)
    wp = np.empty(wb, dtype=np.uint8)
    sp = np.empty(max(sb, 1), dtype=np.uint8)
    wc = np.ascontiguousarray(w_canonical)
    pc = None if pairs_canonical is None else np.ascontiguousarray(pairs_canonical, dtype=np.float32)
    _check(load().qgemm_pack_weights(K, N, _fmt(fmt), _np_ptr(wc), _np_ptr(pc), _np_ptr(wp), wb,
                                     _np_ptr(sp), sb), "qgemm_pack_weights")
    return wp, sp[:sb]


def qgemm_unpack_weights(K: int, N: int, fmt, w_packed: np.ndarray, s_packed: np.ndarray):
    f = _fmt(fmt)
    qb, pf = qgemm_canonical_size(K, N, f)
    q = np.empty(max(qb, 1), dtype=np.uint8)
    pairs = np.empty(max(pf, 1), dtype=np.float32)
    sp = s_packed if s_packed.size else np.zeros(1, np.uint8)
    _check(load().qgemm_unpack_weights(K, N, f, _np_ptr(w_packed), w_packed.nbytes, _np_ptr(sp),
                                       s_packed.nbytes, _np_ptr(q), _np_ptr(pairs)),
           "qgemm_unpack_weights")
    return q[:qb], pairs[:pf]


def qgemm_run(M: int, K: int, N: int, fmt, A, Bq, scales, C, stream=None) -> None:
    """C = A x B on the GPU (torch tensors or raw device addresses)."""
    _check_run_args(M, K, N, fmt, A, Bq, scales, C)
    _check(load().qgemm_run(M, K, N, _fmt(fmt), _dev_ptr(A), _dev_ptr(Bq), _dev_ptr(scales),
                            _dev_ptr(C), _stream(stream)), "qgemm_run")


def qgemm_run_ws(M: int, K: int, N: int, fmt, A, Bq, scales, C, workspace, ws_bytes: int,
                 stream=None) -> None:
    _check_run_args(M, K, N, fmt, A, Bq, scales, C, workspace=workspace, ws_bytes=ws_bytes)
    _check(load().qgemm_run_ws(M, K, N, _fmt(fmt), _dev_ptr(A), _dev_ptr(Bq), _dev_ptr(scales),
                               _dev_ptr(C), _dev_ptr(workspace), ws_bytes, _stream(stream)),
           "qgemm_run_ws")


def qgemm_run_ex(M: int, K: int, N: int, fmt, A, Bq, scales, C, bias=None, residual=None,
                 activation="none", out_type="f32", workspace=None, ws_bytes: int = 0,
                 stream=None) -> None:
    """C = act(A x B + bias + residual) on the GPU; C (and residual) fp32 or fp16
    per out_type. With no workspace the library allocates any scratch the shape
    needs in stream order."""
    _check_run_args(M, K, N, fmt, A, Bq, scales, C, out_type=out_type, bias=bias,
                    residual=residual, workspace=workspace, ws_bytes=ws_bytes)
    epi = Epilogue(_dev_ptr(bias), _dev_ptr(residual),
                   ACTIVATIONS[activation] if isinstance(activation, str) else int(activation),
                   OUT_TYPES[out_type] if isinstance(out_type, str) else int(out_type))
    _check(load().qgemm_run_ex(M, K, N, _fmt(fmt), _dev_ptr(A), _dev_ptr(Bq), _dev_ptr(scales),
                               _dev_ptr(C), ctypes.byref(epi), _dev_ptr(workspace), ws_bytes,
                               _stream(stream)), "qgemm_run_ex")


NOALLOC_SCRATCH_BYTES = 32 << 20   # QGEMM_NOALLOC_SCRATCH_BYTES


def qgemm_run_noalloc(M: int, K: int, N: int, fmt, A, Bq, scales, C, bias=None, residual=None,
                      activation="none", out_type="f32", stream=None) -> None:
    """qgemm_run_ex without any allocation: the scratch the shape needs lives in
    the library's fixed per-GPU array (NOALLOC_SCRATCH_BYTES); calls that may
    overlap on one GPU must be serialised by the caller."""
    _check_run_args(M, K, N, fmt, A, Bq, scales, C, out_type=out_type, bias=bias,
                    residual=residual)
    epi = Epilogue(_dev_ptr(bias), _dev_ptr(residual),
                   ACTIVATIONS[activation] if isinstance(activation, str) else int(activation),
                   OUT_TYPES[out_type] if isinstance(out_type, str) else int(out_type))
    _check(load().qgemm_run_noalloc(M, K, N, _fmt(fmt), _dev_ptr(A), _dev_ptr(Bq), _dev_ptr(scales),
                                    _dev_ptr(C), ctypes.byref(epi), _stream(stream)),
           "qgemm_run_noalloc")


def qgemm_w4a8_debug(M: int, K: int, N: int, A, Bq, scales, C, qa, sa, S, D, workspace,
                     ws_bytes: int, stream=None) -> None:
    _check_run_args(M, K, N, QGEMM_W4A8, A, Bq, scales, C, workspace=workspace, ws_bytes=ws_bytes)
    _need(qa, "qa", (torch.int8, torch.uint8), numel=M * K)
    _need(sa, "sa", (torch.float32,), numel=M)
    _need(S, "S", (torch.int32,), numel=M)
    _need(D, "D", (torch.int32,), numel=M * N)
    _check(load().qgemm_w4a8_debug(M, K, N, _dev_ptr(A), _dev_ptr(Bq), _dev_ptr(scales),
                                   _dev_ptr(C), _dev_ptr(qa), _dev_ptr(sa), _dev_ptr(S),
                                   _dev_ptr(D), _dev_ptr(workspace), ws_bytes, _stream(stream)),
           "qgemm_w4a8_debug")


def qgemm_quantize_weights_device(W, fmt, q=None, pairs=None, stream=None):
    """Device float W [N][K] -> (canonical codes uint8, pairs float32 [N][nblk][2]),
    both device tensors (allocated here unless given)."""
    f = _fmt(fmt)
    N, K = W.shape
    qb, pf = qgemm_canonical_size(K, N, f)
    if q is None:
        q = torch.empty(max(qb, 1), dtype=torch.uint8, device=W.device)
    if pairs is None:
        pairs = torch.empty(max(pf, 1), dtype=torch.float32, device=W.device)
    _check(load().qgemm_quantize_weights_device(K, N, f, _dev_ptr(W), _dev_ptr(q), _dev_ptr(pairs),
                                                _stream(stream)), "qgemm_quantize_weights_device")
    qshape = (N, K) if is_int8(f) else (N, K // 2)
    return q[:qb].view(qshape), pairs[:pf].view(N, pairs_per_channel(f, K), 2)


def qgemm_quantize_pack_device(W, fmt, Bq=None, scales=None, stream=None):
    """Device float W [N][K] -> (packed weights uint8, packed pairs uint8), both
    device tensors in the layout qgemm_run reads."""
    f = _fmt(fmt)
    N, K = W.shape
    wb, sb = qgemm_packed_size(K, N, f)
    if Bq is None:
        Bq = torch.empty(wb, dtype=torch.uint8, device=W.device)
    if scales is None:
        scales = torch.empty(sb, dtype=torch.uint8, device=W.device)
    _check(load().qgemm_quantize_pack_device(K, N, f, _dev_ptr(W), _dev_ptr(Bq), _dev_ptr(scales),
                                             _stream(stream)), "qgemm_quantize_pack_device")
    return Bq, scales


def qgemm_set_gemv_max_m(max_m: int) -> int:
    return load().qgemm_set_gemv_max_m(max_m)


# ---------------------------------------------------------------------------
# Convenience: a packed weight resident on the GPU.
# ---------------------------------------------------------------------------
class PackedWeight:
    """Quantise (or take) a weight, pack it and upload it to the GPU."""

    def __init__(self, fmt, K: int, N: int, w_canonical: np.ndarray,
                 pairs_canonical: np.ndarray | None, device="cuda"):
        self.fmt = _fmt(fmt)
        self.K, self.N = K, N
        wp, sp = qgemm_pack_weights(K, N, self.fmt, w_canonical, pairs_canonical)
        self.Bq = torch.from_numpy(wp).to(device)
        self.scales = torch.from_numpy(sp).to(device) if sp.size else None

    @classmethod
    def from_float(cls, fmt, W: np.ndarray, device="cuda"):
        """W [N][K] float -> quantised by the library's host quantiser."""
        f = _fmt(fmt)
        N, K = W.shape
        if f == QGEMM_F32:
            return cls(f, K, N, np.ascontiguousarray(W.T, dtype=np.float32), None, device)
        q, pairs = qgemm_quantize_weights(W, f)
        return cls(f, K, N, q, pairs, device)

    def __call__(self, A: torch.Tensor, C: torch.Tensor | None = None, stream=None):
        if A.dim() != 2 or A.shape[1] != self.K:
            raise ValueError(f"A: shape {tuple(A.shape)}, expected [M][{self.K}]")
        M = A.shape[0]
        if C is None:
            C = torch.empty((M, self.N), dtype=torch.float32, device=A.device)
        qgemm_run(M, self.K, self.N, self.fmt, A, self.Bq, self.scales, C, stream)
        return C

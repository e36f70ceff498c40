"""Helpers of the GPU parity tests: upload canonical inputs, run the library
through its C ABI, and compare with the oracle to the stated tolerances."""
from __future__ import annotations

import numpy as np
import torch

from weight_quantized_gemm_amd import qgemm as Q

# Tolerances for the fp16/fp32-accumulated paths, measured in fp64 against
# the oracle: max |C - C_ref| <= 1e-2 and ||C - C_ref||_F / ||C_ref||_F <= 2e-3.
MAX_ABS = 1e-2
REL_F = 2e-3


def require_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible to torch")


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run(fmt: str, M: int, K: int, N: int, A: np.ndarray, wc: np.ndarray,
        pairs: np.ndarray | None, stream=None, ws: bool = False) -> np.ndarray:
    """Pack on the host, upload, run qgemm_run (or qgemm_run_ws), return C."""
    wp, sp = Q.qgemm_pack_weights(K, N, fmt, wc, pairs)
    Ad = dev(A) if M * K else torch.empty(0, device="cuda")
    Bd = dev(wp)
    Sd = dev(sp) if sp.size else None
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    if ws:
        nbytes = Q.qgemm_workspace_size(M, K, N, fmt)
        W = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
        Q.qgemm_run_ws(M, K, N, fmt, Ad, Bd, Sd, C, W, nbytes, stream)
    else:
        Q.qgemm_run(M, K, N, fmt, Ad, Bd, Sd, C, stream)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def compare(C: np.ndarray, ref: np.ndarray, what: str = "", max_abs=MAX_ABS, rel_f=REL_F):
    """Asserts both tolerance criteria; returns (max_abs_err, rel_F, wrong/total)."""
    C = C.astype(np.float64)
    ref = ref.astype(np.float64)
    assert C.shape == ref.shape, (C.shape, ref.shape)
    assert np.all(np.isfinite(C)), f"{what}: non-finite outputs"
    err = np.abs(C - ref)
    mx = float(err.max()) if err.size else 0.0
    nrm = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(C - ref) / nrm) if nrm > 0 else float(np.linalg.norm(C - ref))
    wrong = int(np.count_nonzero(err > max_abs))
    assert mx <= max_abs and rel <= rel_f, \
        f"{what}: max_abs={mx:.3e} rel_F={rel:.3e} wrong={wrong}/{err.size}"
    return mx, rel, f"{wrong}/{err.size}"

"""GPU parity of the fused epilogue C = act(A x B + bias + residual), C fp32 or
fp16, through qgemm_run_ex, against the oracle's product followed by the
oracle's epilogue (fp16 outputs rounded to nearest even by the oracle).

Every kernel path is covered: the GEMVs (Int4, Int8, fp16, W4A8 with and
without the fused quantiser), the tiled Int4 / Int8 / fp16 / fp32 / W4A8
GEMMs, every split-K reduce, fp32 K-groups and Int4 / Int8 blocks of 16, 32
and 48 elements. Both
sides start from the oracle's quantisation of the seeded weights (the
library packs it). Tolerances are
the library's (max-abs 1e-2, relative-Frobenius 2e-3); an fp16 output may
differ from the oracle's by one fp16 step where the two round values on
either side of a tie point, which stays inside max-abs for |C| < 16.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import compare, dev, require_gpu
from oracle import oracle as O
from weight_quantized_gemm_amd import qgemm as Q
from weight_quantized_gemm_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    prev = Q.qgemm_set_gemv_max_m(8)
    yield
    Q.qgemm_set_gemv_max_m(prev)


SHAPES = [("f32", 16, 256, 256), ("f32", 8, 2560, 1024), ("f32", 130, 512, 200),
          ("int4b64", 1, 4096, 300), ("int4b64", 96, 1024, 300), ("int4b64", 65, 4096, 256),
          ("int8b0", 3, 1000, 130), ("int8b0", 130, 640, 200), ("w4a8", 100, 640, 256),
          ("f16", 3, 1000, 130), ("f16", 130, 640, 200),
          ("w4a8", 1, 4096, 300), ("w4a8", 6, 2048, 300), ("w4a8", 40, 3072, 300),
          ("int8b0", 32, 2560, 256), ("f16", 9, 4096, 96), ("int4b32", 96, 1024, 300),
          ("int4b64", 3, 9728, 640), ("w4a8", 2, 9728, 640), ("int8b64", 3, 1024, 130),
          ("int8b32", 130, 640, 200), ("int4b16", 96, 1024, 300), ("int8b16", 3, 1024, 130),
          ("int4b48", 2, 2496, 300), ("int4b64", 1000, 640, 2300)]
EPILOGUES = [("bias", "silu", "f32", False), ("residual", "gelu", "f16", False),
             ("bias+residual", "relu", "f32", False), ("bias+residual", "gelu", "f16", True),
             ("bias+residual", "none", "f32", True)]


def _product(fmt, M, K, N, seed):
    """Inputs, packed device weights and the oracle's fp64 product."""
    rng = np.random.default_rng(seed)
    if fmt in ("f32", "f16"):
        A = synth.activations(rng, M, K, fp16=(fmt == "f16"))
        B = synth.float_pattern_weights(K, N) if fmt == "f32" else synth.half_pattern_weights(K, N)
        wp, sp = Q.qgemm_pack_weights(K, N, fmt, B, None)
        return A, dev(wp), None, O.reference(fmt, A, B=B)
    A = synth.activations(rng, M, K, fp16=True)
    q, p = O.quantize(synth.normal_weights(rng, N, K), fmt)
    wp, sp = Q.qgemm_pack_weights(K, N, fmt, q, p)
    return A, dev(wp), dev(sp), O.reference(fmt, A, q=q, pairs=p)


@pytest.mark.parametrize("fmt,M,K,N", SHAPES)
@pytest.mark.parametrize("parts,act,out,inplace", EPILOGUES)
def test_epilogue(fmt, M, K, N, parts, act, out, inplace):
    A, Bd, Sd, P = _product(fmt, M, K, N, seed=M * 3 + K + N)
    rng = np.random.default_rng(M + N)
    odt = np.float16 if out == "f16" else np.float32
    tdt = torch.float16 if out == "f16" else torch.float32
    bias = rng.standard_normal(N).astype(np.float32) if "bias" in parts else None
    res = rng.standard_normal((M, N)).astype(odt) if "residual" in parts else None
    want = O.epilogue(P, bias, res, act, out_f16=(out == "f16"))
    C = torch.full((M, N), float("nan"), dtype=tdt, device="cuda")
    if inplace:
        C.copy_(torch.from_numpy(res))
        res_d = C
    else:
        res_d = dev(res) if res is not None else None
    Q.qgemm_run_ex(M, K, N, fmt, dev(A), Bd, Sd, C, bias=dev(bias) if bias is not None else None,
                   residual=res_d, activation=act, out_type=out)
    torch.cuda.synchronize()
    compare(C.float().cpu().numpy(), want, f"{fmt} {M}x{K}x{N} {parts} {act} {out}")


def test_plain_ex_equals_run():
    """qgemm_run_ex with no epilogue (and with a caller workspace) gives
    exactly what qgemm_run gives, on a split-K shape."""
    M, K, N = 65, 4096, 256
    A, Bd, Sd, _ = _product("int4b64", M, K, N, seed=7)
    Ad = dev(A)
    C1 = torch.empty((M, N), device="cuda")
    C2 = torch.empty((M, N), device="cuda")
    C3 = torch.empty((M, N), device="cuda")
    Q.qgemm_run(M, K, N, "int4b64", Ad, Bd, Sd, C1)
    Q.qgemm_run_ex(M, K, N, "int4b64", Ad, Bd, Sd, C2)
    nb = Q.qgemm_workspace_size(M, K, N, "int4b64")
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    Q.qgemm_run_ex(M, K, N, "int4b64", Ad, Bd, Sd, C3, workspace=ws, ws_bytes=nb)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2) and torch.equal(C1, C3)

"""qgemm_run_noalloc (scratch in the library's fixed per-GPU array) against
qgemm_run_ex with a caller workspace: the same kernels on the same inputs,
so the outputs must be identical, on two calls in a row (the second one
smaller, so it runs on what the first left in the array)."""
import numpy as np
import pytest
import torch

from tests.gpu_helpers import dev, require_gpu
from weight_quantized_gemm_amd import qgemm as Q
from weight_quantized_gemm_amd import synth

pytestmark = pytest.mark.gpu


def _inputs(fmt, M, K, N, seed):
    rng = np.random.default_rng(seed)
    A = synth.activations(rng, M, K, fp16=True)
    q, p = Q.qgemm_quantize_weights(synth.normal_weights(rng, N, K), fmt)
    wp, sp = Q.qgemm_pack_weights(K, N, fmt, q, p)
    return dev(A), dev(wp), dev(sp)


def _both(fmt, M, K, N, seed, **epi):
    A, Bq, S = _inputs(fmt, M, K, N, seed)
    out = torch.float16 if epi.get("out_type") == "f16" else torch.float32
    ws_bytes = Q.qgemm_workspace_size(M, K, N, fmt)
    assert ws_bytes > 0, "the case must use scratch"
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    C_ex = torch.full((M, N), float("nan"), dtype=out, device="cuda")
    C_na = torch.full((M, N), float("nan"), dtype=out, device="cuda")
    Q.qgemm_run_ex(M, K, N, fmt, A, Bq, S, C_ex, workspace=ws, ws_bytes=ws_bytes, **epi)
    Q.qgemm_run_noalloc(M, K, N, fmt, A, Bq, S, C_na, **epi)
    torch.cuda.synchronize()
    return C_ex.cpu().numpy(), C_na.cpu().numpy(), ws_bytes


def test_noalloc_matches_run_ex_on_two_calls():
    require_gpu()
    # first: W4A8 prefill with split-K (activation codes and int32 partials in the scratch)
    ex1, na1, b1 = _both("w4a8", 192, 1024, 512, seed=11)
    assert np.all(np.isfinite(na1))
    assert np.array_equal(ex1, na1)
    # second, smaller: Int4-Block64 with split-K and a fused epilogue
    g = torch.Generator(device="cuda").manual_seed(5)
    bias = torch.randn(256, device="cuda", generator=g)
    ex2, na2, b2 = _both("int4b64", 24, 2048, 256, seed=12, bias=bias, activation="silu")
    assert b2 < b1
    assert np.all(np.isfinite(na2))
    assert np.array_equal(ex2, na2)

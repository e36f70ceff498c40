"""GPU parity of the device quantisers (qgemm_quantize_weights_device and
qgemm_quantize_pack_device, through the C ABI) against the oracle's
quantiser: codes and pairs bit-exact, packed buffers byte-identical to the
host packer's output of the oracle's canonical result (every byte written,
checked by filling the outputs with a marker first).

Inputs: the seeded normal weights at several shapes (several channel tiles,
ragged K and N), plus hand-built blocks that hit the quantiser's corner
cases: constant blocks (scale 0), exact round-half ties, signed zeros in
either order as minimum or maximum, a range whose scale is a float
subnormal, a range near the float limit, and non-finite weights (whose
block gets NaN pairs and zero codes, as the header states)."""
import numpy as np
import pytest
import torch

from gpu_helpers import compare, dev, require_gpu
from oracle import oracle as O
from weight_quantized_gemm_amd import qgemm as Q
from weight_quantized_gemm_amd import synth

pytestmark = pytest.mark.gpu

FMTS = ["int4b64", "int8b0", "w4a8", "int4b0"]
MARK = 0xA5


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _device_canonical(W, fmt):
    N, K = W.shape
    qb, pf = Q.qgemm_canonical_size(K, N, fmt)
    q = torch.full((max(qb, 1),), MARK, dtype=torch.uint8, device="cuda")
    p = torch.full((max(pf, 1),), float("nan"), dtype=torch.float32, device="cuda")
    qd, pd = Q.qgemm_quantize_weights_device(dev(W), fmt, q, p)
    torch.cuda.synchronize()
    return qd.cpu().numpy(), pd.cpu().numpy()


def _device_packed(W, fmt):
    N, K = W.shape
    wb, sb = Q.qgemm_packed_size(K, N, fmt)
    B = torch.full((wb,), MARK, dtype=torch.uint8, device="cuda")
    S = torch.full((sb,), MARK, dtype=torch.uint8, device="cuda")
    Q.qgemm_quantize_pack_device(dev(W), fmt, B, S)
    torch.cuda.synchronize()
    return B.cpu().numpy(), S.cpu().numpy()


def _check_bit_exact(W, fmt, what):
    N, K = W.shape
    q_ref, p_ref = O.quantize(W, fmt)
    q, p = _device_canonical(W, fmt)
    assert np.array_equal(q, q_ref), f"{what}: codes differ at {np.argwhere(q != q_ref)[:4].tolist()}"
    assert np.array_equal(p.view(np.uint32), p_ref.view(np.uint32)), \
        f"{what}: pairs differ at {np.argwhere(p.view(np.uint32) != p_ref.view(np.uint32))[:4].tolist()}"
    wp_ref, sp_ref = Q.qgemm_pack_weights(K, N, fmt, q_ref, p_ref)
    wp, sp = _device_packed(W, fmt)
    assert np.array_equal(wp, wp_ref), f"{what}: packed codes differ at {np.flatnonzero(wp != wp_ref)[:8]}"
    assert np.array_equal(sp, sp_ref), f"{what}: packed pairs differ at {np.flatnonzero(sp != sp_ref)[:8]}"


SHAPES = {
    "int4b64": [(64, 1), (128, 70), (576, 33), (4096, 300)],
    "int4b0": [(64, 1), (128, 70), (640, 40), (4096, 96)],
    "int8b0": [(1, 3), (137, 70), (1001, 9), (4096, 256), (5000, 5)],
    "w4a8": [(2, 1), (70, 70), (1002, 33), (3072, 128), (9000, 7)],
    "int4b128": [(128, 1), (256, 70), (4096, 300)],
    "int4b32": [(64, 1), (128, 70), (4096, 300)],
    "int4b320": [(640, 33), (2560, 40)],
    "int8b64": [(64, 1), (128, 70), (4096, 300)],
    "int8b32": [(64, 1), (128, 70), (4096, 300)],
    "int8b512": [(512, 3), (4096, 70)],
    "int8b192": [(192, 5), (2304, 40)],
    "int4b16": [(64, 1), (128, 70), (4096, 300)],
    "int8b16": [(64, 1), (128, 70), (4096, 300)],
}


@pytest.mark.parametrize("fmt", FMTS + ["int4b32", "int4b128", "int4b320", "int8b64", "int8b32",
                                 "int8b512", "int8b192", "int4b16", "int8b16"])
def test_device_quantizer_bit_exact(fmt):
    for i, (K, N) in enumerate(SHAPES[fmt]):
        rng = np.random.default_rng(700 + i)
        W = synth.normal_weights(rng, N, K)
        print(f"quantize {fmt} K={K} N={N}", flush=True)
        _check_bit_exact(W, fmt, f"{fmt} K={K} N={N}")


def _corner_rows(K):
    """Rows of length K (a multiple of 64) whose 64-blocks hit the quantiser's
    corner cases; for the per-channel formats each row is one block."""
    rows = []
    r = np.zeros(K, np.float32); r[:] = 0.75; rows.append(r)                       # constant
    r = np.tile(np.arange(64, dtype=np.float32) % 16, K // 64); r[1::7] += 0.5     # ties
    r[0], r[-1] = 0.0, 15.0; rows.append(r)
    r = (np.arange(K, dtype=np.float32) % 5) * 0.25; r[0::64] = -0.0; r[1::64] = 0.0; rows.append(r)
    r = (np.arange(K, dtype=np.float32) % 5) * 0.25; r[0::64] = 0.0; r[1::64] = -0.0; rows.append(r)
    r = -(np.arange(K, dtype=np.float32) % 7) * 0.5; r[3::64] = -0.0; r[9::64] = 0.0; rows.append(r)
    r = np.zeros(K, np.float32); r[::2] = -0.0; rows.append(r)                     # all zeros, mixed signs
    r = np.zeros(K, np.float32); r[1::2] = -0.0; rows.append(r)
    r = (np.arange(K) % 16).astype(np.float32) * np.float32(1e-44); rows.append(r)  # subnormal scale
    r = np.linspace(-3.0e38, 3.0e38, K).astype(np.float32); rows.append(r)          # near the float limit
    r = np.zeros(K, np.float32); r[5] = 1.0; rows.append(r)                         # one nonzero
    return np.stack(rows)


@pytest.mark.parametrize("fmt", FMTS + ["int4b32", "int4b128", "int8b64", "int8b32", "int4b16",
                                 "int8b16"])
def test_device_quantizer_corner_cases(fmt):
    for K in ((128, 256) if fmt == "int4b128" else (64, 256)):
        W = _corner_rows(K)
        rng = np.random.default_rng(5)
        # mix corner blocks into random rows so that blocks of one row differ
        W2 = synth.normal_weights(rng, W.shape[0], K)
        W2[:, :64] = W[:, :64]
        for name, M in (("corner", W), ("mixed", W2)):
            print(f"quantize corners {fmt} K={K} {name}", flush=True)
            _check_bit_exact(np.ascontiguousarray(M), fmt, f"{fmt} K={K} {name}")


@pytest.mark.parametrize("fmt", FMTS)
def test_device_quantizer_nonfinite_blocks(fmt):
    K, N = 256, 40
    W = synth.normal_weights(np.random.default_rng(9), N, K)
    bad = {3: np.nan, 17: np.inf, 30: -np.inf}
    for n, x in bad.items():
        W[n, 70] = x                              # k = 70: block 1 of Int4-Block64
    q, p = _device_canonical(W, fmt)
    clean = W.copy()
    for n in bad:
        clean[n, 70] = 0.0
    q_ref, p_ref = O.quantize(clean, fmt)
    bits8 = fmt == "int8b0"
    per_block = fmt == "int4b64"
    for n in range(N):
        for b in range(p_ref.shape[1]):
            k0, k1 = (64 * b, 64 * b + 64) if per_block else (0, K)
            cs = slice(k0, k1) if bits8 else slice(k0 // 2, k1 // 2)
            hit = n in bad and k0 <= 70 < k1
            if hit:
                assert np.isnan(p[n, b]).all(), (n, b)
                assert not q[n, cs].any(), (n, b)
            else:
                assert np.array_equal(p[n, b], p_ref[n, b]), (n, b)
                assert np.array_equal(q[n, cs], q_ref[n, cs]), (n, b)


@pytest.mark.parametrize("fmt", FMTS)
def test_device_quantize_pack_then_run(fmt):
    """Weights quantised and packed on the GPU run through qgemm_run and match
    the oracle's product of the oracle's quantisation."""
    M, K, N = 9, 1024, 200
    rng = np.random.default_rng(40)
    A = synth.activations(rng, M, K, fp16=True)
    W = synth.normal_weights(rng, N, K)
    B, S = Q.qgemm_quantize_pack_device(dev(W), fmt)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    Q.qgemm_run(M, K, N, fmt, dev(A), B, S, C)
    torch.cuda.synchronize()
    q_ref, p_ref = O.quantize(W, fmt)
    compare(C.cpu().numpy(), O.reference(fmt, A, q=q_ref, pairs=p_ref), f"{fmt} quantize+run")


def test_device_quantizer_full_size_decode_weights():
    """The decode workload's weights (K = 4096, N = 11008) quantised and packed
    on the GPU equal the host path's bytes."""
    W = synth.normal_weights(np.random.default_rng(301), 11008, 4096)
    print("quantize int4b64 K=4096 N=11008", flush=True)
    _check_bit_exact(W, "int4b64", "int4b64 4096x11008")

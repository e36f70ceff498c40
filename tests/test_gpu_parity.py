"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Inputs come from the seeded generator; the library's own host quantiser
produces the HIP side's canonical weights and the oracle's quantiser the
oracle side's (the two are bit-identical, checked on the CPU). Tolerances:
max-abs 1e-2 and relative-Frobenius 2e-3 for the fp16/fp32-accumulated
paths; bit-exact for the W4A8 integer intermediates (qa, sa, S, D).
"""
import json
import os

import numpy as np
import pytest
import torch

from gpu_helpers import compare, dev, require_gpu, run
from oracle import oracle as O
from weight_quantized_gemm_amd import qgemm as Q
from weight_quantized_gemm_amd import synth

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    prev = Q.qgemm_set_gemv_max_m(8)
    yield
    Q.qgemm_set_gemv_max_m(prev)


def _case(fmt, M, K, N, seed):
    rng = np.random.default_rng(seed)
    if fmt == "f32":
        A = synth.activations(rng, M, K, fp16=False)
        return A, synth.float_pattern_weights(K, N), None
    if fmt == "f16":
        return synth.activations(rng, M, K, fp16=True), synth.half_pattern_weights(K, N), None
    A = synth.activations(rng, M, K, fp16=True)
    W = synth.normal_weights(rng, N, K)
    return A, W, None


def _quantized_pair(fmt, W):
    q_lib, p_lib = Q.qgemm_quantize_weights(W, fmt)
    q_orc, p_orc = O.quantize(W, fmt)
    assert np.array_equal(q_lib, q_orc) and np.array_equal(p_lib, p_orc)
    return q_lib, p_lib, q_orc, p_orc


def _parity(fmt, M, K, N, seed, rows=None, stream=None, ws=False):
    """Runs one shape on the GPU and checks it (optionally on sampled rows)."""
    A, W, _ = _case(fmt, M, K, N, seed)
    if fmt in ("f32", "f16"):
        C = run(fmt, M, K, N, A, W, None, stream=stream)
        sel = slice(None) if rows is None else rows
        ref = O.reference(fmt, A[sel], B=W)
        return compare(C[sel], ref, f"{fmt} {M}x{K}x{N}")
    q, p, qo, po = _quantized_pair(fmt, W)
    C = run(fmt, M, K, N, A, q, p, stream=stream, ws=ws)
    sel = slice(None) if rows is None else rows
    ref = O.reference(fmt, A[sel], q=qo, pairs=po)
    return compare(C[sel], ref, f"{fmt} {M}x{K}x{N}")


# ---------------------------------------------------------------------------
# The named workloads, in the launch configuration the bench uses.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_named_workload(name):
    fmt, M, K, N, seed = synth.CONFIGS[name]
    inp = synth.make_inputs(name)
    A = inp["A"]
    if fmt == "f32":
        C = run(fmt, M, K, N, A, inp["B"], None)
        compare(C, O.gemm_f32(A, inp["B"]), name)
        return
    q, p, qo, po = _quantized_pair(fmt, inp["W"])
    if fmt == "w4a8":
        nbytes = Q.qgemm_workspace_size(M, K, N, fmt)
        wp, sp = Q.qgemm_pack_weights(K, N, fmt, q, p)
        Ad, Bd, Sd = dev(A), dev(wp), dev(sp)
        C = torch.empty((M, N), dtype=torch.float32, device="cuda")
        qa = torch.empty((M, K), dtype=torch.int8, device="cuda")
        sa = torch.empty(M, dtype=torch.float32, device="cuda")
        S = torch.empty(M, dtype=torch.int32, device="cuda")
        D = torch.empty((M, N), dtype=torch.int32, device="cuda")
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        Q.qgemm_w4a8_debug(M, K, N, Ad, Bd, Sd, C, qa, sa, S, D, ws, nbytes)
        torch.cuda.synchronize()
        qa_o, sa_o, S_o = O.w4a8_actquant(A)
        # activation quantisation of every row, bit-exact
        assert np.array_equal(qa.cpu().numpy(), qa_o)
        assert np.array_equal(sa.cpu().numpy().view(np.uint32), sa_o.view(np.uint32))
        assert np.array_equal(S.cpu().numpy(), S_o)
        # the exact integer product on every output, bit-exact, and C
        D_o = O.w4a8_dot(qa_o, qo)
        assert np.array_equal(D.cpu().numpy().astype(np.int64), D_o)
        ref = O.w4a8_rescale(D_o, sa_o, S_o, po)
        compare(C.cpu().numpy(), ref, name)
        # the plain entry point (library-allocated scratch) gives the same C
        C2 = run(fmt, M, K, N, A, q, p)
        assert np.array_equal(C2, C.cpu().numpy())
        return
    C = run(fmt, M, K, N, A, q, p)
    assert np.all(np.isfinite(C))
    compare(C, O.reference(fmt, A, q=qo, pairs=po), name)


# ---------------------------------------------------------------------------
# Ragged shapes, both dispatch paths, tails over several tiles.
# ---------------------------------------------------------------------------
SMALL_M = [1, 2, 3, 4, 5, 7, 8, 9, 63, 64, 65, 129]


@pytest.mark.parametrize("M", SMALL_M)
def test_f16_shapes(M):
    """fp16 weights: GEMV for M <= 8 up to K = 8192, the tiled GEMM otherwise
    (so K = 9000 takes the GEMM at every M); ragged K and N."""
    for K, N in [(64, 1), (137, 70), (256, 130), (4160, 67), (9000, 40)]:
        _parity("f16", M, K, N, seed=M * 5 + K + N)


@pytest.mark.parametrize("M", [1, 3, 8])
def test_int4_gemv_split_k(M):
    """The Int4 GEMV on shapes with few 32-channel tiles splits K over the
    workgroups of a tile and adds the partial tiles in a fixed order; ragged N,
    passes of 64 blocks, Block0 and blocks of 16, 32 and 48 included."""
    for fmt, K, N in [("int4b64", 9728, 2560), ("int4b64", 2560, 1024), ("int4b64", 4096, 300),
                      ("int4b64", 16384, 70), ("int4b0", 9728, 96), ("int4b32", 9728, 130),
                      ("int4b16", 9728, 130), ("int4b48", 2496, 1024)]:
        _parity(fmt, M, K, N, seed=M * 7 + K + N)


@pytest.mark.parametrize("M", [1, 2, 3, 5, 8])
def test_int4_gemv_k_passes(M):
    """The half-tile Int4 GEMV over K in passes of 64 blocks (K > 4096) with
    enough channel tiles not to split: ragged N, an odd block count in the
    last pass, blocks of 16 and 32; with at most one half tile per CU (N <= 4096 at
    one row group) the sixteen-wave kernel, a two-block last pass among them."""
    for fmt, K, N in [("int4b64", 8192, 4100), ("int4b32", 5120, 1000), ("int4b64", 12352, 4128),
                      ("int4b64", 8320, 4000), ("int4b64", 11008, 4096), ("int4b16", 5120, 1000)]:
        _parity(fmt, M, K, N, seed=M * 23 + K + N)


@pytest.mark.parametrize("M", [1, 3, 8, 9, 64, 65, 129])
def test_int4_other_block_sizes(M):
    """Int4 with blocks of 16, 32, 48, 80, 96, 128, 256 and 320 K-elements (the
    page's blockSize parameter, any multiple of 16 that divides K) through
    the Int4 GEMV and GEMM, split-K shapes included."""
    for fmt, K, N in [("int4b128", 128, 5), ("int4b128", 4096, 256), ("int4b256", 2560, 1024),
                      ("int4b320", 640, 130), ("int4b128", 9728, 96), ("int4b32", 64, 33),
                      ("int4b32", 4096, 300), ("int4b32", 2560, 1024), ("int4b16", 64, 33),
                      ("int4b16", 4096, 300), ("int4b48", 192, 70), ("int4b48", 2496, 1024),
                      ("int4b80", 640, 256), ("int4b96", 3072, 130)]:
        _parity(fmt, M, K, N, seed=M * 17 + K + N)


@pytest.mark.parametrize("M", [9, 16, 31, 32, 33, 48, 64])
def test_int4_skinny(M):
    """The skinny prefill kernel (GEMV threshold < M <= 64: a 32-channel tile of
    every row per workgroup, passes of 16 or 8 blocks double-buffered): one
    and several passes (a short last pass), split K and not, ragged N, pairs
    per 64-block, per 32-half and per 16-quarter."""
    for fmt, K, N in [("int4b64", 64, 33), ("int4b64", 2560, 4096), ("int4b64", 9728, 300),
                      ("int4b64", 4096, 11008), ("int4b0", 1088, 70), ("int4b32", 3072, 1000),
                      ("int4b16", 2560, 130), ("int4b48", 768, 100)]:
        _parity(fmt, M, K, N, seed=M * 29 + K + N)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 9, 64, 65, 129])
def test_int8_block_sizes(M):
    """Int8 with a pair per block of 16, 32, 48, 64, 80, 96, 128, 192 or 320
    K-elements: the
    Int8 GEMV (M <= 4, K <= 8192) adds each 16-code slice with its block's
    pair; the channel-row GEMM dequantises per weight (split-K shapes, K past
    the GEMV's limit, ragged N)."""
    for fmt, K, N in [("int8b64", 64, 5), ("int8b64", 4096, 256), ("int8b32", 2560, 1024),
                      ("int8b128", 4096, 300), ("int8b320", 640, 130), ("int8b64", 9728, 96),
                      ("int8b192", 768, 70), ("int8b32", 8192, 40), ("int8b16", 2560, 1024),
                      ("int8b16", 8192, 40), ("int8b48", 768, 70), ("int8b80", 640, 130),
                      ("int8b96", 4608, 300)]:
        _parity(fmt, M, K, N, seed=M * 19 + K + N)


@pytest.mark.parametrize("M", [1, 3, 8, 9, 64, 65, 129])
def test_int4b0_shapes(M):
    """Int4-Block0 with fp16 activations (per-channel pairs) through the
    Int4 GEMV and GEMM, split-K shapes included."""
    for K, N in [(64, 5), (256, 130), (4096, 256), (2560, 1024)]:
        _parity("int4b0", M, K, N, seed=M * 13 + K + N)


@pytest.mark.parametrize("M", SMALL_M)
def test_int4b64_shapes(M):
    for K, N in [(64, 1), (64, 5), (192, 70), (256, 130), (4160, 67)]:
        _parity("int4b64", M, K, N, seed=M * 7 + K + N)


@pytest.mark.parametrize("fmt", ["f32", "f16", "int8b0", "int4b64", "w4a8"])
@pytest.mark.parametrize("K,N", synth.PAGE_KN)
def test_page_shape_grid(fmt, K, N):
    """Every (K, N) of the benchmark page's default sizes at its M values, every
    format; rows sampled (first, tile edges, last) once M is past 32."""
    for M in synth.PAGE_M:
        rows = None if M <= 32 else sorted({0, 1, 63, 64, M // 2, M - 2, M - 1})
        _parity(fmt, M, K, N, seed=K + N + M, rows=rows)


@pytest.mark.parametrize("M,K,N", [(9, 4160, 67), (65, 4096, 256), (64, 1920, 384),
                                   (33, 9728, 2560), (128, 2560, 1024)])
def test_int4b64_split_k(M, K, N):
    """Shapes with few output tiles split K over several workgroups
    (partials in the workspace, added in a fixed order): parity, run vs
    run_ws and repeat runs bit-identical."""
    assert Q.qgemm_workspace_size(M, K, N, "int4b64") >= 2 * M * N * 4   # the split engages
    A, W, _ = _case("int4b64", M, K, N, seed=M + K + N)
    q, p, qo, po = _quantized_pair("int4b64", W)
    C1 = run("int4b64", M, K, N, A, q, p)
    compare(C1, O.reference("int4b64", A, q=qo, pairs=po), f"split {M}x{K}x{N}")
    C2 = run("int4b64", M, K, N, A, q, p, ws=True)
    C3 = run("int4b64", M, K, N, A, q, p)
    assert np.array_equal(C1, C2) and np.array_equal(C1, C3)


@pytest.mark.parametrize("fmt,M,K,N,sample", [("int4b64", 1000, 640, 2300, False),
                                               ("int4b32", 1000, 640, 2300, False),
                                               ("int4b16", 1024, 320, 2304, False),
                                               ("int4b64", 2000, 1088, 4000, True)])
def test_int4_wide_tiles(fmt, M, K, N, sample):
    """Shapes whose 128 x 128 tiles take fewer rounds of the CUs than 128 x 64
    ones (8 x 18 = 144 tiles in one round against 288 in two; 16 x 32 = 512
    in two against 1008 in four): the wide tile's two-chunk reduction, ragged
    last row and column tiles, and K quarters of unequal length. The largest
    shape is compared on rows spanning every row tile and its edges."""
    rows = sorted({*range(0, M, 61), 127, 128, 1919, 1920, M - 1}) if sample else None
    _parity(fmt, M, K, N, seed=M + K + N, rows=rows)


@pytest.mark.parametrize("M,K,N", [(1000, 256, 4000), (512, 2560, 4096), (200, 8190, 1000)])
def test_w4a8_half_width_tiles(M, K, N):
    """W4A8 shapes whose 128 x 128 tiles fit one round of the CUs (two rows of
    four waves, 64 x 32 each): 256 tiles with ragged last row and column
    tiles (the staged fp32 store's element path), 128 tiles unsplit, and a
    split shape with a ragged K; D bit-exact where checked."""
    _parity("w4a8", M, K, N, seed=M + K + N)
    if M <= 512:
        _w4a8_debug_check(M, K, N, seed=M + K + N + 1, zero_row=3)


@pytest.mark.parametrize("M,K,N,split", [(16, 256, 256, False), (3, 137, 70, False),
                                         (8, 2560, 1024, True), (1, 9728, 64, True),
                                         (40, 640, 100, False), (17, 4096, 4096, True),
                                         (64, 8192, 256, True)])
def test_f32_split_k(M, K, N, split):
    """fp32 shapes with few output tiles spread K over two thread groups per
    workgroup and, when that is still too few, over workgroups (chunks of 64,
    the last one ragged): parity, run vs run_ws and repeats bit-identical."""
    ws = Q.qgemm_workspace_size(M, K, N, "f32")
    assert (ws >= 2 * M * N * 4) if split else ws == 0
    A, W, _ = _case("f32", M, K, N, seed=M + K + N)
    C1 = run("f32", M, K, N, A, W, None)
    compare(C1, O.gemm_f32(A, W), f"f32 split {M}x{K}x{N}")
    C2 = run("f32", M, K, N, A, W, None, ws=True)
    C3 = run("f32", M, K, N, A, W, None)
    assert np.array_equal(C1, C2) and np.array_equal(C1, C3)


@pytest.mark.parametrize("M", [1, 3, 5, 8])
def test_int4b64_gemv_long_k(M):
    """The decode kernel walks K in passes of 64 blocks: K = 9728 (a K of the
    page's shape grid) takes two full passes and a partial third."""
    K, N = 9728, 70
    A, W, _ = _case("int4b64", M, K, N, seed=9728 + M)
    q, p, qo, po = _quantized_pair("int4b64", W)
    C = run("int4b64", M, K, N, A, q, p)
    compare(C, O.reference("int4b64", A, q=qo, pairs=po), f"int4b64 gemv M={M} K={K}")


@pytest.mark.parametrize("K", [64, 128, 192, 256, 320, 384, 448, 512, 576, 640, 1024])
def test_int4b64_tiled_short_k(K):
    """The tiled kernel splits the K-blocks over four waves and pads each
    wave's count to its register ring; every per-wave count from 0 to 4
    blocks (plus a ragged remainder) must match the oracle and be
    bit-identical across calls."""
    M, N = 65, 130
    A, W, _ = _case("int4b64", M, K, N, seed=K)
    q, p, qo, po = _quantized_pair("int4b64", W)
    C1 = run("int4b64", M, K, N, A, q, p)
    C2 = run("int4b64", M, K, N, A, q, p)
    compare(C1, O.reference("int4b64", A, q=qo, pairs=po), f"int4b64 tiled K={K}")
    assert np.array_equal(C1, C2)


@pytest.mark.parametrize("M", SMALL_M)
def test_int8b0_shapes(M):
    for K, N in [(1, 3), (7, 4), (12, 9), (64, 64), (100, 70), (1000, 33), (4100, 6)]:
        _parity("int8b0", M, K, N, seed=M * 11 + K + N)


@pytest.mark.parametrize("M", [1, 2, 3, 31, 32, 33, 127, 128, 129, 300])
def test_w4a8_shapes(M):
    for K, N in [(2, 1), (8, 33), (62, 5), (64, 64), (66, 130), (200, 31), (1030, 257)]:
        _parity("w4a8", M, K, N, seed=M * 13 + K + N)


@pytest.mark.parametrize("fmt", ["int4b64", "int8b0", "f16", "w4a8", "f32"])
def test_many_tiles_with_ragged_edges(fmt):
    """Shapes with enough output tiles that no K split is planned, and a ragged
    last row tile and last column tile: the tiled kernels' store phases (whole
    tile rows per store instruction; the W4A8 GEMM's 64 x 32 blocks through LDS,
    with partial blocks stored element by element) on full and partial tiles."""
    M, K, N = 1000, 256, 4100
    ws = Q.qgemm_workspace_size(M, K, N, fmt)
    assert ws < M * N * 4, "no split-K partial tiles for this shape"
    _parity(fmt, M, K, N, seed=4100 + len(fmt))


@pytest.mark.parametrize("M,K,N", [(1, 1, 1), (3, 137, 70), (16, 256, 256), (65, 17, 129),
                                   (130, 300, 67), (64, 64, 64)])
def test_f32_shapes(M, K, N):
    _parity("f32", M, K, N, seed=M + K + N)


def test_f32_k_zero_writes_zeros():
    C = run("f32", 3, 0, 5, np.zeros((3, 0), np.float32), np.zeros((0, 5), np.float32), None)
    assert np.array_equal(C, np.zeros((3, 5), np.float32))


@pytest.mark.parametrize("fmt", ["int4b64", "int8b0"])
@pytest.mark.parametrize("M", [1, 3, 8])
def test_gemv_and_tiled_paths_agree_with_oracle(fmt, M):
    """M <= 8 runs the GEMV by default; forcing the threshold to 0 sends the
    same call to the MFMA kernel. Both must meet the oracle's tolerance."""
    K, N = 1024, 300
    A, W, _ = _case(fmt, M, K, N, seed=99 + M)
    q, p, qo, po = _quantized_pair(fmt, W)
    ref = O.reference(fmt, A, q=qo, pairs=po)
    C_gemv = run(fmt, M, K, N, A, q, p)
    prev = Q.qgemm_set_gemv_max_m(0)
    try:
        C_mfma = run(fmt, M, K, N, A, q, p)
    finally:
        Q.qgemm_set_gemv_max_m(prev)
    compare(C_gemv, ref, "gemv")
    compare(C_mfma, ref, "mfma")


# ---------------------------------------------------------------------------
# Closed forms through the real kernels.
# ---------------------------------------------------------------------------
def _identity(fmt, K):
    eye = np.eye(K, dtype=np.uint8)
    return eye if fmt == "int8b0" else (eye[:, 0::2] | (eye[:, 1::2] << 4)).astype(np.uint8)


@pytest.mark.parametrize("fmt", ["int4b64", "int8b0"])
def test_identity_weights(fmt):
    """offset 0, scale 1, q = delta_kn: C = A. The Int4-Block64 MFMA path sums
    one nonzero product per output, so it is exact; the paths that regroup
    the product around the channel pair (both GEMVs and the Int8-Block0
    MFMA path, which multiplies the biased codes 1024 + q) remove a bias
    from an fp32 sum, so they are held to the tolerance."""
    K = 128
    rng = np.random.default_rng(5)
    A = rng.standard_normal((70, K)).astype(np.float16)
    q = _identity(fmt, K)
    nblk = K // 64 if fmt == "int4b64" else 1
    p = np.zeros((K, nblk, 2), np.float32)
    p[:, :, 1] = 1.0
    C = run(fmt, 70, K, K, A, q, p)
    if fmt == "int4b64":
        assert np.array_equal(C, A.astype(np.float32))
    else:
        compare(C, A.astype(np.float64), "int8b0 identity")
    C1 = run(fmt, 1, K, K, A[:1], q, p)
    compare(C1, A[:1].astype(np.float64), "gemv identity")


@pytest.mark.parametrize("fmt", ["int4b64", "int8b0"])
@pytest.mark.parametrize("M", [1, 100])
def test_constant_blocks(fmt, M):
    """scale = 0: C[m][n] = sum_b offset[n][b] * sum_{k in b} A[m][k]."""
    K, N = 256, 40
    rng = np.random.default_rng(6)
    A = rng.integers(-4, 5, size=(M, K)).astype(np.float16)
    nblk = K // 64 if fmt == "int4b64" else 1
    p = np.zeros((N, nblk, 2), np.float32)
    p[:, :, 0] = 2.0 ** rng.integers(-3, 3, size=(N, nblk))
    qb, _ = Q.qgemm_canonical_size(K, N, fmt)
    q = rng.integers(0, 256, size=qb).astype(np.uint8)
    C = run(fmt, M, K, N, A, q, p)
    want = A.astype(np.float64).reshape(M, nblk, K // nblk).sum(2) @ p[:, :, 0].T.astype(np.float64)
    compare(C, want, "constant blocks")


def test_w4a8_golden_rows_and_identity():
    """The hand-worked activation rows (ties, zero row, subnormals, the
    near-tie that separates division from reciprocal-multiply) through the
    GPU's quantiser, with identity weights so that D = qa."""
    g = json.load(open(os.path.join(GOLDEN, "w4a8_actquant_rows.json")))
    A = np.array([r["a"] for r in g["rows"]], dtype=np.float16)
    M, K = A.shape
    N = K
    q = _identity("int4b64", K)
    p = np.zeros((N, 1, 2), np.float32)
    p[:, 0, 1] = 1.0
    wp, sp = Q.qgemm_pack_weights(K, N, "w4a8", q, p)
    nbytes = Q.qgemm_workspace_size(M, K, N, "w4a8")
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    qa = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sa = torch.empty(M, dtype=torch.float32, device="cuda")
    S = torch.empty(M, dtype=torch.int32, device="cuda")
    D = torch.empty((M, N), dtype=torch.int32, device="cuda")
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    Q.qgemm_w4a8_debug(M, K, N, dev(A), dev(wp), dev(sp), C, qa, sa, S, D, ws, nbytes)
    torch.cuda.synchronize()
    for i, r in enumerate(g["rows"]):
        assert qa[i].cpu().tolist() == r["qa"], i
        assert int(sa[i].cpu().numpy().view(np.uint32)) == int(r["sa_bits"], 16), i
        assert int(S[i]) == r["S"], i
    assert np.array_equal(D.cpu().numpy(), qa.cpu().numpy().astype(np.int32))
    assert np.array_equal(C.cpu().numpy(), sa.cpu().numpy()[:, None] * qa.cpu().numpy())


def _w4a8_debug_check(M, K, N, seed, zero_row=None):
    A, W, _ = _case("w4a8", M, K, N, seed=seed)
    if zero_row is not None:
        A[zero_row] = 0
    q, p, qo, po = _quantized_pair("w4a8", W)
    wp, sp = Q.qgemm_pack_weights(K, N, "w4a8", q, p)
    nbytes = Q.qgemm_workspace_size(M, K, N, "w4a8")
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    qa = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sa = torch.empty(M, dtype=torch.float32, device="cuda")
    S = torch.empty(M, dtype=torch.int32, device="cuda")
    D = torch.empty((M, N), dtype=torch.int32, device="cuda")
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    Q.qgemm_w4a8_debug(M, K, N, dev(A), dev(wp), dev(sp), C, qa, sa, S, D, ws, nbytes)
    torch.cuda.synchronize()
    Cr, qa_o, sa_o, S_o, D_o = O.w4a8_gemm(A, qo, po)
    assert np.array_equal(qa.cpu().numpy(), qa_o)
    assert np.array_equal(sa.cpu().numpy(), sa_o)
    assert np.array_equal(S.cpu().numpy(), S_o)
    assert np.array_equal(D.cpu().numpy().astype(np.int64), D_o)
    compare(C.cpu().numpy(), Cr, f"w4a8 {M}x{K}x{N}")
    if zero_row is not None:
        assert np.all(C.cpu().numpy()[zero_row] == 0)


@pytest.mark.parametrize("M,K,N", [(1, 3072, 8192), (3, 1000, 70), (5, 9000, 96), (8, 4096, 300)])
def test_w4a8_gemv_debug_bit_exact(M, K, N):
    """The decode-shaped W4A8 GEMV (M <= 8): qa, sa, S and the int32 products
    D bit-exact, ragged K and N, K past 8192 (two passes of four rows)."""
    _w4a8_debug_check(M, K, N, seed=M + K, zero_row=M - 1 if M > 1 else None)


@pytest.mark.parametrize("M", [1, 2, 3, 8])
def test_w4a8_gemv_split_k_debug_bit_exact(M):
    """The W4A8 GEMV on shapes with few 32-channel tiles: past two rows (and at
    two rows past K = 8192) the standalone quantiser's codes, int32 partial
    tiles per K-slice and the exact reduce; one row keeps the fused kernel.
    D bit-exact, ragged K (a partial last record) and ragged N."""
    for K, N in [(9728, 2560), (16384, 70), (12350, 130), (6144, 1000)]:
        _w4a8_debug_check(M, K, N, seed=M * 3 + K + N, zero_row=M - 1 if M > 1 else None)


@pytest.mark.parametrize("M,K,N", [(9, 3072, 512), (40, 9728, 300), (130, 2560, 250), (9, 16000, 64)])
def test_w4a8_split_k_debug_bit_exact(M, K, N):
    """W4A8 GEMM shapes with few output tiles split K into slices whose int32
    partial products are added exactly: D stays bit-exact and C matches.
    K of 9728 and 16000 also take the long-row variants of the activation
    quantiser (24 and 32 chunks per lane), whose qa, sa and S are checked."""
    assert Q.qgemm_workspace_size(M, K, N, "w4a8") > Q.qgemm_workspace_size(M, K, 1, "w4a8")
    _w4a8_debug_check(M, K, N, seed=M + K + N, zero_row=2)


@pytest.mark.parametrize("fmt", ["int8b0", "f16"])
@pytest.mark.parametrize("M", [9, 32, 129])
def test_rows_gemm_split_k(fmt, M):
    """Channel-row GEMM (Int8-Block0, fp16 weights) on shapes with few output
    tiles: K split into slices, each carrying its share of the pair terms,
    added by the fixed-order reduce; ragged K and N."""
    for K, N in [(9728, 96), (4160, 200), (2500, 64)]:
        assert Q.qgemm_workspace_size(M, K, N, fmt) > 0
        _parity(fmt, M, K, N, seed=M + K + N)


def test_w4a8_debug_bit_exact_mid_size():
    M, K, N = 200, 3072, 300
    A, W, _ = _case("w4a8", M, K, N, seed=77)
    A[3] = 0                                   # a zero row
    q, p, qo, po = _quantized_pair("w4a8", W)
    wp, sp = Q.qgemm_pack_weights(K, N, "w4a8", q, p)
    nbytes = Q.qgemm_workspace_size(M, K, N, "w4a8")
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    qa = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sa = torch.empty(M, dtype=torch.float32, device="cuda")
    S = torch.empty(M, dtype=torch.int32, device="cuda")
    D = torch.empty((M, N), dtype=torch.int32, device="cuda")
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    Q.qgemm_w4a8_debug(M, K, N, dev(A), dev(wp), dev(sp), C, qa, sa, S, D, ws, nbytes)
    torch.cuda.synchronize()
    Cr, qa_o, sa_o, S_o, D_o = O.w4a8_gemm(A, qo, po)
    assert np.array_equal(qa.cpu().numpy(), qa_o)
    assert np.array_equal(sa.cpu().numpy(), sa_o)
    assert np.array_equal(S.cpu().numpy(), S_o)
    assert np.array_equal(D.cpu().numpy().astype(np.int64), D_o)
    compare(C.cpu().numpy(), Cr, "w4a8 mid")
    assert np.all(C.cpu().numpy()[3] == 0)


# ---------------------------------------------------------------------------
# Runtime behaviour.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", ["int4b64", "int8b0", "w4a8", "f32", "f16"])
def test_deterministic_and_stream(fmt):
    """Repeated runs are bit-identical (no atomics), also on a side stream
    and through the workspace entry point."""
    M, K, N = (130, 512, 200)
    A, W, _ = _case(fmt, M, K, N, seed=3)
    if fmt in ("f32", "f16"):
        wc, p = W, None
    else:
        wc, p = Q.qgemm_quantize_weights(W, fmt)
    C1 = run(fmt, M, K, N, A, wc, p)
    C2 = run(fmt, M, K, N, A, wc, p)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        C3 = run(fmt, M, K, N, A, wc, p, stream=s)
    C4 = run(fmt, M, K, N, A, wc, p, ws=True)
    assert np.array_equal(C1, C2) and np.array_equal(C1, C3) and np.array_equal(C1, C4)


def test_empty_product_touches_nothing():
    C = torch.full((4, 3), 7.0, device="cuda")
    Q.qgemm_run(0, 64, 3, "int4b64", None, None, None, C)
    Q.qgemm_run(4, 64, 0, "int4b64", None, None, None, C)
    torch.cuda.synchronize()
    assert torch.all(C == 7.0)


def test_errors_leave_output_untouched():
    C = torch.full((2, 8), 7.0, device="cuda")
    A = torch.zeros((2, 64), dtype=torch.float16, device="cuda")
    B = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    with pytest.raises(Q.QGemmError) as e:
        Q.qgemm_run(2, 64, 8, "int4b64", A, B, None, C)     # missing scales
    assert e.value.status == 1
    with pytest.raises(Q.QGemmError) as e:
        Q.qgemm_run(2, 60, 8, "int4b64", A, B, B, C)        # K % 64 != 0
    assert e.value.status == 2
    torch.cuda.synchronize()
    assert torch.all(C == 7.0)


def test_graph_capture_replays_match_eager():
    """The kernels record into a HIP graph (through torch's capture) and
    every replay, with unrelated eager work in between, reproduces the eager
    result bit for bit. W4A8 goes through qgemm_run_ws (qgemm_run allocates
    its scratch and is not meant for capture)."""
    calls = []
    # GEMVs (Int4, Int8, W4A8 fused and unfused), tiled GEMMs, and split-K
    # shapes of every tiled kernel with their reduce (fp32 and W4A8 int32)
    for fmt, M, K, N in [("int4b64", 1, 4096, 1000), ("int4b64", 200, 1024, 300),
                         ("int4b64", 64, 4096, 512),
                         ("int8b0", 3, 1000, 130), ("w4a8", 100, 640, 256),
                         ("w4a8", 1, 4096, 512), ("w4a8", 6, 2048, 300), ("w4a8", 40, 3072, 300),
                         ("int8b0", 32, 2560, 256), ("f16", 9, 4096, 96), ("int4b32", 100, 1024, 300),
                         ("int4b64", 2, 9728, 640), ("w4a8", 3, 9728, 640),
                         ("int8b64", 2, 4096, 300), ("int8b32", 100, 1024, 300)]:
        A, W, _ = _case(fmt, M, K, N, seed=M + N)
        if fmt == "f16":
            wp, sp = Q.qgemm_pack_weights(K, N, fmt, W, None)
        else:
            q, p = Q.qgemm_quantize_weights(W, fmt)
            wp, sp = Q.qgemm_pack_weights(K, N, fmt, q, p)
        nbytes = Q.qgemm_workspace_size(M, K, N, fmt)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
        calls.append((fmt, M, K, N, dev(A), dev(wp), dev(sp) if sp.size else None,
                      torch.empty((M, N), dtype=torch.float32, device="cuda"), ws, nbytes))

    def issue():
        for fmt, M, K, N, A, B, S, C, ws, nb in calls:
            Q.qgemm_run_ws(M, K, N, fmt, A, B, S, C, ws, nb)

    issue()
    torch.cuda.synchronize()
    eager = [c[7].clone() for c in calls]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        issue()
    for rep in range(4):
        for c in calls:
            c[7].fill_(float("nan"))
        x = torch.randn(1 << 20, device="cuda")
        _ = (x * 2).sum().item()
        g.replay()
        torch.cuda.synchronize()
        for c, e in zip(calls, eager):
            assert torch.equal(c[7], e), (rep, c[0], c[1])

"""C-ABI checks that need no GPU: exports, argument validation (every
rejection happens before anything touches the GPU), the host quantiser
against the oracle's quantiser (bit-exact), and packer round trips."""
import ctypes

import numpy as np
import pytest

from oracle import oracle as O
from weight_quantized_gemm_amd import qgemm as Q
from weight_quantized_gemm_amd import synth

FMTS = ["int4b64", "int8b0", "w4a8", "int4b0"]


@pytest.fixture(scope="module")
def lib():
    return Q.load()


def test_every_declared_symbol_is_exported(lib):
    import os
    import re
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "qgemm.h")).read()
    declared = set(re.findall(r"^\s*(?:const char \*|int |qgemm_status )(qgemm_\w+)\(", hdr, re.M))
    assert declared == set(Q.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    assert Q.qgemm_abi_version() == 1


def test_status_strings(lib):
    for code, name in Q.STATUS.items():
        assert Q.qgemm_status_string(code).startswith(name)
    assert Q.qgemm_status_string(12345) == "QGEMM_ERR_UNKNOWN"


def _run(lib, M, K, N, f, A=256, B=256, S=256, C=256, stream=None):
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.qgemm_run(M, K, N, f, v(A), v(B), v(S), v(C), stream)


def test_run_validation_before_device(lib):
    OK, NULL, SHAPE, FMT, ALIGN, DEV = 0, 1, 2, 3, 4, 6
    # unknown format
    assert _run(lib, 1, 64, 4, 7) == FMT
    # shapes
    assert _run(lib, -1, 64, 4, 1) == SHAPE
    assert _run(lib, 1, 63, 4, 1) == SHAPE          # Int4-Block64 needs K % 64 == 0
    assert _run(lib, 1, 0, 4, 1) == SHAPE
    assert _run(lib, 1, 0, 4, 2) == SHAPE
    assert _run(lib, 1, 65, 4, 3) == SHAPE          # W4A8 needs even K
    assert _run(lib, 1, 2 * 1127500, 4, 3) == SHAPE  # int32 D could overflow
    # empty products are valid and touch nothing
    assert _run(lib, 0, 64, 4, 1, None, None, None, None) == OK
    assert _run(lib, 5, 64, 0, 1, None, None, None, None) == OK
    # null pointers
    assert _run(lib, 1, 64, 4, 1, C=None) == NULL
    assert _run(lib, 1, 64, 4, 1, A=None) == NULL
    assert _run(lib, 1, 64, 4, 1, S=None) == NULL
    assert _run(lib, 1, 64, 4, 0, S=256) == FMT      # F32 takes no scales
    # alignment
    assert _run(lib, 1, 64, 4, 1, A=258) == ALIGN
    assert _run(lib, 1, 64, 4, 1, C=260) == ALIGN
    # a valid request on a host without a gfx950 GPU
    import torch
    if not torch.cuda.is_available():
        assert _run(lib, 1, 64, 4, 1) == DEV
        assert _run(lib, 3, 0, 4, 0, S=None) == DEV   # F32 with K = 0 is valid


def test_run_ws_validation(lib):
    v = ctypes.c_void_p
    ws = Q.qgemm_workspace_size(8, 128, 16, "w4a8")
    assert ws > 0 and Q.qgemm_workspace_size(8, 128, 16, "int4b64") == 0
    st = lib.qgemm_run_ws(8, 128, 16, 3, v(256), v(256), v(256), v(256), None, 0, None)
    assert st == 1                                   # W4A8 needs a workspace
    st = lib.qgemm_run_ws(8, 128, 16, 3, v(256), v(256), v(256), v(256), v(512), ws - 1, None)
    assert st == 8                                   # too small
    st = lib.qgemm_run_ws(8, 128, 16, 3, v(256), v(256), v(256), v(256), v(520), ws, None)
    assert st == 4                                   # misaligned


def test_split_k_workspace_plan():
    """Workspace is a function of the shape: Int4 GEMMs with few output tiles
    split K into at most 8 slices and need S partial [M][N] float tiles;
    shapes that fill the GPU need none. Up to M = 64 (the skinny kernel: a
    32-channel tile of every row per workgroup) slices keep >= 8 K-blocks
    of 64 and split while tiles x slices fit the 256 CUs; above, 64 x 128 or
    128 x 64 tiles split below 128 tiles, slices of >= 8 K-blocks."""
    def sz(M, K, N):
        return Q.qgemm_workspace_size(M, K, N, "int4b64")
    assert sz(64, 4096, 512) == 8 * 64 * 512 * 4          # 16 tiles -> 8 slices
    assert sz(64, 1920, 384) == 3 * 64 * 384 * 4          # 30 K-blocks -> 3 slices
    assert sz(32, 2560, 4096) == 2 * 32 * 4096 * 4        # 128 tiles -> 2 slices
    assert sz(48, 4096, 11008) == 2 * 48 * 11008 * 4      # 344 tiles: 64 x 128 tiles, 86 -> 2 slices
    assert sz(32, 9728, 2560) == 3 * 32 * 2560 * 4        # 80 tiles -> 3 slices (240 <= 256)
    assert sz(96, 4096, 512) == 8 * 96 * 512 * 4          # 64 x 128 tiles: 4 -> 8 slices
    assert sz(512, 4096, 4096) == 0                       # 256 tiles fill the GPU
    assert sz(64, 448, 128) == 0                          # 7 K-blocks: too short to split
    assert sz(1, 4096, 4096) == sz(1, 4096, 4096)         # pure function of the shape
    # channel-row GEMM (Int8-Block0, fp16 weights): 128 x 64 tiles, slices of
    # >= 8 K-blocks; W4A8: 128 x 256 tiles, slices of >= 4 stages of 128
    assert Q.qgemm_workspace_size(64, 4096, 512, "int8b0") == 8 * 64 * 512 * 4    # 8 tiles
    assert Q.qgemm_workspace_size(32, 9728, 2560, "f16") == 6 * 32 * 2560 * 4     # 40 tiles
    assert Q.qgemm_workspace_size(512, 2560, 4096, "f16") == 0                    # 256 tiles
    assert Q.qgemm_workspace_size(64, 448, 512, "int8b0") == 0                   # 7 K-blocks
    # Int4 GEMV (M <= 8): fewer than 128 32-channel tiles split K into three or
    # more slices of >= 48 blocks; the size covers the larger of the GEMV and
    # GEMM plans
    assert Q.qgemm_workspace_size(8, 9728, 2560, "int4b64") == 3 * 8 * 2560 * 4   # GEMM plan 3 = GEMV 3
    assert Q.qgemm_workspace_size(2, 16384, 70, "int4b64") == -(-8 * 2 * 70 * 4 // 256) * 256   # GEMM plan 8 > GEMV 5
    assert Q.qgemm_workspace_size(1, 16384, 70, "int4b64") == -(-8 * 1 * 70 * 4 // 256) * 256
    assert Q.qgemm_workspace_size(1, 4096, 11008, "int4b64") == 2 * 11008 * 4     # GEMM plan: 86 tiles of 64 x 128
    w4 = Q.qgemm_workspace_size(32, 9728, 2560, "w4a8")
    assert w4 - Q.qgemm_workspace_size(32, 9728, 32, "w4a8") >= 8 * 32 * 2560 * 4 - 8 * 32 * 32 * 4
    # fp32: 16x64 / 64x64 tiles; below 256 tiles each workgroup has two
    # K-groups, and a cross-workgroup split only when that is still short and
    # every group of every slice keeps four or more 64-wide chunks
    assert Q.qgemm_workspace_size(16, 256, 256, "f32") == 0          # 4 tiles x 2 groups, 2 chunks each
    assert Q.qgemm_workspace_size(8, 2560, 1024, "f32") == 5 * 8 * 1024 * 4   # 40 chunks / (2 x 4)
    assert Q.qgemm_workspace_size(512, 4096, 4096, "f32") == 0       # 512 tiles
    w = Q.qgemm_workspace_size(8, 128, 16, "w4a8")
    assert w == Q.qgemm_workspace_size(8, 128, 16000, "w4a8")   # W4A8 scratch has no N part
    # W4A8 GEMM: shapes with fewer than 128 tiles split K; the slice count
    # minimises 4 us per 1000 K of a slice plus, when
    # split, 4 us + 0.2 us per MB of (slices + 1) x M x N x 4 bytes (the plan
    # is a pure function of the shape); int32 partials follow the quantiser's
    # scratch, so the size less that of N = 1 (up to 8 slices x M x 4 bytes of
    # its own partials) is about slices x M x N x 4
    def w4a8_part(M, K, N):
        return Q.qgemm_workspace_size(M, K, N, "w4a8") - Q.qgemm_workspace_size(M, K, 1, "w4a8")
    assert w4a8_part(512, 2560, 4096) <= 0                     # 64 tiles, yet unsplit (8 MB per slice)
    assert w4a8_part(128, 2560, 9728) <= 0                     # 38 tiles, unsplit
    assert w4a8_part(512, 4096, 2560) >= 3 * 512 * 2560 * 4 - 8 * 512 * 4    # three slices of 80 tiles
    assert w4a8_part(128, 2560, 1024) >= 5 * 128 * 1024 * 4 - 8 * 128 * 4    # five (the K cap)
    # the estimate written out: slices for a shape with few tiles
    def est(M, K, N, sp):
        return 0.004 * K / sp + (0 if sp == 1 else 4 + 0.2 * (sp + 1) * M * N * 4 / 1e6)
    # (tiles of 128 x 128 while those fit 256 CUs, else 128 x 256)
    for M, K, N in [(512, 2560, 4096), (512, 9728, 2560), (128, 9728, 2560), (300, 4096, 1000),
                    (1024, 4096, 4096), (2048, 2048, 2048)]:
        t128 = -(-M // 128) * -(-N // 128)
        tiles = t128 if t128 <= 256 else -(-M // 128) * -(-N // 256)
        if tiles >= 128:
            assert w4a8_part(M, K, N) <= 0, (M, K, N)
            continue
        cap = min(256 // tiles, 8, -(-K // 128) // 4)
        sp = min(range(1, cap + 1), key=lambda s: (est(M, K, N, s), s))
        part = w4a8_part(M, K, N)
        if sp == 1:
            assert part <= 0, (M, K, N)
        else:
            assert sp * M * N * 4 - 8 * M * 4 - 4096 <= part <= sp * M * N * 4 + 4096, (M, K, N, sp)


def test_run_ex_validation(lib):
    """Epilogue checks happen before any device work: unknown activation or
    output type -> ERR_FORMAT, misaligned bias or residual -> ERR_ALIGN, a
    short caller workspace -> ERR_SIZE."""
    v = ctypes.c_void_p
    def ex(act=0, out=0, bias=None, res=None, ws=None, nb=0):
        e = Q.Epilogue(bias, res, act, out)
        return lib.qgemm_run_ex(64, 4096, 512, 1, v(256), v(256), v(256), v(256), ctypes.byref(e),
                                ws, nb, None)
    assert ex(act=4) == 3 and ex(act=-1) == 3 and ex(out=2) == 3
    assert ex(bias=v(260)) == 4 and ex(res=v(264)) == 4
    need = Q.qgemm_workspace_size(64, 4096, 512, "int4b64")
    assert need > 0 and ex(ws=v(512), nb=need - 1) == 8


def test_f16_layout_and_checks(lib):
    """fp16 weights: channel rows [roundup(N,4)][roundup(K,64)] fp16, zero
    padded; pack/unpack round trip; not quantisable; scales must be NULL."""
    K, N = 137, 70
    B = (np.arange(K * N, dtype=np.float64).reshape(K, N) / 997.0).astype(np.float16)
    wb, sb = Q.qgemm_packed_size(K, N, "f16")
    assert sb == 0 and wb == ((72 * 192 * 2 + 255) // 256) * 256
    wp, sp = Q.qgemm_pack_weights(K, N, "f16", B, None)
    rows = wp[: 72 * 192 * 2].view(np.float16).reshape(72, 192)
    assert np.array_equal(rows[:N, :K], B.T) and not rows[N:].any() and not rows[:, K:].any()
    q, _ = Q.qgemm_unpack_weights(K, N, "f16", wp, sp)
    assert np.array_equal(q.view(np.float16).reshape(K, N), B)
    with pytest.raises(Q.QGemmError) as e:
        Q.qgemm_quantize_weights(np.zeros((N, K), np.float32), "f16")
    assert e.value.status == 3
    v = ctypes.c_void_p
    assert lib.qgemm_run(2, K, N, 4, v(256), v(256), v(256), v(256), None) == 3   # scales given


def test_int4b0_packs_as_block64_with_repeated_pairs():
    """Int4-Block0 packs exactly like Int4-Block64 whose every 64-block holds
    the channel's one pair."""
    N, K = 40, 256
    rng = np.random.default_rng(9)
    q, p = Q.qgemm_quantize_weights(synth.normal_weights(rng, N, K), "int4b0")
    assert p.shape == (N * 2,) or p.size == N * 2
    wp0, sp0 = Q.qgemm_pack_weights(K, N, "int4b0", q, p)
    p64 = np.repeat(p.reshape(N, 1, 2), K // 64, axis=1)
    wp1, sp1 = Q.qgemm_pack_weights(K, N, "int4b64", q, p64)
    assert np.array_equal(wp0, wp1) and np.array_equal(sp0, sp1)


def test_sizes():
    assert Q.qgemm_packed_size(4096, 11008, "int4b64") == (22544384, 5636096)
    assert Q.qgemm_packed_size(4096, 100, "int4b64") == (4 * 64 * 1024, 4 * 64 * 256)
    assert Q.qgemm_packed_size(4096, 4096, "int8b0") == (16777216, 32768)
    assert Q.qgemm_packed_size(3072, 8192, "w4a8") == (12582912, 65536)
    assert Q.qgemm_packed_size(256, 256, "f32") == (262144, 0)
    # ragged shapes pad channels and K, then round to 256 bytes
    w, s = Q.qgemm_packed_size(137, 70, "int8b0")
    assert w == 72 * 192 and s == 768
    assert Q.qgemm_canonical_size(4096, 11008, "int4b64") == (11008 * 2048, 11008 * 64 * 2)
    with pytest.raises(Q.QGemmError):
        Q.qgemm_packed_size(100, 8, "int4b64")


@pytest.mark.parametrize("fmt", FMTS + ["int4b16", "int4b32", "int4b48", "int4b128", "int4b192",
                                        "int8b16", "int8b32", "int8b64", "int8b80", "int8b192"])
@pytest.mark.parametrize("shape", [(1, 64), (5, 128), (70, 192), (33, 1024)])
def test_quantizer_matches_oracle_bit_exact(fmt, shape):
    if fmt[:5] in ("int4b", "int8b") and fmt[5:] != "0" and shape[1] % int(fmt[5:]):
        pytest.skip("the block does not divide K")
    N, K = shape
    rng = np.random.default_rng(N * 1000 + K)
    W = synth.normal_weights(rng, N, K)
    W[0, :16] = 0.25                                  # partly constant block
    if N > 2:
        W[2, :] = -0.125                              # a fully constant channel
    q_lib, p_lib = Q.qgemm_quantize_weights(W, fmt)
    q_orc, p_orc = O.quantize(W, fmt)
    assert np.array_equal(q_lib, q_orc)
    assert np.array_equal(p_lib.view(np.uint32), p_orc.view(np.uint32))


def test_quantizer_rejects_nonfinite():
    W = np.zeros((4, 64), np.float32)
    W[1, 3] = np.nan
    with pytest.raises(Q.QGemmError) as e:
        Q.qgemm_quantize_weights(W, "int4b64")
    assert e.value.status == 9
    with pytest.raises(Q.QGemmError):
        Q.qgemm_quantize_weights(np.zeros((4, 64), np.float32), "f32")


@pytest.mark.parametrize("fmt", FMTS + ["f32", "int4b16", "int4b32", "int4b48", "int4b128",
                                        "int4b320", "int8b16", "int8b32", "int8b64", "int8b80",
                                        "int8b96", "int8b320"])
@pytest.mark.parametrize("shape", [(1, 64), (3, 128), (70, 192), (37, 4160)])
def test_pack_unpack_round_trip(fmt, shape):
    N, K = shape
    if fmt[:5] in ("int4b", "int8b") and fmt[5:] != "0" and K % int(fmt[5:]):
        pytest.skip("the block does not divide K")
    rng = np.random.default_rng(K + N)
    if fmt == "f32":
        wc = rng.standard_normal((K, N)).astype(np.float32)
        pc = None
    else:
        qb, pf = Q.qgemm_canonical_size(K, N, fmt)
        wc = rng.integers(0, 256, size=qb).astype(np.uint8)
        pc = rng.standard_normal(pf).astype(np.float32)
    wp, sp = Q.qgemm_pack_weights(K, N, fmt, wc, pc)
    q2, p2 = Q.qgemm_unpack_weights(K, N, fmt, wp, sp)
    assert np.array_equal(q2, wc.reshape(-1).view(np.uint8))
    if pc is not None:
        assert np.array_equal(p2, pc)
    # padding is zero: the packed buffer holds exactly the canonical content
    if fmt.startswith("int8b"):
        assert int(np.count_nonzero(wp)) == int(np.count_nonzero(wc))
    elif fmt != "f32":
        nz = lambda b: int(np.count_nonzero(b & 15) + np.count_nonzero(b >> 4))
        assert nz(wp) == nz(wc)


def test_int4_packed_layout_golden():
    """Record (t, b) of the Int4-Block64 layout is 1 KiB: piece 32 h + c holds
    canonical bytes [32 b + 16 h, +16) of channel 32 t + c; pair record (t, b)
    holds the 32 channels' {offset, scale} of block b."""
    N, K = 40, 128
    nblk = K // 64
    wc = np.arange(N * K // 2, dtype=np.int64).astype(np.uint8).reshape(N, K // 2)
    pc = np.arange(N * nblk * 2, dtype=np.float32).reshape(N, nblk, 2)
    wp, sp = Q.qgemm_pack_weights(K, N, "int4b64", wc, pc)
    assert wp.size == 2 * nblk * 1024 and sp.size == 2 * nblk * 256
    pieces = wp.reshape(-1, 64, 16)
    recs = sp.view(np.float32).reshape(-1, 32, 2)
    for n in range(N):
        t, c = divmod(n, 32)
        for b in range(nblk):
            for half in range(2):
                assert np.array_equal(pieces[t * nblk + b, 32 * half + c],
                                      wc[n, 32 * b + 16 * half: 32 * b + 16 * half + 16])
            assert list(recs[t * nblk + b, c]) == list(pc[n, b])
    # channels 40..63 of the second tile are zero padding
    assert not np.any(pieces[nblk:, :, :][:, [c for c in range(64) if (c % 32) >= 8]])


def test_w4a8_packed_word_order_golden():
    """A W4A8 record holds 32 channels x 64 codes; piece 32 h + c of channel c
    carries, for s = 0, 1, the codes of k = 32 s + 16 h + [0, 16) in bytes
    [8 s, 8 s + 8), and byte i of word w (k0 = 32 s + 16 h + 8 w) holds code
    k0 + i in the low and k0 + 4 + i in the high nibble, so nibble masks give
    codes in natural k order."""
    K, N = 64, 40
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 16, size=(N, K))
    wc = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    pc = np.zeros((N, 1, 2), np.float32)
    wp, _ = Q.qgemm_pack_weights(K, N, "w4a8", wc, pc)
    assert wp.nbytes >= 2 * 1024
    for n in range(N):
        g, c = divmod(n, 32)
        rec = wp[g * 1024:(g + 1) * 1024]
        for h in range(2):
            piece = rec[(32 * h + c) * 16:(32 * h + c + 1) * 16]
            for s in range(2):
                for w in range(2):
                    k0 = 32 * s + 16 * h + 8 * w
                    for i in range(4):
                        byte = int(piece[8 * s + 4 * w + i])
                        assert byte & 15 == codes[n, k0 + i]
                        assert byte >> 4 == codes[n, k0 + 4 + i]
    # channels 40 .. 63 of the second record are padding
    assert not np.any(wp[1024:2048].reshape(2, 32, 16)[:, 8:, :])


def test_device_quantizer_validation_before_device(lib):
    """Every rejection of the device quantisers happens before the GPU is touched."""
    OK, NULL, SHAPE, FMT, ALIGN, DEV = 0, 1, 2, 3, 4, 6
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    for fn in (lib.qgemm_quantize_weights_device, lib.qgemm_quantize_pack_device):
        q = lambda K, N, f, W=256, a=256, b=256: fn(K, N, f, v(W), v(a), v(b), None)
        assert q(64, 4, 0) == FMT                     # float weights are not quantised
        assert q(64, 4, 4) == FMT
        assert q(64, 4, 9) == FMT
        assert q(63, 4, 1) == SHAPE                   # Int4-Block64: K % 64 == 0
        assert q(96, 4, 5) == SHAPE                   # Int4-Block0 packs as Block64
        assert q(65, 4, 3) == SHAPE                   # W4A8: even K
        assert q(0, 4, 2) == SHAPE
        assert q(192, 4, Q.QGEMM_INT4_BLOCK(48)) == FMT    # multiples of 16 other than
        assert q(320, 4, Q.QGEMM_INT8_BLOCK(80)) == FMT    # 16, 32, 64 k: host quantiser
        assert q(384, 4, Q.QGEMM_INT4_BLOCK(96)) == FMT
        assert q(64, 0, 1, None, None, None) == OK    # nothing to do
        assert q(64, 4, 1, W=None) == NULL
        assert q(64, 4, 2, a=None) == NULL
        assert q(64, 4, 3, b=None) == NULL
        assert q(64, 4, 1, W=260) == ALIGN
        assert q(64, 4, 2, a=264) == ALIGN
        assert q(64, 4, 3, b=200) == ALIGN
        import torch
        if not torch.cuda.is_available():
            assert q(64, 4, 1) == DEV


def test_int4_block_sizes_pack_as_block64_with_repeated_pairs():
    """Int4 with block b (a multiple of 64) packs exactly as Int4-Block64 whose
    64-blocks repeat the pair of the b-block holding them, so the Int4 kernels
    read it unchanged; Block64 and Block-K ids behave as INT4_B64 and INT4_B0."""
    N, K = 45, 768
    rng = np.random.default_rng(12)
    W = synth.normal_weights(rng, N, K)
    for b in (128, 256, 384, 768):
        q, p = Q.qgemm_quantize_weights(W, f"int4b{b}")
        assert p.shape == (N, K // b, 2)
        rep = np.repeat(p, b // 64, axis=1)            # one pair per 64-block
        wp0, sp0 = Q.qgemm_pack_weights(K, N, "int4b64", q, rep)
        wp, sp = Q.qgemm_pack_weights(K, N, f"int4b{b}", q, p)
        assert np.array_equal(wp, wp0) and np.array_equal(sp, sp0)
    q64, p64 = Q.qgemm_quantize_weights(W, Q.QGEMM_INT4_BLOCK(64))
    qa, pa = Q.qgemm_quantize_weights(W, "int4b64")
    assert np.array_equal(q64, qa) and np.array_equal(p64, pa)
    qk, pk = Q.qgemm_quantize_weights(W, Q.QGEMM_INT4_BLOCK(K))
    qb0, pb0 = Q.qgemm_quantize_weights(W, "int4b0")
    assert np.array_equal(qk, qb0) and np.array_equal(pk, pb0)


def test_int4_block_size_validation(lib):
    SHAPE, FMT = 2, 3
    size = lambda K, f: lib.qgemm_packed_size(K, 8, f, ctypes.byref(ctypes.c_size_t()),
                                              ctypes.byref(ctypes.c_size_t()))
    assert size(256, Q.QGEMM_INT4_BLOCK(128)) == 0
    assert size(384, Q.QGEMM_INT4_BLOCK(256)) == SHAPE    # the block must divide K
    assert size(256, Q.QGEMM_INT4_BLOCK(32)) == 0         # a pair per half of each 64-block
    assert size(96, Q.QGEMM_INT4_BLOCK(32)) == SHAPE      # the kernels' step: K % 64 == 0
    assert size(256, Q.QGEMM_INT4_BLOCK(16)) == 0         # a pair per quarter of each 64-block
    assert size(192, Q.QGEMM_INT4_BLOCK(48)) == 0         # any multiple of 16 that divides K
    assert size(384, Q.QGEMM_INT4_BLOCK(96)) == 0
    assert size(256, Q.QGEMM_INT4_BLOCK(96)) == SHAPE
    assert size(256, Q.QGEMM_INT4_BLOCK(8)) == FMT        # multiples of 16 only
    assert size(256, Q.QGEMM_INT4_BLOCK(24)) == FMT
    assert size(256, Q.QGEMM_INT4_BLOCK(0)) == FMT
    assert size(256, Q.QGEMM_INT4_BLOCK(-64)) == FMT
    assert Q.qgemm_workspace_size(16, 4096, 256, "int4b128") == \
        Q.qgemm_workspace_size(16, 4096, 256, "int4b64")  # same kernels, same split-K plan


def test_int8_block_sizes_layout_golden(lib):
    """Int8 with block b: codes as channel rows [Np][K] (the Int8-Block0 rows);
    pairs channel-major, one entry per 64-block repeating the pair of the
    b-block that holds it (b = 32, 96: one entry per 32-element half; other
    multiples of 16: one per 16-element quarter)."""
    N, K = 6, 384
    wc = (np.arange(N * K, dtype=np.int64) * 7 % 251).astype(np.uint8).reshape(N, K)
    for b in (16, 32, 48, 64, 96, 128, 384):
        nb = K // b
        pc = np.arange(N * nb * 2, dtype=np.float32).reshape(N, nb, 2) + 1
        wp, sp = Q.qgemm_pack_weights(K, N, f"int8b{b}", wc, pc)
        Np = 8
        assert wp.size == -(-Np * K // 256) * 256
        rows = wp[:Np * K].reshape(Np, K)
        assert np.array_equal(rows[:N], wc) and not np.any(rows[N:])
        H = 1 if b % 64 == 0 else 2 if b % 32 == 0 else 4
        ent = sp.view(np.float32)[:Np * (K // 64) * H * 2].reshape(Np, K // 64 * H, 2)
        for n in range(N):
            for e in range(K // 64 * H):
                k = e * (64 // H)                      # first K-element the entry covers
                assert list(ent[n, e]) == list(pc[n, k // b])
        assert not np.any(ent[N:])                     # padding channels
        assert not np.any(sp.view(np.float32)[Np * (K // 64) * H * 2:])
    SHAPE, FMT = 2, 3
    size = lambda K, f: lib.qgemm_packed_size(K, 8, f, ctypes.byref(ctypes.c_size_t()),
                                              ctypes.byref(ctypes.c_size_t()))
    assert size(256, Q.QGEMM_INT8_BLOCK(128)) == 0
    assert size(384, Q.QGEMM_INT8_BLOCK(256)) == SHAPE    # the block must divide K
    assert size(96, Q.QGEMM_INT8_BLOCK(32)) == SHAPE      # K % 64 == 0
    assert size(256, Q.QGEMM_INT8_BLOCK(16)) == 0         # multiples of 16
    assert size(320, Q.QGEMM_INT8_BLOCK(80)) == 0
    assert size(256, Q.QGEMM_INT8_BLOCK(96)) == SHAPE
    assert size(256, Q.QGEMM_INT8_BLOCK(40)) == FMT
    assert size(256, Q.QGEMM_INT8_BLOCK(-64)) == FMT
    assert Q.qgemm_workspace_size(64, 4096, 512, "int8b64") == \
        Q.qgemm_workspace_size(64, 4096, 512, "int8b0")   # the channel-row kernel's split-K plan


def test_int4_block32_pair_records_golden():
    """Int4 with 32-element blocks: codes as Int4-Block64; pair record (t, b)
    is 512 bytes, entry 32 h + c holding channel 32 t + c's pair for K-elements
    64 b + 32 h .. + 31."""
    N, K = 40, 128
    nblk = K // 32
    wc = np.arange(N * K // 2, dtype=np.int64).astype(np.uint8).reshape(N, K // 2)
    pc = np.arange(N * nblk * 2, dtype=np.float32).reshape(N, nblk, 2)
    wp, sp = Q.qgemm_pack_weights(K, N, "int4b32", wc, pc)
    wp64, _ = Q.qgemm_pack_weights(K, N, "int4b64", wc, np.zeros((N, K // 64, 2), np.float32))
    assert np.array_equal(wp, wp64) and sp.size == 2 * (K // 64) * 512
    recs = sp.view(np.float32).reshape(-1, 2, 32, 2)
    for n in range(N):
        t, c = divmod(n, 32)
        for b in range(K // 64):
            for h in range(2):
                assert list(recs[t * (K // 64) + b, h, c]) == list(pc[n, 2 * b + h])
    assert not np.any(recs[K // 64:, :, 8:, :])        # channels 40..63: zero padding


@pytest.mark.parametrize("b", [16, 48])
def test_int4_quarter_pair_records_golden(b):
    """Int4 with blocks that are multiples of 16 but not of 32: codes as
    Int4-Block64; pair record (t, b64) is 1024 bytes, entry 4 c + j holding
    channel 32 t + c's pair for the quarter K-elements 64 b64 + 16 j .. + 15
    (the two quarters of one 32-element half are adjacent)."""
    N, K = 40, 192
    nblk = K // b
    wc = np.arange(N * K // 2, dtype=np.int64).astype(np.uint8).reshape(N, K // 2)
    pc = np.arange(N * nblk * 2, dtype=np.float32).reshape(N, nblk, 2)
    wp, sp = Q.qgemm_pack_weights(K, N, f"int4b{b}", wc, pc)
    wp64, _ = Q.qgemm_pack_weights(K, N, "int4b64", wc, np.zeros((N, K // 64, 2), np.float32))
    assert np.array_equal(wp, wp64) and sp.size == 2 * (K // 64) * 1024
    recs = sp.view(np.float32).reshape(-1, 32, 4, 2)
    for n in range(N):
        t, c = divmod(n, 32)
        for b64 in range(K // 64):
            for j in range(4):
                k = 64 * b64 + 16 * j
                assert list(recs[t * (K // 64) + b64, c, j]) == list(pc[n, k // b])
    assert not np.any(recs[K // 64:, 8:, :, :])        # channels 40..63: zero padding
    q2, p2 = Q.qgemm_unpack_weights(K, N, f"int4b{b}", wp, sp)
    assert np.array_equal(q2, wc.reshape(-1)) and np.array_equal(p2, pc.reshape(-1))


def test_binding_checks_dtypes_and_sizes_before_the_library():
    """The Python binding rejects device buffers of the wrong element type or
    too few bytes before calling into C, where the kernels would read or write
    past them (CPU tensors stand in: the dtype and size checks come before the
    device check)."""
    import torch
    M, K, N = 4, 128, 64
    wb, sb = Q.qgemm_packed_size(K, N, "int4b64")
    A16 = torch.zeros((M, K), dtype=torch.float16)
    C32 = torch.zeros((M, N), dtype=torch.float32)
    Bq = torch.zeros(wb, dtype=torch.uint8)
    Sc = torch.zeros(sb, dtype=torch.uint8)
    bad = [
        dict(A=torch.zeros((M, K), dtype=torch.float32)),     # fp32 A for an fp16 format
        dict(A=torch.zeros((M, K - 1), dtype=torch.float16)),  # too few A elements
        dict(C=torch.zeros((M, N - 1), dtype=torch.float32)),  # C smaller than M x N
        dict(C=torch.zeros((M, N), dtype=torch.float16)),      # fp16 C with fp32 output
        dict(Bq=torch.zeros(wb - 1, dtype=torch.uint8)),       # packed weights too short
        dict(scales=torch.zeros(sb - 16, dtype=torch.uint8)),  # packed pairs too short
    ]
    for override in bad:
        args = dict(A=A16, Bq=Bq, scales=Sc, C=C32)
        args.update(override)
        with pytest.raises(ValueError):
            Q.qgemm_run(M, K, N, "int4b64", args["A"], args["Bq"], args["scales"], args["C"])
    # the fp32 format takes fp32 A; an fp16 A is rejected
    Bf = torch.zeros(K * N, dtype=torch.float32)
    with pytest.raises(ValueError, match="dtype"):
        Q.qgemm_run(M, K, N, "f32", A16, Bf, None, C32)
    # the fp32 format's B is the [K][N] matrix itself: exactly K*N floats pass
    # (137 x 70 x 4 bytes is not a multiple of the packed size's 256-byte
    # rounding), one float fewer does not
    Kf, Nf = 137, 70
    Af = torch.zeros((M, Kf), dtype=torch.float32)
    Cf = torch.zeros((M, Nf), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        Q.qgemm_run(M, Kf, Nf, "f32", Af, torch.zeros(Kf * Nf, dtype=torch.float32), None, Cf)
    with pytest.raises(ValueError, match="Bq"):
        Q.qgemm_run(M, Kf, Nf, "f32", Af, torch.zeros(Kf * Nf - 1, dtype=torch.float32), None, Cf)
    # epilogue operands: residual in C's type, bias fp32 [N]
    with pytest.raises(ValueError, match="residual"):
        Q.qgemm_run_ex(M, K, N, "int4b64", A16, Bq, Sc, C32,
                       residual=torch.zeros((M, N), dtype=torch.float16))
    with pytest.raises(ValueError, match="bias"):
        Q.qgemm_run_ex(M, K, N, "int4b64", A16, Bq, Sc, C32, bias=torch.zeros(N - 4))
    with pytest.raises(ValueError, match="C"):
        Q.qgemm_run_ex(M, K, N, "int4b64", A16, Bq, Sc, C32, out_type="f16")
    # a workspace smaller than the size claimed for it
    with pytest.raises(ValueError, match="workspace"):
        Q.qgemm_run_ws(M, K, N, "int4b64", A16, Bq, Sc, C32, torch.zeros(16, dtype=torch.uint8), 4096)
    # well-typed CPU tensors get past these checks and stop at the device check
    with pytest.raises(ValueError, match="GPU"):
        Q.qgemm_run(M, K, N, "int4b64", A16, Bq, Sc, C32)


def test_packed_weight_checks_activation_shape():
    import torch
    K, N = 128, 32
    w = Q.PackedWeight.__new__(Q.PackedWeight)
    w.fmt, w.K, w.N = Q.QGEMM_INT4_B64, K, N
    with pytest.raises(ValueError, match="shape"):
        w(torch.zeros((2, K + 64), dtype=torch.float16))


def test_noalloc_rejects_oversized_scratch_before_device(lib):
    """qgemm_run_noalloc refuses a shape whose scratch exceeds its fixed
    per-GPU array with QGEMM_ERR_SIZE, before any device call (no GPU here);
    a shape that fits gets past the size check and stops at the device check."""
    SIZE, DEV = 8, 6
    v = ctypes.c_void_p
    big = (65536, 1024, 64)                      # W4A8 codes alone: 64 MiB
    assert Q.qgemm_workspace_size(*big, "w4a8") > Q.NOALLOC_SCRATCH_BYTES
    st = lib.qgemm_run_noalloc(*big, Q.QGEMM_W4A8, v(256), v(256), v(256), v(256), None, None)
    assert st == SIZE
    small = (64, 1024, 64)
    assert 0 < Q.qgemm_workspace_size(*small, "w4a8") <= Q.NOALLOC_SCRATCH_BYTES
    st = lib.qgemm_run_noalloc(*small, Q.QGEMM_W4A8, v(256), v(256), v(256), v(256), None, None)
    assert st == DEV

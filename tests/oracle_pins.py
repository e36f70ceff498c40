"""Pins that tie the CPU oracle to something other than itself.

Each ``pin_*`` takes a loaded oracle library (the real one, or a deliberately
broken copy built by the mutation tests) and raises AssertionError when the
oracle disagrees with:
  - a library routine on a special case (numpy's fp16 decoding, numpy float64
    and int64 matmul),
  - exact rational brute force on tiny inputs,
  - closed forms (identity weights, constant blocks, all-ones activations with
    the page's float filler, unit rows, hand-worked quantiser ramps),
  - invariants (the quantise/dequantise round trip stays within scale/2),
  - hand-worked fixtures under tests/golden/ (nibble order, W4A8 rows).
The set is chosen so that a dropped term, a wrong sign or index, a transposed
operand, a swapped nibble or pair order or a wrong rounding rule fails at
least one pin (checked by test_oracle_mutants.py).
"""
from __future__ import annotations

import json
import os

import numpy as np

from oracle import brute
from oracle import oracle as O
from weight_quantized_gemm_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rel_close(got, want, scale, tol=1e-12):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    assert np.all(err <= tol * np.maximum(scale, 1e-300)), \
        f"max err {err.max():.3e} vs scale {np.max(scale):.3e}"


def _pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Codes [N][K] (0..15) -> canonical bytes [N][K/2], low nibble first.

    This is the storage reading itself (byte = even | odd << 4), written out
    here only to build test inputs with known codes.
    """
    c = codes.astype(np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


# --------------------------------------------------------------------------
# fp16 decoding
# --------------------------------------------------------------------------
def pin_half_decode_all_patterns(lib):
    """Every binary16 pattern decodes like numpy's own fp16 -> fp64 cast."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = bits.view(np.float16).astype(np.float64)
    got = np.array([lib.orc_half_to_double(int(b)) for b in bits])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


# --------------------------------------------------------------------------
# fp32 product
# --------------------------------------------------------------------------
def pin_f32_brute_force(lib):
    rng = np.random.default_rng(7)
    for (M, K, N) in [(1, 1, 1), (2, 3, 4), (3, 7, 2), (4, 5, 6)]:
        A = rng.standard_normal((M, K)).astype(np.float32)
        B = rng.standard_normal((K, N)).astype(np.float32)
        C = O.gemm_f32(A, B, lib)
        want = brute.to_array(brute.gemm_f32(A, B))
        scale = np.abs(A).astype(np.float64) @ np.abs(B).astype(np.float64)
        _rel_close(C, want, scale)


def pin_f32_numpy_matmul(lib):
    rng = np.random.default_rng(8)
    A = rng.standard_normal((9, 37)).astype(np.float32)
    B = rng.standard_normal((37, 21)).astype(np.float32)
    C = O.gemm_f32(A, B, lib)
    want = A.astype(np.float64) @ B.astype(np.float64)
    scale = np.abs(A).astype(np.float64) @ np.abs(B).astype(np.float64)
    _rel_close(C, want, scale)


def pin_f32_unit_rows(lib):
    """A = unit rows e_i picks row i of B exactly (catches a transposed B)."""
    K, N = 5, 7
    B = synth.float_pattern_weights(K, N)
    A = np.eye(K, dtype=np.float32)[[3, 0, 4]]
    C = O.gemm_f32(A, B, lib)
    assert np.array_equal(C, B[[3, 0, 4]].astype(np.float64))


def pin_f32_ones_closed_form(lib):
    """A = ones with the page's filler: C[m][n] = sum_k ((k*N+n)%127 - 63)/1000.

    The integer sum is exact; the stored B is the float32 nearest to each
    rational, so the two differ by at most K float32 half-ulps of |b| <= 0.063.
    """
    for (K, N) in [(256, 256), (137, 70)]:
        B = synth.float_pattern_weights(K, N)
        A = np.ones((2, K), dtype=np.float32)
        C = O.gemm_f32(A, B, lib)
        k = np.arange(K)[:, None]
        n = np.arange(N)[None, :]
        exact = (((k * N + n) % 127) - 63).sum(axis=0) / 1000.0
        bound = K * 0.063 * 2.0 ** -24 * 1.01
        assert np.all(np.abs(C - exact[None, :]) <= bound)


# --------------------------------------------------------------------------
# quantiser
# --------------------------------------------------------------------------
def pin_quantize_roundtrip(lib):
    """|w - (offset + scale*q)| <= scale/2 for every weight (rounding to nearest)."""
    rng = np.random.default_rng(9)
    W = (rng.standard_normal((13, 256)) * 0.02).astype(np.float32)
    W[0, :64] = 0.5                      # a constant Int4 block
    W[1, 5] = 3.0                        # an outlier
    for fmt, bits, block in [("int4b64", 4, 64), ("int8b0", 8, 256), ("w4a8", 4, 256),
                             ("int8b64", 8, 64), ("int8b32", 8, 32), ("int4b32", 4, 32)]:
        q, pairs = O.quantize(W, fmt, lib)
        N, K = W.shape
        nb = K // block
        codes = q if bits == 8 else np.stack([q & 15, q >> 4], axis=-1).reshape(N, K)
        off = np.repeat(pairs[:, :, 0].astype(np.float64), block, axis=1)
        scl = np.repeat(pairs[:, :, 1].astype(np.float64), block, axis=1)
        rec = off + scl * codes
        err = np.abs(W.astype(np.float64) - rec)
        assert np.all(err <= scl / 2 * (1 + 1e-9) + 0.0)
        assert codes.min() >= 0 and codes.max() <= (1 << bits) - 1
        wb = W.reshape(N, nb, block).astype(np.float64)
        # offset is the block minimum exactly, scale the rounded range / qmax
        assert np.array_equal(pairs[:, :, 0], wb.min(axis=2).astype(np.float32))
        want_scale = ((wb.max(axis=2) - wb.min(axis=2)) / ((1 << bits) - 1)).astype(np.float32)
        assert np.array_equal(pairs[:, :, 1], want_scale)
        # the minimum maps to code 0 and the maximum to the top code
        cb = codes.reshape(N, nb, block)
        has_range = want_scale > 0
        imin = wb.argmin(axis=2)
        imax = wb.argmax(axis=2)
        nn, bb = np.nonzero(has_range)
        assert np.all(cb[nn, bb, imin[nn, bb]] == 0)
        assert np.all(cb[nn, bb, imax[nn, bb]] == (1 << bits) - 1)
    q, pairs = O.quantize(W, "int4b64", lib)
    assert pairs[0, 0, 1] == 0.0 and pairs[0, 0, 0] == np.float32(0.5)
    assert np.all(q[0, :32] == 0)


def pin_quantize_ramps(lib):
    """Hand-worked ramps whose codes are known exactly.

    Int4: w_i = -1 + (i mod 16)/8 -> offset -1, scale 1.875/15 = 0.125, q = i mod 16.
    Int8: w_k = -2 + k/64 over K = 256 -> offset -2, scale 3.984375/255 = 1/64, q = k.
    """
    i = np.arange(64)
    W4 = (-1.0 + (i % 16) / 8.0).astype(np.float32)[None, :]
    q, pairs = O.quantize(W4, "int4b64", lib)
    assert pairs[0, 0, 0] == -1.0 and pairs[0, 0, 1] == 0.125
    assert np.array_equal(q[0], _pack_nibbles((i % 16)[None, :])[0])
    k = np.arange(256)
    W8 = (-2.0 + k / 64.0).astype(np.float32)[None, :]
    q, pairs = O.quantize(W8, "int8b0", lib)
    assert pairs[0, 0, 0] == -2.0 and pairs[0, 0, 1] == 1.0 / 64.0
    assert np.array_equal(q[0], k.astype(np.uint8))


# --------------------------------------------------------------------------
# block-quantised products
# --------------------------------------------------------------------------
def pin_nibble_order_golden(lib):
    """With offset 0, scale 1 and A = e_0 / e_1, C reads back each code."""
    g = _golden("nibble_order.json")
    nbytes = len(g["cases"])
    K = 64
    q = np.zeros((nbytes, K // 2), dtype=np.uint8)
    for n, case in enumerate(g["cases"]):
        q[n, 0] = case["byte"]
    pairs = np.zeros((nbytes, 1, 2), dtype=np.float32)
    pairs[:, :, 1] = 1.0
    A = np.zeros((2, K), dtype=np.float16)
    A[0, 0] = 1.0
    A[1, 1] = 1.0
    C = O.gemm_blockq(A, q, pairs, "int4b64", lib)
    for n, case in enumerate(g["cases"]):
        assert C[0, n] == case["q_even"] and C[1, n] == case["q_odd"]


def _identity_codes(fmt, K):
    eye = np.eye(K, dtype=np.uint8)          # q[n][k] = delta_kn
    return eye if fmt == "int8b0" else _pack_nibbles(eye)


def pin_identity_weights(lib):
    """offset 0, scale 1, q = delta_kn gives C = A exactly (fp16 -> fp64)."""
    rng = np.random.default_rng(10)
    for fmt, K in [("int4b64", 64), ("int4b64", 128), ("int8b0", 48)]:
        A = rng.standard_normal((3, K)).astype(np.float16)
        q = _identity_codes(fmt, K)
        nblk = K // 64 if fmt == "int4b64" else 1
        pairs = np.zeros((K, nblk, 2), dtype=np.float32)
        pairs[:, :, 1] = 1.0
        C = O.gemm_blockq(A, q, pairs, fmt, lib)
        assert np.array_equal(C, A.astype(np.float64))


def pin_constant_blocks(lib):
    """scale = 0: C[m][n] = sum_b offset[n][b] * sum_{k in b} A[m][k].

    Offsets are powers of two and A small integers, so both sides are exact.
    """
    rng = np.random.default_rng(11)
    for fmt, K, N in [("int4b64", 192, 5), ("int8b0", 40, 3)]:
        M = 4
        A = rng.integers(-8, 9, size=(M, K)).astype(np.float16)
        nblk = K // 64 if fmt == "int4b64" else 1
        block = K // nblk
        pairs = np.zeros((N, nblk, 2), dtype=np.float32)
        pairs[:, :, 0] = 2.0 ** rng.integers(-4, 4, size=(N, nblk))
        pairs[:, :, 0] *= np.where(rng.random((N, nblk)) < 0.5, -1, 1)
        qshape = (N, K) if fmt == "int8b0" else (N, K // 2)
        q = rng.integers(0, 256, size=qshape).astype(np.uint8)   # ignored: scale 0
        C = O.gemm_blockq(A, q, pairs, fmt, lib)
        rows = A.astype(np.float64).reshape(M, nblk, block).sum(axis=2)    # [M][nblk]
        want = rows @ pairs[:, :, 0].astype(np.float64).T
        assert np.array_equal(C, want)


def pin_blockq_brute_force(lib):
    rng = np.random.default_rng(12)
    cases = [("int4b64", 4, 64, 64, 1, 3), ("int4b64", 4, 64, 128, 3, 5),
             ("int8b0", 8, None, 12, 2, 4), ("int8b0", 8, None, 64, 3, 2),
             ("int8b64", 8, 64, 192, 2, 3), ("int8b32", 8, 32, 96, 3, 2)]
    for fmt, bits, block, K, M, N in cases:
        block = K if block is None else block
        nblk = K // block
        A = rng.standard_normal((M, K)).astype(np.float16)
        qshape = (N, K) if bits == 8 else (N, K // 2)
        q = rng.integers(0, 256, size=qshape).astype(np.uint8)
        pairs = np.empty((N, nblk, 2), dtype=np.float32)
        pairs[:, :, 0] = rng.standard_normal((N, nblk)) * 0.05
        pairs[:, :, 1] = rng.random((N, nblk)) * 0.01
        C = O.gemm_blockq(A, q, pairs, fmt, lib)
        want = brute.to_array(brute.gemm_blockq(A, q, pairs, bits, block))
        codes = q if bits == 8 else np.stack([q & 15, q >> 4], -1).reshape(N, K)
        wabs = (np.abs(np.repeat(pairs[:, :, 0], block, 1)) +
                np.abs(np.repeat(pairs[:, :, 1], block, 1)) * codes).astype(np.float64)
        scale = np.abs(A.astype(np.float64)) @ wabs.T
        _rel_close(C, want, scale)


# --------------------------------------------------------------------------
# W4A8
# --------------------------------------------------------------------------
def pin_w4a8_actquant_golden(lib):
    g = _golden("w4a8_actquant_rows.json")
    A = np.array([r["a"] for r in g["rows"]], dtype=np.float16)
    assert np.array_equal(A.astype(np.float64), np.array([r["a"] for r in g["rows"]]))
    qa, sa, S = O.w4a8_actquant(A, lib)
    for i, r in enumerate(g["rows"]):
        assert int(sa.view(np.uint32)[i]) == int(r["sa_bits"], 16), i
        assert qa[i].tolist() == r["qa"], (i, qa[i].tolist())
        assert int(S[i]) == r["S"], i


def pin_w4a8_actquant_properties(lib):
    """On random rows: |qa| <= 127, the row maximum maps to +-127, S = sum(qa),
    and qa is the nearest integer to a/sa (|a/sa - qa| <= 1/2)."""
    rng = np.random.default_rng(13)
    A = rng.standard_normal((6, 333)).astype(np.float16)
    qa, sa, S = O.w4a8_actquant(A, lib)
    a32 = A.astype(np.float32)
    amax = np.abs(a32).max(axis=1)
    assert np.array_equal(sa, amax / np.float32(127))
    assert np.all(np.abs(qa.astype(np.int32)) <= 127)
    j = np.abs(a32).argmax(axis=1)
    assert np.all(np.abs(qa[np.arange(6), j]) == 127)
    assert np.array_equal(S, qa.astype(np.int32).sum(axis=1))
    t = a32.astype(np.float64) / sa[:, None].astype(np.float64)
    assert np.all(np.abs(t - qa) <= 0.5 + 1e-6)
    assert np.array_equal(np.sign(qa), np.sign(np.where(np.abs(t) <= 0.5, 0, t)))


def pin_w4a8_dot_numpy(lib):
    """D = qa . q^T equals numpy's int64 matmul with q the decoded int4 codes."""
    rng = np.random.default_rng(14)
    M, K, N = 5, 96, 7
    qa = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    q = rng.integers(0, 256, size=(N, K // 2)).astype(np.uint8)
    D = O.w4a8_dot(qa, q, lib)
    codes = np.stack([q & 15, q >> 4], -1).reshape(N, K).astype(np.int64)
    assert np.array_equal(D, qa.astype(np.int64) @ codes.T)


def pin_w4a8_regrouping(lib):
    """sa*(scale*D + offset*S) equals sum_k (sa*qa)(offset + scale*q) up to fp64 rounding."""
    rng = np.random.default_rng(15)
    M, K, N = 4, 64, 6
    A = rng.standard_normal((M, K)).astype(np.float16)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    q, pairs = O.quantize(W, "w4a8", lib)
    C, qa, sa, S, D = O.w4a8_gemm(A, q, pairs, lib)
    C2 = O.w4a8_dequant_product(qa, sa, q, pairs, lib)
    codes = np.stack([q & 15, q >> 4], -1).reshape(N, K)
    wabs = np.abs(pairs[:, 0, 0:1]).astype(np.float64) + np.abs(pairs[:, 0, 1:2]) * codes
    scale = (np.abs(qa.astype(np.float64)) * sa[:, None]) @ wabs.T
    _rel_close(C, C2, scale, tol=1e-13)


def pin_w4a8_identity(lib):
    """offset 0, scale 1, q = delta_kn (K = N) gives C = sa * qa exactly."""
    rng = np.random.default_rng(16)
    K = 32
    A = rng.standard_normal((3, K)).astype(np.float16)
    q = _pack_nibbles(np.eye(K, dtype=np.uint8))
    pairs = np.zeros((K, 1, 2), dtype=np.float32)
    pairs[:, 0, 1] = 1.0
    C, qa, sa, S, D = O.w4a8_gemm(A, q, pairs, lib)
    assert np.array_equal(D, qa.astype(np.int64))
    assert np.array_equal(C, sa[:, None].astype(np.float64) * qa)


def pin_w4a8_error_bound(lib):
    """|C_w4a8 - C_exact| <= (sa/2) * sum_k |w_kn| (activation rounding only)."""
    rng = np.random.default_rng(17)
    M, K, N = 3, 128, 4
    A = rng.standard_normal((M, K)).astype(np.float16)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    q, pairs = O.quantize(W, "w4a8", lib)
    C = O.w4a8_gemm(A, q, pairs, lib)[0]
    exact = brute.to_array(brute.gemm_blockq(A, q, pairs, 4, K))
    codes = np.stack([q & 15, q >> 4], -1).reshape(N, K)
    w = pairs[:, 0, 0:1].astype(np.float64) + pairs[:, 0, 1:2].astype(np.float64) * codes
    sa = np.abs(A.astype(np.float32)).max(axis=1) / np.float32(127)
    bound = (sa[:, None].astype(np.float64) / 2) * np.abs(w).sum(axis=1)[None, :]
    assert np.all(np.abs(C - exact) <= bound * (1 + 1e-6) + 1e-12)


# --------------------------------------------------------------------------
# Fused epilogue and fp16 output rounding
# --------------------------------------------------------------------------
def pin_epilogue_sum_exact(lib):
    """No activation: small integers (exact in every type) add exactly, with a
    float32 and with an fp16 residual."""
    rng = np.random.default_rng(11)
    P = rng.integers(-50, 50, (3, 5)).astype(np.float64)
    b = rng.integers(-9, 9, 5).astype(np.float32)
    r = rng.integers(-20, 20, (3, 5)).astype(np.float32)
    assert np.array_equal(O.epilogue(P, b, r, "none", lib=lib), P + b + r)
    assert np.array_equal(O.epilogue(P, b, r.astype(np.float16), "none", lib=lib), P + b + r)
    assert np.array_equal(O.epilogue(P, None, None, "none", lib=lib), P)


def pin_epilogue_textbook_values(lib):
    """SiLU(1) = logistic(1) = 0.7310585786300049; GELU(+-1) = +-Phi(+-1) with
    the tabulated normal distribution value Phi(1) = 0.8413447460685429;
    ReLU of (-2.5, -0, 0, 3.25)."""
    x = np.array([[1.0, -1.0]])
    _rel_close(O.epilogue(x, activation="silu", lib=lib), [[0.7310585786300049, -0.2689414213699951]], 1.0)
    _rel_close(O.epilogue(x, activation="gelu", lib=lib), [[0.8413447460685429, -0.15865525393145705]], 1.0)
    r = O.epilogue(np.array([[-2.5, -0.0, 0.0, 3.25]]), activation="relu", lib=lib)
    assert np.array_equal(r, [[0.0, 0.0, 0.0, 3.25]])


def pin_epilogue_odd_parts(lib):
    """x sigma(x) - (-x) sigma(-x) = x and x Phi(x) - (-x) Phi(-x) = x, since
    sigma(x) + sigma(-x) = Phi(x) + Phi(-x) = 1."""
    x = np.linspace(-6, 6, 49)
    X = np.stack([x, -x])
    for act in ("silu", "gelu"):
        y = O.epilogue(X, activation=act, lib=lib)
        _rel_close(y[0] - y[1], x, np.maximum(np.abs(x), 1.0), tol=1e-14)


def pin_epilogue_order(lib):
    """Bias and residual are added before the activation: ReLU(-2 + 0.5 + 1)
    = 0, SiLU(0 + 0 + 1) = logistic(1)."""
    P = np.array([[-2.0, 0.0]])
    b = np.array([0.5, 0.0], np.float32)
    r = np.array([[1.0, 1.0]], np.float32)
    assert O.epilogue(P, b, r, "relu", lib=lib)[0, 0] == 0.0
    _rel_close(O.epilogue(P, b, r, "silu", lib=lib)[0, 1], 0.7310585786300049, 1.0)


def pin_round_half_numpy(lib):
    """Rounding to binary16 matches numpy's float64 -> float16 conversion
    (round to nearest even, overflow to infinity) on random values, exact
    ties, subnormals and the overflow boundary."""
    rng = np.random.default_rng(12)
    vals = list(rng.standard_normal(300) * np.exp2(rng.integers(-26, 17, 300)))
    for e in (-24, -20, -14, -1, 0, 5, 15):            # exact ties at several exponents
        ulp = 2.0 ** max(e - 10, -24)
        base = 2.0 ** e
        vals += [base + ulp / 2, base + 1.5 * ulp, -(base + 2.5 * ulp)]
    vals += [65504.0, 65519.99, 65520.0, -65520.0, 2.0 ** -25, 3 * 2.0 ** -25, 1e-9, 7e4]
    for v in vals:
        got = O.round_half(v, lib=lib)
        want = float(np.float64(v).astype(np.float16))
        assert got == want or (np.isnan(got) and np.isnan(want)), (v, got, want)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]

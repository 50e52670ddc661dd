"""Pins of the CPU oracle to facts outside itself (no GPU needed).

Each test checks the oracle against something it cannot agree with by
construction: hand-worked values, exact rational arithmetic, a library routine
(numpy int64 matmul, PyTorch's float32 -> bf16 cast), a closed-form bound or a
mathematical invariant.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from exact import bf16 as exact_bf16
from exact import f16 as exact_f16
from exact import quantize_row as exact_quantize_row
from quantized_gemm_quantize_amd.inputs import (bf16_bits_to_f32, bsr_from_dense, dense_from_bsr,
                                                f32_to_bf16_bits, make_inputs, make_linear)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bits_to_float(b):
    return float(bf16_bits_to_f32(np.array([b], np.uint16))[0])


# --- hand-worked example ---------------------------------------------------

def test_worked_example_2x3(oracle):
    g = _load("worked_2x3.json")
    x_bits = f32_to_bf16_bits(np.array(g["x"], np.float32))
    assert np.array_equal(bf16_bits_to_f32(x_bits), np.array(g["x"], np.float32))  # exact in bf16
    xq, sx = oracle.quantize_rows_bf16(x_bits)
    assert sx.tolist() == g["x_scale"]
    assert xq.tolist() == g["xq"]
    wq, sw = oracle.quantize_rows_f32(np.array(g["w"], np.float32))
    assert sw.tolist() == g["w_scale"]
    assert wq.tolist() == g["wq"]
    acc = oracle.gemm_i32(xq, wq)
    assert acc.tolist() == g["acc"]
    out = oracle.epilogue_bf16(acc, sx, sw)
    assert bf16_bits_to_f32(out).tolist() == g["out_bf16"]
    # the exact product, rounded by hand-written rational bf16 rounding
    for m in range(2):
        for n in range(2):
            v = Fraction(g["out_exact"][m][n])
            assert v == acc[m, n] * Fraction(float(sx[m])) * Fraction(float(sw[n]))
            assert float(exact_bf16(v)) == g["out_bf16"][m][n]


def test_near_ties_divide_by_stored_fp32_scale(oracle):
    g = _load("near_ties.json")
    for case in g["cases"]:
        row = np.array([[case["absmax"], case["x"]]], np.float32)
        bits = f32_to_bf16_bits(row)
        assert np.array_equal(bf16_bits_to_f32(bits), row)
        q, s = oracle.quantize_rows_bf16(bits)
        assert int(q[0, 0]) == 127
        assert int(q[0, 1]) == case["q"], case
        # the same cases through the fp32 entry (weights)
        q2, s2 = oracle.quantize_rows_f32(row)
        assert int(q2[0, 1]) == case["q"] and s2[0] == s[0]


# --- exact rational reference on small rows --------------------------------

def _special_rows():
    rows = [
        np.zeros(16, np.float32),                                    # all-zero row
        np.full(16, -3.0, np.float32),                               # constant
        np.array([2.0 ** -130, -2.0 ** -131] + [0.0] * 14, np.float32),   # bf16 subnormals
        np.array([1e-38, 5e-39, -2e-39] + [1e-40] * 13, np.float32),      # tiny normals/subnormals
        np.array([3e38, -1.0, 1e30] + [0.5] * 13, np.float32),       # near the top of the range
        np.array([127.0, 63.5, -0.5, 1.5, 2.5, -2.5, 0.0, -0.0] * 2, np.float32),
    ]
    return rows


def test_quantize_matches_exact_rationals(oracle):
    rng = np.random.default_rng(123)
    rows = _special_rows()
    for _ in range(60):
        scale = float(2.0 ** rng.integers(-140, 120))
        rows.append((rng.standard_normal(16) * scale).astype(np.float32))
    for _ in range(40):   # heavy-tailed rows with outliers
        r = rng.standard_normal(16).astype(np.float32)
        r[rng.integers(0, 16)] *= 40
        rows.append(r)
    x = np.stack(rows)
    bits = f32_to_bf16_bits(x)
    xb = bf16_bits_to_f32(bits)
    q, s = oracle.quantize_rows_bf16(bits)
    for m in range(x.shape[0]):
        es, eq = exact_quantize_row([Fraction(float(v)) for v in xb[m]])
        assert Fraction(float(s[m])) == es, m
        assert q[m].tolist() == eq, m
    # fp32 entry on rows that are not bf16-representable
    xf = x + np.float32(1e-3) * rng.standard_normal(x.shape).astype(np.float32)
    qf, sf = oracle.quantize_rows_f32(xf)
    for m in range(xf.shape[0]):
        es, eq = exact_quantize_row([Fraction(float(v)) for v in xf[m]])
        assert Fraction(float(sf[m])) == es and qf[m].tolist() == eq, m


def test_zero_and_subnormal_rows(oracle):
    x = np.zeros((2, 32), np.float32)
    x[1, 3] = 2.0 ** -133          # smallest bf16 subnormal
    x[1, 7] = -(2.0 ** -134) * 3   # not bf16: rounds to -2^-132
    bits = f32_to_bf16_bits(x)
    q, s = oracle.quantize_rows_bf16(bits)
    assert s[0] == 0.0 and not q[0].any()
    assert s[1] > 0.0                    # subnormal scale, not flushed
    assert q[1, 7] == -127 and q[1, 3] == 64   # s = 1032 * 2^-149; 2^-133 / s = 63.504 -> 64
    acc = oracle.gemm_i32(q, np.ones((4, 32), np.int8))
    out = oracle.epilogue_bf16(acc, s, np.ones(4, np.float32))
    assert (out[0] == 0).all()           # +0, not -0


# --- invariants at workload sizes ------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "prefill_outliers"])
def test_quantize_invariants(oracle, name):
    inp = make_inputs(name, M=256 if name != "tiny" else None)
    q, s = oracle.quantize_rows_bf16(inp.x_bits)
    x = bf16_bits_to_f32(inp.x_bits).astype(np.float64)
    s64 = s.astype(np.float64)[:, None]
    err = np.abs(x - q.astype(np.float64) * s64)
    assert (err <= s64 * (0.5 + 2.0 ** -16)).all()
    assert (np.abs(q.astype(np.int32)) <= 127).all()
    assert (np.abs(q.astype(np.int32)).max(axis=1) == 127).all()
    # scale equals absmax/127 to within half an fp32 ulp (correct rounding)
    absmax = np.abs(x).max(axis=1)
    rel = np.abs(s.astype(np.float64) - absmax / 127.0) / (absmax / 127.0)
    assert (rel <= 2.0 ** -24).all()
    wq, sw = oracle.quantize_rows_f32(inp.w)
    errw = np.abs(inp.w.astype(np.float64) - wq.astype(np.float64) * sw.astype(np.float64)[:, None])
    assert (errw <= sw.astype(np.float64)[:, None] * (0.5 + 2.0 ** -16)).all()


# --- integer GEMM -----------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (2, 3, 5), (5, 8, 3), (8, 8, 8), (3, 1, 64), (17, 33, 48)])
def test_gemm_equals_numpy_int64(oracle, M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    xq = rng.integers(-127, 128, (M, K), dtype=np.int8)
    wq = rng.integers(-127, 128, (N, K), dtype=np.int8)
    acc = oracle.gemm_i32(xq, wq)
    ref = xq.astype(np.int64) @ wq.astype(np.int64).T
    assert np.array_equal(acc.astype(np.int64), ref)
    # brute force, element by element, for the tiniest shapes
    if M * N * K <= 512:
        for m in range(M):
            for n in range(N):
                assert acc[m, n] == sum(int(xq[m, k]) * int(wq[n, k]) for k in range(K))


def test_int32_headroom_bound(oracle):
    # 127*127*K stays below 2^31 up to K = 133144; the largest multiple of 16 is 133136
    K = 133136
    ones = np.full((1, K), 127, np.int8)
    acc = oracle.gemm_i32(ones, ones)
    assert int(acc[0, 0]) == 127 * 127 * K and 127 * 127 * K < 2 ** 31
    K2 = 133152
    big = np.full((1, K2), 127, np.int8)
    with pytest.raises(OverflowError):
        oracle.gemm_i32(big, big)
    neg = np.full((1, K2), -127, np.int8)
    with pytest.raises(OverflowError):
        oracle.gemm_i32(big, neg)


def test_int32_headroom_bound_full_int8_range(oracle):
    # -128 * -128 = 2^14 per product (the page's 2^31 / 2^14 remark): 2^14 K < 2^31 up to
    # K = 131071, the largest multiple of 16 being 131056, the library's K limit
    K = 131056
    m128 = np.full((1, K), -128, np.int8)
    acc = oracle.gemm_i32(m128, m128)
    assert int(acc[0, 0]) == 2 ** 14 * K and 2 ** 14 * K < 2 ** 31 <= 2 ** 14 * (K + 16)
    K2 = K + 16
    big = np.full((1, K2), -128, np.int8)
    with pytest.raises(OverflowError):
        oracle.gemm_i32(big, big)


# --- bf16 rounding and the epilogue ----------------------------------------

def test_bf16_rounding_matches_torch_cast(oracle):
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals)]
    ref = f32_to_bf16_bits(vals)
    got = np.array([oracle.bf16_rne_from_f64(float(v)) for v in vals], np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_rounding_ties_and_edges(oracle):
    r = oracle.bf16_rne_from_f64
    assert r(1.0 + 2.0 ** -8) == 0x3F80               # tie -> even (down)
    assert r(1.0 + 3 * 2.0 ** -8) == 0x3F82           # tie -> even (up)
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81  # just above the tie
    assert r(-(1.0 + 2.0 ** -8)) == 0xBF80
    assert r(2.0 ** -134) == 0x0000                   # subnormal tie -> 0
    assert r(3 * 2.0 ** -134) == 0x0002               # subnormal tie -> even
    assert r(2.0 ** -133) == 0x0001
    assert r(2.0 ** 128 - 2.0 ** 119) == 0x7F80       # rounds up to infinity
    assert r(2.0 ** 128 - 2.0 ** 119 - 2.0 ** 100) == 0x7F7F
    assert r(0.0) == 0x0000 and r(-0.0) == 0x8000


def test_epilogue_matches_exact_rationals(oracle):
    rng = np.random.default_rng(11)
    acc = rng.integers(-2 ** 31, 2 ** 31, (40, 50), dtype=np.int64).astype(np.int32)
    acc[0, :5] = [0, 1, -1, 2 ** 24 + 1, -(2 ** 31)]
    sx = (np.abs(rng.standard_normal(40)) * 2.0 ** rng.integers(-30, 10, 40)).astype(np.float32)
    sw = (np.abs(rng.standard_normal(50)) * 2.0 ** rng.integers(-30, 10, 50)).astype(np.float32)
    out = oracle.epilogue_bf16(acc, sx, sw)
    for m in range(40):
        for n in range(50):
            exact = int(acc[m, n]) * Fraction(float(sx[m])) * Fraction(float(sw[n]))
            assert _bits_to_float(out[m, n]) == float(exact_bf16(exact)), (m, n)


# --- addmm epilogue (bias, alpha, beta) ---------------------------------------

def test_addmm_reduces_to_the_plain_epilogue(oracle):
    """alpha = 1 with no bias term (or beta = 0) is the pinned plain epilogue, bit for bit."""
    rng = np.random.default_rng(21)
    acc = rng.integers(-2 ** 31, 2 ** 31, (17, 33), dtype=np.int64).astype(np.int32)
    acc[0, :3] = [0, 1, -1]
    sx = np.abs(rng.standard_normal(17)).astype(np.float32) * 1e-3
    sw = np.abs(rng.standard_normal(33)).astype(np.float32) * 1e-3
    bias = rng.standard_normal(33).astype(np.float32)
    plain = oracle.epilogue_bf16(acc, sx, sw)
    assert np.array_equal(oracle.epilogue_addmm_bf16(acc, sx, sw, None, 1.0, 0.0), plain)
    assert np.array_equal(oracle.epilogue_addmm_bf16(acc, sx, sw, bias, 1.0, 0.0), plain)


def test_addmm_hand_worked(oracle):
    """acc = 100, sx = 0.5, sw = 0.25: acc*sx*sw = 12.5, worked by hand."""
    acc = np.array([[100]], np.int32)
    sx, sw = np.array([0.5], np.float32), np.array([0.25], np.float32)
    cases = [  # bias, alpha, beta, value, bf16 bits
        (-12.5, 2.0, 1.0, 12.5, 0x4148),   # 2 * 12.5 - 12.5
        (-12.5, -1.0, 1.0, -25.0, 0xC1C8),  # -12.5 - 12.5
        (3.0, 2.0, 0.5, 26.5, 0x41D4),      # 25 + 1.5
        (-25.0, 2.0, 1.0, 0.0, 0x0000),     # exact cancellation: +0
    ]
    for b, alpha, beta, value, bits in cases:
        out = oracle.epilogue_addmm_bf16(acc, sx, sw, np.array([b], np.float32), alpha, beta)
        assert int(out[0, 0]) == bits, (b, alpha, beta, hex(int(out[0, 0])))
        assert _bits_to_float(out[0, 0]) == value


def test_addmm_matches_exact_rationals(oracle):
    """alpha*acc*sx[m]*sw[n] + beta*bias[n], evaluated exactly, rounded once to bf16. M != N and
    a bias that varies by channel catch a bias indexed by row or a dropped term."""
    rng = np.random.default_rng(23)
    M, N = 19, 41
    acc = rng.integers(-2 ** 31, 2 ** 31, (M, N), dtype=np.int64).astype(np.int32)
    sx = (np.abs(rng.standard_normal(M)) * 2.0 ** rng.integers(-30, -5, M)).astype(np.float32)
    sw = (np.abs(rng.standard_normal(N)) * 2.0 ** rng.integers(-20, -5, N)).astype(np.float32)
    bias = (rng.standard_normal(N) * 2.0 ** rng.integers(-4, 12, N)).astype(np.float32)
    for alpha, beta in [(1.0, 1.0), (0.75, -2.5), (-3.0, 0.125)]:
        out = oracle.epilogue_addmm_bf16(acc, sx, sw, bias, alpha, beta)
        for m in range(M):
            for n in range(N):
                exact = (Fraction(alpha) * int(acc[m, n]) * Fraction(float(sx[m])) *
                         Fraction(float(sw[n])) + Fraction(beta) * Fraction(float(bias[n])))
                assert _bits_to_float(out[m, n]) == float(exact_bf16(exact)), (alpha, beta, m, n)


def test_dequantized_product_error_bound(oracle):
    """|out - X W^T| is bounded by the quantization errors of X and W plus bf16 rounding."""
    inp = make_linear(24, 40, 96, seed=5)
    xq, sx = oracle.quantize_rows_bf16(inp.x_bits)
    wq, sw = oracle.quantize_rows_f32(inp.w)
    out = bf16_bits_to_f32(oracle.epilogue_bf16(oracle.gemm_i32(xq, wq), sx, sw)).astype(np.float64)
    x = bf16_bits_to_f32(inp.x_bits).astype(np.float64)
    w = inp.w.astype(np.float64)
    xh = xq.astype(np.float64) * sx.astype(np.float64)[:, None]
    wh = wq.astype(np.float64) * sw.astype(np.float64)[:, None]
    bound = np.abs(x - xh) @ np.abs(w).T + np.abs(xh) @ np.abs(w - wh).T
    exact_q = xh @ wh.T
    assert (np.abs(exact_q - x @ w.T) <= bound * (1 + 1e-12) + 1e-300).all()
    assert (np.abs(out - exact_q) <= np.abs(exact_q) * 2.0 ** -8 + 1e-300).all()
    # a transposed or mis-scaled product would break the bound
    assert not (np.abs(exact_q.T[:24, :24] - (x @ w.T)[:24, :24]) <= bound[:24, :24]).all()


def test_small_outputs_survive_bf16(oracle):
    """acc * scale far below 1 keeps its value in bf16 (an int8/int32 output flushes it to 0)."""
    acc = np.array([[3, -5, 1]], np.int32)
    sx = np.array([1e-4], np.float32)
    sw = np.array([1e-3, 1e-3, 1e-3], np.float32)
    out = bf16_bits_to_f32(oracle.epilogue_bf16(acc, sx, sw))
    assert (out != 0).all()
    assert np.allclose(out, acc[0] * 1e-7, rtol=2 ** -8)
    assert (np.rint(acc[0] * 1e-7) == 0).all()


# --- block-sparse weight ----------------------------------------------------

def test_bsr_equals_dense_on_densified_weight(oracle):
    inp = make_linear(40, 256, 192, seed=9, bs=64, zero_frac=0.6)
    xq, sx = oracle.quantize_rows_bf16(inp.x_bits)
    wq, sw = oracle.quantize_rows_f32(inp.w)
    crow, col, values = bsr_from_dense(wq, inp.block_mask, 64)
    assert np.array_equal(dense_from_bsr(crow, col, values, 256, 192), wq * 0 + np.where(
        np.repeat(np.repeat(inp.block_mask, 64, 0), 64, 1), wq, 0))
    acc_bsr = oracle.bsr_gemm_i32(xq, crow, col, values, 256)
    acc_dense = oracle.gemm_i32(xq, dense_from_bsr(crow, col, values, 256, 192))
    assert np.array_equal(acc_bsr, acc_dense)
    assert np.array_equal(acc_bsr.astype(np.int64),
                          xq.astype(np.int64) @ dense_from_bsr(crow, col, values, 256, 192).astype(np.int64).T)


def test_bsr_empty_rows_and_empty_matrix(oracle):
    rng = np.random.default_rng(2)
    xq = rng.integers(-127, 128, (8, 128), dtype=np.int8)
    mask = np.array([[False, False], [True, False], [False, False]])
    w = rng.integers(-127, 128, (192, 128), dtype=np.int8)
    crow, col, values = bsr_from_dense(w, mask, 64)
    assert crow.tolist() == [0, 0, 1, 1] and col.tolist() == [0]
    acc = oracle.bsr_gemm_i32(xq, crow, col, values, 192)
    assert not acc[:, :64].any() and not acc[:, 128:].any()
    assert np.array_equal(acc[:, 64:128].astype(np.int64),
                          xq[:, :64].astype(np.int64) @ w[64:128, :64].astype(np.int64).T)
    crow0 = np.zeros(4, np.int32)
    acc0 = oracle.bsr_gemm_i32(xq, crow0, np.zeros(0, np.int32), np.zeros((0, 64, 64), np.int8), 192)
    assert not acc0.any()


def test_bsr_workload_structure():
    inp = make_inputs("bsr", M=64)
    assert inp.block_mask.shape == (80, 20)
    assert int(inp.block_mask.sum()) == 160
    nz_blocks = np.abs(inp.w).reshape(80, 64, 20, 64).sum(axis=(1, 3)) > 0
    assert np.array_equal(nz_blocks, inp.block_mask)


def test_prefill_outlier_channels():
    inp = make_inputs("prefill_outliers", M=64)
    chans = inp.meta["outlier_channels"]
    assert len(chans) == 41
    x = bf16_bits_to_f32(inp.x_bits)
    ratio = np.abs(x[:, chans]).mean() / np.abs(np.delete(x, chans, axis=1)).mean()
    assert 15 < ratio < 25
    # seeded: the same draw twice
    assert np.array_equal(make_inputs("prefill_outliers", M=64).x_bits, inp.x_bits)
    assert torch.bfloat16 is not None


# --- 2:4 semi-structured weights --------------------------------------------

def test_compress24_hand_worked_rows(oracle):
    """The storage of two 2:4 rows (one 128-column block), worked by hand from its definition."""
    g = _load("sparse24_row.json")
    rows = np.zeros((2, 128), np.int8)
    for grp in range(32):
        p0, p1 = g["pairs"][grp % 6]
        rows[0, 4 * grp + p0] = grp + 1
        rows[0, 4 * grp + p1] = -(grp + 1)
    rows[1] = -rows[0]
    values, meta = oracle.compress24(rows)
    assert values.shape == (1, 2, 64) and meta.shape == (1, 2, 4)
    assert values[0].tolist() == g["values"]
    assert [[int(m) for m in r] for r in meta[0]] == [[int(h, 16) for h in r] for r in g["meta"]]
    assert np.array_equal(oracle.decompress24(values, meta), rows)


def _brute_force_prune24(w: np.ndarray) -> np.ndarray:
    """Keep the two largest |w| of each group of 4 (equal magnitudes in position order)."""
    N, K = w.shape
    out = np.zeros_like(w)
    for n in range(N):
        for g in range(K // 4):
            grp = [int(v) for v in w[n, 4 * g:4 * g + 4]]
            order = sorted(range(4), key=lambda p: (-abs(grp[p]), p))
            for p in order[:2]:
                out[n, 4 * g + p] = grp[p]
    return out


def test_compress24_keeps_the_two_largest_magnitudes(oracle):
    """On a dense int8 matrix the stored weight is the brute-force top-2 selection, ties
    included (small value range so that equal magnitudes are frequent)."""
    rng = np.random.default_rng(24)
    w = rng.integers(-3, 4, size=(9, 384), dtype=np.int8)
    w[0, :8] = -128                                   # int8 extremes
    w[1, :8] = 127
    values, meta = oracle.compress24(w)
    assert np.array_equal(oracle.decompress24(values, meta), _brute_force_prune24(w))


def test_compress24_is_lossless_on_2to4_weights(oracle):
    """The generator's 2:4 weights, quantized per channel, survive the round trip, and every
    nibble lists two distinct positions in increasing order."""
    inp = make_linear(8, 64, 256, seed=7, sparse24=True)
    wq, _ = oracle.quantize_rows_f32(inp.w)
    assert ((wq.reshape(64, -1, 4) != 0).sum(-1) <= 2).all()
    values, meta = oracle.compress24(wq)
    assert np.array_equal(oracle.decompress24(values, meta), wq)
    nib = (meta[..., None] >> (4 * np.arange(8, dtype=np.uint32))) & 15
    assert ((nib & 3) < (nib >> 2)).all()


def test_decompress24_rejects_bad_positions(oracle):
    values = np.zeros((1, 1, 64), np.int8)
    meta = np.array([[[0x44444444, 0x44444441, 0x44444444, 0x44444444]]], np.uint32)  # p0 = 1, p1 = 0
    with pytest.raises(ValueError):
        oracle.decompress24(values, meta)


def test_sparse24_product_matches_float64_matmul(oracle):
    """The 2:4 product (dense GEMM of the decompressed weight) against a float64 matmul of
    the original 2:4 int8 weight."""
    inp = make_linear(5, 32, 128, seed=3, sparse24=True)
    xq, _ = oracle.quantize_rows_bf16(inp.x_bits)
    wq, _ = oracle.quantize_rows_f32(inp.w)
    acc = oracle.gemm_i32(xq, oracle.decompress24(*oracle.compress24(wq)))
    ref = xq.astype(np.float64) @ wq.astype(np.float64).T
    assert np.array_equal(acc.astype(np.float64), ref)


# --- W4A16 (asymmetric group-wise 4-bit weights, bf16 activations) ----------

def _bits(h):
    return np.array([int(h, 16)], np.uint16)


def test_w4a16_dequant_hand_worked(oracle):
    g = _load("w4a16_worked.json")
    c = g["nibbles"]
    w = oracle.w4a16_dequant(np.array([c["bytes"]], np.uint8), _bits(c["scale_bits"])[None, :],
                             _bits(c["zero_bits"])[None, :])
    assert bf16_bits_to_f32(w)[0].tolist() == c["w"]
    for case in ("rounding", "shift_rounding"):
        c = g[case]
        wq4 = np.array([[c["q"] | (c["q"] << 4)]], np.uint8)          # the same code twice
        w = oracle.w4a16_dequant(wq4, _bits(c["scale_bits"])[None, :], _bits(c["zero_bits"])[None, :])
        assert w[0].tolist() == [int(c["w_bits"], 16)] * 2, case
        assert float(bf16_bits_to_f32(w)[0, 0]) == c["w"]


def test_w4a16_dequant_signed_hand_worked(oracle):
    """Signed 4-bit codes (s4): the worked cases of the fixture."""
    g = _load("w4a16_worked.json")
    c = g["nibbles_s4"]
    w = oracle.w4a16_dequant(np.array([c["bytes"]], np.uint8), _bits(c["scale_bits"])[None, :],
                             _bits(c["zero_bits"])[None, :], signed=True)
    assert bf16_bits_to_f32(w)[0].tolist() == c["w"]
    c = g["s4_shift_rounding"]
    wq4 = np.array([[c["q"] | (c["q"] << 4)]], np.uint8)
    w = oracle.w4a16_dequant(wq4, _bits(c["scale_bits"])[None, :], _bits(c["zero_bits"])[None, :],
                             signed=True)
    assert w[0].tolist() == [int(c["w_bits"], 16)] * 2
    assert float(bf16_bits_to_f32(w)[0, 0]) == c["w"]


def _f16_to_fraction(bits: int) -> Fraction:
    """IEEE binary16 bit pattern -> exact value (finite patterns), from the format's layout."""
    e, m = (bits >> 10) & 31, bits & 1023
    v = Fraction(m, 2 ** 24) if e == 0 else Fraction(1024 + m, 2 ** 25) * Fraction(2) ** e
    return -v if bits & 0x8000 else v


def test_f16_rounding_matches_exact(oracle):
    """The oracle's binary16 rounding against the exact rounding on a spread of values:
    normals, subnormals, ties (both parities), the largest finite value and overflow."""
    vals = [0.0, 1.0, -1.0, 0.1, 1 / 3, 65504.0, 65519.99, 65520.0, 2.0 ** -24, 2.0 ** -25,
            3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11,
            -7.3125 * 41 / 4096, 15 - 2.0 ** -11, 1e-8, 12345.678]
    rng = np.random.default_rng(17)
    vals += list(rng.standard_normal(200) * np.exp2(rng.integers(-20, 15, 200)))
    for v in vals:
        bits = oracle.f16_rne_from_f64(v)
        ref = exact_f16(Fraction(v))
        if ref is None:
            assert bits & 0x7FFF == 0x7C00, v          # infinity
        else:
            assert _f16_to_fraction(bits) == ref, v
            if ref == 0:
                assert bits & 0x7FFF == 0


def test_w4a16_dequant_f16_hand_worked(oracle):
    """binary16 scales, zeros and weights: the worked cases of the fixture."""
    g = _load("w4a16_worked.json")
    for case in ("f16_shift_rounding", "f16_rounding"):
        c = g[case]
        wq4 = np.array([[c["q"] | (c["q"] << 4)]], np.uint8)
        w = oracle.w4a16_dequant(wq4, _bits(c["scale_bits"])[None, :],
                                 _bits(c["zero_bits"])[None, :], half=True)
        assert w[0].tolist() == [int(c["w_bits"], 16)] * 2, case
        assert float(_f16_to_fraction(int(w[0, 0]))) == c["w"]


@pytest.mark.parametrize("signed", [False, True])
def test_w4a16_dequant_f16_matches_exact_rationals(oracle, signed):
    """Every binary16 dequantized weight of a random layer against f16(f16(q - z) * s) on
    exact rationals."""
    from quantized_gemm_quantize_amd.inputs import make_w4a16
    inp = make_w4a16(1, 6, 256, G=64, seed=19, signed=signed, half=True)
    w = oracle.w4a16_dequant(inp.wq4, inp.scales, inp.zeros, signed=signed, half=True)
    q = np.empty((6, 256), np.int64)
    q[:, 0::2] = inp.wq4 & 15
    q[:, 1::2] = inp.wq4 >> 4
    if signed:
        q = np.where(q >= 8, q - 16, q)
    for n in range(6):
        for k in range(256):
            sv = _f16_to_fraction(int(inp.scales[n, k // 64]))
            zv = _f16_to_fraction(int(inp.zeros[n, k // 64]))
            ref = exact_f16(exact_f16(int(q[n, k]) - zv) * sv)
            assert _f16_to_fraction(int(w[n, k])) == ref, (n, k)


def test_f16_gemm_matches_exact_sums(oracle):
    """The binary16 product against the exact rational sum rounded once (brute force)."""
    rng = np.random.default_rng(23)
    x = rng.standard_normal((3, 40)).astype(np.float16)
    w = (rng.standard_normal((4, 40)) * 0.05).astype(np.float16)
    out = oracle.f16_gemm(x.view(np.uint16), w.view(np.uint16))
    for m in range(3):
        for n in range(4):
            exact = sum(_f16_to_fraction(int(x.view(np.uint16)[m, k])) *
                        _f16_to_fraction(int(w.view(np.uint16)[n, k])) for k in range(40))
            assert _f16_to_fraction(int(out[m, n])) == exact_f16(exact), (m, n)


def test_w4a16_dequant_signed_agrees_below_eight(oracle):
    """Codes 0..7 mean the same as u4 and s4; codes 8..15 differ (by 16 before the shift)."""
    from quantized_gemm_quantize_amd.inputs import make_w4a16
    inp = make_w4a16(1, 4, 256, G=64, seed=13)
    wu = oracle.w4a16_dequant(inp.wq4, inp.scales, inp.zeros)
    ws = oracle.w4a16_dequant(inp.wq4, inp.scales, inp.zeros, signed=True)
    q = np.empty((4, 256), np.int64)
    q[:, 0::2] = inp.wq4 & 15
    q[:, 1::2] = inp.wq4 >> 4
    assert np.array_equal(wu[q < 8], ws[q < 8])
    assert not np.array_equal(wu[q >= 8], ws[q >= 8])


@pytest.mark.parametrize("signed", [False, True])
def test_w4a16_dequant_matches_exact_rationals(oracle, signed):
    """Every dequantized weight of a random layer against bf16(bf16(q - z) * s) evaluated on
    exact rationals with bf16 rounding written out (the exact module), for u4 and s4 codes."""
    from quantized_gemm_quantize_amd.inputs import make_w4a16
    inp = make_w4a16(1, 6, 256, G=128, seed=9)
    w = oracle.w4a16_dequant(inp.wq4, inp.scales, inp.zeros, signed=signed)
    q = np.empty((6, 256), np.int64)
    q[:, 0::2] = inp.wq4 & 15
    q[:, 1::2] = inp.wq4 >> 4
    if signed:
        q = np.where(q >= 8, q - 16, q)
    s = bf16_bits_to_f32(inp.scales)
    z = bf16_bits_to_f32(inp.zeros)
    for n in range(6):
        for k in range(256):
            sv, zv = Fraction(float(s[n, k // 128])), Fraction(float(z[n, k // 128]))
            ref = exact_bf16(exact_bf16(int(q[n, k]) - zv) * sv)
            assert Fraction(float(bf16_bits_to_f32(w[n:n + 1, k:k + 1])[0, 0])) == ref, (n, k)


def test_bf16_gemm_matches_exact_sums(oracle):
    """The bf16 product against the exact rational sum rounded once to bf16 (brute force)."""
    rng = np.random.default_rng(5)
    x = f32_to_bf16_bits(rng.standard_normal((3, 40)).astype(np.float32))
    w = f32_to_bf16_bits((rng.standard_normal((4, 40)) * 0.05).astype(np.float32))
    out = oracle.bf16_gemm(x, w)
    xf, wf = bf16_bits_to_f32(x), bf16_bits_to_f32(w)
    for m in range(3):
        for n in range(4):
            exact = sum(Fraction(float(xf[m, k])) * Fraction(float(wf[n, k])) for k in range(40))
            got = Fraction(float(bf16_bits_to_f32(out[m:m + 1, n:n + 1])[0, 0]))
            assert got == exact_bf16(exact), (m, n)


def test_w4a16_dequant_group_boundaries(oracle):
    """Each column takes the scale and zero of its own group: a layer whose groups differ
    only in scale dequantizes to q - z times the right group's scale."""
    N, K, G = 2, 256, 64
    q = np.tile(np.arange(16, dtype=np.uint8), (N, K // 16))
    from quantized_gemm_quantize_amd.inputs import pack_u4
    scales = f32_to_bf16_bits(np.array([[1.0, 2.0, 4.0, 8.0], [0.5, 0.25, 0.125, 1.0]], np.float32))
    zeros = f32_to_bf16_bits(np.full((N, K // G), 8.0, np.float32))
    w = bf16_bits_to_f32(oracle.w4a16_dequant(pack_u4(q), scales, zeros))
    s = bf16_bits_to_f32(scales)
    expect = (q.astype(np.float32) - 8.0) * np.repeat(s, G, axis=1)   # exact: small integers x 2^k
    assert np.array_equal(w, expect)

"""Pins of the CPU oracle to facts outside itself (runs without a GPU).

Each test ties one part of ``oracle/`` to a printed value, a closed form, a
library routine, an invariant or exact brute force, chosen so that a plausible
slip (a dropped term, a wrong sign or index, a transposed operand, a wrong bit
order) fails at least one of them.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle_checks import (code_at, e2m1_codebook, e4m3_frac, e8m0_frac, frac_of_storage,
                           read_golden)


# ---------------------------------------------------------------------------
# element / scale decoders
# ---------------------------------------------------------------------------

def test_e2m1_matches_page_codebook():
    book = e2m1_codebook()
    got = oracle.e2m1_value(np.arange(16))
    for c in range(16):
        assert Fraction(float(got[c])) == book[c], c


def test_e4m3_exhaustive_against_torch_fn_and_page_constants():
    b = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_value(b)
    ref = torch.from_numpy(b.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[~both_nan], ref[~both_nan])
    assert int(np.isfinite(ours).sum()) == 254
    for row in read_golden("e4m3_facts.txt"):
        hx, v = row.split()
        got = ours[int(hx, 16)]
        if v == "nan":
            assert np.isnan(got)
        else:
            assert got == float(v) and np.signbit(got) == v.startswith("-"), hx
    # integer-field form, byte by byte
    for byte in range(256):
        f = e4m3_frac(byte)
        if f is None:
            assert np.isnan(ours[byte])
        else:
            assert Fraction(float(ours[byte])) == f


def test_e8m0_against_torch_and_closed_form():
    b = np.arange(256, dtype=np.uint8)
    ours = oracle.e8m0_value(b)
    ref = torch.from_numpy(b.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])
    assert ours[120] == 1.0 / 128 and ours[127] == 1.0 and ours[130] == 8.0
    assert ours[0] == 2.0 ** -127
    for byte in range(255):
        assert Fraction(float(ours[byte])) == e8m0_frac(byte)


def test_e4m3_encoder_reference_against_torch_rne():
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.normal(0, 1, 4000), rng.normal(0, 50, 2000), rng.uniform(-448, 448, 2000),
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 2000),
    ]).astype(np.float32)
    # every exact tie between neighbouring codes (midpoints), positive and negative
    vals = oracle.e4m3_value(np.arange(0x7F))
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids, vals.astype(np.float32)])
    ours = oracle.e4m3_encode_nearest(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    # saturation and NaN, which torch's cast does not define the same way
    sat = oracle.e4m3_encode_nearest(np.array([449.0, 1e6, -1e6, np.inf, -np.inf, np.nan]))
    assert list(sat) == [0x7E, 0x7E, 0xFE, 0x7E, 0xFE, 0x7F]


# ---------------------------------------------------------------------------
# bit layout
# ---------------------------------------------------------------------------

def test_pack_known_answers_from_page_masks():
    for row in read_golden("pack_known_answers.txt"):
        lhs, rhs = row.split("->")
        bits, codes = lhs.split()
        bits = int(bits)
        codes = np.array([int(c) for c in codes.split(",")], dtype=np.uint8)
        expect = np.array([int(h, 16) for h in rhs.split()], dtype=np.uint8)
        # pad to a whole number of bytes is already true for every line
        packed = oracle.pack_codes(codes[None, :], bits)
        assert np.array_equal(packed[0], expect), (bits, codes)
        back = oracle.unpack_codes(expect[None, :], len(codes), bits)
        assert np.array_equal(back[0], codes)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
def test_pack_unpack_roundtrip_and_bitwise_reader(bits):
    rng = np.random.default_rng(bits)
    K = 96
    codes = rng.integers(0, 1 << bits, size=(5, K), dtype=np.uint8)
    codes[0, : min(K, 1 << bits)] = np.arange(min(K, 1 << bits))  # every code value
    packed = oracle.pack_codes(codes, bits)
    assert packed.shape == (5, oracle.packed_row_bytes(K, bits))
    assert np.array_equal(oracle.unpack_codes(packed, K, bits), codes)
    for r in range(5):
        for j in range(K):
            assert code_at(packed[r], j, bits) == codes[r, j]


def test_packed_geometry_matches_pack_factor_rule():
    # mlx quantized_nax.h get_pack_factor / get_bytes_per_pack: 3- and 5-bit
    # codes come 8 per 3 / 5 bytes, 6-bit 4 per 3 bytes, 2/4/8-bit 8/b per byte.
    per = {2: (4, 1), 3: (8, 3), 4: (2, 1), 5: (8, 5), 6: (4, 3), 8: (1, 1)}
    for bits, (pf, bpp) in per.items():
        assert oracle.packed_row_bytes(4096, bits) == 4096 // pf * bpp


# ---------------------------------------------------------------------------
# rounding to the output dtypes
# ---------------------------------------------------------------------------

def _bf16_neighbours_rne(v: float) -> int:
    """Brute force: the bf16 pattern nearest to v (exact comparison with
    Fractions over the two candidates around v), ties to the even pattern."""
    f32 = np.float32(v)
    u = int(np.array([f32]).view(np.uint32)[0])
    lo = u >> 16
    cands = {lo, lo + 1, lo - 1}
    best = None
    for c in sorted(cands):
        if c < 0 or c > 0xFFFF:
            continue
        fv = np.array([c << 16], dtype=np.uint32).view(np.float32)[0]
        if not np.isfinite(fv):
            continue
        d = abs(Fraction(float(fv)) - Fraction(v))
        key = (d, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_bf16_rounding_direct_from_f64():
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.normal(0, 1, 3000), rng.normal(0, 1e-30, 500),
                        rng.normal(0, 1e30, 500)])
    # exact midpoints between bf16 neighbours, plus a nudge that fp32 would lose
    base = np.float32(1.0) + np.float32(2.0 ** -7) * np.arange(64, dtype=np.float32)
    mids = base.astype(np.float64) + 2.0 ** -8
    v = np.concatenate([v, mids, mids + 2.0 ** -40, mids - 2.0 ** -40, -mids])
    got = oracle.round_f64_to_bf16_bits(v)
    for i in range(v.size):
        assert int(got[i]) == _bf16_neighbours_rne(float(v[i])), v[i]
    # the nudged midpoints must not tie (a via-fp32 rounding would get these wrong)
    up = oracle.round_f64_to_bf16_bits(mids + 2.0 ** -40)
    assert np.all(up == oracle.round_f64_to_bf16_bits(base.astype(np.float64) + 2.0 ** -7))


def test_f16_rounding_direct_from_f64():
    one_tie = 1.0 + 2.0 ** -11
    assert oracle.round_f64_to_f16(np.array([one_tie]))[0] == np.float16(1.0)
    assert oracle.round_f64_to_f16(np.array([one_tie + 2.0 ** -40]))[0] == np.float16(1.0 + 2.0 ** -10)
    assert np.isinf(oracle.round_f64_to_f16(np.array([65520.0]))[0])
    assert oracle.round_f64_to_f16(np.array([65519.0]))[0] == np.float16(65504.0)


def test_ulp_of_spacing():
    assert oracle.ulp_of(np.array([np.float32(1.0)]), "f32")[0] == 2.0 ** -23
    assert oracle.ulp_of(np.array([np.float16(1.0)]), "f16")[0] == 2.0 ** -10
    one_bf16 = np.array([0x3F80], dtype=np.uint16)
    assert oracle.ulp_of(one_bf16, "bf16")[0] == 2.0 ** -7
    assert oracle.ulp_of(np.array([0], dtype=np.uint16), "bf16")[0] == 2.0 ** -133


# ---------------------------------------------------------------------------
# the product itself
# ---------------------------------------------------------------------------

def _exact_weights(fmt, K, w, scales, biases, bits, group, dtype, gscale):
    """Fraction weights [N][K] by reading bits one at a time."""
    N = w.shape[0]
    book = e2m1_codebook()
    if fmt == "affine":
        S = frac_of_storage(scales, dtype)
        Bi = frac_of_storage(biases, dtype)
    W = [[None] * K for _ in range(N)]
    for n in range(N):
        for k in range(K):
            if fmt == "affine":
                q = code_at(w[n], k, bits)
                W[n][k] = S[n, k // group] * q + Bi[n, k // group]
            elif fmt == "mxfp4":
                W[n][k] = book[code_at(w[n], k, 4)] * e8m0_frac(int(scales[n, k // 32]))
            elif fmt == "nvfp4":
                g = Fraction(float(np.float32(gscale))) if gscale is not None else Fraction(1)
                W[n][k] = book[code_at(w[n], k, 4)] * e4m3_frac(int(scales[n, k // 16])) * g
            elif fmt == "mxfp8":
                W[n][k] = e4m3_frac(int(w[n, k])) * e8m0_frac(int(scales[n, k // 32]))
    return W


def _small_case(fmt, dtype, bits=4, group=32, B=3, N=8, K=32, seed=0):
    key = f"pin-{fmt}-{dtype}-{bits}-{group}-{seed}"
    if fmt == "affine":
        return workloads.affine_case(99, key, bits=bits, group=group, K=K, N=N, B=B, dtype=dtype)
    if fmt == "mxfp4":
        return workloads.mxfp4_case(99, key, K=K, N=N, B=B, dtype=dtype)
    if fmt == "nvfp4":
        return workloads.nvfp4_case(99, key, K=K, N=N, B=B, dtype=dtype, global_scale=0.75)
    return workloads.mxfp8_case(99, key, K=K, N=N, B=B, dtype=dtype)


def _oracle_y(c):
    W = oracle.dequant(c.fmt, c.K, c.w, c.scales, c.biases, bits=c.bits, group=c.group,
                       dtype=c.dtype, global_scale=c.global_scale)
    return oracle.qmv(c.x, c.dtype, W), W


CASES_8x32 = ([("affine", d, b, 32) for d in ("f32", "f16", "bf16") for b in (2, 3, 4, 5, 6, 8)]
              + [(f, d, 4, 32) for f in ("mxfp4", "nvfp4", "mxfp8") for d in ("f32", "f16", "bf16")])


@pytest.mark.parametrize("fmt,dtype,bits,group", CASES_8x32)
def test_brute_force_8x32_exact(fmt, dtype, bits, group):
    c = _small_case(fmt, dtype, bits=bits, group=group)
    y, _ = _oracle_y(c)
    W = _exact_weights(fmt, c.K, c.w, c.scales, c.biases, bits, group, dtype, c.global_scale)
    X = frac_of_storage(c.x, dtype)
    for b in range(c.B):
        for n in range(c.N):
            exact = sum(X[b, k] * W[n][k] for k in range(c.K))
            mag = sum(abs(X[b, k] * W[n][k]) for k in range(c.K))
            err = abs(Fraction(float(y[b, n])) - exact)
            assert err <= Fraction(c.K) * Fraction(2) ** -53 * mag, (b, n)


def test_affine_identity_exact():
    # sum_k x_k (s q_k + beta) = s sum x q + beta sum x, over one group (mlx
    # quantized_nax.h qdot); checked in exact arithmetic against the oracle.
    c = workloads.affine_case(98, "identity", bits=4, group=64, K=64, N=4, B=2, dtype="bf16")
    y, _ = _oracle_y(c)
    X = frac_of_storage(c.x, "bf16")
    S = frac_of_storage(c.scales, "bf16")
    Bi = frac_of_storage(c.biases, "bf16")
    for b in range(2):
        for n in range(4):
            sxq = sum(X[b, k] * code_at(c.w[n], k, 4) for k in range(64))
            sx = sum(X[b, k] for k in range(64))
            exact = S[n, 0] * sxq + Bi[n, 0] * sx
            assert abs(Fraction(float(y[b, n])) - exact) <= Fraction(2) ** -45 * (abs(exact) + 1)


def test_one_hot_reads_weight_column():
    c = workloads.affine_case(97, "onehot", bits=5, group=32, K=64, N=6, B=1, dtype="f32")
    _, W = _oracle_y(c)
    for k in range(c.K):
        x = np.zeros((1, c.K), dtype=np.float32)
        x[0, k] = 1.0
        y = oracle.qmv(x, "f32", W)
        assert np.array_equal(y[0], W[:, k])
        # and W[:, k] is code k of each row under the page's LSB-first layout
        for n in range(c.N):
            q = code_at(c.w[n], k, 5)
            s = float(c.scales[n, k // 32])
            bb = float(c.biases[n, k // 32])
            assert W[n, k] == s * q + bb


def test_scale_equivariance_powers_of_two():
    c = workloads.mxfp4_case(96, "equi", K=128, N=16, B=2, dtype="bf16")
    y1, _ = _oracle_y(c)
    c.scales = (c.scales + 1).astype(np.uint8)
    y2, _ = _oracle_y(c)
    assert np.array_equal(y2, 2.0 * y1)
    n = workloads.nvfp4_case(96, "equi-nv", K=128, N=16, B=2, dtype="f16", global_scale=1.0)
    ya, _ = _oracle_y(n)
    n.global_scale = 0.5
    yb, _ = _oracle_y(n)
    assert np.array_equal(yb, 0.5 * ya)
    n.global_scale = None
    yc, _ = _oracle_y(n)
    assert np.array_equal(yc, ya)


# the tiny value of each 16-bit type: below half an ulp of 1.0 (bf16 ulp
# 2^-7, f16 ulp 2^-10), so 1 + tiny rounds back to 1 in that type
TINY = {"bf16": 2.0 ** -9, "f16": 2.0 ** -12}


def _sum_in_type(xs, dtype):
    """sum of stored values accumulated in the 16-bit type itself, each
    partial sum rounded to it (the behaviour before the fix)."""
    acc = 0.0
    for k in range(xs.shape[-1]):
        a = acc + oracle.storage_to_f64(xs[0, k:k + 1], dtype)[0]
        acc = oracle.storage_to_f64(oracle.round_f64_to(np.array([a]), dtype), dtype)[0]
    return acc


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_precision_regression_input_is_sensitive(dtype):
    # mlx pull request 4516: sum(x) for the affine bias term must widen each
    # element before adding. One large and many tiny x in a group: summing in
    # the 16-bit type first drops the tiny ones, the oracle keeps them exactly.
    K, group = 64, 64
    tiny = TINY[dtype]
    x = np.full((1, K), tiny, dtype=np.float64)
    x[0, 0] = 1.0
    xs = workloads.to_storage(x, dtype)
    w = np.zeros((1, K // 2), dtype=np.uint8)             # q = 0 everywhere: y = bias * sum(x)
    scales = workloads.to_storage(np.array([[0.01]]), dtype)
    biases = workloads.to_storage(np.array([[1.0]]), dtype)
    W = oracle.dequant_affine(w, scales, biases, K, 4, group, dtype)
    y = oracle.qmv(xs, dtype, W)[0, 0]
    exact = 1.0 + 63 * tiny
    assert y == exact
    # the same sum accumulated in the 16-bit type loses every tiny value
    pre_fix = _sum_in_type(xs, dtype)
    assert pre_fix == 1.0
    r = oracle.round_f64_to(np.array([exact]), dtype)
    ulp = oracle.ulp_of(r, dtype)[0]
    assert abs(pre_fix - exact) > ulp
    # and so does the GPU test's input (large x first in each group of 64)
    K2 = 512
    x2 = np.full((1, K2), tiny)
    x2[0, ::group] = 1.0
    xs2 = workloads.to_storage(x2, dtype)
    for g in range(K2 // group):
        assert _sum_in_type(xs2[:, g * group:(g + 1) * group], dtype) == 1.0
        assert oracle.storage_to_f64(xs2[:, g * group:(g + 1) * group], dtype).sum() == exact


def test_gather_equals_per_slot_and_zero_rows():
    m = workloads.moe_case("affine", "gate_up", E=6, hidden=64, ffn=16, tokens=3, top_k=2)
    Wd = lambda e: oracle.dequant_affine(m.w[e], m.scales[e], m.biases[e], m.K, 4, 64, "bf16")
    lhs = m.lhs.copy()
    rhs = m.rhs.copy()
    rhs[1] = 1000      # expert out of range -> zeros
    lhs[2] = 77        # x row out of range -> zeros
    y = oracle.gather_qmv(m.x, "bf16", lhs, rhs, m.E, m.N, Wd)
    for s in range(lhs.size):
        if s in (1, 2):
            assert not y[s].any()
        else:
            ref = oracle.qmv(m.x[lhs[s]][None, :], "bf16", Wd(int(rhs[s])))[0]
            assert np.array_equal(y[s], ref)


def test_abs_dot_brute_force():
    c = _small_case("mxfp8", "f16", B=2, N=4, K=32, seed=5)
    _, W = _oracle_y(c)
    A = oracle.abs_dot(c.x, "f16", W)
    X = oracle.storage_to_f64(c.x, "f16")
    for b in range(2):
        for n in range(4):
            assert math.isclose(A[b, n], sum(abs(X[b, k] * W[n, k]) for k in range(32)),
                                rel_tol=1e-14)


# ---------------------------------------------------------------------------
# the generators produce what the workload recipe states
# ---------------------------------------------------------------------------

def test_generators_follow_recipes():
    c1 = workloads.small_affine_case()
    assert (c1.K, c1.N, c1.B, c1.bits, c1.group, c1.dtype) == (512, 256, 1, 4, 64, "f32")
    codes = oracle.unpack_codes(c1.w, 512, 4)
    assert set(np.unique(codes)) == set(range(16))
    s = c1.scales.astype(np.float64)
    assert s.min() >= 0.01 and s.max() <= 0.1
    assert np.all(np.abs(c1.biases.astype(np.float64) + 8 * s) <= 0.0100001)
    m3 = workloads.mlp_up_case("mxfp8", 1, N=64)
    assert not np.any((m3.w & 0x7F) == 0x7F)
    assert m3.scales.min() >= 120 and m3.scales.max() <= 130
    n3 = workloads.mlp_up_case("nvfp4", 1, N=64)
    v = oracle.e4m3_value(n3.scales)
    assert np.all(v >= 0) and np.isfinite(v).all() and n3.global_scale == 0.5
    g = workloads.moe_case("mxfp4", "gate_up")
    assert g.lhs.shape == (128,) and g.w.shape == (64, 1536, 2048)
    per_tok = g.rhs.reshape(16, 8)
    assert all(len(set(r)) == 8 for r in per_tok.tolist())
    d = workloads.moe_case("mxfp4", "down")
    assert np.array_equal(d.rhs, g.rhs) and d.w.shape == (64, 4096, 768)
    assert np.array_equal(workloads.route_topk(np.array([[1.0, 3.0, 3.0, 0.0]]), 2), [[1, 2]])


# ---------------------------------------------------------------------------
# qmv_rows: the product restricted to chosen output rows (sampled checks of
# full-size problems use it)
# ---------------------------------------------------------------------------

def _rows_case(fmt, dtype, seed, K=96, N=11, B=2, bits=4, group=32):
    key = f"rows-{fmt}-{dtype}-{bits}-{group}-{seed}"
    if fmt == "affine":
        return workloads.affine_case(98, key, bits=bits, group=group, K=K, N=N, B=B, dtype=dtype)
    if fmt == "mxfp4":
        return workloads.mxfp4_case(98, key, K=K, N=N, B=B, dtype=dtype)
    if fmt == "nvfp4":
        return workloads.nvfp4_case(98, key, K=K, N=N, B=B, dtype=dtype)
    if fmt == "nvfp4-noglobal":
        return workloads.nvfp4_case(98, key, K=K, N=N, B=B, dtype=dtype, global_scale=None)
    if fmt == "mxfp8":
        return workloads.mxfp8_case(98, key, K=K, N=N, B=B, dtype=dtype)
    return workloads.sb_case(fmt, K=K, N=N, B=B, dtype=dtype, key=key)


ROWS_FORMATS = ([("affine", b, g) for b in (2, 3, 4, 5, 6, 8) for g in (32, 64)] +
                [(f, 4, 32) for f in ("mxfp4", "nvfp4", "nvfp4-noglobal", "mxfp8",
                                      "mxfp8_e5m2", "nvfp8", "int4", "mxint8", "fp4_f16")])
ROWS = np.array([10, 0, 3, 3, 7, 10, 1])   # permuted, repeated, first and last row


@pytest.mark.parametrize("fmt,bits,group", ROWS_FORMATS)
def test_qmv_rows_equals_columns_of_full_product(fmt, bits, group):
    # exactly representable inputs (small-integer x; power-of-two affine
    # scales with integer biases): every fp64 sum is exact, so the restricted
    # product must equal the chosen columns of the full one bit for bit, and
    # a row picked with the wrong scale row, an axis mix-up or a dropped
    # global scale shows as a difference
    c = _rows_case(fmt, "f32", 0, K=64 if group == 32 else 128, bits=bits, group=group)
    rng = np.random.default_rng(bits * 100 + group)
    if c.fmt == "affine":
        c.scales = np.ldexp(1.0, rng.integers(-3, 2, size=c.scales.shape)).astype(np.float32)
        c.biases = rng.integers(-8, 9, size=c.biases.shape).astype(np.float32)
    elif c.scales.dtype in (np.float32, np.float16):
        c.scales = np.ldexp(1.0, rng.integers(-6, -2, size=c.scales.shape)).astype(c.scales.dtype)
    c.x = rng.integers(-3, 4, size=c.x.shape).astype(np.float32)
    W = oracle.dequant(c.fmt, c.K, c.w, c.scales, c.biases, bits=c.bits, group=c.group,
                       dtype="f32", global_scale=c.global_scale)
    full = oracle.qmv(c.x, "f32", W)
    part = oracle.qmv_rows(c.fmt, c.x, "f32", c.K, ROWS, c.w, c.scales, c.biases,
                           bits=c.bits, group=c.group, global_scale=c.global_scale)
    assert part.shape == (c.B, ROWS.size)
    assert np.array_equal(part, full[:, ROWS])
    # each chosen column is the loop-by-loop dot product of its own row
    for j, n in enumerate(ROWS):
        for b in range(c.B):
            assert part[b, j] == math.fsum(float(c.x[b, k]) * W[n, k] for k in range(c.K))


@pytest.mark.parametrize("fmt,bits,group", ROWS_FORMATS)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_qmv_rows_random_inputs(fmt, bits, group, dtype):
    # the workload generators' own distributions: equal to the full product's
    # columns up to fp64 summation order
    c = _rows_case(fmt, dtype, 1, K=3 * group if fmt == "affine" else 192, bits=bits, group=group)
    W = oracle.dequant(c.fmt, c.K, c.w, c.scales, c.biases, bits=c.bits, group=c.group,
                       dtype=dtype, global_scale=c.global_scale)
    full = oracle.qmv(c.x, dtype, W)
    A = oracle.abs_dot(c.x, dtype, W)
    part = oracle.qmv_rows(c.fmt, c.x, dtype, c.K, ROWS, c.w, c.scales, c.biases,
                           bits=c.bits, group=c.group, global_scale=c.global_scale)
    assert np.all(np.abs(part - full[:, ROWS]) <= 1e-13 * A[:, ROWS])

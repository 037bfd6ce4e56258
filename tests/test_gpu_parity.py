"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every test names its case before launching anything (see gpu_util.say)."""

from __future__ import annotations

import ctypes
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import (case_to_dev, check, indices_dev, oracle_rows, run_qmv, sample_rows, say,
                      to_dev, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bmv():
    import torch
    import bit_matrix_vector_amd as m
    assert torch.cuda.is_available()
    m.load()  # a machine without the built library must fail here, loudly
    return m


def _sync():
    import torch
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# device codecs: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
def test_device_unpack_bit_exact(bmv, bits):
    say(f"unpack bits={bits}")
    rng = np.random.default_rng(bits)
    K = 256
    codes = rng.integers(0, 1 << bits, size=(37, K), dtype=np.uint8)
    codes[0, : 1 << min(bits, 8)] = np.arange(1 << min(bits, 8))[:K]
    packed = oracle.pack_codes(codes, bits)
    out = bmv.qmv_unpack_codes_device(to_dev(packed), K, bits).cpu().numpy()
    assert np.array_equal(out, codes)


def _f32_bits_equal(got: np.ndarray, want64: np.ndarray):
    want = want64.astype(np.float32)
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn), "NaN positions differ"
    g = got[~gn].view(np.uint32)
    w = want[~wn].view(np.uint32)
    bad = np.flatnonzero(g != w)
    assert bad.size == 0, (f"{bad.size} values differ; e.g. got {got[~gn][bad[:4]]} "
                           f"want {want[~wn][bad[:4]]}")


def _rn32_affine(c):
    """RN_fp32(s*q + b), exact: fp64 when the fp64 sum is exact, else Fraction."""
    q = oracle.unpack_codes(c.w, c.K, c.bits).astype(np.float64)
    g = np.arange(c.K) // c.group
    s = oracle.storage_to_f64(c.scales, c.dtype)[:, g]
    b = oracle.storage_to_f64(c.biases, c.dtype)[:, g]
    p = s * q                               # exact: <= 24 + 8 significant bits
    t = p + b
    bb = t - p
    err = (p - (t - bb)) + (b - bb)         # TwoSum error term
    out = t.astype(np.float32)
    for i in zip(*np.nonzero(err != 0)):
        ex = Fraction(float(p[i])) + Fraction(float(b[i]))
        # nearest fp32 to the exact value, ties to even
        f = np.float32(float(ex))
        cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
        best = min(cands, key=lambda c_: (abs(Fraction(float(c_)) - ex),
                                          int(np.array([c_]).view(np.uint32)[0]) & 1))
        out[i] = best
    return out.astype(np.float64)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("group", [32, 64, 128])
def test_device_dequant_affine_bit_exact(bmv, dtype, bits, group):
    say(f"dequant affine b{bits} g{group} {dtype}")
    c = workloads.affine_case(50, f"dq-{bits}-{group}-{dtype}", bits=bits, group=group, K=256,
                              N=19, B=1, dtype=dtype)
    d = case_to_dev(c)
    wt = bmv.make_weights("affine", d["w"], d["scales"], d["biases"], K=c.K, bits=bits,
                          group_size=group)
    got = bmv.qmv_dequant_device(wt, {"f32": 0, "f16": 1, "bf16": 2}[dtype], "cuda:0")
    _f32_bits_equal(got.cpu().numpy(), _rn32_affine(c))


@pytest.mark.parametrize("dt", [0, 1, 2])
def test_device_dequant_mxfp4_exhaustive(bmv, dt):
    say(f"dequant mxfp4 exhaustive dtype {dt}")
    exps = np.array([0, 1, 2, 100, 120, 126, 127, 128, 130, 200, 253, 254, 255], dtype=np.uint8)
    N = exps.size
    K = 32 * 8
    codes = np.tile(np.arange(16, dtype=np.uint8), (N, K // 16))
    w = oracle.pack_codes(codes, 4)
    scales = np.repeat(exps[:, None], K // 32, axis=1)
    import torch
    wt_w, wt_s = to_dev(w), to_dev(scales)
    wt = bmv.make_weights("mxfp4", wt_w, wt_s, K=K)
    got = bmv.qmv_dequant_device(wt, dt, "cuda:0").cpu().numpy()
    _f32_bits_equal(got, oracle.dequant_mxfp4(w, scales, K))


@pytest.mark.parametrize("dt", [0, 1, 2])
@pytest.mark.parametrize("gscale", [None, 1.0, 0.5, 3.0])
def test_device_dequant_nvfp4_exhaustive(bmv, gscale, dt):
    say(f"dequant nvfp4 exhaustive g={gscale} dtype {dt}")
    import torch
    N = 256                          # every E4M3 scale byte, one per row
    K = 32
    codes = np.tile(np.arange(16, dtype=np.uint8), (N, K // 16))
    w = oracle.pack_codes(codes, 4)
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], K // 16, axis=1)
    gs = None if gscale is None else torch.tensor([gscale], dtype=torch.float32, device="cuda:0")
    dw, ds = to_dev(w), to_dev(scales)
    wt = bmv.make_weights("nvfp4", dw, ds, K=K, global_scale=gs)
    got = bmv.qmv_dequant_device(wt, dt, "cuda:0").cpu().numpy()
    _f32_bits_equal(got, oracle.dequant_nvfp4(w, scales, K, gscale))


@pytest.mark.parametrize("dt", [0, 1, 2])
def test_device_dequant_mxfp8_exhaustive(bmv, dt):
    say(f"dequant mxfp8 exhaustive dtype {dt}")
    exps = np.array([0, 1, 7, 120, 127, 130, 254, 255], dtype=np.uint8)
    K = 256
    w = np.tile(np.arange(256, dtype=np.uint8), (exps.size, 1))
    scales = np.repeat(exps[:, None], K // 32, axis=1)
    dw, ds = to_dev(w), to_dev(scales)
    wt = bmv.make_weights("mxfp8", dw, ds, K=K)
    got = bmv.qmv_dequant_device(wt, dt, "cuda:0").cpu().numpy()
    _f32_bits_equal(got, oracle.dequant_mxfp8(w, scales, K))


# ---------------------------------------------------------------------------
# QMV at small sizes: every output checked
# ---------------------------------------------------------------------------

def _full_check(bmv, c, what):
    say(what)
    y = to_host(run_qmv(bmv, c), c.dtype)
    W = oracle.dequant(c.fmt, c.K, c.w, c.scales, c.biases, bits=c.bits, group=c.group,
                       dtype=c.dtype, global_scale=c.global_scale)
    return check(y, oracle.qmv(c.x, c.dtype, W), oracle.abs_dot(c.x, c.dtype, W), c.dtype, what)


def test_small_affine_full(bmv):
    _full_check(bmv, workloads.small_affine_case(), "small affine b4 g64 K512 N256 f32")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("K,group", [(512, 32), (640, 64), (2304, 128), (4096, 64)])
def test_affine_small_grid(bmv, dtype, bits, K, group):
    for B in (1, 3, 8):
        c = workloads.affine_case(60, f"grid-{dtype}-{bits}-{K}-{group}-{B}", bits=bits,
                                  group=group, K=K, N=77, B=B, dtype=dtype)
        _full_check(bmv, c, f"affine b{bits} g{group} K{K} N77 B{B} {dtype}")


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "mxfp8"])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_block_scaled_small_grid(bmv, fmt, dtype):
    for K, N, B in ((512, 77, 1), (1536, 40, 2), (4096, 33, 5), (2560, 129, 8)):
        key = f"bs-{fmt}-{dtype}-{K}-{N}-{B}"
        if fmt == "mxfp4":
            c = workloads.mxfp4_case(61, key, K=K, N=N, B=B, dtype=dtype)
        elif fmt == "nvfp4":
            c = workloads.nvfp4_case(61, key, K=K, N=N, B=B, dtype=dtype, global_scale=0.5)
        else:
            c = workloads.mxfp8_case(61, key, K=K, N=N, B=B, dtype=dtype)
        _full_check(bmv, c, f"{fmt} K{K} N{N} B{B} {dtype}")


def test_nvfp4_without_global_scale(bmv):
    c = workloads.nvfp4_case(62, "nv-noglobal", K=1024, N=45, B=3, dtype="bf16",
                             global_scale=None)
    _full_check(bmv, c, "nvfp4 no global scale")


# ---------------------------------------------------------------------------
# the chain workload: 8-bit g64 K=2560 bf16, tails, dependent chain
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N", [2560, *workloads.CHAIN_TAILS])
def test_chain_full(bmv, N):
    _full_check(bmv, workloads.chain_case(N), f"chain workload N{N}")


def test_tail_rows_equal_padded_call_bitwise(bmv):
    import torch
    c = workloads.chain_case(2560)
    d = case_to_dev(c)
    say("tail vs padded, affine 8-bit")
    full = bmv.qmv_affine(d["x"], d["w"], d["scales"], d["biases"], 8, 64)
    for n in (1, 3, 5, 7, 8, 9, 12, 17, 63, 65, 100):
        part = bmv.qmv_affine(d["x"], d["w"][:n].contiguous(), d["scales"][:n].contiguous(),
                              d["biases"][:n].contiguous(), 8, 64)
        assert torch.equal(part.view(torch.int16), full[:, :n].view(torch.int16)), n
    for fmt in ("mxfp4", "nvfp4", "mxfp8"):
        c3 = workloads.mlp_up_case(fmt, 2, N=300)
        d3 = case_to_dev(c3)
        say(f"tail vs padded, {fmt}")
        full = run_qmv(bmv, c3, d3)
        for n in (1, 3, 5, 7, 8, 9, 12, 17):
            sub = dict(d3, w=d3["w"][:n].contiguous(), scales=d3["scales"][:n].contiguous())
            c_sub = workloads.QmvCase(c3.fmt, c3.dtype, c3.B, c3.K, n, c3.w[:n], c3.scales[:n],
                                      c3.x, global_scale=c3.global_scale)
            part = run_qmv(bmv, c_sub, sub)
            assert torch.equal(part.view(torch.int16), full[:, :n].view(torch.int16)), (fmt, n)


def test_chain_dependent(bmv):
    import torch
    c = workloads.chain_case(2560)
    d = case_to_dev(c)
    W = oracle.dequant_affine(c.w, c.scales, c.biases, c.K, 8, 64, "bf16")
    bufs = [d["x"].clone(), torch.empty_like(d["x"])]
    say("chain of 100")
    ys = []
    for t in range(100):
        bmv.qmv_affine(bufs[t % 2], d["w"], d["scales"], d["biases"], 8, 64, y=bufs[(t + 1) % 2])
        ys.append(bufs[(t + 1) % 2].clone())
    _sync()
    x_t = c.x
    norms = []
    for t in range(100):
        y_t = to_host(ys[t], "bf16")
        y64 = oracle.qmv(x_t, "bf16", W)
        check(y_t, y64, oracle.abs_dot(x_t, "bf16", W), "bf16", f"chain step {t}")
        norms.append(float(np.linalg.norm(oracle.storage_to_f64(y_t, "bf16"))))
        x_t = y_t
    # the weights preserve the norm in expectation: over 100 calls the chain
    # neither dies out nor blows up (repeated products drift toward the
    # largest eigen-direction, so allow a wide band)
    assert 0.05 * norms[0] < norms[-1] < 20 * norms[0], norms[::10]


# ---------------------------------------------------------------------------
# the MLP projection: K=4096, N=14336, MXFP4 / NVFP4 / MXFP8, B in {1, 4}
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "mxfp8"])
@pytest.mark.parametrize("B", [1, 4])
def test_mlp_up_sampled(bmv, fmt, B):
    c = workloads.mlp_up_case(fmt, B)
    say(f"{fmt} B{B} K4096 N14336")
    y = to_host(run_qmv(bmv, c), c.dtype)
    rows = sample_rows(c.N, 256, seed=B)
    y64, A = oracle_rows(c, rows)
    check(y[:, rows], y64, A, c.dtype, f"{fmt} B{B} K4096 N14336")


def test_block_scale_equivariance_bitwise(bmv):
    import torch
    c = workloads.mlp_up_case("mxfp4", 2, N=512)
    say("mxfp4 exponent +1 doubles y")
    y1 = run_qmv(bmv, c)
    c2 = workloads.QmvCase("mxfp4", c.dtype, c.B, c.K, c.N, c.w, (c.scales + 1).astype(np.uint8),
                           c.x)
    y2 = run_qmv(bmv, c2)
    assert torch.equal(y2.float(), 2 * y1.float())
    n = workloads.mlp_up_case("nvfp4", 2, N=512)
    say("nvfp4 global 0.5 vs 1.0")
    ya = run_qmv(bmv, workloads.QmvCase("nvfp4", n.dtype, n.B, n.K, n.N, n.w, n.scales, n.x,
                                        global_scale=1.0))
    yb = run_qmv(bmv, workloads.QmvCase("nvfp4", n.dtype, n.B, n.K, n.N, n.w, n.scales, n.x,
                                        global_scale=0.5))
    yc = run_qmv(bmv, workloads.QmvCase("nvfp4", n.dtype, n.B, n.K, n.N, n.w, n.scales, n.x,
                                        global_scale=None))
    assert torch.equal(yb.float(), 0.5 * ya.float())
    assert torch.equal(yc.view(torch.int16), ya.view(torch.int16))


# ---------------------------------------------------------------------------
# the affine sweep at full size (sampled rows)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("B", [1, 2, 4, 8])
@pytest.mark.parametrize("group", [32, 64, 128])
@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
def test_affine_sweep_sampled(bmv, bits, group, B, dtype):
    c = workloads.affine_sweep_case(bits, group, B, dtype)
    say(f"affine b{bits} g{group} B{B} {dtype} K=N=4096")
    y = to_host(run_qmv(bmv, c), dtype)
    rows = sample_rows(c.N, 48, seed=bits * 100 + group + B)
    y64, A = oracle_rows(c, rows)
    check(y[:, rows], y64, A, dtype, f"affine b{bits} g{group} B{B} {dtype} K=N=4096")


# the matrix cores take bf16 batches from B = 3 (MXFP4), 4 (NVFP4, MXFP8), and
# f16 batches from B = 5 (MXFP4), 7 (NVFP4, MXFP8)
MC_FIRST = {"mxfp4": 3, "nvfp4": 4, "mxfp8": 4}
MC_FIRST_F16 = {"mxfp4": 5, "nvfp4": 7, "mxfp8": 7}


def test_batch_rows_equal_single_row_calls_bitwise(bmv):
    # on the VALU tile and the one-row kernel: affine codes at any B, and the
    # block-scaled formats below the batch size where the matrix cores take
    # over (MC_FIRST, MC_FIRST_F16; tested below)
    import torch
    cases = [("affine", workloads.affine_sweep_case(3, 64, 8, "bf16", N=256))]
    for fmt in ("mxfp4", "nvfp4", "mxfp8"):
        cases.append((fmt, getattr(workloads, f"{fmt}_case")(73, f"batch-{fmt}-f16", K=4096,
                                                            N=256, B=MC_FIRST_F16[fmt] - 1,
                                                            dtype="f16")))
        cases.append((fmt, workloads.mlp_up_case(fmt, MC_FIRST[fmt] - 1, N=256)))
    for fmt, c in cases:
        d = case_to_dev(c)
        say(f"batch invariance {fmt} {c.dtype} B={c.B}")
        yb = run_qmv(bmv, c, d)
        for b in range(c.B):
            db = dict(d, x=d["x"][b:b + 1].contiguous())
            y1 = run_qmv(bmv, c, db)
            assert torch.equal(y1[0].view(torch.int16), yb[b].view(torch.int16)), (fmt, b)


# ---------------------------------------------------------------------------
# B = 3..8 with bf16 activations and block-scaled weights: the matrix-core QMV
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "mxfp8"])
@pytest.mark.parametrize("B", ["first", 6, 8])
def test_matrix_core_ragged(bmv, fmt, B):
    B = MC_FIRST[fmt] if B == "first" else B
    # K not a multiple of the 256 (FP4) / 128 (FP8) codes of a chunk (a
    # partial chunk at the end of every row), K below one chunk, N not a
    # multiple of the 32-row block, K long enough for several chunks per wave
    for K, N in ((1056, 301), (96, 70), (160, 33), (4096, 33), (8192, 40), (2560, 65)):
        c = workloads.mlp_up_case(fmt, B, K=K, N=N)
        say(f"matrix cores {fmt} B={B} K={K} N={N}")
        y = to_host(run_qmv(bmv, c), c.dtype)
        y64, A = oracle_rows(c, np.arange(N))
        check(y, y64, A, c.dtype, f"matrix cores {fmt} B={B} K={K} N={N}")


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "mxfp8"])
@pytest.mark.parametrize("B", [4, 8])
def test_matrix_core_full_size_sampled(bmv, fmt, B):
    c = workloads.mlp_up_case(fmt, B)
    say(f"matrix cores {fmt} B={B} K4096 N14336")
    y = to_host(run_qmv(bmv, c), c.dtype)
    rows = sample_rows(c.N, 128, seed=8)
    y64, A = oracle_rows(c, rows)
    check(y[:, rows], y64, A, c.dtype, f"matrix cores {fmt} B={B} K4096 N14336")


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "mxfp8"])
def test_matrix_core_bitwise_properties(bmv, fmt):
    # same bits on every call; each activation row's result independent of
    # the other rows (a permuted batch gives the permuted rows, and a row gives
    # the same bits in a batch of 3 as in a batch of 8); rows < n of a call on
    # the first n weight rows equal those of the full call
    import torch
    for K in (2048, 1056):
        c = workloads.mlp_up_case(fmt, 8, K=K, N=200)
        d = case_to_dev(c)
        say(f"matrix cores {fmt} K={K}: repeat, permutation, batch size, tail")
        y1 = run_qmv(bmv, c, d)
        y2 = run_qmv(bmv, c, d)
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
        perm = torch.tensor([5, 2, 7, 0, 1, 6, 3, 4], device=d["x"].device)
        yp = run_qmv(bmv, c, dict(d, x=d["x"][perm].contiguous()))
        assert torch.equal(yp.view(torch.int16), y1[perm].view(torch.int16))
        for sel in ([6, 1, 3, 0, 2], [2, 4, 7, 0, 5, 1]):
            idx = torch.tensor(sel, device=d["x"].device)
            c_sub = workloads.QmvCase(c.fmt, c.dtype, len(sel), c.K, c.N, c.w, c.scales, c.x,
                                      global_scale=c.global_scale)
            ys = run_qmv(bmv, c_sub, dict(d, x=d["x"][idx].contiguous()))
            assert torch.equal(ys.view(torch.int16), y1[idx].view(torch.int16)), sel
        for n in (1, 31, 33, 100):
            sub = dict(d, w=d["w"][:n].contiguous(), scales=d["scales"][:n].contiguous())
            c_sub = workloads.QmvCase(c.fmt, c.dtype, c.B, c.K, n, c.w[:n], c.scales[:n], c.x,
                                      global_scale=c.global_scale)
            part = run_qmv(bmv, c_sub, sub)
            assert torch.equal(part.view(torch.int16), y1[:, :n].view(torch.int16)), n


# ---------------------------------------------------------------------------
# f16 batches on the matrix cores: each activation row enters as two bf16
# columns, its head RN_bf16(x) and the exact remainder x - RN_bf16(x)
# ---------------------------------------------------------------------------

def _f16_case(fmt, B, K, N, key):
    # E8M0 exponents 116..126 keep MXFP8 outputs of K = 4096 rows inside f16
    if fmt == "nvfp4":
        return workloads.nvfp4_case(79, key, K=K, N=N, B=B, dtype="f16", global_scale=0.5)
    return getattr(workloads, f"{fmt}_case")(79, key, K=K, N=N, B=B, dtype="f16",
                                             exp_range=(116, 126))


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "mxfp8"])
@pytest.mark.parametrize("B", ["first", 8])
def test_matrix_core_f16_split(bmv, fmt, B):
    B = MC_FIRST_F16[fmt] if B == "first" else B
    # a partial last chunk, K below one chunk, ragged N, several chunks per
    # wave, and the row kernel's K values (which it hands on from these B)
    for K, N in ((1056, 301), (96, 70), (8192, 40), (4096, 65), (2048, 33)):
        c = _f16_case(fmt, B, K, N, f"mc16-{fmt}-{B}-{K}-{N}")
        say(f"matrix cores f16 {fmt} B={B} K={K} N={N}")
        y = to_host(run_qmv(bmv, c), "f16")
        y64, A = oracle_rows(c, np.arange(N))
        check(y, y64, A, "f16", f"matrix cores f16 {fmt} B={B} K={K} N={N}")


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "mxfp8"])
def test_matrix_core_f16_split_bitwise_properties(bmv, fmt):
    # a row's two columns depend on that row alone: a permuted batch gives the
    # permuted rows, a row gives the same bits in every batch size the matrix
    # cores take, and repeated calls give the same bits
    import torch
    c = _f16_case(fmt, 8, 2048, 200, f"mc16-bits-{fmt}")
    d = case_to_dev(c)
    say(f"matrix cores f16 {fmt}: repeat, permutation, batch size")
    y1 = run_qmv(bmv, c, d)
    assert torch.equal(y1.view(torch.int16), run_qmv(bmv, c, d).view(torch.int16))
    perm = torch.tensor([5, 2, 7, 0, 1, 6, 3, 4], device=d["x"].device)
    yp = run_qmv(bmv, c, dict(d, x=d["x"][perm].contiguous()))
    assert torch.equal(yp.view(torch.int16), y1[perm].view(torch.int16))
    sel = [6, 1, 3, 0, 2, 7, 4][:max(MC_FIRST_F16[fmt], 5)]
    idx = torch.tensor(sel, device=d["x"].device)
    c_sub = workloads.QmvCase(c.fmt, c.dtype, len(sel), c.K, c.N, c.w, c.scales, c.x,
                              global_scale=c.global_scale)
    ys = run_qmv(bmv, c_sub, dict(d, x=d["x"][idx].contiguous()))
    assert torch.equal(ys.view(torch.int16), y1[idx].view(torch.int16)), sel


def test_matrix_core_f16_split_extreme_activations(bmv):
    # activations whose remainders are the largest and smallest the split
    # sees: f16 values with all 10 fraction bits set (remainder 3 bits), the
    # largest finite f16 (65504 = 65536 - 32), subnormals and zeros
    K, N, B = 1024, 64, 8
    c = workloads.mxfp4_case(79, "mc16-extreme-x", K=K, N=N, B=B, dtype="f16",
                             exp_range=(100, 110))
    x = c.x.copy()
    xb = x.view(np.uint16)
    xb[0, :] = 0x3FFF                    # 1.9990234375
    xb[1, ::3] = 0x7BFF                  # 65504
    xb[2, :] = 0x0001                    # 2^-24, the smallest subnormal
    xb[3, ::2] = 0x83FF                  # -(the largest subnormal)
    xb[4, :] = 0
    c.x = x
    say("matrix cores f16: extreme activation values")
    y = to_host(run_qmv(bmv, c), "f16")
    y64, A = oracle_rows(c, np.arange(N))
    check(y, y64, A, "f16", "matrix cores f16 extreme activations")


def _extreme_scale_case(fmt, B, dtype="bf16"):
    """Rows whose scales sit at the ends of their code range: E8M0 0 (2^-127,
    whose products with the smaller E2M1 / E4M3 values are subnormal in
    bf16 and fp32), 1 and 2, and one block with the NaN code (255 for E8M0,
    0x7F for E4M3); NVFP4 rows also hold E4M3 block scales 0x00 (zero) and
    0x01 (2^-9). The other rows keep the workload's scales."""
    K, N = 1088, 40
    if fmt == "mxfp4":
        c = workloads.mxfp4_case(72, f"extreme-{fmt}-{B}-{dtype}", K=K, N=N, B=B, dtype=dtype)
    elif fmt == "mxfp8":
        c = workloads.mxfp8_case(72, f"extreme-{fmt}-{B}-{dtype}", K=K, N=N, B=B, dtype=dtype)
    else:
        c = workloads.nvfp4_case(72, f"extreme-{fmt}-{B}-{dtype}", K=K, N=N, B=B, dtype=dtype)
    sc = c.scales.copy()
    if fmt == "nvfp4":
        sc[0, :] = 0x01
        sc[1, ::2] = 0x00
        sc[2, :] = 0x08               # 2^-6, the smallest normal E4M3
        sc[3, 5] = 0x7F               # NaN block
        sc[4, :] = 0x7E               # 448, the largest
        nan_rows = [3]
    else:
        sc[0, :] = 0
        sc[1, :] = 1
        sc[2, ::2] = 2
        sc[3, 7] = 255                # NaN block
        sc[4, :] = np.where(np.arange(sc.shape[1]) % 2 == 0, 0, 130)
        nan_rows = [3]
    c.scales = sc
    return c, nan_rows


def _check_with_nan_rows(y, c, nan_rows, what):
    assert np.isnan(oracle.storage_to_f64(y[:, nan_rows], c.dtype)).all(), what
    keep = np.setdiff1d(np.arange(c.N), nan_rows)
    y64, A = oracle_rows(c, keep)
    check(y[:, keep], y64, A, c.dtype, what)


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "mxfp8"])
@pytest.mark.parametrize("B", [8, 1, 4])
def test_extreme_scale_codes(bmv, fmt, B):
    # B = 8 (bf16) runs on the matrix cores, B = 1 and 4 on the VALU tile;
    # both must decode the end codes of the scale formats as the oracle does
    c, nan_rows = _extreme_scale_case(fmt, B)
    say(f"extreme scale codes {fmt} B={B} K={c.K} N={c.N}")
    y = to_host(run_qmv(bmv, c), c.dtype)
    _check_with_nan_rows(y, c, nan_rows, f"extreme scales {fmt} B={B}")


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "mxfp8"])
@pytest.mark.parametrize("dtype,B", [("f32", 2), ("f16", 2), ("f16", 8)])
def test_extreme_scale_codes_other_dtypes(bmv, fmt, dtype, B):
    # f16 at B = 8: the matrix cores with the split activation operand
    c, nan_rows = _extreme_scale_case(fmt, B, dtype)
    say(f"extreme scale codes {fmt} B={B} {dtype}")
    # (f16 outputs of the 2^-127-scaled rows underflow to zeros and
    # subnormals; the 1-ulp bar, with the smallest subnormal as the ulp at
    # zero, still applies)
    y = to_host(run_qmv(bmv, c), c.dtype)
    _check_with_nan_rows(y, c, nan_rows, f"extreme scales {fmt} B={B} {dtype}")


# ---------------------------------------------------------------------------
# the MoE workload: routed-MoE gathered QMV
# ---------------------------------------------------------------------------

def _moe_dev(m):
    d = {"x": to_dev(m.x, m.dtype), "w": to_dev(m.w), "lhs": indices_dev(m.lhs),
         "rhs": indices_dev(m.rhs)}
    d["scales"] = to_dev(m.scales, m.dtype if m.fmt == "affine" else None)
    d["biases"] = to_dev(m.biases, m.dtype) if m.biases is not None else None
    return d


def _moe_weights(bmv, m, d):
    return bmv.make_weights(m.fmt, d["w"], d["scales"], d["biases"], K=m.K, bits=m.bits,
                            group_size=m.group)


@pytest.mark.parametrize("fmt", ["mxfp4", "affine"])
@pytest.mark.parametrize("proj", ["gate_up", "down"])
def test_moe_gather(bmv, fmt, proj):
    m = workloads.moe_case(fmt, proj)
    d = _moe_dev(m)
    say(f"MoE gather {fmt} {proj}")
    y = to_host(bmv.gather_qmv(d["x"], _moe_weights(bmv, m, d), d["lhs"], d["rhs"]), m.dtype)
    rows = sample_rows(m.N, 24, seed=5)
    for s in range(m.lhs.size):
        c = m.expert_case(int(m.rhs[s]))
        c.x = m.x[int(m.lhs[s])][None, :]
        c.B = 1
        y64, A = oracle_rows(c, rows)
        check(y[s:s + 1, rows], y64, A, m.dtype, f"gather {fmt} {proj} slot {s}")


@pytest.mark.parametrize("fmt", ["mxfp4", "affine"])
def test_gather_equals_single_calls_bitwise(bmv, fmt):
    import torch
    m = workloads.moe_case(fmt, "gate_up", E=16, hidden=1024, ffn=96, tokens=12, top_k=4)
    d = _moe_dev(m)
    say(f"gather vs single calls {fmt}")
    yg = bmv.gather_qmv(d["x"], _moe_weights(bmv, m, d), d["lhs"], d["rhs"])
    for s in range(m.lhs.size):
        e, r = int(m.rhs[s]), int(m.lhs[s])
        x1 = d["x"][r:r + 1].contiguous()
        if fmt == "affine":
            y1 = bmv.qmv_affine(x1, d["w"][e], d["scales"][e], d["biases"][e], 4, 64)
        else:
            y1 = bmv.qmv_fp_mxfp4(x1, d["w"][e], d["scales"][e])
        assert torch.equal(y1[0].view(torch.int16), yg[s].view(torch.int16)), s


def test_gather_out_of_range_rows_are_zero(bmv):
    import torch
    m = workloads.moe_case("mxfp4", "gate_up", E=8, hidden=512, ffn=64, tokens=5, top_k=3)
    m.rhs = m.rhs.copy()
    m.lhs = m.lhs.copy()
    m.rhs[2] = 8               # expert == n_experts
    m.rhs[4] = 0xFFFFFFFF      # far out of range
    m.lhs[6] = 5               # x row == n_x_rows
    d = _moe_dev(m)
    say("gather out-of-range indices")
    y = bmv.gather_qmv(d["x"], _moe_weights(bmv, m, d), d["lhs"], d["rhs"])
    yh = to_host(y, "bf16")
    Wd = lambda e: oracle.dequant_mxfp4(m.w[e], m.scales[e], m.K)
    y64 = oracle.gather_qmv(m.x, "bf16", m.lhs, m.rhs, m.E, m.N, Wd)
    for s in (2, 4, 6):
        assert not yh[s].any()
    A = np.zeros_like(y64)
    for s in range(m.lhs.size):
        if s in (2, 4, 6):
            continue
        A[s] = oracle.abs_dot(m.x[int(m.lhs[s])][None, :], "bf16", Wd(int(m.rhs[s])))[0]
    keep = [s for s in range(m.lhs.size) if s not in (2, 4, 6)]
    check(yh[keep], y64[keep], A[keep], "bf16", "gather with invalid slots")


def _moe_dev_any(m):
    d = _moe_dev(m)
    if m.fmt == "nvfp4" and m.global_scale is not None:
        import torch
        d["gscale"] = torch.tensor([m.global_scale], dtype=torch.float32, device="cuda:0")
    return d


def _single_call(bmv, m, d, e, x1):
    """One-row QMV of expert e through the plain entry point of its format."""
    if m.fmt == "affine":
        return bmv.qmv_affine(x1, d["w"][e], d["scales"][e], d["biases"][e], m.bits, m.group)
    if m.fmt == "mxfp4":
        return bmv.qmv_fp_mxfp4(x1, d["w"][e], d["scales"][e])
    if m.fmt == "nvfp4":
        return bmv.qmv_fp_nvfp4(x1, d["w"][e], d["scales"][e], d.get("gscale"))
    return bmv.qmv_fp_mxfp8(x1, d["w"][e], d["scales"][e])


def _gather_case_check(bmv, m, what, bad_slots=()):
    """gather_qmv on m: every valid slot against the oracle and bit for bit
    against a one-row call of its expert; slots in bad_slots (an index out
    of range) must be zero rows."""
    import torch
    d = _moe_dev_any(m)
    wt = bmv.make_weights(m.fmt, d["w"], d["scales"], d["biases"], K=m.K, bits=m.bits,
                          group_size=m.group, global_scale=d.get("gscale"))
    say(f"{what}: {m.fmt} {m.dtype} E={m.E} K={m.K} N={m.N} slots={m.lhs.size}")
    yg = bmv.gather_qmv(d["x"], wt, d["lhs"], d["rhs"])
    yh = to_host(yg, m.dtype)
    for s in range(m.lhs.size):
        if s in bad_slots:
            assert not np.any(yh[s]), s
            continue
        e, r = int(m.rhs[s]), int(m.lhs[s])
        c = m.expert_case(e)
        c.x = m.x[r][None, :]
        c.B = 1
        y64, A = oracle_rows(c, np.arange(m.N))
        check(yh[s:s + 1], y64, A, m.dtype, f"{what} slot {s}")
        y1 = _single_call(bmv, m, d, e, d["x"][r:r + 1].contiguous())
        a = y1[0].view(torch.int32 if m.dtype == "f32" else torch.int16)
        b = yg[s].view(torch.int32 if m.dtype == "f32" else torch.int16)
        assert torch.equal(a, b), f"{what}: slot {s} differs from the one-row call"


@pytest.mark.parametrize("fmt,gscale", [("nvfp4", 0.5), ("nvfp4", None), ("mxfp8", None),
                                        ("mxfp4", None), ("affine", None)])
@pytest.mark.parametrize("dtype", ["f16", "f32", "bf16"])
def test_gather_formats_and_dtypes(bmv, fmt, gscale, dtype):
    m = workloads.moe_case(fmt, "gate_up", E=8, hidden=1024, ffn=96, tokens=6, top_k=3,
                           dtype=dtype, global_scale=gscale)
    _gather_case_check(bmv, m, f"gather {fmt} g={gscale} {dtype}")


@pytest.mark.parametrize("fmt,dtype,K", [("mxfp4", "f32", 4096), ("nvfp4", "f32", 4096),
                                         ("affine", "f32", 4096), ("mxfp8", "bf16", 10240),
                                         ("mxfp4", "bf16", 10240), ("affine", "f16", 10240)])
def test_gather_multi_slab(bmv, fmt, dtype, K):
    # a chunk of two x rows of K values no longer fits the gather's LDS stage
    # (f32 K=4096: 32 KB of x plus the scales; 16-bit K=10240: 40 KB), so the
    # gather runs the tile slab by slab; out-of-range ids must still give
    # zero rows
    m = workloads.moe_case(fmt, "gate_up", E=6, hidden=K, ffn=70, tokens=5, top_k=2,
                           dtype=dtype)
    m.rhs = m.rhs.copy()
    m.lhs = m.lhs.copy()
    m.rhs[3] = m.E            # expert == n_experts
    m.lhs[7] = 5              # x row == n_x_rows
    _gather_case_check(bmv, m, f"gather multi-slab K={K}", bad_slots=(3, 7))


# ---------------------------------------------------------------------------
# layout, precision and edge cases
# ---------------------------------------------------------------------------

def test_one_hot_reads_each_weight(bmv):
    import torch
    c = workloads.affine_case(70, "onehot-gpu", bits=5, group=32, K=64, N=9, B=1, dtype="f32")
    d = case_to_dev(c)
    W = oracle.dequant_affine(c.w, c.scales, c.biases, 64, 5, 32, "f32")
    say("one-hot x, affine 5-bit")
    for k in range(64):
        x = torch.zeros((1, 64), dtype=torch.float32, device="cuda:0")
        x[0, k] = 1.0
        y = bmv.qmv_affine(x, d["w"], d["scales"], d["biases"], 5, 32).cpu().numpy()[0]
        # x = e_k: y[n] = s*q + b*1 computed in fp32, which is RN(s*q + b) up to
        # the fp32 fold; compare with the exact weight to 2 fp32 ulps
        assert np.allclose(y, W[:, k], rtol=2 ** -22, atol=0), k


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6])
def test_bias_sum_precision(bmv, dtype, bits):
    # one large and many small x in each group: summing x in the 16-bit type
    # before widening loses the small ones (mlx pull request 4516)
    # the small value lies below half an ulp of 1.0 in each type (bf16 2^-9,
    # f16 2^-12), so every 16-bit partial sum drops it
    K, N, group = 512, 16, 64
    rng = np.random.default_rng(bits)
    x64 = np.full((1, K), 2.0 ** -9 if dtype == "bf16" else 2.0 ** -12)
    x64[0, ::group] = 1.0
    w = rng.integers(0, 256, size=(N, K * bits // 8), dtype=np.uint8)
    s64 = np.full((N, K // group), 1e-3)
    b64 = np.full((N, K // group), 1.0)
    c = workloads.QmvCase("affine", dtype, 1, K, N, w, workloads.to_storage(s64, dtype),
                          workloads.to_storage(x64, dtype),
                          biases=workloads.to_storage(b64, dtype), bits=bits, group=group)
    _full_check(bmv, c, f"bias-sum precision b{bits} {dtype}")


def test_output_guard_bytes_untouched(bmv):
    import torch
    c = workloads.chain_case(17)
    d = case_to_dev(c)
    say("guard bytes around y")
    buf = torch.full((1, 17 + 64), -7.0, dtype=torch.bfloat16, device="cuda:0")
    y = buf[:, 32:32 + 17]
    out = torch.empty((1, 17), dtype=torch.bfloat16, device="cuda:0")
    bmv.qmv_affine(d["x"], d["w"], d["scales"], d["biases"], 8, 64, y=out)
    flat = buf.view(-1)
    flat_y = flat[32:32 + 17]
    bmv.qmv_affine(d["x"], d["w"], d["scales"], d["biases"], 8, 64, y=flat_y.view(1, 17))
    _sync()
    assert torch.all(flat[:32] == -7.0) and torch.all(flat[32 + 17:] == -7.0)
    assert torch.equal(flat_y.view(torch.int16), out[0].view(torch.int16))


def test_k_zero_gives_zeros_and_empty_calls(bmv):
    import torch
    say("K=0 / N=0 / B=0")
    x = torch.empty((2, 0), dtype=torch.bfloat16, device="cuda:0")
    w = torch.empty((5, 0), dtype=torch.uint8, device="cuda:0")
    s = torch.empty((5, 0), dtype=torch.bfloat16, device="cuda:0")
    y = torch.full((2, 5), 3.0, dtype=torch.bfloat16, device="cuda:0")
    bmv.qmv_affine(x, w, s, s, 4, 64, y=y)
    assert torch.all(y == 0)
    x2 = torch.randn((0, 64), device="cuda:0").to(torch.bfloat16)
    w2 = torch.zeros((5, 32), dtype=torch.uint8, device="cuda:0")
    s2 = torch.zeros((5, 1), dtype=torch.bfloat16, device="cuda:0")
    assert bmv.qmv_affine(x2, w2, s2, s2, 4, 64).shape == (0, 5)


def test_nan_scale_codes_give_nan_rows(bmv):
    import torch
    c = workloads.mxfp4_case(71, "nan-mx", K=256, N=8, B=1, dtype="f32")
    c.scales = c.scales.copy()
    c.scales[3, 2] = 255
    say("E8M0 255 -> NaN row")
    y = run_qmv(bmv, c).cpu().numpy()[0]
    assert np.isnan(y[3]) and np.isfinite(np.delete(y, 3)).all()
    n = workloads.nvfp4_case(71, "nan-nv", K=256, N=8, B=1, dtype="f32", global_scale=None)
    n.scales = n.scales.copy()
    n.scales[5, 1] = 0x7F
    say("E4M3 0x7F -> NaN row")
    y = run_qmv(bmv, n).cpu().numpy()[0]
    assert np.isnan(y[5]) and np.isfinite(np.delete(y, 5)).all()

"""GPU parity of the fused RMSNorm + QMV.

Primary target: the plain fp64 definition y = W . rmsnorm(x) (no rounding
anywhere), with the bound derived from the one rounding of the staged
activation (`check_fused_norm`). Extra check: this kernel stages
RN_T(x * gamma) and multiplies the row's fp32 result by r, so it must also
meet the plain QMV bar against r * (W . RN_T(x * gamma)) in fp64 (tighter,
and specific to that staging)."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import case_to_dev, check, check_fused_norm, sample_rows, say, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bmv():
    import bit_matrix_vector_amd as m
    m.load()
    return m


def _case(fmt, bits, group, B, K, N, dtype, key):
    if fmt == "affine":
        return workloads.affine_case(10, key, bits=bits, group=group, K=K, N=N, B=B, dtype=dtype)
    if fmt == "mxfp4":
        return workloads.mxfp4_case(10, key, K=K, N=N, B=B, dtype=dtype)
    if fmt == "nvfp4":
        return workloads.nvfp4_case(10, key, K=K, N=N, B=B, dtype=dtype)
    return workloads.mxfp8_case(10, key, K=K, N=N, B=B, dtype=dtype)


def _gamma(K, dtype, key):
    rng = workloads.rng_for(10, f"gamma-{key}")
    return workloads.to_storage(rng.uniform(0.5, 1.5, size=K), dtype)


def _run(bmv, c, gamma, eps, rows=None):
    d = case_to_dev(c)
    blk = {"affine": c.group, "mxfp4": 32, "nvfp4": 16, "mxfp8": 32}[c.fmt]
    wt = bmv.make_weights(c.fmt, d["w"], d["scales"], d.get("biases"), K=c.K, bits=c.bits,
                          group_size=blk, global_scale=d.get("gscale"))
    # x scaled away from unit RMS so the normalization matters
    x = workloads.to_storage(oracle.storage_to_f64(c.x, c.dtype) * 3.0, c.dtype)
    y = bmv.qmv_rmsnorm_qmv(to_dev(x, c.dtype), wt, to_dev(gamma, c.dtype), eps)
    rows = np.arange(c.N) if rows is None else rows
    W = oracle.dequant(c.fmt, c.K, c.w[rows], c.scales[rows],
                       None if c.biases is None else c.biases[rows], bits=c.bits, group=c.group,
                       dtype=c.dtype, global_scale=c.global_scale)
    # the plain definition, and the staged form of this kernel
    y_def = oracle.rmsnorm_qmv(x, c.dtype, gamma, eps, W)
    A_def = oracle.rmsnorm_qmv_abs(x, c.dtype, gamma, eps, W)
    xg = oracle.gamma_stored(x, c.dtype, gamma)
    r = oracle.rms_factor(x, c.dtype, eps)[:, None]
    return y, (y_def, A_def), (r * oracle.qmv(xg, c.dtype, W), r * oracle.abs_dot(xg, c.dtype, W))


def _check(y_host, plain, staged, dtype, what):
    check_fused_norm(y_host, plain[0], plain[1], dtype, what)
    check(y_host, staged[0], staged[1], dtype, what + " (staged form)")


CASES = ([("affine", b, 64) for b in (2, 3, 4, 8)] + [("affine", 4, 32), ("affine", 5, 128)] +
         [("mxfp4", 4, 32), ("nvfp4", 4, 16), ("mxfp8", 8, 32)])


@pytest.mark.parametrize("fmt,bits,group", CASES)
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_rmsnorm_qmv(bmv, fmt, bits, group, dtype):
    K = {32: 1056, 16: 1056, 64: 1088, 128: 1152}[group]
    for B, eps in ((1, 1e-6), (3, 1e-2)):
        key = f"{fmt}-{bits}-{group}-{dtype}-{B}"
        say(f"rmsnorm_qmv {key} B={B} N=300 K={K} eps={eps}")
        c = _case(fmt, bits, group, B, K, 300, dtype, key)
        gamma = _gamma(K, dtype, key)
        y, plain, staged = _run(bmv, c, gamma, eps)
        _check(to_host(y, dtype), plain, staged, dtype, f"rmsnorm_qmv {key}")


@pytest.mark.parametrize("fmt,bits,group,dtype",
                         [("mxfp4", 4, 32, "f32"), ("affine", 4, 64, "f32"),
                          ("mxfp8", 8, 32, "bf16")])
def test_rmsnorm_qmv_b8_multi_slab(bmv, fmt, bits, group, dtype):
    # B = 8 rows of K = 4096 exceed one LDS stage (f32: 128 KB), so x is
    # normalized slab by slab; gamma must follow each slab's offset
    key = f"slab-{fmt}-{dtype}"
    say(f"rmsnorm_qmv {key} B=8 K=4096 N=257")
    c = _case(fmt, bits, group, 8, 4096, 257, dtype, key)
    gamma = _gamma(4096, dtype, key)
    y, plain, staged = _run(bmv, c, gamma, 1e-5)
    _check(to_host(y, dtype), plain, staged, dtype, f"rmsnorm_qmv {key}")


def test_rmsnorm_qmv_full_size_sampled(bmv):
    say("rmsnorm_qmv mxfp4 bf16 B=1 K=4096 N=14336 sampled rows")
    c = _case("mxfp4", 4, 32, 1, 4096, 14336, "bf16", "full")
    gamma = _gamma(4096, "bf16", "full")
    rows = sample_rows(c.N)
    y, plain, staged = _run(bmv, c, gamma, 1e-6, rows=rows)
    _check(to_host(y, "bf16")[:, rows], plain, staged, "bf16", "rmsnorm_qmv full size")


def test_rmsnorm_qmv_unit_rms_equals_plain_qmv(bmv):
    # x = +-1 and eps = 0 make r exactly 1, so the fused call must equal the
    # plain QMV of RN_T(x * gamma) bit for bit (same staged values, same tile)
    import torch
    for fmt, bits, group in (("affine", 4, 64), ("mxfp4", 4, 32), ("nvfp4", 4, 16)):
        say(f"rmsnorm_qmv unit rms vs qmv {fmt} bf16 B=2 K=2048 N=512")
        c = _case(fmt, bits, group, 2, 2048, 512, "bf16", f"unit-{fmt}")
        signs = workloads.rng_for(10, f"signs-{fmt}").integers(0, 2, size=(2, 2048)) * 2 - 1
        x = workloads.to_storage(signs.astype(np.float64), "bf16")
        gamma = _gamma(2048, "bf16", f"unit-{fmt}")
        d = case_to_dev(c)
        blk = {"affine": c.group, "mxfp4": 32, "nvfp4": 16}[fmt]
        wt = bmv.make_weights(fmt, d["w"], d["scales"], d.get("biases"), K=c.K, bits=c.bits,
                              group_size=blk, global_scale=d.get("gscale"))
        y = bmv.qmv_rmsnorm_qmv(to_dev(x, "bf16"), wt, to_dev(gamma, "bf16"), 0.0)
        xg = to_dev(oracle.gamma_stored(x, "bf16", gamma), "bf16")
        if fmt == "affine":
            y0 = bmv.qmv_affine(xg, d["w"], d["scales"], d["biases"], 4, 64)
        elif fmt == "mxfp4":
            y0 = bmv.qmv_fp_mxfp4(xg, d["w"], d["scales"])
        else:
            y0 = bmv.qmv_fp_nvfp4(xg, d["w"], d["scales"], d["gscale"])
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y0.view(torch.int16)), fmt


def test_rmsnorm_qmv_k_zero(bmv):
    import torch
    say("rmsnorm_qmv K=0")
    wt = bmv.make_weights("mxfp4", torch.zeros((5, 0), dtype=torch.uint8, device="cuda:0"),
                          torch.zeros((5, 0), dtype=torch.uint8, device="cuda:0"), K=0)
    x = torch.zeros((2, 0), dtype=torch.bfloat16, device="cuda:0")
    g = torch.zeros((0,), dtype=torch.bfloat16, device="cuda:0")
    y = torch.full((2, 5), 7.0, dtype=torch.bfloat16, device="cuda:0")
    bmv.qmv_rmsnorm_qmv(x, wt, g, 1e-6, y=y)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0


# bf16 batches of the MX formats from the matrix-core threshold on (MXFP4 3,
# NVFP4 and MXFP8 4) run the fused norm on the matrix cores: whole chunks
# (K = 4096) and a partial last chunk (K = 1088), tail rows (N = 300)
@pytest.mark.parametrize("fmt,bits,group", [("mxfp4", 4, 32), ("nvfp4", 4, 16), ("mxfp8", 8, 32)])
@pytest.mark.parametrize("B", [4, 8])
@pytest.mark.parametrize("K", [4096, 1088])
def test_rmsnorm_qmv_matrix_cores(bmv, fmt, bits, group, B, K):
    key = f"mc-{fmt}-{B}-{K}"
    say(f"rmsnorm_qmv matrix cores {fmt} bf16 B={B} K={K} N=300")
    c = _case(fmt, bits, group, B, K, 300, "bf16", key)
    gamma = _gamma(K, "bf16", key)
    y, plain, staged = _run(bmv, c, gamma, 1e-6)
    _check(to_host(y, "bf16"), plain, staged, "bf16", f"rmsnorm_qmv {key}")


# f16 batches from B = 5 (MXFP4, NVFP4) or 6 (MXFP8) run the fused norm on the
# matrix cores too, the staged RN_f16(x * gamma) split into a bf16 head and its
# exact remainder; E8M0 exponents 114..124 keep the f16 outputs finite
@pytest.mark.parametrize("fmt,bits,group", [("mxfp4", 4, 32), ("nvfp4", 4, 16), ("mxfp8", 8, 32)])
@pytest.mark.parametrize("B", ["first", 8])
@pytest.mark.parametrize("K", [4096, 1088])
def test_rmsnorm_qmv_matrix_cores_f16(bmv, fmt, bits, group, B, K):
    B = {"mxfp4": 5, "nvfp4": 5, "mxfp8": 6}[fmt] if B == "first" else B
    key = f"mc16-{fmt}-{B}-{K}"
    say(f"rmsnorm_qmv matrix cores {fmt} f16 B={B} K={K} N=300")
    if fmt == "nvfp4":
        c = workloads.nvfp4_case(10, key, K=K, N=300, B=B, dtype="f16")
    else:
        c = getattr(workloads, f"{fmt}_case")(10, key, K=K, N=300, B=B, dtype="f16",
                                             exp_range=(114, 124))
    gamma = _gamma(K, "f16", key)
    y, plain, staged = _run(bmv, c, gamma, 1e-6)
    _check(to_host(y, "f16"), plain, staged, "f16", f"rmsnorm_qmv {key}")


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "mxfp8"])
def test_rmsnorm_qmv_matrix_cores_f16_unit_rms_equals_plain_qmv(bmv, fmt):
    # f16, B = 8: the fused and the plain call both split the same staged
    # values on the matrix cores, so with r exactly 1 they agree bit for bit
    import torch
    say(f"rmsnorm_qmv unit rms vs qmv {fmt} f16 B=8 K=4096 N=300 (matrix cores)")
    key = f"unit-mc16-{fmt}"
    if fmt == "nvfp4":
        c = workloads.nvfp4_case(10, key, K=4096, N=300, B=8, dtype="f16")
    else:
        c = getattr(workloads, f"{fmt}_case")(10, key, K=4096, N=300, B=8, dtype="f16",
                                             exp_range=(114, 124))
    signs = workloads.rng_for(10, f"signs-mc16-{fmt}").integers(0, 2, size=(8, 4096)) * 2 - 1
    x = workloads.to_storage(signs.astype(np.float64), "f16")
    gamma = _gamma(4096, "f16", key)
    d = case_to_dev(c)
    blk = {"mxfp4": 32, "nvfp4": 16, "mxfp8": 32}[fmt]
    wt = bmv.make_weights(fmt, d["w"], d["scales"], None, K=c.K, bits=c.bits, group_size=blk,
                          global_scale=d.get("gscale"))
    y = bmv.qmv_rmsnorm_qmv(to_dev(x, "f16"), wt, to_dev(gamma, "f16"), 0.0)
    xg = to_dev(oracle.gamma_stored(x, "f16", gamma), "f16")
    if fmt == "mxfp4":
        y0 = bmv.qmv_fp_mxfp4(xg, d["w"], d["scales"])
    elif fmt == "nvfp4":
        y0 = bmv.qmv_fp_nvfp4(xg, d["w"], d["scales"], d["gscale"])
    else:
        y0 = bmv.qmv_fp_mxfp8(xg, d["w"], d["scales"])
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y0.view(torch.int16)), fmt


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "mxfp8"])
def test_rmsnorm_qmv_matrix_cores_unit_rms_equals_plain_qmv(bmv, fmt):
    # as the VALU-tile case above, at B = 4: the fused and the plain call both
    # run on the matrix cores, in the same order, so with r exactly 1 they
    # must agree bit for bit
    import torch
    say(f"rmsnorm_qmv unit rms vs qmv {fmt} bf16 B=4 K=4096 N=300 (matrix cores)")
    c = _case(fmt, 4 if fmt != "mxfp8" else 8, {"mxfp4": 32, "nvfp4": 16, "mxfp8": 32}[fmt], 4,
              4096, 300, "bf16", f"unit-mc-{fmt}")
    signs = workloads.rng_for(10, f"signs-mc-{fmt}").integers(0, 2, size=(4, 4096)) * 2 - 1
    x = workloads.to_storage(signs.astype(np.float64), "bf16")
    gamma = _gamma(4096, "bf16", f"unit-mc-{fmt}")
    d = case_to_dev(c)
    blk = {"mxfp4": 32, "nvfp4": 16, "mxfp8": 32}[fmt]
    wt = bmv.make_weights(fmt, d["w"], d["scales"], None, K=c.K, bits=c.bits, group_size=blk,
                          global_scale=d.get("gscale"))
    y = bmv.qmv_rmsnorm_qmv(to_dev(x, "bf16"), wt, to_dev(gamma, "bf16"), 0.0)
    xg = to_dev(oracle.gamma_stored(x, "bf16", gamma), "bf16")
    if fmt == "mxfp4":
        y0 = bmv.qmv_fp_mxfp4(xg, d["w"], d["scales"])
    elif fmt == "nvfp4":
        y0 = bmv.qmv_fp_nvfp4(xg, d["w"], d["scales"], d["gscale"])
    else:
        y0 = bmv.qmv_fp_mxfp8(xg, d["w"], d["scales"])
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y0.view(torch.int16)), fmt

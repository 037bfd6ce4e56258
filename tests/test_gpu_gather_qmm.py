"""GPU parity of gather_qmm (the routed-expert product for many slots, on the
matrix cores) against the oracle's gathered product, with the QMV parity bar
per slot (A = sum_k |x[lhs[s], k] W[rhs[s]][n, k]|)."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import check, indices_dev, say, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bmv():
    import bit_matrix_vector_amd as m
    m.load()
    return m


def _stack(fmt, E, K, N, dtype, key):
    """Expert-stacked weights from E single-matrix cases."""
    cases = []
    for e in range(E):
        k = f"{key}-e{e}"
        if fmt == "affine":
            cases.append(workloads.affine_case(11, k, bits=4, group=64, K=K, N=N, B=1,
                                               dtype=dtype))
        elif fmt == "mxfp4":
            cases.append(workloads.mxfp4_case(11, k, K=K, N=N, B=1, dtype=dtype))
        elif fmt == "nvfp4":
            cases.append(workloads.nvfp4_case(11, k, K=K, N=N, B=1, dtype=dtype,
                                              global_scale=0.5))
        else:
            cases.append(workloads.mxfp8_case(11, k, K=K, N=N, B=1, dtype=dtype))
    w = np.stack([c.w for c in cases])
    sc = np.stack([c.scales for c in cases])
    bi = np.stack([c.biases for c in cases]) if fmt == "affine" else None
    return cases[0], w, sc, bi


def _routes(n_tokens, top_k, E, key, sort):
    rng = workloads.rng_for(11, f"routes-{key}")
    logits = rng.normal(size=(n_tokens, E))
    rhs = workloads.route_topk(logits, top_k).reshape(-1)
    lhs = np.arange(rhs.size) // top_k
    if sort:   # slots grouped by expert (stable), as a prefill dispatcher lays them out
        order = np.argsort(rhs, kind="stable")
        rhs, lhs = rhs[order], lhs[order]
    return lhs.astype(np.uint32), rhs.astype(np.uint32)


def _run_and_check(bmv, fmt, dtype, E, K, N, n_tokens, top_k, sort, key, tweak=None):
    c0, w, sc, bi = _stack(fmt, E, K, N, dtype, key)
    x = workloads.to_storage(workloads.rng_for(11, f"x-{key}").normal(size=(n_tokens, K)), dtype)
    lhs, rhs = _routes(n_tokens, top_k, E, key, sort)
    if tweak is not None:
        tweak(lhs, rhs)
    import torch
    dw = to_dev(w)
    dsc = to_dev(sc, dtype if fmt == "affine" else None)
    dbi = to_dev(bi, dtype) if bi is not None else None
    gs = (torch.tensor([c0.global_scale], dtype=torch.float32, device="cuda:0")
          if fmt == "nvfp4" else None)
    blk = {"affine": 64, "mxfp4": 32, "nvfp4": 16, "mxfp8": 32}[fmt]
    wt = bmv.make_weights(fmt, dw, dsc, dbi, K=K, bits=c0.bits, group_size=blk, global_scale=gs)
    y = bmv.gather_qmm(to_dev(x, dtype), wt, indices_dev(lhs), indices_dev(rhs))
    yh = to_host(y, dtype)

    def W(e):
        return oracle.dequant(fmt, K, w[e], sc[e], None if bi is None else bi[e], bits=c0.bits,
                              group=c0.group, dtype=dtype, global_scale=c0.global_scale)
    y64 = oracle.gather_qmv(x, dtype, lhs, rhs, E, N, W)
    A = np.zeros_like(y64)
    valid = []
    cache = {}
    for s in range(lhs.size):
        e, r = int(rhs[s]), int(lhs[s])
        if e >= E or r >= n_tokens:
            assert not yh[s].any(), f"slot {s}: out-of-range ids must give zeros"
            continue
        if e not in cache:
            cache[e] = W(e)
        A[s] = oracle.abs_dot(x[r][None, :], dtype, cache[e])[0]
        valid.append(s)
    check(yh[valid], y64[valid], A[valid], dtype, f"gather_qmm {key}")
    return yh


@pytest.mark.parametrize("fmt", ["affine", "mxfp4", "nvfp4", "mxfp8"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_gather_qmm_sorted(bmv, fmt, dtype):
    # 40 tokens x top-4 of 8 experts = 160 slots, grouped by expert
    key = f"sorted-{fmt}-{dtype}"
    say(f"gather_qmm {key} E=8 K=1088 N=300 slots=160")
    _run_and_check(bmv, fmt, dtype, 8, 1088, 300, 40, 4, True, key)


@pytest.mark.parametrize("fmt", ["affine", "mxfp4"])
def test_gather_qmm_unsorted(bmv, fmt):
    # token-major slot order: every tile mixes experts
    key = f"unsorted-{fmt}"
    say(f"gather_qmm {key} E=8 K=1024 N=257 slots=120")
    _run_and_check(bmv, fmt, "bf16", 8, 1024, 257, 30, 4, False, key)


def test_gather_qmm_out_of_range_rows_are_zero(bmv):
    def tweak(lhs, rhs):
        rhs[3] = 8              # expert == n_experts
        rhs[70] = 0xFFFFFFFF    # far out of range
        lhs[100] = 40           # x row == n_x_rows
    say("gather_qmm out-of-range ids")
    _run_and_check(bmv, "mxfp4", "bf16", 8, 1024, 200, 40, 4, True, "oor", tweak)


def test_gather_qmm_large_tiles(bmv):
    # 512 tokens x top-2 of 4 experts = 1024 slots (128-row tiles)
    key = "large"
    say("gather_qmm mxfp8 E=4 K=2048 N=2048 slots=1024")
    yh = _run_and_check(bmv, "mxfp8", "bf16", 4, 2048, 2048, 512, 2, True, key)
    assert np.isfinite(oracle.storage_to_f64(yh, "bf16")).all()


def test_gather_qmm_moe_shape(bmv):
    # the MoE workload's gate/up projection (64 experts, hidden 4096, ffn
    # 1536), 64 tokens x top-8, slots sorted by expert; sampled slots checked
    m = workloads.moe_case("mxfp4", "gate_up", tokens=64)
    order = np.argsort(m.rhs, kind="stable")
    lhs, rhs = m.lhs[order], m.rhs[order]
    say("gather_qmm MoE gate/up mxfp4 64 tokens top-8 sorted")
    dev = [to_dev(m.w), to_dev(m.scales)]   # kept alive while the struct is used
    wt = bmv.make_weights("mxfp4", dev[0], dev[1], None, K=m.K, bits=4, group_size=32)
    y = bmv.gather_qmm(to_dev(m.x, "bf16"), wt, indices_dev(lhs), indices_dev(rhs))
    yh = to_host(y, "bf16")
    rng = np.random.default_rng(0)
    slots = np.unique(np.concatenate([np.arange(4), np.arange(lhs.size - 4, lhs.size),
                                      rng.choice(lhs.size, 24, replace=False)]))
    for s in slots:
        e, r = int(rhs[s]), int(lhs[s])
        We = oracle.dequant_mxfp4(m.w[e], m.scales[e], m.K)
        y64 = oracle.qmv(m.x[r][None, :], "bf16", We)
        A = oracle.abs_dot(m.x[r][None, :], "bf16", We)
        check(yh[s:s + 1], y64, A, "bf16", f"MoE gather_qmm slot {s}")

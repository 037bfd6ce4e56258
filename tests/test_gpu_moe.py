"""GPU parity of the fused routed-MoE decode block against the oracle.

Stage 1 (gate/up + SwiGLU) is checked against the fp64 activation of the fp64
projections. The tolerance follows from the arithmetic: the projections carry
fp32 accumulation error (bounded by 2^-20 of sum|x*w|, a margin over the
2^-22 floor of the QMV checks), which the activation passes on through its
partial derivatives (d mid/dg = silu'(g) u, d mid/du = silu(g)); evaluating
silu and the product in fp32 adds a few fp32 ulps (2^-21 |mid|); then mid is
rounded to T (one ulp of T). Stage 2 (down, summed over a token's slots) is
checked on the mid rows the GPU produced, with the QMV parity bar."""

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


class Dev:
    """A MoeMatrix on the device and its qmv_weights_t (tensors kept alive)."""

    def __init__(self, bmv, c, m):
        import torch
        self.w = to_dev(m.w)
        self.s = to_dev(m.scales, c.dtype if c.fmt == "affine" else None)
        self.b = to_dev(m.biases, c.dtype) if m.biases is not None else None
        self.g = (torch.tensor([m.global_scale], dtype=torch.float32, device="cuda:0")
                  if m.global_scale is not None else None)
        blk = {"affine": c.group, "mxfp4": 32, "nvfp4": 16, "mxfp8": 32}[c.fmt]
        self.wt = bmv.make_weights(c.fmt, self.w, self.s, self.b, K=m.K, bits=c.bits,
                                   group_size=blk, global_scale=self.g)


def W_of(c, m):
    cache = {}

    def f(e):
        if e not in cache:
            cache[e] = oracle.dequant(c.fmt, m.K, m.w[e], m.scales[e],
                                      None if m.biases is None else m.biases[e], c.bits,
                                      c.group, c.dtype, m.global_scale)
        return cache[e]
    return f


def check_mid(c, mid_dev, clamp, slots=None):
    """Stage-1 bar (see module docstring) on all slots or the listed ones."""
    Wg, Wu = W_of(c, c.gate), W_of(c, c.up)
    ids = c.ids
    if slots is not None:
        toks = sorted({s // ids.shape[1] for s in slots})
        sub_x, sub_ids = c.x[toks], ids[toks]
    else:
        toks, sub_x, sub_ids = list(range(ids.shape[0])), c.x, ids
    g, u = oracle.gate_up_projections(sub_x, c.dtype, sub_ids, c.E, Wg, Wu)
    x64 = np.abs(oracle.storage_to_f64(sub_x, c.dtype))
    k = ids.shape[1]
    Ag = np.zeros_like(g)
    Au = np.zeros_like(u)
    for ti, t in enumerate(toks):
        for j in range(k):
            e = int(ids[t, j])
            if e < c.E:
                Ag[ti * k + j] = np.abs(Wg(e)) @ x64[ti]
                Au[ti * k + j] = np.abs(Wu(e)) @ x64[ti]
    mid = oracle.swiglu(g, u, clamp)
    mid[(sub_ids.reshape(-1) >= c.E)] = 0.0
    gc = np.minimum(g, clamp) if clamp > 1e-6 else g
    uc = np.clip(u, -clamp, clamp) if clamp > 1e-6 else u
    sig = 1.0 / (1.0 + np.exp(-np.clip(gc, -700, 700)))
    dsilu = sig * (1.0 + gc * (1.0 - sig))
    D = (np.abs(dsilu * uc) * 2.0 ** -20 * Ag + np.abs(oracle.silu(gc)) * 2.0 ** -20 * Au
         + 2.0 ** -21 * np.abs(mid))
    got_all = to_host(mid_dev, c.dtype)
    rows = [t * k + j for t in toks for j in range(k)]
    got = oracle.storage_to_f64(got_all[rows], c.dtype)
    if c.dtype == "f32":
        bad = np.abs(got - mid) > 1e-5 * np.abs(mid) + D
    else:
        r = oracle.round_f64_to(mid, c.dtype)
        bad = np.abs(got - oracle.storage_to_f64(r, c.dtype)) > oracle.ulp_of(r, c.dtype) + D
    assert not bad.any(), (f"mid: {int(bad.sum())} elements outside the bound; first "
                           f"{np.argwhere(bad)[:3].tolist()} got {got[bad][:3]} want {mid[bad][:3]}")
    return got_all


def run_block(bmv, c, clamp=0.0):
    import torch
    G, U, Dn = Dev(bmv, c, c.gate), Dev(bmv, c, c.up), Dev(bmv, c, c.down)
    x = to_dev(c.x, c.dtype)
    ids = indices_dev(c.ids).reshape(c.ids.shape)
    route = torch.from_numpy(c.route).to("cuda:0")
    mid = bmv.qmv_moe_gate_up_swiglu(x, G.wt, U.wt, ids, clamp)
    y = bmv.qmv_moe_down_reduce(mid, Dn.wt, ids, route)
    torch.cuda.synchronize()
    return mid, y, (G, U, Dn)


def check_y(c, mid_host, y_dev, toks=None):
    Wd = W_of(c, c.down)
    T, k = c.ids.shape
    toks = list(range(T)) if toks is None else toks
    rows = [t * k + j for t in toks for j in range(k)]
    y64, A = oracle.moe_down_reduce(mid_host[rows], c.dtype, c.ids[toks], c.route[toks], c.E, Wd)
    check(to_host(y_dev, c.dtype)[toks], y64, A, c.dtype, "moe down")


CASES = [("mxfp4", "bf16"), ("mxfp4", "f16"), ("mxfp4", "f32"), ("affine", "bf16"),
         ("affine", "f32"), ("nvfp4", "bf16")]


@pytest.mark.parametrize("fmt,dtype", CASES)
def test_moe_block_small(bmv, fmt, dtype):
    say(f"moe block {fmt} {dtype} E=8 hidden=1024 ffn=320 T=5 top3")
    c = workloads.moe_block_case(fmt, E=8, hidden=1024, ffn=320, tokens=5, top_k=3, dtype=dtype,
                                 key="small")
    mid, y, _ = run_block(bmv, c)
    mid_host = check_mid(c, mid, 0.0)
    check_y(c, mid_host, y)


def test_moe_block_clamp(bmv):
    say("moe block mxfp4 bf16 clamp 0.5")
    c = workloads.moe_block_case("mxfp4", E=8, hidden=1024, ffn=320, tokens=4, top_k=2,
                                 key="clamp")
    mid, y, _ = run_block(bmv, c, clamp=0.5)
    mid_host = check_mid(c, mid, 0.5)
    check_y(c, mid_host, y)


def test_moe_block_ragged_rows(bmv):
    # hidden and ffn that are not multiples of the row tiles
    say("moe block mxfp4 bf16 hidden=1056 ffn=352")
    c = workloads.moe_block_case("mxfp4", E=6, hidden=1056, ffn=352, tokens=3, top_k=4,
                                 key="ragged")
    mid, y, _ = run_block(bmv, c)
    mid_host = check_mid(c, mid, 0.0)
    check_y(c, mid_host, y)


def test_moe_block_out_of_range_ids(bmv):
    say("moe block mxfp4 bf16 with out-of-range expert ids")
    c = workloads.moe_block_case("mxfp4", E=8, hidden=512, ffn=256, tokens=4, top_k=3,
                                 key="oor")
    c.ids[1, 2] = 8
    c.ids[3, :] = 1000       # a token with no valid expert: y row must be 0
    mid, y, _ = run_block(bmv, c)
    mid_host = check_mid(c, mid, 0.0)
    assert not oracle.storage_to_f64(mid_host[1 * 3 + 2], "bf16").any()
    check_y(c, mid_host, y)
    assert not oracle.storage_to_f64(to_host(y, "bf16")[3], "bf16").any()


@pytest.mark.parametrize("fmt", ["mxfp4", "affine"])
def test_moe_block_full_size_sampled(bmv, fmt):
    # the MoE workload's block (64 experts, hidden 4096, ffn 1536, 16 tokens, top-8);
    # the oracle checks tokens 0, 7 and 15
    say(f"moe block {fmt} bf16 full size")
    c = workloads.moe_block_case(fmt, key="full")
    mid, y, _ = run_block(bmv, c)
    toks = [0, 7, 15]
    k = c.ids.shape[1]
    mid_host = check_mid(c, mid, 0.0, slots=[t * k for t in toks])
    check_y(c, mid_host, y, toks=toks)


def test_moe_down_top1_unit_weight_equals_qmv(bmv):
    # with one slot per token and router weight 1 the down step is a plain QMV
    # of that slot's expert: same lanes, units and reduction, so bit for bit
    import torch
    say("moe down top-1, weight 1 vs qmv_fp_mxfp4")
    c = workloads.moe_block_case("mxfp4", E=4, hidden=2048, ffn=1536, tokens=3, top_k=1,
                                 key="top1")
    Dn = Dev(bmv, c, c.down)
    mid = to_dev(workloads.to_storage(np.random.default_rng(5).normal(size=(3, 1536)), "bf16"),
                 "bf16")
    ids = indices_dev(c.ids).reshape(c.ids.shape)
    ones = torch.ones((3, 1), dtype=torch.float32, device="cuda:0")
    y = bmv.qmv_moe_down_reduce(mid, Dn.wt, ids, ones)
    for t in range(3):
        e = int(c.ids[t, 0])
        ref = bmv.qmv_fp_mxfp4(mid[t:t + 1], Dn.w[e], Dn.s[e])
        assert torch.equal(y[t:t + 1].view(torch.int16), ref.view(torch.int16))


def test_moe_gate_up_zero_k(bmv):
    import torch
    say("moe gate/up K=0")
    G = bmv.QmvWeights(bmv.QMV_MXFP4, 4, 32, 4, 64, 0, None, None, None, None)
    x = torch.empty((2, 0), dtype=torch.bfloat16, device="cuda:0")
    ids = torch.zeros((2, 2), dtype=torch.int32, device="cuda:0")
    mid = torch.full((4, 64), 7.0, dtype=torch.bfloat16, device="cuda:0")
    bmv.qmv_moe_gate_up_swiglu(x, G, G, ids, 0.0, mid=mid)
    assert not mid.float().abs().sum().item()

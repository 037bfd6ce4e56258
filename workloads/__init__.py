"""Seeded synthetic inputs for the QMV workloads (NumPy, host memory).

Shared by the tests, the benchmark and the smoke check. This module holds no
part of the product's arithmetic: it draws random bytes and values and stores
them in the input dtypes, nothing more. Packed weight codes are drawn as
uniform random bytes, which makes every code of any width 2..8 uniform over
{0 .. 2^b - 1} without any packing step (each code is a bit field of a
uniform random bit stream).

Every draw comes from np.random.default_rng(SeedSequence([cfg_id,
crc32(case_key)])) in the fixed order codes -> scales -> biases -> x, so a case
is reproducible from its (cfg_id, key) alone.

Workloads (shapes and value distributions):
  cfg 1  affine 4-bit, group 64, K=512, N=256, B=1, f32 x ~ N(0,1);
         q uniform, scales ~ U(0.01, 0.1), bias = -8*scale + U(-0.01, 0.01)
  cfg 2  affine 8-bit, group 64, K=2560, bf16 x ~ N(0,1), N=2560 plus tails
         N in {1,3,5,12,17}; norm-preserving scales for a 100-call chain
  cfg 3  block-scaled, bf16 x ~ N(0,1), K=4096, N=14336, B in {1,4}:
         MXFP4 (E2M1 codes uniform, E8M0 exponents uniform 120..130),
         NVFP4 (E4M3 block scales ~ |N(0,1)|, fp32 global scale 0.5),
         MXFP8 (E4M3 codes uniform over the 254 finite bytes, E8M0 120..130)
  cfg 4  affine sweep: bits {2,3,4,5,6,8} x group {32,64,128}, K=N=4096,
         B {1,2,4,8}, x dtype {f32,f16,bf16}; scales ~ U(0.005, 0.05),
         biases ~ N(0, 0.05)
  cfg 5  routed MoE: 64 experts, hidden 4096, expert FFN 1536 (gate/up
         4096->1536, down 1536->4096), MXFP4 and 4-bit affine g64; 16 tokens,
         top-8 experts per token from N(0,1) router logits; bf16 x
"""

from __future__ import annotations

import zlib
from dataclasses import dataclass, field

import numpy as np

DTYPES = ("f32", "f16", "bf16")
AFFINE_BITS = (2, 3, 4, 5, 6, 8)
AFFINE_GROUPS = (32, 64, 128)


def rng_for(cfg_id: int, case_key: str) -> np.random.Generator:
    seq = np.random.SeedSequence([int(cfg_id), zlib.crc32(case_key.encode())])
    return np.random.default_rng(seq)


# ---------------------------------------------------------------------------
# storing drawn fp64 values in the input dtypes
# ---------------------------------------------------------------------------

def to_storage(v64: np.ndarray, dtype: str) -> np.ndarray:
    """Store fp64 draws as T. f32 / f16 use NumPy's casts; bf16 is returned as
    uint16 bit patterns, rounded to nearest-even from the fp32 pattern (these
    are random inputs, so the path they take to a bf16 value is immaterial)."""
    v64 = np.asarray(v64, dtype=np.float64)
    if dtype == "f32":
        return v64.astype(np.float32)
    if dtype == "f16":
        return v64.astype(np.float16)
    if dtype == "bf16":
        u = v64.astype(np.float32).view(np.uint32).astype(np.uint64)
        u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
        return u.astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def storage_nbytes(dtype: str) -> int:
    return {"f32": 4, "f16": 2, "bf16": 2}[dtype]


def _e4m3_byte_for(v: np.ndarray) -> np.ndarray:
    """Pick the E4M3 byte for non-negative draws v (used only to draw NVFP4
    block scales): round to nearest-even on the 3-bit-mantissa grid, saturating
    at 448; draws below 2^-10 become 0."""
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros(v.shape, dtype=np.uint8)
    big = v >= 448.0
    sub = (v < 2.0 ** -6) & ~big
    nrm = ~big & ~sub
    out[big] = 0x7E
    out[sub] = np.rint(v[sub] * 2.0 ** 9).astype(np.uint8)      # 0..8 (8 = 2^-6)
    _, ex = np.frexp(v[nrm])
    e = ex.astype(np.int64) - 1
    m = np.rint((v[nrm] / np.ldexp(1.0, e.astype(np.int32)) - 1.0) * 8.0).astype(np.int64)
    e = np.where(m == 8, e + 1, e)
    m = np.where(m == 8, 0, m)
    code = np.minimum(((e + 7) << 3) | m, 0x7E)
    out[nrm] = code.astype(np.uint8)
    return out


# ---------------------------------------------------------------------------
# case containers
# ---------------------------------------------------------------------------

@dataclass
class QmvCase:
    """One QMV problem in host memory. `fmt` is 'affine' | 'mxfp4' | 'nvfp4' |
    'mxfp8'; `x` [B, K] and affine `scales`/`biases` are stored in `dtype`;
    block scales are uint8; `global_scale` is a Python float or None."""
    fmt: str
    dtype: str
    B: int
    K: int
    N: int
    w: np.ndarray
    scales: np.ndarray
    x: np.ndarray
    biases: np.ndarray | None = None
    bits: int = 4
    group: int = 32
    global_scale: float | None = None
    key: str = ""
    meta: dict = field(default_factory=dict)

    def algorithmic_bytes(self) -> int:
        """Bytes one call must move: packed weights + scales (+ biases) + x
        read + y written."""
        t = storage_nbytes(self.dtype)
        n = self.w.nbytes + self.scales.nbytes
        if self.biases is not None:
            n += self.biases.nbytes
        return n + self.B * self.K * t + self.B * self.N * t


def affine_case(cfg_id: int, key: str, *, bits: int, group: int, K: int, N: int, B: int,
                dtype: str, scale_range=(0.005, 0.05), bias_mode: str = "normal",
                bias_sigma: float = 0.05) -> QmvCase:
    """Affine problem. bias_mode: 'normal' (biases ~ N(0, bias_sigma)),
    'centred8' (bias = -8*scale + U(-0.01, 0.01), with the stored scale), or
    'chain' (weights for a dependent chain of calls: scale = s0*U(0.5, 1.5),
    bias = -127.5*scale + scale*U(-0.5, 0.5), so w = scale*(q - 127.5 + u)
    has mean square scale^2 * (Var(q) + 1/12) = scale^2 * 73.9^2 for 8-bit q;
    s0 = 1 / (73.9 * sqrt(K * 13/12)) makes E[w^2] = 1/K, i.e. each call
    preserves the norm of x in expectation (13/12 = E[U(0.5, 1.5)^2]))."""
    rng = rng_for(cfg_id, key)
    w = rng.integers(0, 256, size=(N, K * bits // 8), dtype=np.uint8)
    G = K // group
    if bias_mode == "chain":
        s0 = 1.0 / (73.9 * np.sqrt(K * 13.0 / 12.0))
        s64 = s0 * rng.uniform(0.5, 1.5, size=(N, G))
    else:
        s64 = rng.uniform(scale_range[0], scale_range[1], size=(N, G))
    scales = to_storage(s64, dtype)
    if bias_mode == "normal":
        b64 = rng.normal(0.0, bias_sigma, size=(N, G))
    elif bias_mode == "centred8":
        s_stored = _stored_f64(scales, dtype)
        b64 = -8.0 * s_stored + rng.uniform(-0.01, 0.01, size=(N, G))
    elif bias_mode == "chain":
        s_stored = _stored_f64(scales, dtype)
        b64 = -127.5 * s_stored + s_stored * rng.uniform(-0.5, 0.5, size=(N, G))
    else:
        raise ValueError(bias_mode)
    biases = to_storage(b64, dtype)
    x = to_storage(rng.normal(0.0, 1.0, size=(B, K)), dtype)
    return QmvCase("affine", dtype, B, K, N, w, scales, x, biases=biases, bits=bits,
                   group=group, key=key)


def _stored_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def mxfp4_case(cfg_id: int, key: str, *, K: int, N: int, B: int, dtype: str = "bf16",
               exp_range=(120, 130)) -> QmvCase:
    rng = rng_for(cfg_id, key)
    w = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(exp_range[0], exp_range[1] + 1, size=(N, K // 32), dtype=np.uint8)
    x = to_storage(rng.normal(0.0, 1.0, size=(B, K)), dtype)
    return QmvCase("mxfp4", dtype, B, K, N, w, scales, x, key=key)


def nvfp4_case(cfg_id: int, key: str, *, K: int, N: int, B: int, dtype: str = "bf16",
               global_scale: float | None = 0.5) -> QmvCase:
    rng = rng_for(cfg_id, key)
    w = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = _e4m3_byte_for(np.abs(rng.normal(0.0, 1.0, size=(N, K // 16))))
    x = to_storage(rng.normal(0.0, 1.0, size=(B, K)), dtype)
    return QmvCase("nvfp4", dtype, B, K, N, w, scales, x, global_scale=global_scale, key=key)


def mxfp8_case(cfg_id: int, key: str, *, K: int, N: int, B: int, dtype: str = "bf16",
               exp_range=(120, 130)) -> QmvCase:
    rng = rng_for(cfg_id, key)
    # uniform over the 254 finite E4M3 bytes: skip 0x7F and 0xFF
    r = rng.integers(0, 254, size=(N, K), dtype=np.int64)
    w = (r + (r >= 0x7F)).astype(np.uint8)
    scales = rng.integers(exp_range[0], exp_range[1] + 1, size=(N, K // 32), dtype=np.uint8)
    x = to_storage(rng.normal(0.0, 1.0, size=(B, K)), dtype)
    return QmvCase("mxfp8", dtype, B, K, N, w, scales, x, key=key)


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def small_affine_case() -> QmvCase:
    """Affine 4-bit g64, K=512, N=256, one f32 activation row."""
    return affine_case(1, "c1", bits=4, group=64, K=512, N=256, B=1, dtype="f32",
                       scale_range=(0.01, 0.1), bias_mode="centred8")


CHAIN_TAILS = (1, 3, 5, 12, 17)


def chain_case(N: int = 2560) -> QmvCase:
    """Affine 8-bit g64, K=2560, bf16: the decode-chain matrix (N=2560, or a
    narrow tail N), with norm-preserving weights so 100 chained calls stay finite."""
    return affine_case(2, f"c2-N{N}", bits=8, group=64, K=2560, N=N, B=1, dtype="bf16",
                       bias_mode="chain")


def mlp_up_case(fmt: str, B: int, K: int = 4096, N: int = 14336) -> QmvCase:
    """An MLP up projection (K=4096, N=14336) in MXFP4, NVFP4 (global 0.5) or
    MXFP8, B bf16 activation rows."""
    key = f"c3-{fmt}-B{B}"
    if fmt == "mxfp4":
        return mxfp4_case(3, key, K=K, N=N, B=B)
    if fmt == "nvfp4":
        return nvfp4_case(3, key, K=K, N=N, B=B, global_scale=0.5)
    if fmt == "mxfp8":
        return mxfp8_case(3, key, K=K, N=N, B=B)
    raise ValueError(fmt)


def affine_sweep_case(bits: int, group: int, B: int, dtype: str, K: int = 4096,
                      N: int = 4096) -> QmvCase:
    """One point of the affine sweep: bits x group x B x activation dtype at K=N=4096."""
    return affine_case(4, f"c4-b{bits}-g{group}-B{B}-{dtype}", bits=bits, group=group, K=K,
                       N=N, B=B, dtype=dtype)


@dataclass
class MoeCase:
    """Routed-MoE gathered QMV inputs for one projection. Weights are
    expert-stacked: w [E, N, row_bytes], scales [E, N, K/block] (+ biases)."""
    fmt: str
    dtype: str
    E: int
    K: int
    N: int
    w: np.ndarray
    scales: np.ndarray
    x: np.ndarray                 # [n_x_rows, K]
    lhs: np.ndarray               # [n_slots] uint32: x row per slot
    rhs: np.ndarray               # [n_slots] uint32: expert per slot
    biases: np.ndarray | None = None
    bits: int = 4
    group: int = 64
    key: str = ""
    global_scale: float | None = None   # NVFP4: one fp32 scale shared by all experts

    def expert_case(self, e: int) -> QmvCase:
        """Expert e's matrix as a QMV problem with x rows all of x."""
        return QmvCase(self.fmt, self.dtype, self.x.shape[0], self.K, self.N, self.w[e],
                       self.scales[e], self.x,
                       biases=None if self.biases is None else self.biases[e],
                       bits=self.bits, group=self.group, global_scale=self.global_scale,
                       key=f"{self.key}-e{e}")

    def distinct_experts(self) -> np.ndarray:
        r = self.rhs.astype(np.int64)
        return np.unique(r[(r >= 0) & (r < self.E)])

    def algorithmic_bytes(self) -> int:
        """Weights of the distinct experts used (each read once) + x rows read
        per slot + y written + both index arrays."""
        t = storage_nbytes(self.dtype)
        d = len(self.distinct_experts())
        per = self.w[0].nbytes + self.scales[0].nbytes
        if self.biases is not None:
            per += self.biases[0].nbytes
        ns = self.lhs.shape[0]
        return d * per + ns * self.K * t + ns * self.N * t + 8 * ns


def route_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """Top-k expert ids per token by descending logit (softmax is monotone, so
    ranking the logits ranks the router probabilities); ties go to the lower
    expert index. Returns [tokens, k] int64."""
    order = np.argsort(-logits, axis=1, kind="stable")
    return order[:, :k]


def moe_case(fmt: str, proj: str, *, E: int = 64, hidden: int = 4096, ffn: int = 1536,
             tokens: int = 16, top_k: int = 8, dtype: str = "bf16",
             global_scale: float | None = 0.5) -> MoeCase:
    """proj 'gate_up': K=hidden, N=ffn, x = token activations [tokens, hidden],
    slot s = (token s // top_k, its (s % top_k)-th expert). proj 'down':
    K=ffn, N=hidden, x = per-slot hidden states [tokens*top_k, ffn] ~ N(0,1),
    lhs[s] = s. The routing (router logits ~ N(0,1), top_k) is drawn from its
    own stream so both projections share it. Formats: 'mxfp4' and 'affine'
    (4-bit g64) as the MoE workload states, and for wider parity coverage
    'nvfp4' (E4M3 |N(0,1)| block scales, `global_scale`) and 'mxfp8' (finite
    E4M3 codes, E8M0 120..130), drawn like the MLP projection's weights."""
    route_rng = rng_for(5, "c5-router")
    logits = route_rng.normal(0.0, 1.0, size=(tokens, E))
    experts = route_topk(logits, top_k)                      # [tokens, top_k]
    rhs = experts.reshape(-1).astype(np.uint32)
    n_slots = tokens * top_k
    if proj == "gate_up":
        K, N = hidden, ffn
        lhs = (np.arange(n_slots) // top_k).astype(np.uint32)
        n_x = tokens
    elif proj == "down":
        K, N = ffn, hidden
        lhs = np.arange(n_slots, dtype=np.uint32)
        n_x = n_slots
    else:
        raise ValueError(proj)
    key = f"c5-{fmt}-{proj}"
    rng = rng_for(5, key)
    if fmt == "mxfp4":
        w = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
        scales = rng.integers(120, 131, size=(E, N, K // 32), dtype=np.uint8)
        biases = None
        bits, group = 4, 32
    elif fmt == "affine":
        bits, group = 4, 64
        w = rng.integers(0, 256, size=(E, N, K * bits // 8), dtype=np.uint8)
        scales = to_storage(rng.uniform(0.005, 0.05, size=(E, N, K // group)), dtype)
        biases = to_storage(rng.normal(0.0, 0.05, size=(E, N, K // group)), dtype)
    elif fmt == "nvfp4":
        w = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
        scales = _e4m3_byte_for(np.abs(rng.normal(0.0, 1.0, size=(E, N, K // 16))))
        biases = None
        bits, group = 4, 16
    elif fmt == "mxfp8":
        r = rng.integers(0, 254, size=(E, N, K), dtype=np.int64)   # the 254 finite bytes
        w = (r + (r >= 0x7F)).astype(np.uint8)
        scales = rng.integers(120, 131, size=(E, N, K // 32), dtype=np.uint8)
        biases = None
        bits, group = 8, 32
    else:
        raise ValueError(fmt)
    x = to_storage(rng.normal(0.0, 1.0, size=(n_x, K)), dtype)
    return MoeCase(fmt, dtype, E, K, N, w, scales, x, lhs, rhs, biases=biases, bits=bits,
                   group=group, key=key, global_scale=global_scale if fmt == "nvfp4" else None)


# ---------------------------------------------------------------------------
# Quantize-from-float inputs: float weight matrices [N, K] in T.
# ---------------------------------------------------------------------------
def quant_weights(cfg_id: int, key: str, N: int, K: int, dtype: str = "bf16",
                  special_rows: bool = True) -> np.ndarray:
    """Weights ~ N(0, sigma_n^2) with a log-normal spread of row scales
    (sigma_n = 0.02 * exp(N(0, 1))), stored in T. With special_rows the first
    rows (when N allows) are, in order: a constant row; an all-zero row with
    signed zeros; a row of midpoints between neighbouring E2M1 values in blocks
    whose largest magnitude is 6; the same for E4M3 with 448; a row whose
    groups span [0, 3] with values k + 0.5 (midpoints of a unit step); and a
    row of magnitudes near 2^-130 (fp32 subnormals)."""
    rng = rng_for(cfg_id, key)
    sig = 0.02 * np.exp(rng.normal(0.0, 1.0, size=(N, 1)))
    w = rng.normal(0.0, 1.0, size=(N, K)) * sig
    if special_rows and K >= 32:
        rows = []
        rows.append(np.full(K, 0.3125))
        z = np.zeros(K)
        z[1::2] = -0.0
        rows.append(z)
        mids_e2m1 = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -5.0])
        r = np.resize(mids_e2m1, K)
        r[::32] = 6.0
        rows.append(r)
        mids_e4m3 = np.array([1.0625, 2.125, 0.015625 * 1.5, 2.0 ** -10, 3.0 * 2.0 ** -10,
                              -1.0625, 300.0, 432.0])
        r = np.resize(mids_e4m3, K)
        r[::32] = 448.0
        rows.append(r)
        r = np.resize(np.array([0.0, 3.0, 0.5, 1.5, 2.5, 1.0, 2.0]), K)
        rows.append(r)
        rows.append(rng.normal(0.0, 1.0, size=K) * 2.0 ** -130)
        for i, r in enumerate(rows[:N]):
            w[i] = r
    return to_storage(w, dtype)


# ---------------------------------------------------------------------------
# Fused routed-MoE decode block inputs.
# ---------------------------------------------------------------------------
@dataclass
class MoeMatrix:
    """One expert-stacked projection: w [E, N, row_bytes], scales [E, N, K/blk]
    (+ biases for affine, + an fp32 global scale for NVFP4)."""
    N: int
    K: int
    w: np.ndarray
    scales: np.ndarray
    biases: np.ndarray | None = None
    global_scale: float | None = None


@dataclass
class MoeBlockCase:
    fmt: str
    dtype: str
    E: int
    hidden: int
    ffn: int
    x: np.ndarray          # [tokens, hidden] T
    ids: np.ndarray        # [tokens, top_k] uint32
    route: np.ndarray      # [tokens, top_k] float32
    gate: MoeMatrix
    up: MoeMatrix
    down: MoeMatrix
    bits: int = 4
    group: int = 64

    def matrix_bytes(self, m: MoeMatrix) -> int:
        per = m.w[0].nbytes + m.scales[0].nbytes + (0 if m.biases is None else m.biases[0].nbytes)
        return per


def _moe_matrix(rng, fmt: str, E: int, N: int, K: int, dtype: str, bits: int, group: int,
                gs: float) -> MoeMatrix:
    """Expert weights for the fused-block cases, sized so that projections of
    x ~ N(0, 1) land near 1 (where silu is curved): MXFP4 E8M0 exponents
    116..122; affine scales U(0.001, 0.01) with biases -7.5 s + N(0, s);
    NVFP4 block scales |N(0, 0.03)| as E4M3 with the given global scale."""
    if fmt == "mxfp4":
        w = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
        sc = rng.integers(116, 123, size=(E, N, K // 32), dtype=np.uint8)
        return MoeMatrix(N, K, w, sc)
    if fmt == "nvfp4":
        w = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
        sc = _e4m3_byte_for(np.abs(rng.normal(0.0, 0.03, size=(E, N, K // 16))) / gs)
        return MoeMatrix(N, K, w, sc, global_scale=gs)
    if fmt == "affine":
        w = rng.integers(0, 256, size=(E, N, K * bits // 8), dtype=np.uint8)
        s = rng.uniform(0.001, 0.01, size=(E, N, K // group))
        b = -7.5 * s + s * rng.normal(0.0, 1.0, size=s.shape)
        return MoeMatrix(N, K, w, to_storage(s, dtype), to_storage(b, dtype))
    raise ValueError(fmt)


def moe_block_case(fmt: str, *, E: int = 64, hidden: int = 4096, ffn: int = 1536,
                   tokens: int = 16, top_k: int = 8, dtype: str = "bf16", key: str = "",
                   bits: int = 4, group: int = 64) -> MoeBlockCase:
    """The routed-MoE block of the MoE workload (64 experts, hidden 4096, ffn 1536,
    16 tokens, top-8) with separate gate / up / down stacks. Routing: logits
    ~ N(0, 1) [tokens, E], top_k by logit, router weights = softmax of the
    selected logits (renormalised over the top_k, fp64, stored fp32)."""
    rng = rng_for(6, f"moe-block-{fmt}-{dtype}-{key}")
    logits = rng.normal(0.0, 1.0, size=(tokens, E))
    ids = route_topk(logits, top_k)
    sel = np.take_along_axis(logits, ids, axis=1)
    ex = np.exp(sel - sel.max(axis=1, keepdims=True))
    route = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)
    gate = _moe_matrix(rng, fmt, E, ffn, hidden, dtype, bits, group, 0.5)
    up = _moe_matrix(rng, fmt, E, ffn, hidden, dtype, bits, group, 0.25)
    down = _moe_matrix(rng, fmt, E, hidden, ffn, dtype, bits, group, 0.5)
    x = to_storage(rng.normal(0.0, 1.0, size=(tokens, hidden)), dtype)
    return MoeBlockCase(fmt, dtype, E, hidden, ffn, x, ids.astype(np.uint32), route, gate, up,
                        down, bits, group)


# ---------------------------------------------------------------------------
# The other Track-1 block-scaled formats (symmetric: element x block scale).
# ---------------------------------------------------------------------------
SB_FORMATS = {  # name -> (element, block, scale storage); as in the audit's table
    "mxfp8_e5m2": ("e5m2", 32, "e8m0"), "nvfp8": ("e4m3", 16, "f32"),
    "fp4": ("e2m1", 32, "f32"), "fp8_e4m3": ("e4m3", 32, "f32"),
    "fp8_e5m2": ("e5m2", 32, "f32"), "nvfp8_f16": ("e4m3", 16, "f16"),
    "fp4_f16": ("e2m1", 32, "f16"), "fp8_e4m3_f16": ("e4m3", 32, "f16"),
    "fp8_e5m2_f16": ("e5m2", 32, "f16"),
    **{f"int{n}": (f"int{n}", 64, "f32") for n in (2, 3, 4, 5, 6, 8)},
    **{f"int{n}_f16": (f"int{n}", 64, "f16") for n in (2, 3, 4, 5, 6, 8)},
    **{f"mxint{n}": (f"int{n}", 32, "e8m0") for n in (2, 3, 4, 5, 6, 8)},
}

# scale ranges per element, so products stay near 1: U(lo, hi) for FP32 / FP16
# scales (E5M2's reach f16 subnormals); E8M0 bytes for the mxfp8 / mxint forms
_SB_SCALE_RANGE = {"e2m1": (0.01, 0.1), "e4m3": (5e-4, 5e-3), "e5m2": (2e-6, 2e-5)}


def sb_case(fmt: str, *, K: int, N: int, B: int, dtype: str = "bf16", key: str = "") -> QmvCase:
    """A symmetric block-scaled QMV case: codes uniform over the element's
    finite codes (E4M3 without 0x7F/0xFF, E5M2 without exponent 31), scales
    drawn per element, x ~ N(0, 1) in T."""
    elem, block, kind = SB_FORMATS[fmt]
    bits = 4 if elem == "e2m1" else (8 if elem.startswith("e") else int(elem[3:]))
    rng = rng_for(7, f"sb-{fmt}-{dtype}-{key}")
    w = rng.integers(0, 256, size=(N, K * bits // 8), dtype=np.uint8)
    if elem == "e4m3":
        w[(w & 0x7F) == 0x7F] = 0x7E
    if elem == "e5m2":
        bad = ((w >> 2) & 0x1F) == 31
        w[bad] = w[bad] & 0x83        # exponent 0: a subnormal
    nb = K // block
    if kind == "e8m0":
        lo, hi = (114, 122) if elem == "e5m2" else (120, 130)
        scales = rng.integers(lo, hi, size=(N, nb), dtype=np.uint8)
    else:
        a, b = _SB_SCALE_RANGE.get(elem, (0.005, 0.05))
        s = rng.uniform(a, b, size=(N, nb))
        scales = s.astype(np.float32) if kind == "f32" else s.astype(np.float16)
    x = to_storage(rng.normal(0.0, 1.0, size=(B, K)), dtype)
    return QmvCase(fmt, dtype, B, K, N, w, scales, x, bits=bits, group=block, key=fmt)

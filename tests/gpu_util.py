"""Helpers of the GPU parity tests: moving seeded host cases to the device,
calling the library through its binding, and the tolerance checks."""

from __future__ import annotations

import sys

import numpy as np

import oracle

TORCH_DT = None


def say(msg: str) -> None:
    """Name the case before its GPU work, so a failing run says which one."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


# Elements that passed only through a documented allowance, per case: the
# suite's terminal summary prints them (tests/conftest.py), so they reach the
# run's record even under `pytest -q`.
TOLERANCE_NOTES: list[tuple[str, str, int, int]] = []


def note(what: str, kind: str, count: int, total: int) -> None:
    """Record `count` of `total` elements of case `what` that took allowance
    `kind`; also printed at once."""
    TOLERANCE_NOTES.append((what, kind, int(count), int(total)))
    say(f"{what}: {count} of {total} elements {kind}")


def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def to_dev(a: np.ndarray, dtype: str | None = None, device: str = "cuda:0"):
    """Host storage -> device tensor. dtype names a T storage (bf16 arrays are
    uint16 bit patterns); None keeps raw bytes / integers."""
    import torch
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    if dtype in ("f32", "f16") or dtype is None:
        return torch.from_numpy(a).to(device)
    raise ValueError(dtype)


def to_host(t, dtype: str) -> np.ndarray:
    """Device output -> host storage (bf16 as uint16 bits)."""
    import torch
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def indices_dev(a: np.ndarray, device: str = "cuda:0"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).to(device)


def run_qmv(bmv, c, dev=None, y=None):
    """Run the library on a workloads.QmvCase; returns the device output."""
    import torch
    if dev is None:
        dev = case_to_dev(c)
    if c.fmt == "affine":
        return bmv.qmv_affine(dev["x"], dev["w"], dev["scales"], dev["biases"], c.bits,
                              c.group, y=y)
    if c.fmt == "mxfp4":
        return bmv.qmv_fp_mxfp4(dev["x"], dev["w"], dev["scales"], y=y)
    if c.fmt == "nvfp4":
        return bmv.qmv_fp_nvfp4(dev["x"], dev["w"], dev["scales"], dev.get("gscale"), y=y)
    if c.fmt == "mxfp8":
        return bmv.qmv_fp_mxfp8(dev["x"], dev["w"], dev["scales"], y=y)
    if c.fmt in bmv.BLOCK_FORMATS:
        return bmv.qmv_fp_block(dev["x"], dev["w"], dev["scales"], c.fmt, y=y)
    raise ValueError(c.fmt)


def case_to_dev(c):
    import torch
    d = {"x": to_dev(c.x, c.dtype), "w": to_dev(c.w)}
    if c.fmt == "affine":
        d["scales"] = to_dev(c.scales, c.dtype)
        d["biases"] = to_dev(c.biases, c.dtype)
    elif c.scales.dtype == np.float32:
        d["scales"] = to_dev(c.scales, "f32")
    elif c.scales.dtype == np.float16:
        d["scales"] = to_dev(c.scales, "f16")
    else:
        d["scales"] = to_dev(c.scales)
    if c.fmt == "nvfp4" and c.global_scale is not None:
        d["gscale"] = torch.tensor([c.global_scale], dtype=torch.float32, device="cuda:0")
    return d


def oracle_rows(c, rows):
    """fp64 oracle y[:, rows] and the magnitude sums A for those rows."""
    rows = np.asarray(rows, dtype=np.int64)
    W = oracle.dequant(c.fmt, c.K, c.w[rows], c.scales[rows],
                       None if c.biases is None else c.biases[rows], bits=c.bits,
                       group=c.group, dtype=c.dtype, global_scale=c.global_scale)
    return oracle.qmv(c.x, c.dtype, W), oracle.abs_dot(c.x, c.dtype, W)


def sample_rows(N: int, n: int = 64, seed: int = 0) -> np.ndarray:
    """First rows, last rows (the ragged end of the grid) and random ones."""
    rng = np.random.default_rng(seed)
    head = np.arange(min(N, 8))
    tail = np.arange(max(0, N - 8), N)
    mid = rng.choice(N, size=min(N, n), replace=False)
    return np.unique(np.concatenate([head, tail, mid]))


def check(y_stored: np.ndarray, y64: np.ndarray, A: np.ndarray, dtype: str, what: str):
    """The parity bar.

    f32: normwise max|y - y^| / max|y^| <= 1e-5, and elementwise
         |y - y^| <= 1e-5 |y^| + 2^-22 A (A = sum_k |x w|, a floor that only
         matters under cancellation).
    f16 / bf16: |y - RN_T(y^)| <= ulp_T(RN_T(y^)); an element outside that
         passes only as a near-cancellation case, |y - y^| <= ulp_T(y)/2 +
         2^-22 A, and such elements are counted and reported, never hidden.
    Returns the number of near-cancellation elements."""
    y = oracle.storage_to_f64(y_stored, dtype)
    assert y.shape == y64.shape, (y.shape, y64.shape)
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    if dtype == "f32":
        scale = max(float(np.max(np.abs(y64))), 1e-300)
        norm = float(np.max(np.abs(y - y64))) / scale
        assert norm <= 1e-5, f"{what}: normwise relative error {norm:.3g} > 1e-5"
        err = np.abs(y - y64)
        bad = err > 1e-5 * np.abs(y64) + 2.0 ** -22 * A
        assert not bad.any(), (
            f"{what}: {int(bad.sum())} elements outside 1e-5 rel + 2^-22 A; first at "
            f"{np.argwhere(bad)[:3].tolist()} got {y[bad][:3]} want {y64[bad][:3]}")
        return 0
    r = oracle.round_f64_to(y64, dtype)
    r64 = oracle.storage_to_f64(r, dtype)
    ok = np.abs(y - r64) <= oracle.ulp_of(r, dtype)
    near = ~ok & (np.abs(y - y64) <= oracle.ulp_of(y_stored, dtype) / 2 + 2.0 ** -22 * A)
    bad = ~ok & ~near
    assert not bad.any(), (
        f"{what}: {int(bad.sum())} elements beyond 1 ulp; first at "
        f"{np.argwhere(bad)[:3].tolist()} got {y[bad][:3]} want {y64[bad][:3]}")
    n_near = int(near.sum())
    if n_near:
        note(what, "near-cancellation (beyond 1 ulp, within ulp/2 + 2^-22 A)", n_near, y.size)
    assert n_near <= max(2, y.size // 100), f"{what}: too many near-cancellation elements"
    return n_near


# unit roundoff of each activation type: one rounding to it moves a value by
# at most this fraction of its magnitude
UNIT_ROUNDOFF = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def check_fused_norm(y_stored: np.ndarray, y_def: np.ndarray, A_def: np.ndarray, dtype: str,
                     what: str) -> None:
    """Parity of a fused RMSNorm + QMV against the plain fp64 definition
    y_def = W . rmsnorm(x) (no intermediate rounding), A_def = sum_k |W xn|.

    A fused kernel stages the normalized activation in T once: each staged
    value differs from the exact one by at most the unit roundoff u_T of T,
    which moves a dot product by at most u_T * A_def. The fp32 sums (the
    dot product, the row's sum of squares and r) add at most 2^-17 * A_def
    (a chain of fewer than 128 fp32 additions); 2^-15 keeps a factor 4 of
    margin. Then the result is rounded to T once (ulp_T(y)/2). So every
    element must satisfy |y - y_def| <= ulp_T(y)/2 + (u_T + 2^-15) A_def, and
    f32 outputs also the normwise 1e-5 bar. Elements beyond one ulp of
    RN_T(y_def) are counted and reported."""
    y = oracle.storage_to_f64(y_stored, dtype)
    assert y.shape == y_def.shape, (y.shape, y_def.shape)
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    err = np.abs(y - y_def)
    half = 0.0 if dtype == "f32" else oracle.ulp_of(y_stored, dtype) / 2
    bound = half + (UNIT_ROUNDOFF[dtype] + 2.0 ** -15) * A_def
    bad = err > bound
    assert not bad.any(), (
        f"{what}: {int(bad.sum())} elements beyond the staging bound; first at "
        f"{np.argwhere(bad)[:3].tolist()} got {y[bad][:3]} want {y_def[bad][:3]}")
    if dtype == "f32":
        scale = max(float(np.max(np.abs(y_def))), 1e-300)
        norm = float(np.max(err)) / scale
        assert norm <= 1e-5, f"{what}: normwise relative error {norm:.3g} > 1e-5"
        return
    r = oracle.round_f64_to(y_def, dtype)
    beyond = int((np.abs(y - oracle.storage_to_f64(r, dtype)) > oracle.ulp_of(r, dtype)).sum())
    if beyond:
        note(what, "beyond 1 ulp of RN_T(plain definition), within the staging bound",
             beyond, y.size)

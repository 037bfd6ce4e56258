"""Launches from several host threads at once.

Kernels that stage more than 64 KB of dynamic LDS raise their limit on first
use, per device, under a lock. Here the matrix-core QMV (B = 8, bf16) runs
with four row lengths (96 to 144 KB of LDS) and two formats. All the calls are
released together from one thread each. Every call must succeed, and each
result must equal, bit for bit, the same call made alone afterwards. A few
sampled rows are also checked against the oracle.
"""
from __future__ import annotations

import threading

import numpy as np
import pytest

import workloads
from gpu_util import case_to_dev, check, oracle_rows, run_qmv, sample_rows, say, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bmv():
    import torch
    import bit_matrix_vector_amd as m
    assert torch.cuda.is_available()
    m.load()  # a machine without the built library must fail here, loudly
    return m


def test_concurrent_launches_with_large_lds(bmv):
    import torch
    cases = []
    for fmt in ("mxfp8", "nvfp4"):
        for K in (5120, 6144, 7168, 8192):
            c = workloads.mlp_up_case(fmt, 8, K=K, N=96)
            cases.append((c, case_to_dev(c)))
    torch.cuda.synchronize()
    say(f"{len(cases)} threads: b8 matrix cores, K 5120..8192, mxfp8 and nvfp4")

    outs = [None] * len(cases)
    errors = []
    start = threading.Barrier(len(cases))

    def work(i):
        try:
            c, d = cases[i]
            start.wait(timeout=60)
            outs[i] = run_qmv(bmv, c, d)
            torch.cuda.synchronize()
        except Exception as e:  # reported below, with the case
            errors.append(f"case {i}: {e!r}")

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a launching thread did not finish"
    assert not errors, errors

    for i, (c, d) in enumerate(cases):
        alone = run_qmv(bmv, c, d)
        torch.cuda.synchronize()
        assert torch.equal(outs[i].view(torch.int16), alone.view(torch.int16)), \
            f"{c.fmt} K={c.K}: the concurrent result differs from the call alone"
        rows = sample_rows(c.N, 8, seed=i)
        y = to_host(outs[i], c.dtype)
        y64, A = oracle_rows(c, rows)
        check(y[:, rows], y64, A, c.dtype, f"threads {c.fmt} K={c.K}")

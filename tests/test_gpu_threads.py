"""Launches from several host threads at once.

Kernels that stage more than 64 KB of dynamic LDS raise their limit on first
use, per device, under a lock. Here the VALU QMV tile with eight f32
activation rows (one lane group's slab of x alone fills 64 KB, so each
launch asks for 64 KB plus the tile's scales: 65 KB for MXFP8, 66 KB for
NVFP4) runs with four row lengths and two formats, so four threads race to
raise each kernel's limit. All the calls are released together from one
thread each. Every
call must succeed, and each result must equal, bit for bit, the same call
made alone afterwards. A few sampled rows are also checked against the oracle.

The body runs in a fresh child process, so these launches are the first of
their kernel instances in that process and the locked raise of the LDS limit
really happens there (in the suite's own process an earlier test may already
have raised it).
"""
from __future__ import annotations

import os
import subprocess
import sys
import threading

import numpy as np
import pytest

import workloads
from gpu_util import case_to_dev, check, oracle_rows, run_qmv, sample_rows, say, to_host

pytestmark = pytest.mark.gpu


def _concurrent_launches_with_large_lds(bmv):
    import torch
    cases = []
    for fmt in ("mxfp8", "nvfp4"):
        for K in (5120, 6144, 7168, 8192):
            make = workloads.mxfp8_case if fmt == "mxfp8" else workloads.nvfp4_case
            c = make(74, f"threads-{fmt}-{K}", K=K, N=96, B=8, dtype="f32")
            cases.append((c, case_to_dev(c)))
    torch.cuda.synchronize()
    say(f"{len(cases)} threads: f32 B=8 VALU tile, K 5120..8192, mxfp8 and nvfp4")

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
        assert torch.equal(outs[i].view(torch.int32), alone.view(torch.int32)), \
            f"{c.fmt} K={c.K}: the concurrent result differs from the call alone"
        rows = sample_rows(c.N, 8, seed=i)
        y = to_host(outs[i], c.dtype)
        y64, A = oracle_rows(c, rows)
        check(y[:, rows], y64, A, c.dtype, f"threads {c.fmt} K={c.K}")


def test_concurrent_launches_with_large_lds():
    here = os.path.dirname(os.path.abspath(__file__))
    env = dict(os.environ)
    env["PYTHONPATH"] = os.pathsep.join([os.path.dirname(here), here,
                                         env.get("PYTHONPATH", "")])
    say("child process: first launches of the large-LDS QMV tile from 8 threads")
    r = subprocess.run([sys.executable, os.path.abspath(__file__)], env=env,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, f"child exited with {r.returncode}:\n{r.stdout[-3000:]}"
    assert "CONCURRENT-LAUNCHES-OK" in r.stdout


if __name__ == "__main__":
    import bit_matrix_vector_amd as _m
    _m.load()
    _concurrent_launches_with_large_lds(_m)
    print("CONCURRENT-LAUNCHES-OK", flush=True)

"""Benchmark of the quantized matrix-vector product on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline workload: MXFP4 QMV, batch 1, K=4096, N=14336, bf16 activations.
A step is one call of the library's entry point (host validation + launch +
kernel). Weights are cold: each step reads a different one of >= 1 GiB of
resident weight copies, so nothing is served from the 256 MB Infinity Cache.

Printed: one JSON line with the headline metric, the roofline of the kernel
(algorithmic bytes / HIP-event kernel time vs 8 TB/s), the oracle timed on the
host (cpu_baseline) and the other K=4096 batch-1 cases for context.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "QMV µs/call + achieved HBM GB/s (% of peak), batch 1, K=4096"


def _dev(a, dtype=None):
    import torch
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(a).to("cuda:0")


class Runner:
    """Pre-marshalled calls of one case over rotating weight copies."""

    def __init__(self, bmv, case, min_bytes: int = 1 << 30):
        import torch
        self.case = case
        self.lib = bmv.load()
        self.x = _dev(case.x, case.dtype)
        w0 = _dev(case.w)
        s0 = _dev(case.scales, case.dtype if case.fmt == "affine" else None)
        b0 = _dev(case.biases, case.dtype) if case.biases is not None else None
        per = w0.nbytes + s0.nbytes + (b0.nbytes if b0 is not None else 0)
        self.copies = max(2, -(-min_bytes // per))
        self.w = [w0] + [w0.clone() for _ in range(self.copies - 1)]
        self.s = [s0] + [s0.clone() for _ in range(self.copies - 1)]
        self.b = None if b0 is None else [b0] + [b0.clone() for _ in range(self.copies - 1)]
        self.g = (torch.tensor([case.global_scale], dtype=torch.float32, device="cuda:0")
                  if case.fmt == "nvfp4" and case.global_scale is not None else None)
        self.y = torch.empty((case.B, case.N), dtype=self.x.dtype, device="cuda:0")
        self.dt = {"f32": 0, "f16": 1, "bf16": 2}[case.dtype]
        vp = ctypes.c_void_p
        self.args = []
        for i in range(self.copies):
            common = (vp(self.x.data_ptr()), vp(self.w[i].data_ptr()), vp(self.s[i].data_ptr()))
            if case.fmt == "affine":
                self.args.append(common + (vp(self.b[i].data_ptr()), case.bits, case.group,
                                           vp(self.y.data_ptr())))
            elif case.fmt == "nvfp4":
                self.args.append(common + (vp(self.g.data_ptr()) if self.g is not None else None,
                                           vp(self.y.data_ptr())))
            else:
                self.args.append(common + (vp(self.y.data_ptr()),))
        if case.fmt in bmv.BLOCK_FORMATS:
            code, el, block = bmv.BLOCK_FORMATS[case.fmt]
            lib = self.lib

            def fn(stream, dt, B, K, N, x, w, s, y):
                return lib.qmv_fp_block(stream, dt, code, el, block, B, K, N, x, w, s, y)
            self.fn = fn
        else:
            self.fn = {"affine": self.lib.qmv_affine, "mxfp4": self.lib.qmv_fp_mxfp4,
                       "nvfp4": self.lib.qmv_fp_nvfp4, "mxfp8": self.lib.qmv_fp_mxfp8}[case.fmt]
        self.bytes = case.algorithmic_bytes()

    def call(self, i: int, stream) -> None:
        c = self.case
        st = self.fn(stream, self.dt, c.B, c.K, c.N, *self.args[i % self.copies])
        if st != 0:
            raise RuntimeError(self.lib.qmv_last_error().decode())

    def free(self):
        self.w = self.s = self.b = None


class GatherRunner:
    """Pre-marshalled gather_qmv calls over rotating copies of the expert-
    stacked weights (the MoE workload)."""

    def __init__(self, bmv, m, min_bytes: int = 1 << 29):
        import torch
        self.m = m
        self.lib = bmv.load()
        self.x = _dev(m.x, m.dtype)
        self.lhs = torch.from_numpy(m.lhs.view(np.int32)).to("cuda:0")
        self.rhs = torch.from_numpy(m.rhs.view(np.int32)).to("cuda:0")
        w0 = _dev(m.w)
        s0 = _dev(m.scales, m.dtype if m.fmt == "affine" else None)
        b0 = _dev(m.biases, m.dtype) if m.biases is not None else None
        per = w0.nbytes + s0.nbytes + (b0.nbytes if b0 is not None else 0)
        self.copies = max(2, -(-min_bytes // per))
        self.keep = []
        self.wts = []
        for i in range(self.copies):
            w = w0 if i == 0 else w0.clone()
            sc = s0 if i == 0 else s0.clone()
            bi = None if b0 is None else (b0 if i == 0 else b0.clone())
            self.keep.append((w, sc, bi))
            self.wts.append(bmv.make_weights(m.fmt, w, sc, bi, K=m.K, bits=m.bits,
                                             group_size=m.group))
        self.y = torch.empty((m.lhs.size, m.N), dtype=self.x.dtype, device="cuda:0")
        self.dt = {"f32": 0, "f16": 1, "bf16": 2}[m.dtype]
        self.bytes = m.algorithmic_bytes()

    def call(self, i: int, stream) -> None:
        vp = ctypes.c_void_p
        st = self.lib.gather_qmv(stream, self.dt, ctypes.byref(self.wts[i % self.copies]),
                                 vp(self.x.data_ptr()), self.x.shape[0],
                                 vp(self.lhs.data_ptr()), vp(self.rhs.data_ptr()),
                                 self.m.lhs.size, vp(self.y.data_ptr()))
        if st != 0:
            raise RuntimeError(self.lib.qmv_last_error().decode())

    def free(self):
        self.keep = self.wts = None


class QvmRunner:
    """Pre-marshalled qvm calls (y[1, K] = x[1, N] . W[N, K]) over rotating
    weight copies (>= 1 GiB) and one workspace. Bytes: weights + scales once,
    x, y, and the fp32 row-split partials written and read back."""

    def __init__(self, bmv, case, min_bytes: int = 1 << 30):
        import torch
        self.lib = bmv.load()
        c = case
        self.c = c
        w0 = _dev(c.w)
        s0 = _dev(c.scales, c.dtype if c.fmt == "affine" else None)
        b0 = _dev(c.biases, c.dtype) if c.biases is not None else None
        per = w0.nbytes + s0.nbytes + (b0.nbytes if b0 is not None else 0)
        self.copies = max(2, -(-min_bytes // per))
        blk = {"affine": c.group, "mxfp4": 32, "nvfp4": 16, "mxfp8": 32}[c.fmt]
        self.keep, self.wts = [], []
        for i in range(self.copies):
            w = w0 if i == 0 else w0.clone()
            sc = s0 if i == 0 else s0.clone()
            bi = None if b0 is None else (b0 if i == 0 else b0.clone())
            self.keep.append((w, sc, bi))
            self.wts.append(bmv.make_weights(c.fmt, w, sc, bi, K=c.K, bits=c.bits,
                                             group_size=blk))
        self.x = _dev(workloads_x(c.N, c.dtype), c.dtype)
        self.y = torch.empty((1, c.K), dtype=self.x.dtype, device="cuda:0")
        self.need = int(self.lib.qmv_qvm_workspace_bytes(1, c.K, c.N))
        self.ws = torch.empty((self.need // 4,), dtype=torch.float32, device="cuda:0")
        self.dt = {"f32": 0, "f16": 1, "bf16": 2}[c.dtype]
        tb = 4 if c.dtype == "f32" else 2
        self.bytes = per + c.N * tb + c.K * tb + 2 * self.need

    def call(self, i: int, stream) -> None:
        vp = ctypes.c_void_p
        st = self.lib.qmv_qvm(stream, self.dt, ctypes.byref(self.wts[i % self.copies]), 1,
                              vp(self.x.data_ptr()), vp(self.y.data_ptr()),
                              vp(self.ws.data_ptr()), self.need)
        if st != 0:
            raise RuntimeError(self.lib.qmv_last_error().decode())

    def free(self):
        self.keep = self.wts = None


class NormRunner(Runner):
    """The fused RMSNorm + QMV over the same rotating weight copies as the
    plain QMV case; bytes add gamma once."""

    def __init__(self, bmv, case, min_bytes: int = 1 << 30):
        super().__init__(bmv, case, min_bytes)
        import workloads
        g = workloads.rng_for(8, "bench-gamma").uniform(0.5, 1.5, size=case.K)
        self.gamma = _dev(workloads.to_storage(g, case.dtype), case.dtype)
        blk = {"affine": case.group, "mxfp4": 32, "nvfp4": 16, "mxfp8": 32}[case.fmt]
        self.wts = [bmv.make_weights(case.fmt, self.w[i], self.s[i],
                                     None if self.b is None else self.b[i], K=case.K,
                                     bits=case.bits, group_size=blk, global_scale=self.g)
                    for i in range(self.copies)]
        self.bytes += case.K * (2 if case.dtype != "f32" else 4)

    def call(self, i: int, stream) -> None:
        vp = ctypes.c_void_p
        st = self.lib.qmv_rmsnorm_qmv(stream, self.dt, ctypes.byref(self.wts[i % self.copies]),
                                      self.case.B, vp(self.x.data_ptr()),
                                      vp(self.gamma.data_ptr()), ctypes.c_float(1e-6),
                                      vp(self.y.data_ptr()))
        if st != 0:
            raise RuntimeError(self.lib.qmv_last_error().decode())


class QmmRunner:
    """Pre-marshalled qmm calls (y[M, N] = x[M, K] . W[N, K]^T) over rotating
    weight copies (>= 1 GiB). Bytes: weights + scales once, x, y, and the fp32
    split partials written and read back; flops 2 M N K."""

    def __init__(self, bmv, case, M: int, min_bytes: int = 1 << 30):
        import torch
        import workloads
        self.lib = bmv.load()
        c = case
        w0 = _dev(c.w)
        s0 = _dev(c.scales, c.dtype if c.fmt == "affine" else None)
        b0 = _dev(c.biases, c.dtype) if c.biases is not None else None
        per = w0.nbytes + s0.nbytes + (b0.nbytes if b0 is not None else 0)
        self.copies = max(2, -(-min_bytes // per))
        blk = {"affine": c.group, "mxfp4": 32, "nvfp4": 16, "mxfp8": 32}[c.fmt]
        self.keep, self.wts = [], []
        for i in range(self.copies):
            w = w0 if i == 0 else w0.clone()
            sc = s0 if i == 0 else s0.clone()
            bi = None if b0 is None else (b0 if i == 0 else b0.clone())
            self.keep.append((w, sc, bi))
            self.wts.append(bmv.make_weights(c.fmt, w, sc, bi, K=c.K, bits=c.bits,
                                             group_size=blk))
        xs = workloads.rng_for(8, "bench-qmm-x").normal(size=(M, c.K))
        self.x = _dev(workloads.to_storage(xs, c.dtype), c.dtype)
        self.y = torch.empty((M, c.N), dtype=self.x.dtype, device="cuda:0")
        self.M = M
        self.dt = {"f16": 1, "bf16": 2}[c.dtype]
        self.need = int(self.lib.qmv_qmm_workspace_bytes(M, c.K, c.N, self.wts[0].format))
        self.ws = torch.empty((max(self.need, 4) // 4,), dtype=torch.float32, device="cuda:0")
        # partials written and read back when K is split
        self.bytes = per + 2 * M * (c.K + c.N) + 2 * self.need
        self.flops = 2 * M * c.N * c.K

    def call(self, i: int, stream) -> None:
        vp = ctypes.c_void_p
        st = self.lib.qmv_qmm(stream, self.dt, ctypes.byref(self.wts[i % self.copies]), self.M,
                              vp(self.x.data_ptr()), vp(self.y.data_ptr()),
                              vp(self.ws.data_ptr()), self.need)
        if st != 0:
            raise RuntimeError(self.lib.qmv_last_error().decode())

    def free(self):
        self.keep = self.wts = None


class GatherQmmRunner:
    """gather_qmm over the MoE workload's gate/up stack (64 experts, hidden
    4096, ffn 1536) with `tokens` x top-8 slots sorted by expert, over
    rotating copies of the stack. Bytes: the distinct experts' matrices once,
    x rows per slot, y; flops 2 slots N K."""

    def __init__(self, bmv, tokens: int, min_bytes: int = 1 << 30):
        import numpy as np
        import torch
        import workloads
        self.lib = bmv.load()
        m = workloads.moe_case("mxfp4", "gate_up", tokens=tokens)
        order = np.argsort(m.rhs, kind="stable")
        lhs, rhs = m.lhs[order], m.rhs[order]
        w0, s0 = _dev(m.w), _dev(m.scales)
        per = w0.nbytes + s0.nbytes
        self.copies = max(2, -(-min_bytes // per))
        self.keep = [(w0, s0)] + [(w0.clone(), s0.clone()) for _ in range(self.copies - 1)]
        self.wts = [bmv.make_weights("mxfp4", w, sc, None, K=m.K, bits=4, group_size=32)
                    for (w, sc) in self.keep]
        self.x = _dev(m.x, "bf16")
        self.lhs = torch.from_numpy(lhs.view(np.int32).copy()).cuda()
        self.rhs = torch.from_numpy(rhs.view(np.int32).copy()).cuda()
        self.n_slots = int(lhs.size)
        self.y = torch.empty((self.n_slots, m.N), dtype=torch.bfloat16, device="cuda:0")
        d = len(np.unique(rhs))
        self.bytes = d * (per // m.E) + self.n_slots * 2 * (m.K + m.N)
        self.flops = 2 * self.n_slots * m.N * m.K
        self.n_x = m.x.shape[0]

    def call(self, i: int, stream) -> None:
        vp = ctypes.c_void_p
        st = self.lib.gather_qmm(stream, 2, ctypes.byref(self.wts[i % self.copies]),
                                 vp(self.x.data_ptr()), self.n_x, vp(self.lhs.data_ptr()),
                                 vp(self.rhs.data_ptr()), self.n_slots, vp(self.y.data_ptr()))
        if st != 0:
            raise RuntimeError(self.lib.qmv_last_error().decode())

    def free(self):
        self.keep = self.wts = None


def workloads_x(n: int, dtype: str):
    import workloads
    return workloads.to_storage(workloads.rng_for(8, "bench-qvm-x").normal(size=(1, n)), dtype)


class QuantRunner:
    """Pre-marshalled quantize-from-float calls: a bf16 [N, K] weight matrix
    (rotating copies over >= 512 MiB, so every call reads from HBM) to one of
    the packed formats. Bytes: the input read once plus packed codes and
    scales written (NVFP4 reads the input twice, once for the tensor maximum;
    only one read is counted)."""

    def __init__(self, bmv, fmt: str, N: int = 14336, K: int = 4096, min_bytes: int = 1 << 29):
        import torch
        import workloads
        self.lib = bmv.load()
        self.fmt, self.N, self.K = fmt, N, K
        w0 = _dev(workloads.quant_weights(30, f"bench-quant-{fmt}", N, K, "bf16",
                                          special_rows=False), "bf16")
        self.copies = max(2, -(-min_bytes // w0.nbytes))
        self.ws = [w0] + [w0.clone() for _ in range(self.copies - 1)]
        dev = "cuda:0"
        bits = {"affine4": 4, "mxfp4": 4, "nvfp4": 4, "mxfp8": 8}[fmt]
        self.packed = torch.empty((N, K * bits // 8), dtype=torch.uint8, device=dev)
        if fmt == "affine4":
            self.sc = torch.empty((N, K // 64), dtype=torch.bfloat16, device=dev)
            self.bi = torch.empty_like(self.sc)
            out = self.packed.nbytes + 2 * self.sc.nbytes
        else:
            blk = 16 if fmt == "nvfp4" else 32
            self.sc = torch.empty((N, K // blk), dtype=torch.uint8, device=dev)
            self.gs = torch.empty((1,), dtype=torch.float32, device=dev)
            out = self.packed.nbytes + self.sc.nbytes
        self.bytes = w0.nbytes + out

    def call(self, i: int, stream) -> None:
        vp = ctypes.c_void_p
        w = vp(self.ws[i % self.copies].data_ptr())
        P, S = vp(self.packed.data_ptr()), vp(self.sc.data_ptr())
        if self.fmt == "affine4":
            st = self.lib.qmv_quantize_affine(stream, 2, self.N, self.K, w, 4, 64, P, S,
                                              vp(self.bi.data_ptr()))
        elif self.fmt == "mxfp4":
            st = self.lib.qmv_quantize_mxfp4(stream, 2, self.N, self.K, w, P, S)
        elif self.fmt == "mxfp8":
            st = self.lib.qmv_quantize_mxfp8(stream, 2, self.N, self.K, w, P, S)
        else:
            st = self.lib.qmv_quantize_nvfp4(stream, 2, self.N, self.K, w, P, S,
                                             vp(self.gs.data_ptr()))
        if st != 0:
            raise RuntimeError(self.lib.qmv_last_error().decode())

    def free(self):
        self.ws = None


class MoeBlockRunner:
    """The fused routed-MoE decode block of the MoE workload (64 experts, hidden 4096,
    ffn 1536, 16 tokens, top-8): gate/up + SwiGLU, then the per-token down sum
    (two launches per call), over two copies of the three expert stacks
    (~0.6 GB each for MXFP4, beyond the 256 MB Infinity Cache). Bytes: the
    distinct experts' gate, up and down matrices once, x, mid written and read,
    y, expert ids and router weights."""

    def __init__(self, bmv, fmt: str, copies: int = 2):
        import torch
        import workloads
        self.lib = bmv.load()
        c = workloads.moe_block_case(fmt, key="bench")
        self.c = c
        dev = "cuda:0"
        blk = {"affine": c.group, "mxfp4": 32, "nvfp4": 16}[fmt]
        self.keep, self.wts = [], []
        for i in range(copies):
            trip = []
            for m in (c.gate, c.up, c.down):
                w = _dev(m.w)
                sc = _dev(m.scales, c.dtype if fmt == "affine" else None)
                bi = _dev(m.biases, c.dtype) if m.biases is not None else None
                gs = (torch.tensor([m.global_scale], dtype=torch.float32, device=dev)
                      if m.global_scale is not None else None)
                self.keep.append((w, sc, bi, gs))
                trip.append(bmv.make_weights(fmt, w, sc, bi, K=m.K, bits=c.bits,
                                             group_size=blk, global_scale=gs))
            self.wts.append(trip)
        self.copies = copies
        self.x = _dev(c.x, c.dtype)
        self.ids = torch.from_numpy(c.ids.view(np.int32)).to(dev)
        self.route = torch.from_numpy(c.route).to(dev)
        T, k = c.ids.shape
        self.T, self.k = T, k
        self.mid = torch.empty((T * k, c.ffn), dtype=self.x.dtype, device=dev)
        self.y = torch.empty((T, c.hidden), dtype=self.x.dtype, device=dev)
        d = len(np.unique(c.ids))
        tb = 2
        self.bytes = (d * (c.matrix_bytes(c.gate) + c.matrix_bytes(c.up) + c.matrix_bytes(c.down))
                      + T * c.hidden * tb + 2 * T * k * c.ffn * tb + T * c.hidden * tb
                      + T * k * 8)
        self.distinct = d

    def call(self, i: int, stream) -> None:
        vp = ctypes.c_void_p
        g, u, d = self.wts[i % self.copies]
        st = self.lib.qmv_moe_gate_up_swiglu(stream, 2, ctypes.byref(g), ctypes.byref(u),
                                             vp(self.x.data_ptr()), self.T,
                                             vp(self.ids.data_ptr()), self.k, 0.0,
                                             vp(self.mid.data_ptr()))
        if st == 0:
            st = self.lib.qmv_moe_down_reduce(stream, 2, ctypes.byref(d), vp(self.mid.data_ptr()),
                                              self.T, vp(self.ids.data_ptr()),
                                              vp(self.route.data_ptr()), self.k,
                                              vp(self.y.data_ptr()))
        if st != 0:
            raise RuntimeError(self.lib.qmv_last_error().decode())

    def free(self):
        self.keep = self.wts = None


def time_chain(bmv, N: int = 2560, steps: int = 100) -> dict:
    """A dependent chain of 100 calls (8-bit affine g64, K=2560, bf16), each
    output the next input (for N < K it overwrites the first N values of the
    other buffer); same weights every call (warm), as in a decode loop. Timed
    as plain launches and as one HIP graph."""
    import torch
    import workloads
    c = workloads.chain_case(N)
    lib = bmv.load()
    x = _dev(c.x, "bf16")
    w, s, b = _dev(c.w), _dev(c.scales, "bf16"), _dev(c.biases, "bf16")
    bufs = [x.clone(), x.clone()]
    vp = ctypes.c_void_p

    def chain(stream):
        for t in range(steps):
            st = lib.qmv_affine(stream, 2, 1, c.K, c.N, vp(bufs[t % 2].data_ptr()),
                                vp(w.data_ptr()), vp(s.data_ptr()), vp(b.data_ptr()), 8, 64,
                                vp(bufs[(t + 1) % 2].data_ptr()))
            if st != 0:
                raise RuntimeError(lib.qmv_last_error().decode())

    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(3):
        chain(sp)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    reps = 20
    t0.record()
    for _ in range(reps):
        chain(sp)
    t1.record()
    torch.cuda.synchronize()
    plain = t0.elapsed_time(t1) * 1e3 / (reps * steps)
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=cs):
        chain(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    t0.record()
    for _ in range(reps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    graph = t0.elapsed_time(t1) * 1e3 / (reps * steps)
    del g
    return {"case": f"chain of 100: affine 8b g64 K=2560 N={N} bf16, warm weights",
            "bytes": c.algorithmic_bytes(), "us_per_call_plain": plain,
            "us_per_call_graph": graph, "gbps_graph": c.algorithmic_bytes() / graph / 1e3}


GRAPH_LAUNCHES = 256     # launches captured in one HIP graph
MIN_REPLAYS = 8          # graph replays timed (each on its own event pair)
HEADLINE_WARM_S = 3.0    # untimed graph replays before the headline and ceilings


def time_chain_cold(bmv, N: int = 2560, steps: int = 100) -> dict:
    """The dependent chain of 100 calls (8-bit affine g64, K=2560, bf16) with
    100 distinct weight matrices, call t reading matrix t (about 700 MB in
    all, beyond the 256 MB Infinity Cache, so each call streams its weights
    from HBM). Timed as plain launches and as one HIP graph."""
    import torch
    import workloads
    c = workloads.chain_case(N)
    lib = bmv.load()
    x = _dev(c.x, "bf16")
    w0, s0, b0 = _dev(c.w), _dev(c.scales, "bf16"), _dev(c.biases, "bf16")
    ws = [w0] + [w0.clone() for _ in range(steps - 1)]
    ss = [s0] + [s0.clone() for _ in range(steps - 1)]
    bs = [b0] + [b0.clone() for _ in range(steps - 1)]
    bufs = [x.clone(), x.clone()]
    vp = ctypes.c_void_p

    def chain(stream):
        for t in range(steps):
            st = lib.qmv_affine(stream, 2, 1, c.K, c.N, vp(bufs[t % 2].data_ptr()),
                                vp(ws[t].data_ptr()), vp(ss[t].data_ptr()), vp(bs[t].data_ptr()),
                                8, 64, vp(bufs[(t + 1) % 2].data_ptr()))
            if st != 0:
                raise RuntimeError(lib.qmv_last_error().decode())

    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(3):
        chain(sp)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    reps = 20
    t0.record()
    for _ in range(reps):
        chain(sp)
    t1.record()
    torch.cuda.synchronize()
    plain = t0.elapsed_time(t1) * 1e3 / (reps * steps)
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=cs):
        chain(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    t0.record()
    for _ in range(reps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    graph = t0.elapsed_time(t1) * 1e3 / (reps * steps)
    del g, ws, ss, bs
    return {"case": f"chain of 100: affine 8b g64 K=2560 N={N} bf16, 100 distinct weights (cold)",
            "bytes": c.algorithmic_bytes(), "us_per_call_plain": plain,
            "us_per_call_graph": graph, "gbps_graph": c.algorithmic_bytes() / graph / 1e3,
            "pct_peak": round(100 * c.algorithmic_bytes() / graph / 1e3 / PEAK_HBM_GBPS, 1)}


def time_case(runner: Runner, steps: int, warmup: int, warm_s: float = 0.0) -> dict:
    """Per-call time of back-to-back launches on one stream.

    us_per_call: a HIP graph of GRAPH_LAUNCHES launches (rotating weight
    copies) is replayed max(MIN_REPLAYS, ceil(steps / GRAPH_LAUNCHES))
    times, each replay between its own pair of events on the launch stream;
    the figure is the median replay's time per launch. `steps` is a minimum,
    so a small --steps still times whole 256-launch graphs. With warm_s > 0
    the graph is first replayed, untimed, for that many seconds, so the timed
    replays run at the clocks of sustained work (a GPU that was idle, or
    running the CPU-side checks, takes a while to reach them: the headline
    measured 7.06 us as the first case of a run and 6.81 us after a minute of
    other work, same library, same box; run straight after the GPU test
    suite, 6.98 us after a one-second warm-up, 6.65 us in a fresh process).
    us_per_call_plain: max(steps, 512) plain launches, one event pair."""
    import torch
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    for i in range(warmup):
        runner.call(i, sp)
    torch.cuda.synchronize()

    # (1) plain stream order
    n_plain = max(steps, 512)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(n_plain):
        runner.call(i, sp)
    t1.record()
    torch.cuda.synchronize()
    wall_us = t0.elapsed_time(t1) * 1e3 / n_plain

    # (2) the launches captured once in a HIP graph and replayed
    g = torch.cuda.CUDAGraph()
    cap_stream = torch.cuda.Stream()
    cap_stream.wait_stream(stream)
    with torch.cuda.graph(g, stream=cap_stream):
        csp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for i in range(GRAPH_LAUNCHES):
            runner.call(i, csp)
    torch.cuda.synchronize()
    reps = max(MIN_REPLAYS, -(-steps // GRAPH_LAUNCHES))
    g.replay()
    torch.cuda.synchronize()
    warm_replays = 0
    if warm_s > 0:
        t_end = time.perf_counter() + warm_s
        while time.perf_counter() < t_end:
            for _ in range(8):
                g.replay()
            torch.cuda.synchronize()
            warm_replays += 8
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) * 1e3 / GRAPH_LAUNCHES for a, b in ev)
    graph_us = per[len(per) // 2]

    del g
    return {
        "bytes": runner.bytes,
        "us_per_call_plain": wall_us,
        "us_per_call": graph_us,
        "us_per_call_replays": [round(v, 3) for v in (per[0], per[-1])],
        "timed": f"median of {reps} replays of a {GRAPH_LAUNCHES}-launch graph"
                 + (f" after {warm_replays} untimed replays ({warm_s:g} s)" if warm_replays else "")
                 + f"; {n_plain} plain launches",
        "gbps": runner.bytes / graph_us / 1e3,
        "gbps_plain": runner.bytes / wall_us / 1e3,
        "copies": runner.copies,
    }


def time_stream_read(bmv, nbytes: int, steps: int, warmup: int, min_bytes: int = 1 << 30,
                     unroll: int = 8):
    """A plain 16-byte streaming read of `nbytes` per launch over rotating,
    distinct buffers (cold HBM), with an event pair around each launch; the
    size sweep uses it."""
    import torch
    lib = bmv.load()
    nbytes = (nbytes + 15) // 16 * 16
    copies = max(2, -(-min_bytes // nbytes))
    buf = torch.empty(copies * nbytes, dtype=torch.uint8, device="cuda:0")
    buf.random_(0, 256)
    sink = torch.zeros(65536, dtype=torch.int32, device="cuda:0")
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def call(i):
        st = lib.qmv_bench_stream_read(sp, ctypes.c_void_p(buf.data_ptr() + (i % copies) * nbytes),
                                       nbytes, ctypes.c_void_p(sink.data_ptr()), unroll)
        if st != 0:
            raise RuntimeError(f"stream read launch failed: {st}")

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        call(i)
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / steps
    del buf
    return {"bytes": nbytes, "us_per_call": us, "gbps": nbytes / us / 1e3, "copies": copies,
            "unroll": unroll}


READ_DESIGNS = {
    0: "one-shot, 256 threads x 2 loads", 1: "one-shot, 256 x 4", 2: "one-shot, 256 x 8",
    3: "one-shot, 512 x 4", 4: "one-shot, 1024 x 2", 5: "one-shot, 64 x 8",
    6: "one-shot, 256 x 4, XCD-contiguous blocks", 7: "32 contiguous bytes per lane",
    8: "64 contiguous bytes per lane", 9: "grid-stride, 256 blocks x 4 loads",
    10: "grid-stride, 512 x 4", 11: "grid-stride, 1024 x 4", 12: "grid-stride, 2048 x 4",
    13: "grid-stride, 256 x 8", 14: "grid-stride, 512 x 8",
    15: "rows: 8 lanes per 128-byte line", 16: "rows: 16x16 MFMA operand layout",
    17: "rows: the one-row QMV's loads (weights + scales)",
    18: "rows: the one-row QMV's loads + its 2-byte-per-row write",
    19: "rows: the one-row QMV's loads + write, XCD-chunked blocks",
}


CEILING_DESIGN = 0
# The one-row QMV's own loads followed by the 2-byte-per-row write a QMV makes
# (in its XCD-chunked block order): the same launch without the arithmetic.
RW_CEILING_DESIGN = 19
RW_CEILING_BYTES = 14336 * 2176


class ReadRunner:
    """One read design over rotating, distinct buffers (cold HBM), with the
    Runner interface time_case expects."""

    def __init__(self, bmv, nbytes: int, design: int, min_bytes: int = 1 << 30):
        import torch
        self.lib = bmv.load()
        self.nbytes = nbytes
        self.copies = max(2, -(-min_bytes // nbytes))
        self.buf = torch.empty(self.copies * nbytes, dtype=torch.uint8, device="cuda:0")
        self.buf.random_(0, 256)
        self.sink = torch.zeros(65536, dtype=torch.int32, device="cuda:0")
        self.design = design
        self.bytes = nbytes

    def call(self, i: int, stream) -> None:
        st = self.lib.qmv_bench_read_design(
            stream, ctypes.c_void_p(self.buf.data_ptr() + (i % self.copies) * self.nbytes),
            self.nbytes, ctypes.c_void_p(self.sink.data_ptr()), self.design)
        if st != 0:
            raise RuntimeError(f"read design {self.design} failed: {st}")

    def free(self):
        self.buf = None


def read_designs(bmv, steps: int) -> list[dict]:
    """Every read design at the headline's byte counts: the 31,232,000
    algorithmic bytes, the 29,360,128 weight bytes for the row patterns
    (which need whole 2048-byte rows), and weights plus scales (31,195,136)
    for the one-row QMV's pattern; timed like the QMV (graph replays)."""
    out = []
    for d, name in READ_DESIGNS.items():
        nbytes = 14336 * 2176 if d >= 17 else 14336 * 2048 if d >= 15 else 31232000
        r = ReadRunner(bmv, nbytes, d)
        res = time_case(r, steps, 20)
        r.free()
        res.update(design=d, name=name)
        out.append(res)
        print(f"[read] design {d:2d} {name:42s} {nbytes / 1e6:7.3f} MB "
              f"{res['us_per_call']:7.3f} us {res['gbps']:7.1f} GB/s", file=sys.stderr, flush=True)
    return out


def ceiling_sweep(bmv, steps: int, warmup: int) -> None:
    """Streaming-read time against size and per-lane unroll (to stderr)."""
    for mb in (1, 4, 8, 16, 31.232, 64, 128, 256, 1024):
        for u in (4, 8, 16):
            r = time_stream_read(bmv, int(mb * 1e6), steps, warmup, unroll=u,
                                 min_bytes=max(1 << 30, 2 * int(mb * 1e6)))
            print(f"[ceiling] {mb:8.3f} MB unroll {u:2d}: {r['us_per_call']:9.2f} us "
                  f"{r['gbps']:8.1f} GB/s", file=sys.stderr, flush=True)


KERNEL_SOURCES = ("qmv_kernels.cuh", "qmv_device.h", "qmv_common.h", "qmv_inst.hip",
                  "qmv_dispatch.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_mxfp4_b1_k4096_n14336.md")


def _code_only(text: str) -> str:
    """C++ source with its comments removed and whitespace runs collapsed (a
    comment-only edit leaves the kernel's code, and so this text, unchanged).
    String literals in these sources hold no comment markers."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_fingerprint() -> str:
    """sha256 (first 16 hex digits) of the QMV kernel sources' code, comments
    and layout left out."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "bit_matrix_vector_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def committed_traffic():
    """HBM bytes per launch of the headline kernel from the committed counter
    summary, or None if there is none or it was taken on other kernel sources."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    vals = {}
    for line in (l.strip() for l in text.splitlines()):
        if line.startswith("traffic_bytes_per_launch:"):
            vals["t"] = float(line.split(":", 1)[1])
        if line.startswith("kernel_fingerprint:"):
            vals["f"] = line.split(":", 1)[1].strip()
    if vals.get("f") != kernel_fingerprint() or "t" not in vals:
        return None
    return round(vals["t"])


def pmc_workload(bmv, n: int, batch: int = 1, dtype: str = "bf16", moe: str | None = None) -> None:
    """Launch sequence for hardware-counter runs: n copies of 64 MiB (the
    calibration kernel of known size), then n launches of the MXFP4 QMV at
    K=4096, N=14336 with `batch` activation rows of `dtype` (bf16, B=1: the
    headline; f16 activations take the one-row kernel up to B=4 and the VALU
    tile or the split-operand matrix cores above it, for comparison with the
    matrix-core kernel that bf16 takes from B=3)."""
    import torch
    import workloads
    lib = bmv.load()
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nbytes = 64 << 20
    src = torch.empty(nbytes * 4, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    for i in range(n):
        st = lib.qmv_bench_copy(sp, ctypes.c_void_p(src.data_ptr() + (i % 4) * nbytes),
                                ctypes.c_void_p(dst.data_ptr()), nbytes)
        assert st == 0
    torch.cuda.synchronize()
    del src, dst
    if moe is not None:
        # the MoE gather of one projection instead (`moe` = "fmt:proj")
        fmt, proj = moe.split(":")
        r = GatherRunner(bmv, workloads.moe_case(fmt, proj))
        for i in range(n):
            r.call(i, sp)
        torch.cuda.synchronize()
        print(f"[pmc] {n} copies of {nbytes} bytes, then {n} MoE gather {fmt} {proj} launches "
              f"of {r.bytes} algorithmic bytes", flush=True)
        return
    case = (workloads.mlp_up_case("mxfp4", batch) if dtype == "bf16" else
            workloads.mxfp4_case(3, f"c3-mxfp4-B{batch}-{dtype}", K=4096, N=14336, B=batch,
                                 dtype=dtype))
    r = Runner(bmv, case)
    for i in range(n):
        r.call(i, sp)
    torch.cuda.synchronize()
    print(f"[pmc] {n} copies of {nbytes} bytes, then {n} MXFP4 B={batch} {dtype} launches of "
          f"{r.bytes} "
          f"algorithmic bytes; kernel fingerprint {kernel_fingerprint()}", flush=True)


def summarize_trace(trace_csv: str, kernel_substr: str) -> str:
    """Markdown summary of a rocprofv3 kernel trace for kernels whose name
    contains kernel_substr: duration statistics and the back-to-back period."""
    import csv
    rows = [r for r in csv.DictReader(open(trace_csv)) if kernel_substr in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    st = np.array([int(r["Start_Timestamp"]) for r in rows], dtype=np.int64)
    en = np.array([int(r["End_Timestamp"]) for r in rows], dtype=np.int64)
    d = (en - st) / 1e3
    per = np.diff(st) / 1e3
    back = per[per < 4 * np.median(per)]
    name = rows[0]["Kernel_Name"] if rows else "-"
    return "\n".join([
        f"kernel: `{name}`",
        f"dispatches: {len(rows)}",
        f"duration us: mean {d.mean():.3f}, p10 {np.percentile(d, 10):.3f}, "
        f"p50 {np.median(d):.3f}, p90 {np.percentile(d, 90):.3f}, min {d.min():.3f}, "
        f"max {d.max():.3f}",
        f"back-to-back start-to-start us (gaps > 4x median dropped): mean {back.mean():.3f}, "
        f"p50 {np.median(back):.3f}",
        f"VGPRs {rows[0]['VGPR_Count'] if rows else '-'}, grid {rows[0]['Grid_Size_X'] if rows else '-'}"
        f", workgroup {rows[0]['Workgroup_Size_X'] if rows else '-'}",
    ])


def summarize_trace_table(trace_csv: str) -> str:
    """Markdown table of every kernel in a rocprofv3 kernel trace, one line per
    (kernel, grid): dispatches and duration statistics in microseconds."""
    import csv
    import re
    groups = {}
    for r in csv.DictReader(open(trace_csv)):
        key = (r["Kernel_Name"], r["Grid_Size_X"], r["Grid_Size_Y"])
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = ["| kernel | grid | dispatches | mean us | p10 | p50 | p90 |", "|---|---|---|---|---|---|---|"]
    for (name, gx, gy), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        d = np.array(d)
        short = re.sub(r"\(qmv::LaunchParams.*", "", name).replace("qmv::(anonymous namespace)::", "")
        short = short.replace("void ", "")
        out.append(f"| `{short[:70]}` | {gx}x{gy} | {len(d)} | {d.mean():.2f} | "
                   f"{np.percentile(d, 10):.2f} | {np.median(d):.2f} | {np.percentile(d, 90):.2f} |")
    return "\n".join(out)


def summarize_counters(fetch_csv: str, write_csv: str, copy_bytes: int, alg_bytes: int,
                       kernel: str = "qmv_kernel") -> str:
    """Markdown summary of FETCH_SIZE / WRITE_SIZE per dispatch for the copy
    kernel (calibration, `copy_bytes` read and written) and the QMV kernel
    whose name contains `kernel`."""
    import csv

    def med(path, counter, sub):
        v = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
             if r["Counter_Name"] == counter and sub in r["Kernel_Name"]]
        return float(np.median(v)), len(v)

    fc, nfc = med(fetch_csv, "FETCH_SIZE", "copy_kernel")
    fq, nfq = med(fetch_csv, "FETCH_SIZE", kernel)
    wc, nwc = med(write_csv, "WRITE_SIZE", "copy_kernel")
    wq, nwq = med(write_csv, "WRITE_SIZE", kernel)
    kib = copy_bytes / 1024
    ff, wf = kib / fc, kib / wc
    t = (fq * ff + wq * wf) * 1024
    return "\n".join([
        f"copy kernel ({copy_bytes} bytes read, {copy_bytes} written): FETCH_SIZE {fc:.1f} KiB "
        f"(n={nfc}), WRITE_SIZE {wc:.1f} KiB (n={nwc}) -> scale factors fetch {ff:.4f}, "
        f"write {wf:.4f}",
        f"{kernel}: FETCH_SIZE {fq:.1f} KiB (n={nfq}), WRITE_SIZE {wq:.1f} KiB (n={nwq}) per "
        f"dispatch (medians)",
        f"traffic_bytes_per_launch: {t:.0f}",
        f"algorithmic_bytes_per_launch: {alg_bytes}",
        f"traffic / algorithmic: {t / alg_bytes:.4f}",
        f"kernel_fingerprint: {kernel_fingerprint()}",
    ])


def summarize_pmc_table(counter_csv: str) -> str:
    """Markdown table of a rocprofv3 counter collection: for every kernel (by
    name and grid), the median per dispatch of each counter collected."""
    import csv
    import re
    groups = {}
    names = []
    for r in csv.DictReader(open(counter_csv)):
        key = (r["Kernel_Name"], r.get("Grid_Size", r.get("Grid_Size_X", "")))
        c = r["Counter_Name"]
        if c not in names:
            names.append(c)
        groups.setdefault(key, {}).setdefault(c, []).append(float(r["Counter_Value"]))
    out = ["| kernel | grid | dispatches | " + " | ".join(names) + " |",
           "|---|---|---|" + "---|" * len(names)]
    for (name, grid), by in sorted(groups.items(), key=lambda kv: kv[0]):
        short = re.sub(r"\(qmv::.*", "", name).replace("qmv::(anonymous namespace)::", "")
        short = short.replace("void ", "")
        n = max(len(v) for v in by.values())
        vals = [f"{np.median(by[c]):.0f}" if c in by else "-" for c in names]
        out.append(f"| `{short[:60]}` | {grid} | {n} | " + " | ".join(vals) + " |")
    return "\n".join(out)


def check_once(bmv, case) -> None:
    """The timed entry point gives the oracle's answer on sampled rows."""
    import oracle
    import torch
    x = _dev(case.x, case.dtype)
    w = _dev(case.w)
    s = _dev(case.scales)
    y = bmv.qmv_fp_mxfp4(x, w, s)
    rows = np.arange(0, case.N, 97)
    got = oracle.storage_to_f64(y.cpu().view(torch.int16).numpy().view(np.uint16)[:, rows], "bf16")
    want = oracle.qmv_rows("mxfp4", case.x, "bf16", case.K, rows, case.w, case.scales)
    rel = np.max(np.abs(got - want)) / np.max(np.abs(want))
    if not rel < 2 ** -7:
        raise RuntimeError(f"bench case disagrees with the oracle (rel {rel:.3g})")


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_calls(case, budget_s: float, threads: int | None) -> tuple[int, float, int]:
    """Whole calls of the oracle on `case` (decode every weight row to fp64,
    then the product, in chunks of 2048 rows) until `budget_s` seconds have
    passed, with the BLAS/OpenMP pools limited to `threads` (None: as the
    process starts them). Returns (calls, seconds, threads the pools used)."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    ctx = threadpool_limits(threads) if threads is not None else None
    try:
        used = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        calls = 0
        t0 = time.perf_counter()
        while True:
            for r0 in range(0, case.N, 2048):
                rows = np.arange(r0, min(case.N, r0 + 2048))
                oracle.qmv_rows(case.fmt, case.x, case.dtype, case.K, rows, case.w, case.scales,
                                case.biases, bits=case.bits, group=case.group,
                                global_scale=case.global_scale)
            calls += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        return calls, time.perf_counter() - t0, used
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)


def cpu_baseline(case, budget_s: float = 10.0) -> dict:
    """The fp64 oracle on the host, timed on whole calls of the headline case:
    once with the BLAS/OpenMP pools at every core the process may use, once
    on one core. The oracle is a plain NumPy reference: its decode runs on
    one thread either way, only its final product uses the BLAS pool."""
    nproc = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    legs = {}
    for name, threads in (("all", nproc), ("one", 1)):
        calls, el, used = _oracle_calls(case, budget_s, threads)
        legs[name] = {"value": round(case.algorithmic_bytes() * calls / el / 1e9, 4),
                      "unit": "GB/s", "cores": used, "us_per_call": round(el / calls * 1e6),
                      "calls": calls, "seconds": round(el, 1)}
    a = legs["all"]
    return {"value": a["value"], "unit": "GB/s", "cores": a["cores"], "kind": "oracle",
            "sample": f"{a['calls']} whole calls of the headline case ({case.N} rows x "
                      f"K={case.K}) in {a['seconds']} s, {a['us_per_call']} us/call",
            "single_core": legs["one"], "nproc": nproc, "cpu_model": _cpu_model()}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="also time the whole affine sweep (K=N=4096) to stderr")
    ap.add_argument("--ceiling-sweep", action="store_true",
                    help="only sweep the streaming-read ceiling over sizes and exit")
    ap.add_argument("--read-designs", action="store_true",
                    help="only time every read design at the headline's byte count, then the "
                         "headline QMV, and exit")
    ap.add_argument("--pmc-workload", type=int, default=0, metavar="N",
                    help="only run the counter workload (N copies, N headline launches)")
    ap.add_argument("--pmc-batch", type=int, default=1, metavar="B",
                    help="activation rows of the counter workload's QMV (default 1)")
    ap.add_argument("--pmc-dtype", default="bf16", choices=("bf16", "f16"),
                    help="activation type of the counter workload's QMV (default bf16)")
    ap.add_argument("--pmc-moe", metavar="FMT:PROJ",
                    help="counter workload: the MoE gather (e.g. mxfp4:gate_up) instead of "
                         "the QMV")
    ap.add_argument("--summarize-pmc-table", metavar="COUNTER_CSV",
                    help="print per-kernel medians of every counter in a rocprofv3 counter "
                         "collection and exit (no GPU)")
    ap.add_argument("--summarize-trace-table", metavar="TRACE_CSV",
                    help="print a per-kernel duration table of a rocprofv3 kernel trace")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_CSV", "KERNEL"),
                    help="print a summary of a rocprofv3 kernel trace and exit (no GPU)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the calibrated FETCH/WRITE summary and exit (no GPU)")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(*args.summarize_trace))
        return 0
    if args.summarize_trace_table:
        print(summarize_trace_table(args.summarize_trace_table))
        return 0
    if args.summarize_pmc_table:
        print(summarize_pmc_table(args.summarize_pmc_table))
        return 0
    if args.summarize_counters:
        K, N, B = 4096, 14336, args.pmc_batch
        alg = N * K // 2 + N * K // 32 + B * K * 2 + B * N * 2   # codes + E8M0 + x + y
        # the MXFP4 K=4096 kernels: the one-row kernel up to B=2 (bf16) or 4
        # (f16), the matrix cores above
        kernel = "qmv_row_kernel" if B <= (4 if args.pmc_dtype == "f16" else 2) else \
            "qmv_mfma_kernel"
        print(summarize_counters(*args.summarize_counters, copy_bytes=64 << 20, alg_bytes=alg,
                                 kernel=kernel))
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the QMV path here has "
              "no multi-GPU mode", file=sys.stderr)
        return 2

    import torch
    import bit_matrix_vector_amd as bmv
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    bmv.load()
    if args.ceiling_sweep:
        ceiling_sweep(bmv, min(args.steps, 200), 10)
        return 0
    if args.read_designs:
        designs = read_designs(bmv, args.steps)
        head = workloads.mlp_up_case("mxfp4", 1)
        r = Runner(bmv, head)
        q = time_case(r, args.steps, args.warmup, warm_s=HEADLINE_WARM_S)
        r.free()
        print(json.dumps({"read_designs": designs, "qmv_headline": q}), flush=True)
        return 0
    if args.pmc_workload:
        pmc_workload(bmv, args.pmc_workload, args.pmc_batch, args.pmc_dtype, args.pmc_moe)
        return 0
    head = workloads.mlp_up_case("mxfp4", 1)
    check_once(bmv, head)
    runner = Runner(bmv, head)
    res = time_case(runner, args.steps, args.warmup, warm_s=HEADLINE_WARM_S)
    runner.free()
    print(f"[bench] headline mxfp4 B1: {json.dumps(res)}", file=sys.stderr, flush=True)

    ceiling = rw_ceiling = None
    if not args.no_ceiling:
        # The fastest read design measured at this byte count (one-shot grid,
        # 256 threads, two 16-byte loads per lane), timed like the QMV.
        rr = ReadRunner(bmv, head.algorithmic_bytes(), CEILING_DESIGN)
        ceiling = time_case(rr, args.steps, args.warmup, warm_s=HEADLINE_WARM_S)
        rr.free()
        ceiling.update(design=CEILING_DESIGN, name=READ_DESIGNS[CEILING_DESIGN])
        print(f"[bench] stream-read ceiling: {json.dumps(ceiling)}", file=sys.stderr, flush=True)
        rr = ReadRunner(bmv, RW_CEILING_BYTES, RW_CEILING_DESIGN)
        rw_ceiling = time_case(rr, args.steps, args.warmup, warm_s=HEADLINE_WARM_S)
        rr.free()
        rw_ceiling.update(design=RW_CEILING_DESIGN, name=READ_DESIGNS[RW_CEILING_DESIGN])
        print(f"[bench] read+write ceiling: {json.dumps(rw_ceiling)}", file=sys.stderr,
              flush=True)

    cases = []
    if not args.headline_only:
        for name, c in (("nvfp4 B1 K4096 N14336 bf16", workloads.mlp_up_case("nvfp4", 1)),
                        ("mxfp8 B1 K4096 N14336 bf16", workloads.mlp_up_case("mxfp8", 1)),
                        ("affine 4b g64 B1 K4096 N4096 bf16", workloads.affine_sweep_case(4, 64, 1, "bf16")),
                        ("mxfp4 B2 K4096 N14336 bf16 (one-row kernel)", workloads.mlp_up_case("mxfp4", 2)),
                        ("nvfp4 B3 K4096 N14336 bf16 (one-row kernel)", workloads.mlp_up_case("nvfp4", 3)),
                        ("mxfp8 B4 K4096 N14336 bf16 (one-row kernel)", workloads.mlp_up_case("mxfp8", 4)),
                        ("mxfp4 B4 K4096 N14336 bf16 (matrix cores)", workloads.mlp_up_case("mxfp4", 4)),
                        ("mxfp4 B8 K4096 N14336 bf16 (matrix cores)", workloads.mlp_up_case("mxfp4", 8)),
                        ("mxfp4 B8 K4096 N14336 f16 (matrix cores, split x)",
                         workloads.mxfp4_case(3, "c3-mxfp4-B8-f16", K=4096, N=14336, B=8,
                                              dtype="f16")),
                        *((f"{f} B1 K4096 N14336 bf16",
                           workloads.sb_case(f, K=4096, N=14336, B=1, key="bench"))
                          for f in ("mxfp8_e5m2", "nvfp8", "fp8_e5m2_f16", "int4", "mxint8"))):
            r = Runner(bmv, c)
            cr = time_case(r, max(200, args.steps // 4), args.warmup)
            r.free()
            cr["case"] = name
            cr["pct_peak"] = round(100 * cr["gbps"] / PEAK_HBM_GBPS, 1)
            cases.append(cr)
            print(f"[bench] {name}: {json.dumps(cr)}", file=sys.stderr, flush=True)

    if not args.headline_only:
        for fmt, proj in (("mxfp4", "gate_up"), ("mxfp4", "down"), ("affine", "gate_up"),
                          ("affine", "down")):
            m = workloads.moe_case(fmt, proj)
            r = GatherRunner(bmv, m)
            cr = time_case(r, max(100, args.steps // 10), 10)
            r.free()
            cr["case"] = (f"MoE gather {fmt} {proj}: 64 experts, {m.lhs.size} slots, "
                          f"{len(m.distinct_experts())} distinct, K={m.K} N={m.N} bf16")
            cr["pct_peak"] = round(100 * cr["gbps"] / PEAK_HBM_GBPS, 1)
            cases.append(cr)
            print(f"[bench] {cr['case']}: {json.dumps(cr)}", file=sys.stderr, flush=True)
        for fmt in ("mxfp4", "affine"):
            r = MoeBlockRunner(bmv, fmt)
            cr = time_case(r, max(100, args.steps // 10), 10)
            cr["case"] = (f"fused MoE block {fmt} (64 experts, hidden 4096, ffn 1536, "
                          f"16 tokens x top-8, {r.distinct} distinct): gate/up+SwiGLU, down sum; "
                          "2 launches")
            r.free()
            cr["pct_peak"] = round(100 * cr["gbps"] / PEAK_HBM_GBPS, 1)
            cases.append(cr)
            print(f"[bench] {cr['case']}: {json.dumps(cr)}", file=sys.stderr, flush=True)
        for n in (2560,) + workloads.CHAIN_TAILS:
            ch = time_chain(bmv, n)
            cases.append(ch)
            print(f"[bench] {ch['case']}: {json.dumps(ch)}", file=sys.stderr, flush=True)
        ch = time_chain_cold(bmv, 2560)
        cases.append(ch)
        print(f"[bench] {ch['case']}: {json.dumps(ch)}", file=sys.stderr, flush=True)
        for name, c in (("rmsnorm+qmv mxfp4 B1 K=4096 N=14336 bf16", workloads.mlp_up_case("mxfp4", 1)),
                        ("rmsnorm+qmv affine 4b g64 B1 K=N=4096 bf16",
                         workloads.affine_sweep_case(4, 64, 1, "bf16"))):
            r = NormRunner(bmv, c)
            cr = time_case(r, max(200, args.steps // 4), args.warmup)
            r.free()
            cr["case"] = name
            cr["pct_peak"] = round(100 * cr["gbps"] / PEAK_HBM_GBPS, 1)
            cases.append(cr)
            print(f"[bench] {name}: {json.dumps(cr)}", file=sys.stderr, flush=True)
        for name, c in (("qvm mxfp4 N=14336 K=4096 B1 bf16", workloads.mlp_up_case("mxfp4", 1)),
                        ("qvm affine 4b g64 N=K=4096 B1 bf16", workloads.affine_sweep_case(4, 64, 1, "bf16"))):
            r = QvmRunner(bmv, c)
            cr = time_case(r, max(200, args.steps // 4), args.warmup)
            r.free()
            cr["case"] = name
            cr["pct_peak"] = round(100 * cr["gbps"] / PEAK_HBM_GBPS, 1)
            cases.append(cr)
            print(f"[bench] {name}: {json.dumps(cr)}", file=sys.stderr, flush=True)
        for name, c, M in (("qmm mxfp4 M=32 K=4096 N=14336 bf16", workloads.mlp_up_case("mxfp4", 1), 32),
                           ("qmm mxfp4 M=256 K=4096 N=14336 bf16", workloads.mlp_up_case("mxfp4", 1), 256),
                           ("qmm affine 4b g64 M=256 K=N=4096 bf16",
                            workloads.affine_sweep_case(4, 64, 1, "bf16"), 256)):
            r = QmmRunner(bmv, c, M)
            cr = time_case(r, max(200, args.steps // 4), args.warmup)
            r.free()
            cr["case"] = name
            cr["pct_peak"] = round(100 * cr["gbps"] / PEAK_HBM_GBPS, 1)
            cr["tflops"] = round(r.flops / (cr["us_per_call"] * 1e-6) / 1e12, 1)
            cases.append(cr)
            print(f"[bench] {name}: {json.dumps(cr)}", file=sys.stderr, flush=True)
        r = GatherQmmRunner(bmv, 256)
        cr = time_case(r, max(100, args.steps // 10), args.warmup)
        r.free()
        cr["case"] = "gather_qmm mxfp4 MoE gate/up (64 experts, K=4096, N=1536), 2048 slots sorted"
        cr["pct_peak"] = round(100 * cr["gbps"] / PEAK_HBM_GBPS, 1)
        cr["tflops"] = round(r.flops / (cr["us_per_call"] * 1e-6) / 1e12, 1)
        cases.append(cr)
        print(f"[bench] {cr['case']}: {json.dumps(cr)}", file=sys.stderr, flush=True)
        for fmt in ("mxfp4", "nvfp4", "mxfp8", "affine4"):
            r = QuantRunner(bmv, fmt)
            cr = time_case(r, max(100, args.steps // 10), 10)
            r.free()
            cr["case"] = f"quantize bf16 [14336, 4096] -> {fmt}" + (" g64" if fmt == "affine4" else "")
            cr["pct_peak"] = round(100 * cr["gbps"] / PEAK_HBM_GBPS, 1)
            cases.append(cr)
            print(f"[bench] {cr['case']}: {json.dumps(cr)}", file=sys.stderr, flush=True)
    if args.sweep:
        for bits in workloads.AFFINE_BITS:
            for group in workloads.AFFINE_GROUPS:
                for B in (1, 2, 4, 8):
                    for dt in workloads.DTYPES:
                        c = workloads.affine_sweep_case(bits, group, B, dt)
                        r = Runner(bmv, c, min_bytes=1 << 29)
                        cr = time_case(r, 200, 10)
                        r.free()
                        cr["case"] = f"affine sweep b{bits} g{group} B{B} {dt} K=N=4096"
                        cr["pct_peak"] = round(100 * cr["gbps"] / PEAK_HBM_GBPS, 1)
                        print(f"[sweep] {json.dumps(cr)}", file=sys.stderr, flush=True)

    cpu = None if args.no_cpu_baseline else cpu_baseline(head)
    traffic = committed_traffic()
    line = {
        "metric": METRIC,
        "value": round(res["gbps"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["us_per_call"] / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4(e2m1,e8m0) x bf16 -> f32 accumulate",
        "data": "synthetic",
        "config": {"workload": "MXFP4 QMV, batch 1, K=4096, N=14336, bf16 x/y, cold HBM "
                               f"({res['copies']} rotating weight copies)",
                   "B": 1, "K": 4096, "N": 14336, "format": "mxfp4"},
        "us_per_call": round(res["us_per_call"], 3),
        "us_per_call_plain_launch": round(res["us_per_call_plain"], 3),
        "us_per_call_replay_range": res["us_per_call_replays"],
        "timed": res["timed"],
        "pct_peak": round(100 * res["gbps"] / PEAK_HBM_GBPS, 1),
        "roofline": {"bound": "hbm", "achieved": round(res["gbps"], 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(res["gbps"] / PEAK_HBM_GBPS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "stream_read_ceiling": None if ceiling is None else {
            "gbps": round(ceiling["gbps"], 1), "us_per_call": round(ceiling["us_per_call"], 3),
            "design": ceiling["name"], "timed": ceiling["timed"],
            "qmv_frac_of_ceiling": round(res["gbps"] / ceiling["gbps"], 4)},
        "read_write_ceiling": None if rw_ceiling is None else {
            "us_per_call": round(rw_ceiling["us_per_call"], 3), "design": rw_ceiling["name"],
            "bytes_read": RW_CEILING_BYTES, "bytes_written": 14336 * 2,
            "timed": rw_ceiling["timed"],
            "qmv_frac_of_ceiling": round(rw_ceiling["us_per_call"] / res["us_per_call"], 4)},
        "cases": cases,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

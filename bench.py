"""Benchmark of the N:M sparsification hot path on one MI355X.

One step = one pass of the whole path on the Hessian soft-mask workload (hessian24):
  1-3. Hutchinson estimate D [28672, 8192] of the Hessian diagonal of ||X W^T||^2 from the
     calibration rows X [1024, 8192], 8 Rademacher probes (two bf16 MFMA products per probe),
     the score S = (D + eps) W^2 per weight and the per-tensor mean and standard deviation
     of S (f64), in one call whose second product writes S and its moments (D is never
     stored)
  4-5. the temperature-sigmoid gate annealed over 8 steps (L_mid per step) and projected to
     the 2:4 hard mask, and W packed under that mask (bf16 values + 2-bit in-group indices),
     in one call whose pass over S also packs W
  6. the structured-sparse GEMM Y = X W_hat^T at M = 8192 tokens.
Inputs are synthetic (seeded, LLM-shaped) and resident in HBM before timing.  The step's
launches are captured once into a HIP graph; every timed step runs after a 1 GiB read that
evicts L2 and the 256 MB Infinity Cache (outside the timed events).

Prints ONE JSON line.  value = dense-equivalent TFLOP per step (Hutchinson's products,
2 * 2 * P * R * K * n = 7.70 TFLOP, plus the SpMM's 2 * M * R * K = 3.85 TFLOP) divided by
the step time.  The line also carries per-kernel HIP-event timings, the roofline of the
dominant launch, every other workload's rows (llama24, tiny24, slide68, ternary68 and
hessian24 stage by stage, each cold), and the CPU oracle timed on a row sample of the step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
EPS = 1e-6
# hessian24
R, K, N_CAL, M_TOK = 28672, 8192, 1024, 8192
PAGES_CONTEXT = {
    "note": "speedups the pages quote, on the hardware they name; context only, not targets",
    "SparseForge": "2:4 end-to-end inference 1.40x-1.44x vs dense on NVIDIA H800 (TensorRT-LLM)",
    "SALR": "up to 1.7x inference vs dense LoRA at 50% sparsity (hardware not named)",
    "Sparse-BitNet": "6:8 kernels up to 1.30x vs dense (1.09x-1.30x) on NVIDIA A100 and B200",
    "SlideSparse": "6:8 end-to-end 1.33x (INT8, NVIDIA A100); bound N/(N-1) = 1.33x",
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU-oracle sample time (all threads)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    p.add_argument("--no-rows", action="store_true", help="skip the per-row measurements of every workload")
    p.add_argument("--no-dense", action="store_true", help="skip the hipBLASLt dense context")
    p.add_argument("--eager", action="store_true",
                   help="time the step as individual launches instead of one HIP-graph replay")
    p.add_argument("--pmc-pass", action="store_true",
                   help="run one step plus a plain 256 MiB copy (for HBM counter scaling) and exit")
    p.add_argument("--rows-only", action="store_true", help="run the per-row measurements only (for profiling)")
    return p.parse_args()


class Step:
    """Preallocated buffers and the raw C-ABI calls of one hessian24 step."""

    def __init__(self, nm, torch, synth, dev):
        self.nm, self.torch, self.synth = nm, torch, synth
        r = nm.raw
        bf, f32, u8 = torch.bfloat16, torch.float32, torch.uint8
        self.P, self.steps = synth.HESSIAN24_PROBES, synth.HESSIAN24_STEPS
        self.Xc = synth.hessian24_calib(N_CAL, K).to(dev)
        self.W = synth.hessian24_weight(R, K).to(dev)
        self.X = synth.activations_bf16(4, M_TOK, K).to(dev)
        self.S = torch.empty((R, K), dtype=f32, device=dev)
        self.st = torch.empty(2, dtype=torch.float64, device=dev)
        self.hm = torch.empty((R, K // 8), dtype=u8, device=dev)
        self.lm = torch.empty(self.steps, dtype=torch.float64, device=dev)
        self.vals = torch.empty((R, K // 2), dtype=bf, device=dev)
        self.idx = torch.empty((R, K // 32), dtype=torch.int32, device=dev)
        self.Y = torch.empty((M_TOK, R), dtype=bf, device=dev)

        def ws(n):
            return torch.empty(max(1, int(n)), dtype=u8, device=dev)
        self.ws_h = ws(r.nm_hutchinson_score_workspace(N_CAL, K, R, self.P))
        self.ws_g = ws(r.nm_gate_workspace(R, K, self.steps))
        self.ws_y = ws(r.nm_spmm_workspace(M_TOK, K, R, 0, nm.NM_BF16))
        torch.cuda.synchronize()

    def launches(self):
        """(name, callable taking a stream handle) in step order."""
        nm, r, sy = self.nm, self.nm.raw, self.synth

        def chk(st):
            if st != 0:
                raise nm.NMError(st, nm.last_error())

        return [
            ("hutchinson+score+stats", lambda s: chk(r.nm_hutchinson_score(
                self.Xc.data_ptr(), N_CAL, K, K, R, self.P, sy.HESSIAN24_SEED, self.W.data_ptr(), nm.NM_BF16, K,
                sy.HESSIAN24_EPS, self.S.data_ptr(), K, self.st.data_ptr(), self.ws_h.data_ptr(), self.ws_h.numel(),
                s))),
            ("gate+pack", lambda s: chk(r.nm_gate_pack(
                self.S.data_ptr(), R, K, K, self.st.data_ptr(), 2, 4, sy.HESSIAN24_T0, sy.HESSIAN24_RHO, self.steps,
                self.steps - 1, None, K, self.hm.data_ptr(), K // 8, self.lm.data_ptr(), self.W.data_ptr(),
                nm.NM_BF16, K, nm.NM_BF16, self.vals.data_ptr(), K // 2, self.idx.data_ptr(), K // 32,
                self.ws_g.data_ptr(), self.ws_g.numel(), s))),
            (f"spmm M={M_TOK}", lambda s: chk(r.nm_spmm(
                self.X.data_ptr(), nm.NM_BF16, M_TOK, K, K, self.vals.data_ptr(), nm.NM_BF16, self.idx.data_ptr(), R,
                K // 2, K // 32, 0, None, 1.0, self.Y.data_ptr(), nm.NM_BF16, R, self.ws_y.data_ptr(),
                self.ws_y.numel(), s))),
        ]

    def run(self, stream):
        for _, f in self.launches():
            f(stream)

    def outputs(self):
        return [self.S, self.st, self.hm, self.lm, self.vals, self.idx, self.Y]

    def snapshot(self):
        return [t.clone() for t in self.outputs()]

    def clear_outputs(self):
        for t in self.outputs():
            t.zero_()

    def same(self, ref):
        return all(self.torch.equal(a, b) for a, b in zip(self.outputs(), ref))


HUTCH_FLOPS = 2 * 2 * 8 * R * K * N_CAL            # two products per probe, 8 probes
SPMM_DENSE_EQ = 2 * M_TOK * R * K                   # dense-equivalent work of the sparse product
# the gate's work per score, in full-rate lane operations.  A step with a sigmoid: the scale,
# one 2^x (4: quarter rate), 1 + e, one reciprocal (4), the blend toward h (2) and m (1 - m)
# (2); with rho = 1/2 every step after the first squares the previous exponential (1) in
# place of the scale and the 2^x; the last step (beta = 1) blends nothing.
GATE_OPS_PER_STEP = 1 + 4 + 1 + 4 + 2 + 2


def gate_ops(steps, rho):
    if steps < 2:
        return 0
    later = 1 + 1 + 4 + 2 + 2 if rho == 0.5 else GATE_OPS_PER_STEP
    return GATE_OPS_PER_STEP + (steps - 2) * later
# VALU issue rate: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz full-rate lane operations per
# second; a transcendental (2^x, 1/x) issues at a quarter of that rate.
VALU_PEAK_GOPS = 256 * 4 * 16 * 2.4


def algorithmic_work(steps, rho):
    """Per-launch algorithmic bytes (HBM-bound kernels), lane operations (VALU) or flops."""
    return {
        # the two products' flops; bytes of the fused score: read W (2 B), write S (4 B) per weight
        "hutchinson+score+stats": dict(bound="mfma", flops=HUTCH_FLOPS, flops_dense_eq=HUTCH_FLOPS, bytes=R * K * 6),
        # per weight: the gate's lane operations over all steps (the pack's few are not
        # counted); bytes: read S (4 B) and W (2 B), write the mask bit, 2 of 4 values (1 B)
        # and 2-bit indices (0.125 B)
        "gate+pack": dict(bound="alu", ops=R * K * gate_ops(steps, rho), bytes=int(R * K * 7.25)),
        f"spmm M={M_TOK}": dict(bound="mfma", flops=SPMM_DENSE_EQ // 2, flops_dense_eq=SPMM_DENSE_EQ,
                                bytes=R * K // 2 * 2 + R * K // 32 * 4 + M_TOK * K * 2 + M_TOK * R * 2),
    }


def cpu_model():
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(target_s: float):
    """The oracle on the step restricted to a sample of output rows (Hutchinson rows, their
    score, the statistics and gate of the sampled scores, the pack, and the masked product of
    those rows with all 8192 tokens), in the step's unit (dense-equivalent TFLOP/s); once on
    every host thread and once on one."""
    import numpy as np

    import oracle as O
    import synth

    import torch

    def bits(t):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)

    Xc = bits(synth.hessian24_calib(N_CAL, K))
    W = bits(synth.hessian24_weight(R, K))
    X = bits(synth.activations_bf16(4, M_TOK, K))
    P, steps = synth.HESSIAN24_PROBES, synth.HESSIAN24_STEPS
    per_row = 2 * 2 * P * K * N_CAL + 2 * M_TOK * K    # dense-equivalent flops per output row

    def run(nrows):
        rows = np.linspace(0, R - 1, nrows).astype(np.int64)
        t0 = time.perf_counter()
        D = O.hutchinson_rows(Xc, P, synth.HESSIAN24_SEED, rows).astype(np.float32)
        Wr = np.ascontiguousarray(W[rows])
        S = O.score(Wr, D, synth.HESSIAN24_EPS)
        mu, sg = O.stats(S)
        _, hm, _ = O.gate_anneal(S, mu, sg, 2, 4, synth.HESSIAN24_T0, synth.HESSIAN24_RHO, steps)
        O.pack(Wr, hm, 2, 4)
        O.masked_matmul(X, Wr, hm)
        return time.perf_counter() - t0

    threads = O.num_threads()
    out = dict(unit="TFLOP/s", kind="oracle", cpu=cpu_model(), threads_available=os.cpu_count())
    t8 = run(threads)
    rows_all = int(max(threads, min(4096, threads * target_s / max(t8, 1e-3))))
    t = run(rows_all)
    out.update(value=rows_all * per_row / t / 1e12, cores=threads,
               sample=f"hessian24 step on {rows_all} evenly spaced output rows of 28672 (Hutchinson rows with 8 "
                      f"probes, score, statistics and gate of the sampled scores, pack, masked product with all "
                      f"8192 tokens), {t:.1f} s on {threads} threads; full step extrapolated "
                      f"{t * R / rows_all:.0f} s")
    O.set_threads(1)
    try:
        t1 = run(2)
        rows_1 = int(max(2, min(256, 2 * target_s / 3 / max(t1, 1e-3))))
        t1 = run(rows_1)
        out["one_thread"] = dict(value=rows_1 * per_row / t1 / 1e12, rows=rows_1, seconds=round(t1, 1))
    finally:
        O.set_threads(threads)
    return out


INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 MFMA


def measure_rows(nm, torch, synth, dev, reps: int = 5):
    """Every hot-path row at the full size of each workload: kernel time from HIP events
    around the raw C call (median of `reps`, each after a 1 GiB read that evicts L2 and
    the Infinity Cache: a read leaves no dirty lines whose write-back would overlap the
    timed call, as a 1 GiB write does), with its algorithmic bytes or flops and the
    roofline fraction."""
    r = nm.raw
    bf, f32, i8, i32, u8 = torch.bfloat16, torch.float32, torch.int8, torch.int32, torch.uint8
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    flush = torch.zeros(1 << 27, dtype=torch.int64, device=dev)   # 1 GiB
    out = []

    def chk(st):
        if st != 0:
            raise nm.NMError(st, nm.last_error())

    def timed(f):
        ts = []
        for i in range(reps):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            f()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return sorted(ts)[len(ts) // 2]

    def streamed(make, operands):
        """Per-call time with launches back to back, each call on its own copy of the weight
        operands: enough copies that they fill twice the 256 MB Infinity Cache, so every call
        reads its weight from HBM (as a model's consecutive layers do).  Median of 3 passes
        over the copies, each pass one HIP-event interval."""
        nbytes = sum(t.numel() * t.element_size() for t in operands)
        n = max(4, min(64, -(-(512 << 20) // nbytes)))
        copies = [tuple(t.clone() for t in operands) for _ in range(n)]
        calls = [make(*c) for c in copies]
        for c in calls:
            c()
        ts = []
        for _ in range(3):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for c in calls:
                c()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3 / n)
        del copies, calls
        return sorted(ts)[1], n

    def row(cfg, rowid, name, f, bound, work, stream_of=None):
        t = timed(f)
        e = dict(config=cfg, row=rowid, name=name, us=round(t * 1e6, 2), bound=bound)
        if bound == "hbm":
            e["GBps"] = round(work / t / 1e9, 1)
            e["frac"] = round(e["GBps"] / HBM_PEAK_GBPS, 4)
            if stream_of is not None:   # (factory of a call on given weight operands, the operands)
                ts, n = streamed(*stream_of)
                e["us_stream"] = round(ts * 1e6, 2)
                e["frac_stream"] = round(work / ts / 1e9 / HBM_PEAK_GBPS, 4)
                e["stream_copies"] = n
        elif bound == "mfma":
            e["TFLOPs"] = round(work / t / 1e12, 2)
            e["frac"] = round(e["TFLOPs"] / BF16_PEAK_TFLOPS, 4)
        elif bound == "mfma_i8":
            e["TOPs"] = round(work / t / 1e12, 2)
            e["frac"] = round(e["TOPs"] / INT8_PEAK_TOPS, 4)
        elif bound == "mfma_fp8":
            e["TFLOPs"] = round(work / t / 1e12, 2)
            e["frac"] = round(e["TFLOPs"] / FP8_PEAK_TFLOPS, 4)
        elif bound == "alu":
            e["GOPs"] = round(work / t / 1e9, 1)
            e["frac"] = round(e["GOPs"] / VALU_PEAK_GOPS, 4)
        else:  # launch-latency bound: absolute time only
            e["GBps"] = round(work / t / 1e9, 3)
        out.append(e)

    def ws_for(n):
        return torch.empty(max(int(n), 1), dtype=u8, device=dev)

    def spmm(X, xdt, M, K, vals, vdt, idx, R, Ns, Y, ydt, xs=None, a=1.0, ws=None):
        Kl = K // 8 * 12 if Ns else K
        return lambda: chk(r.nm_spmm(X.data_ptr(), xdt, M, K, K, vals.data_ptr(), vdt, idx.data_ptr(), R, Kl // 2,
                                     Kl // 32, Ns, None if xs is None else xs.data_ptr(), a, Y.data_ptr(), ydt, R,
                                     None if ws is None else ws.data_ptr(), 0 if ws is None else ws.numel(), sh))

    # ---- llama24: H from X_cal, fused Hessian score / top-2 of 4 / pack, SpMM at M in {1, 16, 128, 2048}
    K = 4096
    Xcal = synth.llama24_calib(512, K).to(dev)
    H = torch.empty(K, dtype=f32, device=dev)
    row("llama24", "A1", "colsumsq 512x4096", lambda: chk(r.nm_hdiag_colsumsq(
        Xcal.data_ptr(), nm.NM_BF16, 512, K, K, H.data_ptr(), None, 0, sh)), "latency", 512 * K * 2 + K * 4)
    for lname, R, tid in (("W_a", 4096, 0), ("W_b", 11008, 1)):
        W = synth.llama24_weight(R, K, tensor_id=tid).to(dev)
        vals, idx, mask = (torch.empty((R, K // 2), dtype=bf, device=dev),
                           torch.empty((R, K // 32), dtype=i32, device=dev), torch.empty((R, K // 8), dtype=u8, device=dev))
        def prune_pack(Wc, R=R, vals=vals, idx=idx, mask=mask):
            return lambda: chk(r.nm_prune_pack(
                Wc.data_ptr(), nm.NM_BF16, K, H.data_ptr(), 0, EPS, nm.NM_SCORE_HESSIAN, Wc.data_ptr(), nm.NM_BF16, K, R,
                K, 2, 4, mask.data_ptr(), K // 8, nm.NM_BF16, vals.data_ptr(), K // 2, idx.data_ptr(), K // 32, sh))
        row("llama24", "A3+A7+A8", f"prune_pack {lname} {R}x{K}", prune_pack(W), "hbm", int(R * K * 3.25) + K * 4,
            stream_of=(prune_pack, (W,)))
        for M in (1, 16, 128, 2048):
            X = synth.activations_bf16(1, M, K).to(dev)
            Y = torch.empty((M, R), dtype=bf, device=dev)
            ws = ws_for(r.nm_spmm_workspace(M, K, R, 0, nm.NM_BF16))
            f = spmm(X, nm.NM_BF16, M, K, vals, nm.NM_BF16, idx, R, 0, Y, nm.NM_BF16, ws=ws)
            if M <= 128:
                row("llama24", "A12", f"spmm {lname} M={M}", f, "hbm", R * K // 2 * 2 + R * K // 32 * 4 + M * K * 2 + M * R * 2,
                    stream_of=(lambda v, i, X=X, Y=Y, ws=ws, M=M, R=R: spmm(X, nm.NM_BF16, M, K, v, nm.NM_BF16, i, R, 0, Y,
                                                                           nm.NM_BF16, ws=ws), (vals, idx)))
            else:
                row("llama24", "A12", f"spmm {lname} M={M}", f, "mfma", 2 * M * R * K // 2)
            del X, Y, ws
        del W, vals, idx, mask
    del Xcal, H

    # ---- tiny24: fused Hessian score / top-2 of 4 / pack from fp32 W, SpMM at M = 16 (launch-latency bound)
    W, H, X = synth.tiny24_inputs()
    W, H, X = W.to(dev), H.to(dev), X.to(dev)
    R, K = W.shape
    vals, idx, mask = (torch.empty((R, K // 2), dtype=bf, device=dev), torch.empty((R, K // 32), dtype=i32, device=dev),
                       torch.empty((R, K // 8), dtype=u8, device=dev))
    row("tiny24", "A3+A7+A8", "prune_pack 256x256 (f32 -> bf16)", lambda: chk(r.nm_prune_pack(
        W.data_ptr(), nm.NM_F32, K, H.data_ptr(), 0, EPS, nm.NM_SCORE_HESSIAN, W.data_ptr(), nm.NM_F32, K, R, K, 2, 4,
        mask.data_ptr(), K // 8, nm.NM_BF16, vals.data_ptr(), K // 2, idx.data_ptr(), K // 32, sh)), "latency",
        R * K * 5.25)
    Y = torch.empty((16, R), dtype=bf, device=dev)
    ws = ws_for(r.nm_spmm_workspace(16, K, R, 0, nm.NM_BF16))
    row("tiny24", "A12", "spmm 256x256 M=16", spmm(X, nm.NM_BF16, 16, K, vals, nm.NM_BF16, idx, R, 0, Y, nm.NM_BF16, ws=ws),
        "latency", R * K * 1.125 + 16 * K * 2 + 16 * R * 2)

    # ---- slide68: 6:8 by |W| + sliding-window decomposition; lifted SpMM
    R, K, Ns = 14336, 4096, 4
    Kl = K // 8 * 12
    W = synth.slide68_weight(R, K).to(dev)
    vals, idx, mask = (torch.empty((R, Kl // 2), dtype=bf, device=dev), torch.empty((R, Kl // 32), dtype=i32, device=dev),
                       torch.empty((R, K // 8), dtype=u8, device=dev))
    row("slide68", "A3+A7+A9", "prune_slide 14336x4096 (6:8 -> 3 windows)", lambda: chk(r.nm_prune_slide(
        W.data_ptr(), nm.NM_BF16, K, None, 0, 0.0, nm.NM_SCORE_MAGNITUDE, W.data_ptr(), nm.NM_BF16, K, R, K, Ns,
        mask.data_ptr(), K // 8, nm.NM_BF16, vals.data_ptr(), Kl // 2, idx.data_ptr(), Kl // 32, sh)), "hbm",
        R * K * (2 + 1.5 + 0.1875 + 0.125))
    for M in (1, 64, 512, 4096):
        X = synth.activations_bf16(2, M, K).to(dev)
        Y = torch.empty((M, R), dtype=bf, device=dev)
        ws = ws_for(r.nm_spmm_workspace(M, K, R, Ns, nm.NM_BF16))
        f = spmm(X, nm.NM_BF16, M, K, vals, nm.NM_BF16, idx, R, Ns, Y, nm.NM_BF16, ws=ws)
        if M <= 64:
            row("slide68", "A11+A12", f"spmm lifted 14336x4096 M={M}", f, "hbm", R * K * 1.6875 + M * K * 2 + M * R * 2,
                stream_of=(lambda v, i, X=X, Y=Y, ws=ws, M=M: spmm(X, nm.NM_BF16, M, K, v, nm.NM_BF16, i, R, Ns, Y,
                                                                  nm.NM_BF16, ws=ws), (vals, idx)))
        else:
            row("slide68", "A11+A12", f"spmm lifted 14336x4096 M={M}", f, "mfma", 2 * M * R * Kl // 2)
    # the same layer with a stacked rank-64 low-rank adapter pair (SALR section 3):
    # Y = X W_hat^T + bf16(X A^T) B^T; flops: the sparse product + X A^T + u B^T
    rank, M = 64, 4096
    A, B = synth.adapter_bf16(2, rank, K, R)
    A, B = A.to(dev), B.to(dev)
    X = synth.activations_bf16(2, M, K).to(dev)
    Y = torch.empty((M, R), dtype=bf, device=dev)
    wsl = ws_for(r.nm_spmm_lowrank_workspace(M, K, R, Ns, rank))
    row("slide68", "NEXT-3", f"spmm lifted + rank-{rank} adapter 14336x4096 M={M}", lambda: chk(r.nm_spmm_lowrank(
        X.data_ptr(), M, K, K, vals.data_ptr(), idx.data_ptr(), R, Kl // 2, Kl // 32, Ns, A.data_ptr(), K,
        B.data_ptr(), rank, rank, Y.data_ptr(), nm.NM_BF16, R, wsl.data_ptr(), wsl.numel(), sh)), "mfma",
        2 * M * R * Kl // 2 + 2 * M * K * rank + 2 * M * R * rank)
    del A, B, X, Y, wsl
    # bitmap format (SALR section 4): the same 6:8 weight without the sliding-window
    # expansion, and an unstructured 50% magnitude mask of it; decode into LDS + dense MFMA.
    # Unstructured mask: |W| above the tensor's median (torch setup, not timed).
    keep = W.abs() > W.abs().flatten().float().median().to(W.dtype)
    umask = (keep.view(R, K // 8, 8).to(torch.int32) << torch.arange(8, device=dev, dtype=torch.int32)).sum(-1)
    umask = umask.to(u8).contiguous()
    popc = torch.tensor([bin(i).count("1") for i in range(256)], dtype=torch.int64, device=dev)
    for label, mk in (("6:8", mask), ("unstructured 50%", umask)):
        rown = popc[mk.long()].sum(1)
        nnz, ldvb = int(rown.sum()), (int(rown.max()) + 63) // 64 * 64   # values stored; row capacity
        bvals = torch.zeros((R, ldvb), dtype=bf, device=dev)
        boffs = torch.empty((R, K // 64 + 1), dtype=i32, device=dev)
        row("slide68", "NEXT-4", f"bitmap encode 14336x4096 ({label})", lambda: chk(r.nm_bitmap_encode(
            W.data_ptr(), nm.NM_BF16, R, K, K, mk.data_ptr(), K // 8, bvals.data_ptr(), ldvb, boffs.data_ptr(),
            K // 64 + 1, sh)), "hbm", R * K * 2 + R * K // 8 + nnz * 2 + R * (K // 64 + 1) * 4)
        for M in (1, 4096):
            X = synth.activations_bf16(2, M, K).to(dev)
            Y = torch.empty((M, R), dtype=bf, device=dev)
            wsb = ws_for(r.nm_spmm_bitmap_workspace(M, K, R))
            f = (lambda X=X, Y=Y, wsb=wsb, M=M: chk(r.nm_spmm_bitmap(
                X.data_ptr(), M, K, K, bvals.data_ptr(), ldvb, mk.data_ptr(), K // 8, boffs.data_ptr(), K // 64 + 1,
                R, Y.data_ptr(), nm.NM_BF16, R, wsb.data_ptr(), wsb.numel(), sh)))
            if M == 1:
                row("slide68", "NEXT-4", f"spmm bitmap 14336x4096 ({label}) M={M}", f, "hbm",
                    nnz * 2 + R * K // 8 + R * (K // 64 + 1) * 4 + M * K * 2 + M * R * 2)
            else:
                row("slide68", "NEXT-4", f"spmm bitmap 14336x4096 ({label}) M={M}", f, "mfma", 2 * M * R * K)
            del X, Y, wsb
        del bvals, boffs, rown
    del keep, umask, popc
    # FP8 e4m3 precision of the same layer (SlideSparse section 3): the weight's codes slide-packed
    # under the |W| mask, the activation quantised per token and lifted once, the product over K'
    Wq = W.to(torch.float8_e4m3fn)
    vq = torch.empty((R, Kl // 2), dtype=torch.float8_e4m3fn, device=dev)
    row("slide68", "NEXT-2", "prune_slide 14336x4096 (|W| mask on fp8 codes)", lambda: chk(r.nm_prune_slide(
        W.data_ptr(), nm.NM_BF16, K, None, 0, 0.0, nm.NM_SCORE_MAGNITUDE, Wq.data_ptr(), nm.NM_FP8, K, R, K, Ns,
        mask.data_ptr(), K // 8, nm.NM_FP8, vq.data_ptr(), Kl // 2, idx.data_ptr(), Kl // 32, sh)), "hbm",
        R * K * (2 + 1 + 0.75 + 0.1875 + 0.125))
    del Wq
    for M in (1, 4096):
        X = synth.activations_bf16(2, M, K).to(dev)
        XL = torch.empty((M, Kl), dtype=torch.float8_e4m3fn, device=dev)
        sx = torch.empty(M, dtype=f32, device=dev)
        if M > 1:
            row("slide68", "NEXT-2", f"quant_lift {M}x{K} bf16 -> fp8 lifted + s_x", lambda: chk(r.nm_quant_lift(
                X.data_ptr(), nm.NM_BF16, M, K, K, Ns, nm.NM_FP8, XL.data_ptr(), Kl, sx.data_ptr(), sh)), "hbm",
                M * K * 2 + M * Kl + M * 4)
        else:
            chk(r.nm_quant_lift(X.data_ptr(), nm.NM_BF16, M, K, K, Ns, nm.NM_FP8, XL.data_ptr(), Kl, sx.data_ptr(), sh))
        Y = torch.empty((M, R), dtype=bf, device=dev)
        ws = ws_for(r.nm_spmm_workspace(M, Kl, R, 0, nm.NM_FP8))
        f = spmm(XL, nm.NM_FP8, M, Kl, vq, nm.NM_FP8, idx, R, 0, Y, nm.NM_BF16, xs=sx, a=1.0, ws=ws)
        if M <= 64:
            row("slide68", "NEXT-2", f"spmm fp8 lifted 14336x4096 M={M}", f, "hbm",
                R * Kl * (0.5 + 0.0625) + M * Kl + 4 * M + M * R * 2,
                stream_of=(lambda v, i, XL=XL, sx=sx, Y=Y, ws=ws, M=M: spmm(XL, nm.NM_FP8, M, Kl, v, nm.NM_FP8, i, R, 0,
                                                                           Y, nm.NM_BF16, xs=sx, a=1.0, ws=ws),
                           (vq, idx)))
        else:
            row("slide68", "NEXT-2", f"spmm fp8 lifted 14336x4096 M={M}", f, "mfma_fp8", 2 * M * R * Kl // 2)
        del X, XL, sx, Y
    del W, vals, vq, idx, mask

    # ---- ternary68: 6:8 mask from |W_fp| on the ternary code, alpha = mean|W_fp|, int8 SpMM
    R, K, Ns = 6912, 2560, 4
    Kl = K // 8 * 12
    Wf, Wt = synth.ternary68_weights(R, K)
    Wf, Wt = Wf.to(dev), Wt.to(dev)
    vals, idx, mask = (torch.empty((R, Kl // 2), dtype=i8, device=dev), torch.empty((R, Kl // 32), dtype=i32, device=dev),
                       torch.empty((R, K // 8), dtype=u8, device=dev))
    def prune_slide_t(Wfc, Wtc):
        return lambda: chk(r.nm_prune_slide(
            Wfc.data_ptr(), nm.NM_BF16, K, None, 0, 0.0, nm.NM_SCORE_MAGNITUDE, Wtc.data_ptr(), nm.NM_I8, K, R, K, Ns,
            mask.data_ptr(), K // 8, nm.NM_I8, vals.data_ptr(), Kl // 2, idx.data_ptr(), Kl // 32, sh))
    row("ternary68", "A3+A7+A9+A10", "prune_slide 6912x2560 (|W_fp| mask on W_t)", prune_slide_t(Wf, Wt), "hbm",
        R * K * (2 + 1 + 0.75 + 0.1875 + 0.125), stream_of=(prune_slide_t, (Wf, Wt)))
    alpha = torch.empty(1, dtype=f32, device=dev)
    wsa = ws_for(r.nm_stats_workspace(R, K))
    def absmean(Wfc):
        return lambda: chk(r.nm_absmean(Wfc.data_ptr(), nm.NM_BF16, R, K, K, alpha.data_ptr(), wsa.data_ptr(),
                                        wsa.numel(), sh))
    row("ternary68", "A10", "absmean 6912x2560", absmean(Wf), "hbm", R * K * 2, stream_of=(absmean, (Wf,)))
    # the online step before the int8 product, from bf16 activations (SlideSparse 2B/2C)
    Mq = 2048
    Xb = synth.ternary68_activations_bf16(Mq, K).to(dev)
    XLq = torch.empty((Mq, Kl), dtype=i8, device=dev)
    sxq = torch.empty(Mq, dtype=f32, device=dev)
    row("ternary68", "NEXT-1", f"quant_lift {Mq}x{K} bf16 -> int8 lifted + s_x", lambda: chk(r.nm_quant_lift(
        Xb.data_ptr(), nm.NM_BF16, Mq, K, K, Ns, nm.NM_I8, XLq.data_ptr(), Kl, sxq.data_ptr(), sh)), "hbm",
        Mq * K * 2 + Mq * Kl + Mq * 4)
    del Xb, XLq, sxq
    a = float(alpha.cpu())
    for M in (1, 256, 2048):
        Xq, sx = synth.ternary68_activations(M, K)
        Xq, sx = Xq.to(dev), sx.to(dev)
        Y = torch.empty((M, R), dtype=f32, device=dev)
        ws = ws_for(r.nm_spmm_workspace(M, K, R, Ns, nm.NM_I8))
        f = spmm(Xq, nm.NM_I8, M, K, vals, nm.NM_I8, idx, R, Ns, Y, nm.NM_F32, xs=sx, a=a, ws=ws)
        if M <= 256:
            row("ternary68", "A11+A13", f"spmm int8 lifted 6912x2560 M={M}", f, "hbm",
                R * K * (0.75 + 0.09375) + M * K + 4 * M + 4 * M * R,
                stream_of=(lambda v, i, Xq=Xq, sx=sx, Y=Y, ws=ws, M=M: spmm(Xq, nm.NM_I8, M, K, v, nm.NM_I8, i, R, Ns, Y,
                                                                           nm.NM_F32, xs=sx, a=a, ws=ws), (vals, idx)))
        else:
            row("ternary68", "A11+A13", f"spmm int8 lifted 6912x2560 M={M}", f, "mfma_i8", 2 * M * R * Kl // 2)
    del Wf, Wt, vals, idx, mask

    # ---- hessian24, stage by stage (each cold; the same launches as the headline step)
    R, K, n, P = 28672, 8192, 1024, synth.HESSIAN24_PROBES
    Xc = synth.hessian24_calib(n, K).to(dev)
    W = synth.hessian24_weight(R, K).to(dev)
    D = torch.empty((R, K), dtype=f32, device=dev)
    wsh = ws_for(r.nm_hutchinson_workspace(n, K, R, P))
    row("hessian24", "A2", "hutchinson 28672x8192, 8 probes, X 1024x8192", lambda: chk(r.nm_hdiag_hutchinson(
        Xc.data_ptr(), n, K, K, R, P, synth.HESSIAN24_SEED, D.data_ptr(), K, wsh.data_ptr(), wsh.numel(), sh)),
        "mfma", 2 * P * 2 * R * K * n)
    del wsh
    S = torch.empty((R, K), dtype=f32, device=dev)
    st = torch.empty(2, dtype=torch.float64, device=dev)
    wsf = ws_for(r.nm_hutchinson_score_workspace(n, K, R, P))
    row("hessian24", "A2+A3+A4", "hutchinson + score + statistics (fused, diagonal not stored)", lambda: chk(
        r.nm_hutchinson_score(Xc.data_ptr(), n, K, K, R, P, synth.HESSIAN24_SEED, W.data_ptr(), nm.NM_BF16, K,
                              synth.HESSIAN24_EPS, S.data_ptr(), K, st.data_ptr(), wsf.data_ptr(), wsf.numel(), sh)),
        "mfma", 2 * P * 2 * R * K * n)
    del wsf
    row("hessian24", "A3", "score (H+eps) W^2, per-weight H", lambda: chk(r.nm_score(
        W.data_ptr(), nm.NM_BF16, R, K, K, D.data_ptr(), K, synth.HESSIAN24_EPS, nm.NM_SCORE_HESSIAN, S.data_ptr(), K,
        sh)), "hbm", R * K * 10)
    del D
    wss = ws_for(r.nm_stats_workspace(R, K))
    row("hessian24", "A4", "score mean/std (f64)", lambda: chk(r.nm_score_stats(
        S.data_ptr(), R, K, K, st.data_ptr(), wss.data_ptr(), wss.numel(), sh)), "hbm", R * K * 4)
    hm = torch.empty((R, K // 8), dtype=u8, device=dev)
    steps = synth.HESSIAN24_STEPS
    lm = torch.empty(steps, dtype=torch.float64, device=dev)
    wsg = ws_for(r.nm_gate_workspace(R, K, steps))
    vals, idx = torch.empty((R, K // 2), dtype=bf, device=dev), torch.empty((R, K // 32), dtype=i32, device=dev)
    row("hessian24", "A5+A6+A7", "gate/anneal -> 2:4 hard mask", lambda: chk(r.nm_gate(
        S.data_ptr(), R, K, K, st.data_ptr(), 2, 4, synth.HESSIAN24_T0, synth.HESSIAN24_RHO, steps, steps - 1, None, K,
        hm.data_ptr(), K // 8, lm.data_ptr(), wsg.data_ptr(), wsg.numel(), sh)), "alu",
        R * K * gate_ops(steps, synth.HESSIAN24_RHO))
    row("hessian24", "A8", "pack 28672x8192 from the hard mask", lambda: chk(r.nm_pack(
        W.data_ptr(), nm.NM_BF16, R, K, K, hm.data_ptr(), K // 8, 2, 4, nm.NM_BF16, vals.data_ptr(), K // 2,
        idx.data_ptr(), K // 32, 0, sh)), "hbm", R * K * 3.25)
    row("hessian24", "A5-A8", "gate/anneal -> 2:4 hard mask + pack (fused, as in the step)", lambda: chk(r.nm_gate_pack(
        S.data_ptr(), R, K, K, st.data_ptr(), 2, 4, synth.HESSIAN24_T0, synth.HESSIAN24_RHO, steps, steps - 1, None, K,
        hm.data_ptr(), K // 8, lm.data_ptr(), W.data_ptr(), nm.NM_BF16, K, nm.NM_BF16, vals.data_ptr(), K // 2,
        idx.data_ptr(), K // 32, wsg.data_ptr(), wsg.numel(), sh)), "alu", R * K * gate_ops(steps, synth.HESSIAN24_RHO))
    del S
    M = 8192
    X = synth.activations_bf16(4, M, K).to(dev)
    Y = torch.empty((M, R), dtype=bf, device=dev)
    ws = ws_for(r.nm_spmm_workspace(M, K, R, 0, nm.NM_BF16))
    row("hessian24", "A12", "spmm 28672x8192 M=8192", spmm(X, nm.NM_BF16, M, K, vals, nm.NM_BF16, idx, R, 0, Y,
                                                            nm.NM_BF16, ws=ws), "mfma", 2 * M * R * K // 2)
    return out


def traffic_for(key: str, files):
    """HBM bytes per launch from committed rocprofv3 counter runs, if none of the kernel
    sources has changed since they were taken."""
    f = ROOT / "profiles" / "traffic.json"
    if not f.exists():
        return None
    try:
        d = json.loads(f.read_text())
        e = d.get(key)
        if not e:
            return None
        h = hashlib.sha256()
        for name in files:
            h.update((ROOT / "semi_structured_sparsity_amd" / "csrc" / name).read_bytes())
        if h.hexdigest() != e["source_sha256"]:
            return None
        return int(e["bytes_per_launch"])
    except Exception:
        return None


# kernel sources of each launch (for the staleness check of committed counter figures)
SOURCES = {"hutchinson+score+stats": ("k_hutch.hip", "k_spmm.hip", "k_gate.hip"), "gate+pack": ("k_gate.hip",),
           f"spmm M={M_TOK}": ("k_spmm.hip",)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the hot path runs on a single MI355X "
              "and is not sharded across GPUs.", file=sys.stderr)
        sys.exit(2)
    import torch

    import semi_structured_sparsity_amd as nm
    import synth

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    if args.rows_only:
        print(json.dumps({"rows": measure_rows(nm, torch, synth, dev)}))
        return
    st = Step(nm, torch, synth, dev)

    if args.pmc_pass:
        st.run(sh)
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
        a.copy_(b)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_pass": "done", "copy_bytes": 256 << 20}))
        return

    # The step's launches are captured once into a HIP graph and replayed, so the timed
    # region measures the GPU rather than Python's launch overhead.  The replay is checked
    # bit for bit against an eager run of the same step.
    graph_ok = None
    if args.eager:
        run_step = lambda: st.run(sh)
    else:
        st.run(sh)
        torch.cuda.synchronize()
        ref = st.snapshot()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            st.run(torch.cuda.current_stream(dev).cuda_stream)
        st.clear_outputs()
        g.replay()
        torch.cuda.synchronize()
        graph_ok = st.same(ref)
        del ref
        if not graph_ok:
            print("graph replay differs from the eager step", file=sys.stderr)
            sys.exit(1)
        run_step = g.replay

    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)   # 1 GiB, read before every timed step

    def evict():
        flush.sum()

    for _ in range(args.warmup):
        evict()
        run_step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in ev:
        evict()
        e0.record(stream)
        run_step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    ms = sum(step_ms) / len(step_ms)
    # the same steps back to back (warm caches), for comparison
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    for _ in range(args.steps):
        run_step()
    w1.record(stream)
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1) / args.steps

    # per-launch durations: HIP events around each C call on the launch stream, eager, each
    # step after the same eviction
    launches = st.launches()
    kev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in launches]
           for _ in range(args.steps)]
    for s in range(args.steps):
        evict()
        for j, (_, f) in enumerate(launches):
            kev[s][j][0].record(stream)
            f(sh)
            kev[s][j][1].record(stream)
    torch.cuda.synchronize()
    work = algorithmic_work(st.steps, synth.HESSIAN24_RHO)
    kernels = []
    for j, (name, _) in enumerate(launches):
        t_s = sum(kev[s][j][0].elapsed_time(kev[s][j][1]) for s in range(args.steps)) / args.steps * 1e-3
        w = work[name]
        k = dict(name=name, us=round(t_s * 1e6, 2), bound=w["bound"])
        if "bytes" in w:
            k["GBps"] = round(w["bytes"] / t_s / 1e9, 1)
        if "flops" in w:
            k["TFLOPs"] = round(w["flops"] / t_s / 1e12, 2)
            k["eff_TFLOPs"] = round(w["flops_dense_eq"] / t_s / 1e12, 2)
        if w["bound"] == "hbm":
            k["frac"] = round(k["GBps"] / HBM_PEAK_GBPS, 4)
        elif w["bound"] == "mfma":
            k["frac"] = round(k["TFLOPs"] / BF16_PEAK_TFLOPS, 4)
        else:
            k["GOPs"] = round(w["ops"] / t_s / 1e9, 1)
            k["frac"] = round(k["GOPs"] / VALU_PEAK_GOPS, 4)
        kernels.append(k)
    dom = max(kernels, key=lambda k: k["us"])
    wd = work[dom["name"]]
    if dom["bound"] == "hbm":
        roof = dict(bound="hbm", achieved=dom["GBps"], peak=HBM_PEAK_GBPS, unit="GB/s", frac=dom["frac"])
    else:
        roof = dict(bound="mfma", achieved=dom["TFLOPs"], peak=BF16_PEAK_TFLOPS, unit="TFLOP/s", frac=dom["frac"])
    roof["kernel"] = dom["name"]
    roof["traffic"] = traffic_for(dom["name"], SOURCES[dom["name"]])
    roof["algorithmic"] = wd.get("flops", wd.get("bytes"))

    mp = [k for k in kernels if k["name"] in ("gate+pack",)]
    mp_bytes = sum(work[k["name"]]["bytes"] for k in mp)
    mp_us = sum(k["us"] for k in mp)

    dense_ctx = None
    if not args.no_dense:
        # context only (never on the library path): hipBLASLt dense bf16 GEMMs of the same shapes
        # -- the SpMM's dense equivalent, and Hutchinson's two products per probe (8 probes
        # stacked along the rows)
        def tmm(f, reps=5):
            for _ in range(2):
                f()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                f()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / reps
        Wt = st.W.t()
        d_spmm = tmm(lambda: torch.matmul(st.X, Wt))
        V = torch.randint(0, 2, (st.P * R, K), device=dev, dtype=torch.int8).to(torch.bfloat16) * 2 - 1
        XcT = st.Xc.t().contiguous()
        U = torch.empty((st.P * R, N_CAL), dtype=torch.bfloat16, device=dev)
        d_u = tmm(lambda: torch.matmul(V, XcT, out=U))
        G = torch.empty((st.P * R, K), dtype=torch.bfloat16, device=dev)
        d_g = tmm(lambda: torch.matmul(U, st.Xc, out=G))
        del V, U, G, XcT
        kd = {k["name"]: k["us"] for k in kernels}
        dense_ctx = dict(
            what="torch.matmul (hipBLASLt) dense bf16 GEMMs of the same shapes; context only",
            spmm_dense_us=round(d_spmm, 1), spmm_sparse_us=kd[f"spmm M={M_TOK}"],
            spmm_sparse_speedup=round(d_spmm / kd[f"spmm M={M_TOK}"], 3),
            hutchinson_dense_products_us=round(d_u + d_g, 1), hutchinson_score_us=kd["hutchinson+score+stats"],
            hutchinson_vs_dense=round((d_u + d_g) / kd["hutchinson+score+stats"], 3))
        torch.cuda.empty_cache()

    flops_step = HUTCH_FLOPS + SPMM_DENSE_EQ
    rows = None if args.no_rows else measure_rows(nm, torch, synth, dev)
    cpu = None if args.no_cpu else cpu_baseline(args.cpu_seconds)
    line = {
        "metric": "N:M SpMM effective TFLOP/s + mask/pack GB/s, as % of MI355X roofline",
        "value": round(flops_step / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "hessian24: W 28672x8192 bf16 ~0.015 N(0,1), Hutchinson diagonal of ||X W^T||^2 "
                               "from X 1024x8192 with 8 Rademacher probes, score (D+eps) W^2, per-tensor z-score, "
                               "sigmoid gate T0=0.5 annealed over 8 steps to a 2:4 hard mask, pack, SpMM at M=8192",
                   "pattern": "2:4", "R": R, "K": K, "calibration_rows": N_CAL, "tokens": M_TOK, "probes": st.P},
        "cache": "cold: a 1 GiB read evicts L2 and the Infinity Cache before every timed step (not timed)",
        "warm_ms_per_step": round(warm_ms, 4),
        "wall_s": round(wall, 3),
        "step_flops": flops_step,
        "spmm_effective_TFLOPs": next(k["eff_TFLOPs"] for k in kernels if k["name"].startswith("spmm")),
        "maskpack_GBps": round(mp_bytes / (mp_us * 1e-6) / 1e9, 1),
        "maskpack_frac_hbm": round(mp_bytes / (mp_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "timing": "eager launches" if args.eager else "HIP graph replay of the whole step (checked equal to an "
                                                      "eager step); HIP events on the launch stream",
        "roofline": roof,
        "dense_context": dense_ctx,
        "pages_context": PAGES_CONTEXT,
        "kernels": kernels,
        "rows": rows,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()

"""Benchmark of the N:M sparsification hot path on one MI355X.

One step = one pass of the whole path on the 2:4 bf16 Llama-7B-shaped layers:
  1. H = column sums of squares of the calibration activations X_cal [512, 4096]
  2. fused Hessian score (H + eps) W^2 -> top-2 of 4 -> packed bf16 values +
     2-bit indices (+ mask bits), for W_a [4096, 4096] and W_b [11008, 4096]
  3. the structured-sparse GEMM Y = X W_hat^T on both packed layers at
     M = 1, 16, 128 and 2048 tokens.
Inputs are synthetic (seeded, LLM-shaped) and resident in HBM before timing.

Prints ONE JSON line.  value = dense-equivalent SpMM TFLOP per step (2*M*R*K
summed over the eight products) divided by the whole step time.  The line also
carries per-kernel HIP-event timings, the roofline of the dominant kernel and
the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
TOKENS = (1, 16, 128, 2048)
LAYERS = (("W_a", 4096, 0), ("W_b", 11008, 1))
K = 4096
N_CAL = 512
EPS = 1e-6


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU-oracle sample time")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    p.add_argument("--no-rows", action="store_true", help="skip the per-row measurements on the other workloads")
    p.add_argument("--eager", action="store_true",
                   help="time the step as individual launches instead of one HIP-graph replay")
    p.add_argument("--streams", choices=("one", "layers", "small"), default="layers",
                   help="capture the step on one stream, or forked after H into the two layers' chains "
                        "(default), or the few-token products beside the 2048-token ones")
    p.add_argument("--pmc-pass", action="store_true",
                   help="run one step plus a plain 256 MiB copy (for HBM counter scaling) and exit")
    return p.parse_args()


class Step:
    """Preallocated buffers and the raw C-ABI calls of one step."""

    def __init__(self, nm, torch, synth, dev):
        self.nm, self.torch = nm, torch
        bf = torch.bfloat16
        self.Xcal = synth.llama24_calib(N_CAL, K).to(dev)
        self.H = torch.empty(K, dtype=torch.float32, device=dev)
        self.ws_h = torch.empty(max(1, nm.raw.nm_colsumsq_workspace(N_CAL, K)), dtype=torch.uint8, device=dev)
        self.layers = []
        for name, R, tid in LAYERS:
            W = synth.llama24_weight(R, K, tensor_id=tid).to(dev)
            vals = torch.empty((R, K // 2), dtype=bf, device=dev)
            idx = torch.empty((R, K // 32), dtype=torch.int32, device=dev)
            mask = torch.empty((R, K // 8), dtype=torch.uint8, device=dev)
            self.layers.append(dict(name=name, R=R, W=W, vals=vals, idx=idx, mask=mask))
        self.X = {M: synth.activations_bf16(1, M, K).to(dev) for M in TOKENS}
        self.Y = {(l["name"], M): torch.empty((M, l["R"]), dtype=bf, device=dev) for l in self.layers for M in TOKENS}
        for l in self.layers:   # one workspace per layer: the two layers' chains may run concurrently
            need = max(nm.raw.nm_spmm_workspace(M, K, l["R"], 0, nm.NM_BF16) for M in TOKENS)
            l["ws"] = torch.empty(max(1, need), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    def launches(self):
        """(kernel name, callable) in step order; each callable takes a stream handle.
        The first launch (H) feeds both layers; after it, each layer's launches depend
        only on that layer's earlier launches."""
        nm, r = self.nm, self.nm.raw
        out = []

        def chk(st):
            if st != 0:
                raise nm.NMError(st, nm.last_error())

        def colsumsq(stream):
            chk(r.nm_hdiag_colsumsq(self.Xcal.data_ptr(), nm.NM_BF16, N_CAL, K, K, self.H.data_ptr(),
                                    self.ws_h.data_ptr(), self.ws_h.numel(), stream))
        out.append(("colsumsq", colsumsq))
        for l in self.layers:
            def prune(stream, l=l):
                chk(r.nm_prune_pack(l["W"].data_ptr(), nm.NM_BF16, K, self.H.data_ptr(), 0, EPS, nm.NM_SCORE_HESSIAN,
                                    l["W"].data_ptr(), nm.NM_BF16, K, l["R"], K, 2, 4, l["mask"].data_ptr(), K // 8,
                                    nm.NM_BF16, l["vals"].data_ptr(), K // 2, l["idx"].data_ptr(), K // 32, stream))
            out.append((f"prune_pack {l['name']}", prune))
        for l in self.layers:
            for M in TOKENS:
                def spmm(stream, l=l, M=M):
                    Y = self.Y[(l["name"], M)]
                    chk(r.nm_spmm(self.X[M].data_ptr(), nm.NM_BF16, M, K, K, l["vals"].data_ptr(), nm.NM_BF16,
                                  l["idx"].data_ptr(), l["R"], K // 2, K // 32, 0, None, 1.0, Y.data_ptr(), nm.NM_BF16,
                                  l["R"], l["ws"].data_ptr(), l["ws"].numel(), stream))
                out.append((f"spmm {l['name']} M={M}", spmm))
        return out

    def run(self, stream):
        for _, f in self.launches():
            f(stream)

    def run_two(self, main, side, split="layers"):
        """The step on two torch streams, forked after H and joined at the end, so that
        independent kernels can share the GPU.  split="layers": W_a's chain on `main`,
        W_b's on `side`.  split="small": H and both packs on `main`, then the two
        2048-token products on `main` and the few-token products on `side`."""
        torch = self.torch
        launches = self.launches()
        fork = torch.cuda.Event()
        if split == "layers":
            launches[0][1](main.cuda_stream)
            fork.record(main)
            side.wait_event(fork)
            for name, f in launches[1:]:
                f((main if self.layers[0]["name"] in name else side).cuda_stream)
        else:
            rest = []
            for name, f in launches:
                if name.startswith("spmm"):
                    rest.append((name, f))
                else:
                    f(main.cuda_stream)
            fork.record(main)
            side.wait_event(fork)
            big = f"M={TOKENS[-1]}"
            for name, f in sorted(rest, key=lambda t: not t[0].endswith(big) or "W_a" in t[0]):
                f((main if name.endswith(big) else side).cuda_stream)
        join = torch.cuda.Event()
        join.record(side)
        main.wait_event(join)

    def outputs(self):
        out = [self.H]
        for l in self.layers:
            out += [l["vals"], l["idx"], l["mask"]]
        return out + list(self.Y.values())

    def snapshot(self):
        return [t.clone() for t in self.outputs()]

    def clear_outputs(self):
        for t in self.outputs():
            t.zero_()

    def same(self, ref):
        return all(self.torch.equal(a, b) for a, b in zip(self.outputs(), ref))


def algorithmic_work():
    """Per-launch algorithmic bytes (HBM-bound kernels) or flops (GEMMs)."""
    w = {"colsumsq": dict(bound="hbm", bytes=N_CAL * K * 2 + K * 4)}
    for name, R, _ in LAYERS:
        # read W (2 B) ; write 2 of 4 values (1 B), 2-bit indices (0.125 B), mask bit (0.125 B) per weight; read H
        w[f"prune_pack {name}"] = dict(bound="hbm", bytes=int(R * K * 3.25) + K * 4)
        for M in TOKENS:
            packed = R * K // 2 * 2 + R * K // 32 * 4
            w[f"spmm {name} M={M}"] = dict(
                # up to 128 tokens the product is bound by the packed weight's HBM stream
                bound="hbm" if M <= 128 else "mfma",
                flops_dense_eq=2 * M * R * K,          # dense-equivalent work
                flops=2 * M * R * K // 2,              # multiply-adds on kept weights only (2 of 4)
                bytes=packed + M * K * 2 + M * R * 2)  # packed weight + X + Y
    return w


def cpu_baseline(target_s: float):
    """The oracle on a row sample of the same step, scaled to dense-eq TFLOP/s."""
    import numpy as np

    import oracle as O
    import synth

    import torch

    def bits(t):
        return t.view(torch.int16).numpy().view(np.uint16)

    Xcal = bits(synth.llama24_calib(N_CAL, K))
    Ws = {name: bits(synth.llama24_weight(R, K, tensor_id=tid)) for name, R, tid in LAYERS}
    Xs = {M: bits(synth.activations_bf16(1, M, K)) for M in TOKENS}

    def run(rows):
        t0 = time.perf_counter()
        H = O.colsumsq(Xcal).astype(np.float32)
        flops = 0
        for name, R, tid in LAYERS:
            W = np.ascontiguousarray(Ws[name][:rows])
            S = O.score(W, H, EPS)
            mask = O.topn_mask(S, 2, 4)
            O.pack(W, mask, 2, 4)
            for M in TOKENS:
                O.masked_matmul(Xs[M], W, mask)
                flops += 2 * M * rows * K
        return time.perf_counter() - t0, flops

    # time a small sample, then size the real one to the target
    t_small, _ = run(8)
    rows = int(max(8, min(4096, 8 * target_s / max(t_small, 1e-3))))
    t, flops = run(rows)
    return dict(value=flops / t / 1e12, unit="TFLOP/s", cores=O.num_threads(), kind="oracle",
                sample=f"whole step on the first {rows} output rows of each layer (H, score, top-2 of 4, pack, "
                       f"and the masked matmul at M=1,16,128,2048), {t:.1f} s")


INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 MFMA
# VALU issue rate: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz full-rate lane operations per
# second; a transcendental (2^x, 1/x) issues at a quarter of that rate.
VALU_PEAK_GOPS = 256 * 4 * 16 * 2.4
# the gate's work per score and step, in full-rate lane operations: one 2^x and one
# reciprocal (4 each), then the scale, 1 + e, the blend toward h (2) and m (1 - m) (2)
GATE_OPS_PER_STEP = 4 + 4 + 1 + 1 + 2 + 2


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

    def row(cfg, rowid, name, f, bound, work):
        t = timed(f)
        e = dict(config=cfg, row=rowid, name=name, us=round(t * 1e6, 2), bound=bound)
        if bound == "hbm":
            e["GBps"] = round(work / t / 1e9, 1)
            e["frac"] = round(e["GBps"] / HBM_PEAK_GBPS, 4)
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
            row("slide68", "A11+A12", f"spmm lifted 14336x4096 M={M}", f, "hbm", R * K * 1.6875 + M * K * 2 + M * R * 2)
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
                R * Kl * (0.5 + 0.0625) + M * Kl + 4 * M + M * R * 2)
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
    row("ternary68", "A3+A7+A9+A10", "prune_slide 6912x2560 (|W_fp| mask on W_t)", lambda: chk(r.nm_prune_slide(
        Wf.data_ptr(), nm.NM_BF16, K, None, 0, 0.0, nm.NM_SCORE_MAGNITUDE, Wt.data_ptr(), nm.NM_I8, K, R, K, Ns,
        mask.data_ptr(), K // 8, nm.NM_I8, vals.data_ptr(), Kl // 2, idx.data_ptr(), Kl // 32, sh)), "hbm",
        R * K * (2 + 1 + 0.75 + 0.1875 + 0.125))
    alpha = torch.empty(1, dtype=f32, device=dev)
    wsa = ws_for(r.nm_stats_workspace(R, K))
    row("ternary68", "A10", "absmean 6912x2560", lambda: chk(r.nm_absmean(
        Wf.data_ptr(), nm.NM_BF16, R, K, K, alpha.data_ptr(), wsa.data_ptr(), wsa.numel(), sh)), "hbm", R * K * 2)
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
                R * K * (0.75 + 0.09375) + M * K + 4 * M + 4 * M * R)
        else:
            row("ternary68", "A11+A13", f"spmm int8 lifted 6912x2560 M={M}", f, "mfma_i8", 2 * M * R * Kl // 2)
    del Wf, Wt, vals, idx, mask

    # ---- hessian24: Hutchinson diagonal, score, z-score statistics, gate/anneal, pack, SpMM M = 8192
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
    row("hessian24", "A3", "score (H+eps) W^2, per-weight H", lambda: chk(r.nm_score(
        W.data_ptr(), nm.NM_BF16, R, K, K, D.data_ptr(), K, synth.HESSIAN24_EPS, nm.NM_SCORE_HESSIAN, S.data_ptr(), K,
        sh)), "hbm", R * K * 10)
    del D
    st = torch.empty(2, dtype=torch.float64, device=dev)
    wss = ws_for(r.nm_stats_workspace(R, K))
    row("hessian24", "A4", "score mean/std (f64)", lambda: chk(r.nm_score_stats(
        S.data_ptr(), R, K, K, st.data_ptr(), wss.data_ptr(), wss.numel(), sh)), "hbm", R * K * 4)
    hm = torch.empty((R, K // 8), dtype=u8, device=dev)
    steps = synth.HESSIAN24_STEPS
    lm = torch.empty(steps, dtype=torch.float64, device=dev)
    wsg = ws_for(r.nm_gate_workspace(R, K, steps))
    row("hessian24", "A5+A6+A7", "gate/anneal -> 2:4 hard mask", lambda: chk(r.nm_gate(
        S.data_ptr(), R, K, K, st.data_ptr(), 2, 4, synth.HESSIAN24_T0, synth.HESSIAN24_RHO, steps, steps - 1, None, K,
        hm.data_ptr(), K // 8, lm.data_ptr(), wsg.data_ptr(), wsg.numel(), sh)), "alu", R * K * steps * GATE_OPS_PER_STEP)
    del S
    vals, idx = torch.empty((R, K // 2), dtype=bf, device=dev), torch.empty((R, K // 32), dtype=i32, device=dev)
    row("hessian24", "A8", "pack 28672x8192 from the hard mask", lambda: chk(r.nm_pack(
        W.data_ptr(), nm.NM_BF16, R, K, K, hm.data_ptr(), K // 8, 2, 4, nm.NM_BF16, vals.data_ptr(), K // 2,
        idx.data_ptr(), K // 32, 0, sh)), "hbm", R * K * 3.25)
    M = 8192
    X = synth.activations_bf16(4, M, K).to(dev)
    Y = torch.empty((M, R), dtype=bf, device=dev)
    ws = ws_for(r.nm_spmm_workspace(M, K, R, 0, nm.NM_BF16))
    row("hessian24", "A12", "spmm 28672x8192 M=8192", spmm(X, nm.NM_BF16, M, K, vals, nm.NM_BF16, idx, R, 0, Y,
                                                            nm.NM_BF16, ws=ws), "mfma", 2 * M * R * K // 2)
    return out


def traffic_for(kernel_file: str, kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if the kernel
    source has not changed since they were taken."""
    f = ROOT / "profiles" / "traffic.json"
    if not f.exists():
        return None
    try:
        d = json.loads(f.read_text())
        e = d.get(kernel)
        if not e:
            return None
        src = (ROOT / "semi_structured_sparsity_amd" / "csrc" / kernel_file).read_bytes()
        if hashlib.sha256(src).hexdigest() != e["source_sha256"]:
            return None
        return int(e["bytes_per_launch"])
    except Exception:
        return None


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
    st = Step(nm, torch, synth, dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    if args.pmc_pass:
        st.run(sh)
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
        a.copy_(b)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_pass": "done", "copy_bytes": 256 << 20}))
        return

    # The step's launches are captured once into a HIP graph and replayed, so the timed
    # region measures the GPU rather than Python's launch overhead.  The replay is
    # checked bit for bit against an eager run of the same step.
    graph_ok = None
    if args.eager:
        run_step = lambda: st.run(sh)
    else:
        st.run(sh)
        torch.cuda.synchronize()
        ref = st.snapshot()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(dev)
        with torch.cuda.graph(g):
            cur = torch.cuda.current_stream(dev)
            if args.streams == "one":
                st.run(cur.cuda_stream)
            else:
                st.run_two(cur, side, args.streams)
        st.clear_outputs()
        g.replay()
        torch.cuda.synchronize()
        graph_ok = st.same(ref)
        if not graph_ok:
            print("graph replay differs from the eager step", file=sys.stderr)
            sys.exit(1)
        run_step = g.replay

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall / args.steps * 1e3

    # per-kernel durations: HIP events around each launch on the launch stream
    launches = st.launches()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in launches]
          for _ in range(args.steps)]
    for s in range(args.steps):
        for j, (_, f) in enumerate(launches):
            ev[s][j][0].record(stream)
            f(sh)
            ev[s][j][1].record(stream)
    torch.cuda.synchronize()
    work = algorithmic_work()
    kernels = []
    for j, (name, _) in enumerate(launches):
        t_ms = sum(ev[s][j][0].elapsed_time(ev[s][j][1]) for s in range(args.steps)) / args.steps
        w = work[name]
        k = dict(name=name, us=round(t_ms * 1e3, 2), bound=w["bound"])
        k["GBps"] = round(w["bytes"] / (t_ms * 1e-3) / 1e9, 1)
        if "flops" in w:
            k["eff_TFLOPs"] = round(w["flops_dense_eq"] / (t_ms * 1e-3) / 1e12, 2)
            k["TFLOPs"] = round(w["flops"] / (t_ms * 1e-3) / 1e12, 2)
        k["frac"] = round(k["GBps"] / HBM_PEAK_GBPS if w["bound"] == "hbm" else k["TFLOPs"] / BF16_PEAK_TFLOPS, 4)
        kernels.append(k)
    dom = max(kernels, key=lambda k: k["us"])
    wd = work[dom["name"]]
    if dom["bound"] == "hbm":
        kfile = "k_prune.hip"
        roof = dict(bound="hbm", achieved=dom["GBps"], peak=HBM_PEAK_GBPS, unit="GB/s", frac=dom["frac"])
    else:
        kfile = "k_spmm.hip"
        roof = dict(bound="mfma", achieved=dom["TFLOPs"], peak=BF16_PEAK_TFLOPS, unit="TFLOP/s", frac=dom["frac"])
    roof["kernel"] = dom["name"]
    roof["traffic"] = traffic_for(kfile, dom["name"])

    spmm_flops = sum(w["flops_dense_eq"] for n, w in work.items() if n.startswith("spmm"))
    maskpack = [k for k in kernels if k["name"].startswith("prune_pack")]
    mp_bytes = sum(work[k["name"]]["bytes"] for k in maskpack)
    mp_us = sum(k["us"] for k in maskpack)
    spmm_us = sum(k["us"] for k in kernels if k["name"].startswith("spmm"))

    # context only (never on the library path): hipBLASLt's dense bf16 GEMM of the dominant
    # product's shape, X [2048, 4096] x W_b^T, with the same HIP-event timing
    Xd, Wd = st.X[TOKENS[-1]], st.layers[-1]["W"]
    for _ in range(3):
        torch.matmul(Xd, Wd.t())
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        torch.matmul(Xd, Wd.t())
    e1.record(stream)
    torch.cuda.synchronize()
    dense_us = e0.elapsed_time(e1) * 1e3 / args.steps
    dense_ctx = dict(what=f"torch.matmul (hipBLASLt) dense bf16, same shape as {dom['name']}; context only",
                     us=round(dense_us, 2), sparse_us=dom["us"],
                     sparse_speedup=round(dense_us / dom["us"], 3))

    rows = None if args.no_rows else measure_rows(nm, torch, synth, dev)
    cpu = None if args.no_cpu else cpu_baseline(args.cpu_seconds)
    line = {
        "metric": "N:M SpMM effective TFLOP/s + mask/pack GB/s, as % of MI355X roofline",
        "value": round(spmm_flops / (ms * 1e-3) / 1e12, 3),
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
        "config": {"workload": "llama24: 2:4 bf16 Llama-7B-shaped layers W 4096x4096 and 11008x4096 (1% outlier "
                               "input channels x20), H from X_cal 512x4096, fused score/top-2-of-4/pack, "
                               "SpMM at M in {1,16,128,2048}",
                   "pattern": "2:4", "K": K, "tokens": list(TOKENS)},
        "spmm_effective_TFLOPs": round(spmm_flops / (spmm_us * 1e-6) / 1e12, 2),
        "maskpack_GBps": round(mp_bytes / (mp_us * 1e-6) / 1e9, 1),
        "maskpack_frac_hbm": round(mp_bytes / (mp_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "timing": "eager launches" if args.eager else (
            "HIP graph replay of the whole step" + {
                "one": " on one stream",
                "layers": ", the two layers' chains on two streams after H",
                "small": ", the few-token products on a second stream beside the 2048-token ones"}[args.streams] +
            " (checked equal to an eager step)"),
        "roofline": roof,
        "dense_context": dense_ctx,
        "kernels": kernels,
        "rows": rows,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()

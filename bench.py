#!/usr/bin/env python3
"""Benchmark of the int4 group-quantized decode matvec path on one MI355X.

A step is one pass over every call of the hot path, each on its own weights:
  split4   x[4096] . W[6656, 4096]  -> 4096/1024/1024/512 routed outputs (gs 128)
  gated    silu(x . Wg) * (x . Wu), Wg, Wu [14336, 4096]                (gs 128)
  down     h[14336] . Wd[4096, 14336]  (h = the gated output)           (gs 128)
  norm     RMSNorm(a_a + a_b) * w_norm . W[151936, 4096]  (LM head)     (gs 128)
  lanes    X[M, 5120] . W[25600, 5120] for M = 1, 2, 4, 8, a weight copy each (gs 64)
The step is captured once in a HIP graph and replayed; weights are re-read
from HBM every step (a step streams ~0.8 GB, far beyond the 256 MB MALL).

value = effective GB/s of the step = algorithmic bytes per step / time per step,
where algorithmic bytes = packed codes N*K/2 + fp32 scales and zeros
N*(K/gs)*8 + fp32 activations in + fp32 outputs out (what the method must move).

Next-row calls (the fused variants beside the hot path) are timed the same
way and reported under "next_rows"; they are not part of the step:
  dual     x[4096] . W0, W1 [4096, 4096]                                 (gs 128), and M = 4 lanes
  gated4   silu(X . Wg) * (X . Wu) for M = 4 lanes, the c3 gate/up weights (gs 128)
  mlp      gated + down in one launch (int4_mlp), the c3 weights            (gs 128)
  sig      (a * sigmoid(gate))[4096] . W[4096, 4096]                      (gs 128)
  swiglu   (silu(gate) * up)[8192] . W[4096, 8192]                        (gs 128)
  normswi  silu(x . Wg) * (x . Wu), x = RMSNorm(a_a + a_b) * w_norm, [14336, 4096] (gs 128)
  embed    rows ids[T] of an int4 table [151936, 4096] dequantized, T = 1 and 4096 (gs 128);
           bytes = ids + the T rows' codes, scales and zeros + the fp32 output
  prefill  X[T, 4096] . W[4096, 4096]^T for T = 512 and 4096 (gs 128) on the matrix cores;
           reported as useful TFLOP/s (2 T N K flops per call, prep launch included)

One GPU's share of every call of the step under an 8-way split (columns; K
for the down projection; synth.SHARD8) is timed as well, each call alone and
the eight together as one graph ("one_gpu_share_of_8"; --no-shards skips it):
context for how the path would shard, not the metric.

Each call also gets a warm number (the same buffers every call, labelled
cache-resident: calls under 256 MB then run from the MALL).  The single
1024x1024 matvec (gs 128) is timed the same way as a row of its own, outside
the step.

stream_read_ceiling: a plain streaming read of each call's algorithmic bytes
(the library's probe kernel, best of a few launch shapes, rotating >= 1 GiB)
is timed too; each row's pct_of_stream_read is that read's time over the
call's time.

Per-call durations: each call is also timed alone, in a graph of back-to-back
calls cycling over >= 1 GiB of device copies of its buffers, with HIP events
on the stream the kernels run on.  The norm LM head call is the dominant
kernel; its roofline entry uses that measured duration.

cpu_baseline: the CPU oracle (plain C, fp64 dot products) over every column
of every call of the step on all its OpenMP threads, and on one thread over a
bounded sample (the first fraction f of every call's columns); each the
median of three passes, in GB/s of algorithmic bytes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "int4 GEMV µs/call + effective HBM GB/s (% of MI355X peak), 1 GPU"
PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
PEAK_FP16_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak
MALL_ROTATE_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "norm_lmhead_151936x4096_traffic.md")
KERNEL_SRC = [os.path.join(ROOT, "int4_group_quantized_quant_amd", "csrc", f)
              for f in ("kernels.hip", "device_common.h")]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def alg_bytes(N, K, gs, in_floats, out_floats):
    return N * K // 2 + N * (K // gs) * 8 + 4 * in_floats + 4 * out_floats


def kernel_source_hash() -> str:
    """sha256 (first 16 hex digits) of the norm kernel's sources (kernels.hip
    and the device helpers it includes) with comments and blank space
    removed, so comment edits keep a counter summary valid."""
    src = ""
    for path in KERNEL_SRC:
        with open(path) as f:
            src += f.read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = " ".join(src.split())
    return hashlib.sha256(src.encode()).hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch of the norm kernel from the committed rocprofv3 PMC
    summary, or None when the summary is missing or the kernel changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


# ---------------------------------------------------------------- workload

class Call:
    """One library call with its buffers and algorithmic bytes."""

    def __init__(self, name, nbytes, fn, sets_fn, weight_bytes):
        self.name = name
        self.nbytes = nbytes
        self.fn = fn            # fn(buffer_set) enqueues the call
        self.sets_fn = sets_fn  # sets_fn(r) -> list of r buffer sets (device copies)
        self.weight_bytes = weight_bytes


def build_single(q4, torch, dev):
    """The single 1024x1024 matvec (gs 128): a per-call row of its own, not part
    of the step (it moves 0.6 MB, so it measures launch latency, not HBM)."""
    c1 = synth.CONFIGS["c1"]
    i1 = synth.c1_inputs()
    w1 = q4.int4_quantize_pack(torch.from_numpy(i1["W"]).to(dev), c1["gs"])
    x1 = torch.from_numpy(i1["x"]).to(dev)
    y1 = torch.empty(c1["N"], device=dev)
    sets = lambda r: [tuple(w1)] + [tuple(t.clone() for t in w1) for _ in range(r - 1)]
    return Call(f"single {c1['N']}x{c1['K']}", alg_bytes(c1["N"], c1["K"], c1["gs"], c1["K"], c1["N"]),
                lambda s: q4.int4_matvec(x1, *s, Y=y1), sets, sum(t.numel() * 4 for t in w1))


def build_workload(q4, torch, dev):
    c2, c3, c4, c5 = (synth.CONFIGS[k] for k in ("c2", "c3", "c4", "c5"))
    calls = []
    quant_times = []

    def quantize(W, gs):
        Wd = torch.from_numpy(W).to(dev)
        q4.int4_quantize_pack(Wd[:1], gs)  # first launch of this kernel: code loading, not timed
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        out = q4.int4_quantize_pack(Wd, gs)
        e1.record()
        torch.cuda.synchronize()
        quant_times.append((W.size, W.shape[0] * (W.shape[1] // gs), e0.elapsed_time(e1) * 1e-3))
        del Wd
        return out

    def clones(tensors, r):
        sets = [tuple(tensors)]
        for _ in range(r - 1):
            sets.append(tuple(t.clone() for t in tensors))
        return sets

    # split4
    log("generating and quantizing split4 weights 6656x4096")
    i2 = synth.c2_inputs()
    w2 = quantize(i2["W"], c2["gs"])
    x2 = torch.from_numpy(i2["x"]).to(dev)
    outs2 = tuple(torch.empty(n, device=dev) for n in (4096, 1024, 1024, 512))
    b2 = alg_bytes(c2["N"], c2["K"], c2["gs"], c2["K"], c2["N"])

    def f2(s):
        q4.int4_matvec_split4(s[0], s[1], s[2], s[3], c2["n0"], c2["n1"], c2["n2"], outs=outs2)
    calls.append(Call("split4 6656x4096", b2, f2, lambda r: clones((x2, *w2), r),
                      sum(t.numel() * 4 for t in w2)))

    # gated + down
    log("generating and quantizing gated MLP weights 2x14336x4096 and down 4096x14336")
    i3 = synth.c3_inputs()
    wg = quantize(i3["Wg"], c3["gs"])
    wu = quantize(i3["Wu"], c3["gs"])
    wd = quantize(i3["Wd"], c3["gs"])
    x3 = torch.from_numpy(i3["x"]).to(dev)
    h3 = torch.empty(c3["N"], device=dev)
    y3 = torch.empty(c3["Nd"], device=dev)
    b3g = 2 * alg_bytes(c3["N"], c3["K"], c3["gs"], 0, 0) + 4 * c3["K"] + 4 * c3["N"]
    b3d = alg_bytes(c3["Nd"], c3["Kd"], c3["gs"], c3["Kd"], c3["Nd"])

    def f3g(s):
        q4.int4_matvec_gated(s[0], *s[1:7], h=s[7])

    def f3d(s):
        q4.int4_matvec(s[0], s[1], s[2], s[3], Y=s[4])
    calls.append(Call("gated 2x14336x4096", b3g, f3g,
                      lambda r: [(x3, *c[:6], h3) for c in clones((*wg, *wu), r)],
                      sum(t.numel() * 4 for t in (*wg, *wu))))
    calls.append(Call("down 4096x14336", b3d, f3d,
                      lambda r: [(h3, *c, y3) for c in clones(wd, r)],
                      sum(t.numel() * 4 for t in wd)))

    # norm LM head
    log("generating and quantizing the LM head 151936x4096 (the largest call)")
    i4 = synth.c4_inputs()
    w4 = quantize(i4["W"], c4["gs"])
    del i4["W"]
    a4 = [torch.from_numpy(i4[k]).to(dev) for k in ("a_a", "a_b", "w_norm")]
    y4 = torch.empty(c4["N"], device=dev)
    r4 = torch.empty(c4["K"], device=dev)
    n4 = torch.empty(c4["K"], device=dev)
    b4 = alg_bytes(c4["N"], c4["K"], c4["gs"], 3 * c4["K"], c4["N"] + 2 * c4["K"])

    def f4(s):
        q4.int4_matvec_norm(*a4, c4["eps"], s[0], s[1], s[2], y=y4, residual_out=r4, norm_out=n4)
    calls.append(Call("norm LM head 151936x4096", b4, f4, lambda r: clones(w4, r),
                      sum(t.numel() * 4 for t in w4)))

    # lanes: one weight copy per M so no call re-reads another's weights from cache
    log("generating and quantizing lane weights 25600x5120 gs=64")
    i5 = synth.c5_inputs(8)
    w5 = quantize(i5["W"], c5["gs"])
    X5 = torch.from_numpy(i5["X"]).to(dev)
    for M in c5["Ms"]:
        wM = tuple(t.clone() for t in w5)
        XM = X5[:M].contiguous()
        YM = torch.empty((M, c5["N"]), device=dev)
        bM = alg_bytes(c5["N"], c5["K"], c5["gs"], M * c5["K"], M * c5["N"])

        def f5(s, YM=YM):
            q4.int4_matvec(s[0], s[1], s[2], s[3], Y=YM)
        calls.append(Call(f"lanes M={M} 25600x5120", bM, f5,
                          lambda r, XM=XM, wM=wM: [(XM, *c) for c in clones(wM, r)],
                          sum(t.numel() * 4 for t in wM)))
    del w5
    quant = {"elements": int(sum(n for n, _, _ in quant_times)),
             "groups": int(sum(g for _, g, _ in quant_times)),
             "seconds": float(sum(t for _, _, t in quant_times))}
    return calls, quant, {"y4": y4, "a4": a4, "w4": w4}


def build_next(q4, torch, dev):
    """Calls of the fused variants next to the hot path (timed alone, not in the step)."""
    n1, n2, n3, n4 = (synth.NEXT[k] for k in ("n1", "n2", "n3", "n4"))
    calls = []

    def quantize(W, gs):
        return q4.int4_quantize_pack(torch.from_numpy(W).to(dev), gs)

    def clones(tensors, r):
        sets = [tuple(tensors)]
        for _ in range(r - 1):
            sets.append(tuple(t.clone() for t in tensors))
        return sets

    def wbytes(ws):
        return sum(t.numel() * 4 for t in ws)

    log("generating and quantizing next-row weights (dual, gated inputs, norm + SwiGLU)")
    i1 = synth.n1_inputs()
    w1 = (*quantize(i1["W0"], n1["gs"]), *quantize(i1["W1"], n1["gs"]))
    x1 = torch.from_numpy(i1["x"]).to(dev)
    y1 = (torch.empty(n1["N"], device=dev), torch.empty(n1["N"], device=dev))
    b1 = 2 * alg_bytes(n1["N"], n1["K"], n1["gs"], 0, n1["N"]) + 4 * n1["K"]
    calls.append(Call(f"dual 2x{n1['N']}x{n1['K']}", b1,
                      lambda s: q4.int4_matvec_dual(x1, *s, y0=y1[0], y1=y1[1]),
                      lambda r: clones(w1, r), wbytes(w1)))

    # M = 4 decode lanes of the same calls (matrix-core kernel).
    X1 = torch.from_numpy(synth.lanes(0x604, 4, n1["K"])).to(dev)
    Y1 = (torch.empty((4, n1["N"]), device=dev), torch.empty((4, n1["N"]), device=dev))
    b1m = 2 * alg_bytes(n1["N"], n1["K"], n1["gs"], 0, 4 * n1["N"]) + 4 * 4 * n1["K"]
    calls.append(Call(f"dual M=4 2x{n1['N']}x{n1['K']}", b1m,
                      lambda s: q4.int4_matvec_dual(X1, *s, y0=Y1[0], y1=Y1[1]),
                      lambda r: clones(w1, r), wbytes(w1)))

    i2 = synth.n2_inputs()
    w2 = quantize(i2["W"], n2["gs"])
    a2 = [torch.from_numpy(i2[k]).to(dev) for k in ("a", "gate")]
    y2 = torch.empty(n2["N"], device=dev)
    b2 = alg_bytes(n2["N"], n2["K"], n2["gs"], 2 * n2["K"], n2["N"])
    calls.append(Call(f"sigmoid-gated {n2['N']}x{n2['K']}", b2,
                      lambda s: q4.int4_matvec_sigmoid_gated(*a2, *s, y=y2),
                      lambda r: clones(w2, r), wbytes(w2)))

    i3 = synth.n3_inputs()
    w3 = quantize(i3["W"], n3["gs"])
    a3 = [torch.from_numpy(i3[k]).to(dev) for k in ("gate", "up")]
    y3 = torch.empty(n3["N"], device=dev)
    b3 = alg_bytes(n3["N"], n3["K"], n3["gs"], 2 * n3["K"], n3["N"])
    calls.append(Call(f"swiglu-gated {n3['N']}x{n3['K']}", b3,
                      lambda s: q4.int4_matvec_swiglu_gated(*a3, *s, y=y3),
                      lambda r: clones(w3, r), wbytes(w3)))

    i3g = synth.c3_inputs()
    c3 = synth.CONFIGS["c3"]
    w3g = (*quantize(i3g["Wg"], c3["gs"]), *quantize(i3g["Wu"], c3["gs"]))
    w3d = quantize(i3g["Wd"], c3["gs"])
    x3 = torch.from_numpy(i3g["x"]).to(dev)
    del i3g
    # The whole MLP block (gated pass + down projection) in one launch; the
    # bytes are those of the two separate calls (h written, then read).
    h3m = torch.empty(c3["N"], device=dev)
    y3m = torch.empty(c3["Nd"], device=dev)
    ws3 = torch.zeros(q4.int4_mlp_workspace_bytes() // 4, dtype=torch.int32, device=dev)
    b3f = (2 * alg_bytes(c3["N"], c3["K"], c3["gs"], 0, 0) + 4 * c3["K"] + 4 * c3["N"]
           + alg_bytes(c3["Nd"], c3["Kd"], c3["gs"], c3["Kd"], c3["Nd"]))
    calls.append(Call(f"MLP fused 2x{c3['N']}x{c3['K']} + {c3['Nd']}x{c3['Kd']}", b3f,
                      lambda s: q4.int4_mlp(x3, *s, h=h3m, y=y3m, workspace=ws3),
                      lambda r: clones((*w3g, *w3d), r), wbytes((*w3g, *w3d))))
    X3 = torch.from_numpy(synth.lanes(0x305, 4, c3["K"])).to(dev)
    H3 = torch.empty((4, c3["N"]), device=dev)
    b3m = 2 * alg_bytes(c3["N"], c3["K"], c3["gs"], 0, 0) + 4 * 4 * c3["K"] + 4 * 4 * c3["N"]
    calls.append(Call(f"gated M=4 2x{c3['N']}x{c3['K']}", b3m,
                      lambda s: q4.int4_matvec_gated_lanes(X3, *s, H=H3),
                      lambda r: clones(w3g, r), wbytes(w3g)))

    i4 = synth.n4_inputs()
    w4 = (*quantize(i4["Wg"], n4["gs"]), *quantize(i4["Wu"], n4["gs"]))
    a4 = [torch.from_numpy(i4[k]).to(dev) for k in ("a_a", "a_b", "w_norm")]
    h4 = torch.empty(n4["N"], device=dev)
    r4 = torch.empty(n4["K"], device=dev)
    b4 = 2 * alg_bytes(n4["N"], n4["K"], n4["gs"], 0, 0) + 4 * (3 * n4["K"] + n4["N"] + n4["K"])
    calls.append(Call(f"norm+swiglu 2x{n4['N']}x{n4['K']}", b4,
                      lambda s: q4.int4_matvec_norm_swiglu(*a4, n4["eps"], *s, h=h4, residual_out=r4),
                      lambda r: clones(w4, r), wbytes(w4)))

    i5 = synth.n5_inputs()
    n5 = synth.NEXT["n5"]
    w5 = quantize(i5["W"], n5["gs"])
    del i5["W"]
    for T in n5["Ts"]:
        ids = torch.from_numpy(i5["ids"][:T].copy()).to(dev)
        out = torch.empty((T, n5["K"]), device=dev)
        b5 = 4 * T + T * (n5["K"] // 2 + (n5["K"] // n5["gs"]) * 8) + 4 * T * n5["K"]
        calls.append(Call(f"embedding T={T} {n5['N']}x{n5['K']}", b5,
                          lambda s, ids=ids, out=out: q4.int4_embedding_gather(ids, *s, out=out),
                          lambda r: clones(w5, r), wbytes(w5)))

    # Per-layer-embedding rows gathered from a page-locked host table: the
    # table never enters HBM, so its copies are not rotated; the rows of
    # every call are different tokens (rotating id sets), and the bytes are
    # the T rows read over the host link plus ids and output.
    n7 = synth.NEXT["n7"]
    i7 = synth.n7_inputs()
    t7 = i7["table"]
    for T in n7["Ts"]:
        out = torch.empty((T, n7["K"]), device=dev)
        b7 = 4 * T + T * (n7["K"] // 2 + (n7["K"] // n7["gs"]) * 8) + 4 * T * n7["K"]
        id_sets = lambda r, T=T: [(torch.from_numpy(synth.token_ids(0xC10 + i, T, n7["N"])).to(dev),)
                                  for i in range(r)]
        calls.append(Call(f"PLE gather from a pinned host table T={T} {n7['N']}x{n7['K']}", b7,
                          lambda s, t7=t7, out=out: q4.int4_embedding_gather_host(s[0], *t7, out=out),
                          id_sets, 16 * 1024 * 1024))

    n6 = synth.NEXT["n6"]
    i6 = synth.n6_inputs(max(n6["Ts"]))
    w6 = quantize(i6["W"], n6["gs"])
    for T in n6["Ts"]:
        X6 = torch.from_numpy(i6["X"][:T].copy()).to(dev)
        Y6 = torch.empty((T, n6["N"]), device=dev)
        ws6 = torch.empty(q4.int4_gemm_workspace_bytes(T, n6["N"], n6["K"], n6["gs"]),
                          dtype=torch.uint8, device=dev)
        b6 = alg_bytes(n6["N"], n6["K"], n6["gs"], T * n6["K"], T * n6["N"])
        c6 = Call(f"prefill GEMM T={T} {n6['N']}x{n6['K']}", b6,
                  lambda s, X6=X6, Y6=Y6, ws6=ws6: q4.int4_gemm(X6, *s, Y=Y6, workspace=ws6),
                  lambda r: clones(w6, r), wbytes(w6))
        c6.flops = 2 * T * n6["N"] * n6["K"]
        calls.append(c6)
    return calls


def build_shards(q4, torch, dev):
    """One GPU's share of every call of the step under an 8-way split
    (synth.SHARD8): the same kernels at the shapes one of eight GPUs would
    run.  The down projection's partial y would be summed across GPUs (one
    16 KB all-reduce, not built here: one GPU only)."""
    sh = synth.SHARD8
    c2, c3, c4, c5 = (synth.CONFIGS[k] for k in ("c2", "c3", "c4", "c5"))
    w = synth.shard8_inputs()
    calls = []

    def quantize(W, gs):
        return q4.int4_quantize_pack(torch.from_numpy(W).to(dev), gs)

    def clones(tensors, r):
        sets = [tuple(tensors)]
        for _ in range(r - 1):
            sets.append(tuple(t.clone() for t in tensors))
        return sets

    def wbytes(ws):
        return sum(t.numel() * 4 for t in ws)

    s2 = sh["split4"]
    w2 = quantize(w["W2"], s2["gs"])
    x2 = torch.from_numpy(synth.normal_f32(0x201, c2["K"])).to(dev)
    o2 = tuple(torch.empty(n, device=dev) for n in (s2["n0"], s2["n1"] - s2["n0"], s2["n2"] - s2["n1"],
                                                     s2["N"] - s2["n2"]))
    calls.append(Call(f"split4 {s2['N']}x{s2['K']}", alg_bytes(s2["N"], s2["K"], s2["gs"], s2["K"], s2["N"]),
                      lambda s: q4.int4_matvec_split4(x2, *s, s2["n0"], s2["n1"], s2["n2"], outs=o2),
                      lambda r: clones(w2, r), wbytes(w2)))
    sg, sd = sh["gated"], sh["down"]
    wgu = (*quantize(w["Wg"], sg["gs"]), *quantize(w["Wu"], sg["gs"]))
    x3 = torch.from_numpy(synth.normal_f32(0x301, c3["K"])).to(dev)
    h3 = torch.empty(sg["N"], device=dev)
    calls.append(Call(f"gated 2x{sg['N']}x{sg['K']}",
                      2 * alg_bytes(sg["N"], sg["K"], sg["gs"], 0, 0) + 4 * sg["K"] + 4 * sg["N"],
                      lambda s: q4.int4_matvec_gated(x3, *s, h=h3), lambda r: clones(wgu, r), wbytes(wgu)))
    wd = quantize(w["Wd"], sd["gs"])
    y3 = torch.empty(sd["N"], device=dev)
    calls.append(Call(f"down (K share) {sd['N']}x{sd['K']}",
                      alg_bytes(sd["N"], sd["K"], sd["gs"], sd["K"], sd["N"]),
                      lambda s: q4.int4_matvec(h3, *s, Y=y3), lambda r: clones(wd, r), wbytes(wd)))
    # The same gate/up and down shares as one launch (int4_mlp): reported
    # beside the share step, not in it.
    ws3 = torch.zeros(q4.int4_mlp_workspace_bytes() // 4, dtype=torch.int32, device=dev)
    h3m = torch.empty(sg["N"], device=dev)
    y3m = torch.empty(sd["N"], device=dev)
    mlp = Call(f"MLP fused 2x{sg['N']}x{sg['K']} + {sd['N']}x{sd['K']}",
               2 * alg_bytes(sg["N"], sg["K"], sg["gs"], 0, 0) + 4 * sg["K"] + 4 * sg["N"]
               + alg_bytes(sd["N"], sd["K"], sd["gs"], sd["K"], sd["N"]),
               lambda s: q4.int4_mlp(x3, *s, h=h3m, y=y3m, workspace=ws3),
               lambda r: clones((*wgu, *wd), r), wbytes((*wgu, *wd)))
    mlp.in_step = False
    calls.append(mlp)
    s4 = sh["lmhead"]
    w4 = quantize(w["W4"], s4["gs"])
    i4 = {k: torch.from_numpy(v).to(dev) for k, v in (
        ("a_a", synth.normal_f32(0x401, c4["K"])), ("a_b", synth.normal_f32(0x402, c4["K"])),
        ("w_norm", synth.uniform_f32(0x403, c4["K"], 0.5, 1.5)))}
    y4 = torch.empty(s4["N"], device=dev)
    r4 = torch.empty(s4["K"], device=dev)
    n4 = torch.empty(s4["K"], device=dev)
    calls.append(Call(f"norm LM head {s4['N']}x{s4['K']}",
                      alg_bytes(s4["N"], s4["K"], s4["gs"], 3 * s4["K"], s4["N"] + 2 * s4["K"]),
                      lambda s: q4.int4_matvec_norm(i4["a_a"], i4["a_b"], i4["w_norm"], s4["eps"], *s, y=y4,
                                                    residual_out=r4, norm_out=n4),
                      lambda r: clones(w4, r), wbytes(w4)))
    s5 = sh["lanes"]
    w5 = quantize(w["W5"], s5["gs"])
    X5 = torch.from_numpy(synth.lanes(0x501, 8, c5["K"])).to(dev)
    for M in s5["Ms"]:
        wM = tuple(t.clone() for t in w5)
        XM = X5[:M].contiguous()
        YM = torch.empty((M, s5["N"]), device=dev)
        calls.append(Call(f"lanes M={M} {s5['N']}x{s5['K']}",
                          alg_bytes(s5["N"], s5["K"], s5["gs"], M * s5["K"], M * s5["N"]),
                          lambda s, XM=XM, YM=YM: q4.int4_matvec(XM, *s, Y=YM),
                          lambda r, wM=wM: clones(wM, r), wbytes(wM)))
    return calls


# ---------------------------------------------------------------- timing

def capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # eager warm-up on the capture stream (device queries, attributes)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_call(torch, call, replays=6):
    """Average duration of one call, from back-to-back calls over rotating copies."""
    r = max(2, min(64, -(-MALL_ROTATE_BYTES // max(call.weight_bytes, 1))))
    sets = call.sets_fn(r)
    g = capture(torch, lambda: [call.fn(s) for s in sets])
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (replays * r)
    del g, sets
    return us, r


def time_call_warm(torch, call, n=32, replays=6):
    """Average duration of one call repeated on the same buffers (cache-resident
    where the call's bytes fit the 256 MB MALL)."""
    s0 = call.sets_fn(1)[0]
    g = capture(torch, lambda: [call.fn(s0) for _ in range(n)])
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e3 / (replays * n)


# Launch shapes tried for the streaming-read ceiling: (blocks per CU, waves
# per block, 16-byte loads in flight per lane); the fastest is reported.
STREAM_SHAPES = ((1, 8, 4), (1, 16, 2), (2, 8, 2), (1, 8, 2), (2, 4, 4))


def stream_read_ceiling(q4, torch, dev, sizes, cus):
    """Time of one plain streaming read of each size (the library's probe
    kernel: buffer loads, XOR checksum, persistent grid), over rotating
    slices of >= 1 GiB so the MALL cannot serve it, best over STREAM_SHAPES."""
    out = {}
    sink = torch.empty(2 * cus, dtype=torch.int32, device=dev)
    for nbytes in sorted(set(sizes)):
        n16 = -(-nbytes // 16) * 16
        r = max(2, min(64, -(-MALL_ROTATE_BYTES // n16)))
        buf = torch.ones(r * n16 // 4, dtype=torch.float32, device=dev)
        best = None
        for bpc, waves, unroll in STREAM_SHAPES:
            blocks = bpc * cus

            def reads():
                for i in range(r):
                    q4.int4_probe_stream_read(buf[i * n16 // 4:(i + 1) * n16 // 4], sink[:blocks], blocks,
                                              waves, unroll)
            g = capture(torch, reads)
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(4):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (4 * r)
            if best is None or us < best[0]:
                best = (us, bpc, waves, unroll)
            del g
        out[nbytes] = {"us": round(best[0], 3), "GBps": round(nbytes / best[0] / 1e3, 1),
                       "shape": f"{best[1]} block(s)/CU x {best[2]} waves, {best[3]} loads in flight per lane"}
        log(f"streaming read {nbytes / 1e6:9.1f} MB {best[0]:9.2f} us {nbytes / best[0] / 1e3:8.1f} GB/s")
        del buf
    torch.cuda.empty_cache()
    return out


def cpu_baseline(single_budget_s=3.0):
    """The oracle (plain C, fp64 dot products) on the step's calls: all of every
    call on all the threads OpenMP gives it, and a bounded sample on one
    thread; each the median of three passes."""
    import oracle
    c2, c3, c4, c5 = (synth.CONFIGS[k] for k in ("c2", "c3", "c4", "c5"))

    def prep(frac):
        items = []
        W = synth.weights(0x202, max(1, int(c2["N"] * frac)), c2["K"])
        items.append(("matvec", synth.normal_f32(0x201, c2["K"]), oracle.quantize_pack(W, 128),
                      c2["K"], 128, 1))
        for seed in (0x302, 0x303):
            W = synth.weights(seed, max(1, int(c3["N"] * frac)), c3["K"])
            items.append(("matvec", synth.normal_f32(0x301, c3["K"]), oracle.quantize_pack(W, 128),
                          c3["K"], 128, 1))
        W = synth.weights(0x304, max(1, int(c3["Nd"] * frac)), c3["Kd"])
        items.append(("matvec", synth.normal_f32(0x30A, c3["Kd"]), oracle.quantize_pack(W, 128),
                      c3["Kd"], 128, 1))
        W = synth.weights(0x404, max(1, int(c4["N"] * frac)), c4["K"])
        items.append(("norm", None, oracle.quantize_pack(W, 128), c4["K"], 128, 1))
        del W
        W = synth.weights(0x502, max(1, int(c5["N"] * frac)), c5["K"])
        w5 = oracle.quantize_pack(W, 64)
        for M in c5["Ms"]:
            items.append(("matvec", synth.lanes(0x501, M, c5["K"]), w5, c5["K"], 64, M))
        return items

    i4 = synth.c4_inputs(N=1)

    def run(items):
        nbytes = 0
        t0 = time.perf_counter()
        for kind, x, (q, s, z), K, gs, M in items:
            N = q.shape[0]
            if kind == "norm":
                oracle.norm(i4["a_a"], i4["a_b"], i4["w_norm"], 1e-6, q, s, z, K, gs)
                nbytes += alg_bytes(N, K, gs, 3 * K, N + 2 * K)
            else:
                oracle.matvec(x, q, s, z, K, gs)
                nbytes += alg_bytes(N, K, gs, M * K, M * N)
        return nbytes, time.perf_counter() - t0

    def median3(items):
        runs = sorted((run(items) for _ in range(3)), key=lambda bt: bt[0] / bt[1])
        return runs[1]

    threads = oracle.max_threads()
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    full = prep(1.0)
    nb_all, dt_all = median3(full)
    del full
    log(f"cpu baseline: whole step on {threads} threads, {dt_all:.2f}s per pass (median of 3)")
    oracle.set_threads(1)
    try:
        probe = 0.002
        nb, dt = run(prep(probe))
        frac = min(1.0, probe * single_budget_s / max(dt, 1e-6))
        items = prep(frac)
        nb_one, dt_one = median3(items)
    finally:
        oracle.set_threads(threads)
    log(f"cpu baseline: f={frac:.4f} of the step on one thread, {dt_one:.2f}s per pass (median of 3)")
    return {"value": round(nb_all / dt_all / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": (f"every column of every call of the step ({nb_all / 1e6:.1f} MB algorithmic), "
                       f"median of 3 passes of {dt_all:.2f} s, {threads} OpenMP threads over output columns; "
                       "plain C oracle, fp64 dot products"),
            "host_cpus": os.cpu_count(), "host_cpus_usable": affinity,
            "single_thread": {"value": round(nb_one / dt_one / 1e9, 3), "unit": "GB/s", "cores": 1,
                              "sample": (f"first {frac:.4f} of the columns of every call of the step "
                                         f"({nb_one / 1e6:.1f} MB algorithmic), median of 3 passes "
                                         f"of {dt_one:.2f} s")}}


# Calls the counter probe launches, in this order, each PROBE_REPS times on
# rotating weight copies: (label, kind, N, K, gs, M).  The labels name the
# rows of the counter summaries in profiles/.
PROBE_CALLS = (
    ("split4 6656x4096", "split4", 6656, 4096, 128, 1),
    ("gated 2x14336x4096", "gated", 14336, 4096, 128, 1),
    ("down 4096x14336", "plain", 4096, 14336, 128, 1),
    ("norm LM head 151936x4096", "norm", 151936, 4096, 128, 1),
    ("lanes M=1 25600x5120", "plain", 25600, 5120, 64, 1),
    ("lanes M=2 25600x5120", "plain", 25600, 5120, 64, 2),
    ("lanes M=4 25600x5120", "plain", 25600, 5120, 64, 4),
    ("lanes M=8 25600x5120", "plain", 25600, 5120, 64, 8),
    ("MLP fused 2x14336x4096 + 4096x14336", "mlp", 14336, 4096, 128, 1),
    ("prefill GEMM T=512 4096x4096", "gemm", 4096, 4096, 128, 512),
    ("prefill GEMM T=4096 4096x4096", "gemm", 4096, 4096, 128, 4096),
)
PROBE_REPS = 5
PROBE_COPY_BYTES = 1 << 28


def counter_probe(q4, torch, dev):
    """Launches for hardware-counter runs: every call of the step, the fused
    MLP block and the prefill GEMM (whose prep launch comes first each time),
    PROBE_REPS times each on rotating weight copies (random codes:
    the bytes a launch moves do not depend on the values), then PROBE_REPS
    plain elementwise copies of PROBE_COPY_BYTES whose bytes are known, used
    to calibrate the FETCH_SIZE / WRITE_SIZE counters.  Prints the dispatch
    order on stderr."""
    g = torch.Generator(device=dev)
    g.manual_seed(4)

    def triplet(N, K, gs):
        q = torch.randint(-2**31, 2**31 - 1, (N, K // 8), dtype=torch.int32, device=dev, generator=g)
        s_ = torch.rand((N, K // gs), device=dev, generator=g) * 1e-2
        z = torch.randint(0, 16, (N, K // gs), device=dev, generator=g).float()
        return q, s_, z

    def vec(*shape):
        return torch.randn(*shape, device=dev, generator=g)

    copies = 2
    for label, kind, N, K, gs, M in PROBE_CALLS:
        if kind == "gated":
            sets = [(*triplet(N, K, gs), *triplet(N, K, gs)) for _ in range(copies)]
            x, h = vec(K), torch.empty(N, device=dev)
            fn = lambda w: q4.int4_matvec_gated(x, *w, h=h)
        elif kind == "mlp":
            sets = [(*triplet(N, K, gs), *triplet(N, K, gs), *triplet(K, N, gs)) for _ in range(copies)]
            x, h, y = vec(K), torch.empty(N, device=dev), torch.empty(K, device=dev)
            ws = torch.zeros(q4.int4_mlp_workspace_bytes() // 4, dtype=torch.int32, device=dev)
            fn = lambda w: q4.int4_mlp(x, *w, h=h, y=y, workspace=ws)
        elif kind == "norm":
            sets = [triplet(N, K, gs) for _ in range(copies)]
            a = [vec(K) for _ in range(3)]
            y, r, n = (torch.empty(m, device=dev) for m in (N, K, K))
            fn = lambda w: q4.int4_matvec_norm(*a, 1e-6, *w, y=y, residual_out=r, norm_out=n)
        elif kind == "gemm":
            sets = [triplet(N, K, gs) for _ in range(copies)]
            X, Y = vec(M, K), torch.empty((M, N), device=dev)
            ws = torch.empty(q4.int4_gemm_workspace_bytes(M, N, K, gs), dtype=torch.uint8, device=dev)
            fn = lambda w: q4.int4_gemm(X, *w, Y=Y, workspace=ws)
        elif kind == "split4":
            sets = [triplet(N, K, gs) for _ in range(copies)]
            x = vec(K)
            outs = tuple(torch.empty(m, device=dev) for m in (4096, 1024, 1024, 512))
            fn = lambda w: q4.int4_matvec_split4(x, *w, 4096, 5120, 6144, outs=outs)
        else:
            sets = [triplet(N, K, gs) for _ in range(copies)]
            X, Y = vec(M, K), torch.empty((M, N), device=dev)
            fn = lambda w: q4.int4_matvec(X, *w, Y=Y)
        for i in range(PROBE_REPS):
            fn(sets[i % copies])
        torch.cuda.synchronize()
        log(f"counter probe: {PROBE_REPS} x {label}")
        del sets
        torch.cuda.empty_cache()
    src = torch.empty(PROBE_COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(PROBE_REPS):
        torch.mul(src, 1.0, out=dst)  # one elementwise kernel: reads and writes PROBE_COPY_BYTES
    torch.cuda.synchronize()
    log(f"counter probe: {PROBE_REPS} x elementwise copy of {PROBE_COPY_BYTES} bytes")


# Shapes of the fixed-cost sweep: (label, kind, K, gs, column counts).  The
# split4 rows keep the 6656-column call's routing proportions.
FIXED_COST_SWEEPS = (
    ("one-lane matvec K=5120 gs64 (the lanes M=1 kernel)", "plain", 5120, 64,
     (256, 1024, 2048, 4096, 8192, 12800, 19200, 25600)),
    ("split4 K=4096 gs128", "split4", 4096, 128, (256, 832, 1664, 3328, 4992, 6656)),
)
FIXED_COST_K = (1024, 2048, 4096, 8192, 16384)  # one-lane K sweep at 256 columns, gs 128


def fit_line(xs, ys):
    """Least-squares y = a + b x."""
    n = len(xs)
    mx, my = sum(xs) / n, sum(ys) / n
    b = sum((x - mx) * (y - my) for x, y in zip(xs, ys)) / sum((x - mx) ** 2 for x in xs)
    return my - b * mx, b


def fixed_cost(q4, torch, dev, cus):
    """Splits a call's time into a part that does not grow with the bytes it
    streams and a part that does: each sweep times the call at several column
    counts (rotating copies, as the per-call rows) and the streaming-read probe
    at the same byte counts, and fits t = a + b * bytes to both.  The probe's
    intercept is the fixed cost of any launch that reads memory (dispatch,
    first round trip to HBM, drain); the call's intercept minus the probe's is
    what the call adds once per launch (activation staging, the partial-sum
    epilogue).  A K sweep at 256 columns shows how the staging grows with K."""
    g = torch.Generator(device=dev)
    g.manual_seed(5)

    def triplet(N, K, gs):
        q = torch.randint(-2**31, 2**31 - 1, (N, K // 8), dtype=torch.int32, device=dev, generator=g)
        s_ = torch.rand((N, K // gs), device=dev, generator=g) * 1e-2
        z = torch.randint(0, 16, (N, K // gs), device=dev, generator=g).float()
        return q, s_, z

    def call_for(kind, N, K, gs):
        w = triplet(N, K, gs)
        x = torch.randn(K, device=dev, generator=g)
        nbytes = alg_bytes(N, K, gs, K, N)
        sets = lambda r: [w] + [tuple(t.clone() for t in w) for _ in range(r - 1)]
        wb = sum(t.numel() * 4 for t in w)
        if kind == "split4":
            n0, n1, n2 = (N * 4096) // 6656, (N * 5120) // 6656, (N * 6144) // 6656
            outs = tuple(torch.empty(m, device=dev) for m in (n0, n1 - n0, n2 - n1, N - n2))
            return Call(f"split4 {N}x{K}", nbytes, lambda s: q4.int4_matvec_split4(x, *s, n0, n1, n2, outs=outs),
                        sets, wb)
        y = torch.empty(N, device=dev)
        return Call(f"matvec {N}x{K}", nbytes, lambda s: q4.int4_matvec(x, *s, Y=y), sets, wb)

    out = {"method": "t = a + b * bytes fitted to the call and to the streaming-read probe at the "
                     "same byte counts; a_call - a_probe is what the call adds once per launch",
           "sweeps": {}, "k_sweep": {}}
    for label, kind, K, gs, Ns in FIXED_COST_SWEEPS:
        rows = []
        for N in Ns:
            c = call_for(kind, N, K, gs)
            us, _ = time_call(torch, c)
            rows.append((N, c.nbytes, us))
            log(f"fixed-cost sweep {label}: N={N} {us:.2f} us")
            del c
            torch.cuda.empty_cache()
        probe = stream_read_ceiling(q4, torch, dev, [b for _, b, _ in rows], cus)
        xs = [b for _, b, _ in rows]
        a_k, b_k = fit_line(xs, [us for _, _, us in rows])
        a_p, b_p = fit_line(xs, [probe[b]["us"] for b in xs])
        out["sweeps"][label] = {
            "rows": [{"N": N, "alg_bytes": b, "us": round(us, 3), "probe_us": probe[b]["us"]}
                     for N, b, us in rows],
            "call_intercept_us": round(a_k, 3), "call_slope_GBps": round(1e-3 / b_k, 1),
            "probe_intercept_us": round(a_p, 3), "probe_slope_GBps": round(1e-3 / b_p, 1),
            "call_adds_per_launch_us": round(a_k - a_p, 3)}
        log(f"fixed-cost {label}: call {a_k:.2f} us + bytes at {1e-3 / b_k:.0f} GB/s; probe {a_p:.2f} us "
            f"+ bytes at {1e-3 / b_p:.0f} GB/s")
    for K in FIXED_COST_K:
        c = call_for("plain", 256, K, 128)
        us, _ = time_call(torch, c)
        out["k_sweep"][str(K)] = {"N": 256, "alg_bytes": c.nbytes, "us": round(us, 3)}
        log(f"fixed-cost K sweep: 256x{K} {us:.2f} us")
        del c
        torch.cuda.empty_cache()
    probe = stream_read_ceiling(q4, torch, dev, [v["alg_bytes"] for v in out["k_sweep"].values()], cus)
    for v in out["k_sweep"].values():
        v["probe_us"] = probe[v["alg_bytes"]]["us"]
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (the JSON then carries cpu_baseline null)")
    ap.add_argument("--no-shards", action="store_true",
                    help="skip the 1/8-share calls (the JSON then carries one_gpu_share_of_8 null); "
                         "a kernel trace then holds only the full-size launches of each kernel")
    ap.add_argument("--counter-probe", action="store_true",
                    help="only launch every call of the step and the fused MLP block, then a plain "
                         "256 MiB device copy, 5 times each, for rocprofv3 --pmc runs (prints no JSON)")
    ap.add_argument("--fixed-cost", action="store_true",
                    help="only run the fixed-cost sweeps (calls and the streaming-read probe at several "
                         "sizes, fitted to a + b * bytes) and print them as one JSON line")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the int4 matvec path here has no multi-GPU "
              "mode (it would shard by output columns, and the MLP down projection by K with "
              "one small all-reduce per layer; the JSON reports one GPU's share of an 8-way "
              "split); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import int4_group_quantized_quant_amd as q4

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name} {getattr(props, 'gcnArchName', '?')} CUs={props.multi_processor_count}")

    if args.counter_probe:
        counter_probe(q4, torch, dev)
        return
    if args.fixed_cost:
        print(json.dumps({"fixed_cost": fixed_cost(q4, torch, dev, props.multi_processor_count)}), flush=True)
        return

    calls, quant, keep = build_workload(q4, torch, dev)
    step_bytes = sum(c.nbytes for c in calls)

    # Per-call durations (rotating copies, graphs of back-to-back calls); the
    # single small matvec is timed the same way but is not part of the step.
    per_call = {}
    for c in [build_single(q4, torch, dev)] + calls:
        us, r = time_call(torch, c)
        warm = time_call_warm(torch, c)
        per_call[c.name] = {"us_per_call": round(us, 3), "GBps": round(c.nbytes / us / 1e3, 1),
                            "pct_peak": round(100 * c.nbytes / us / 1e3 / PEAK_GBS, 1),
                            "alg_bytes": c.nbytes, "rotating_copies": r,
                            "warm_us_per_call": round(warm, 3),
                            "dtype": ("f32 activations split into fp16 hi + lo on the matrix cores, "
                                      "fp32 accumulation" if re.search(r"M=[2-8]", c.name) else "f32")}
        log(f"{c.name:28s} {us:9.2f} us  {c.nbytes / us / 1e3:8.1f} GB/s  "
            f"({100 * c.nbytes / us / 1e3 / PEAK_GBS:5.1f}% of 8 TB/s)")

    # Next-row calls, timed alone (not part of the step).
    next_rows = {}
    for c in build_next(q4, torch, dev):
        us, r = time_call(torch, c)
        next_rows[c.name] = {"us_per_call": round(us, 3), "GBps": round(c.nbytes / us / 1e3, 1),
                             "pct_peak": round(100 * c.nbytes / us / 1e3 / PEAK_GBS, 1),
                             "alg_bytes": c.nbytes, "rotating_copies": r}
        flops = getattr(c, "flops", None)
        if flops:
            tf = flops / us / 1e6
            next_rows[c.name].update({"alg_flops": flops, "TFLOPs": round(tf, 1),
                                      "pct_fp16_mfma_peak": round(100 * tf / PEAK_FP16_TFLOPS, 1)})
            log(f"{c.name:28s} {us:9.2f} us  {tf:8.1f} TFLOP/s ({100 * tf / PEAK_FP16_TFLOPS:5.1f}% of "
                f"the 2.5 PFLOP/s fp16 matrix peak; two fp16 products per term)  [next row]")
            continue
        log(f"{c.name:28s} {us:9.2f} us  {c.nbytes / us / 1e3:8.1f} GB/s  "
            f"({100 * c.nbytes / us / 1e3 / PEAK_GBS:5.1f}% of 8 TB/s)  [next row, not in the step]")
        del c
    torch.cuda.empty_cache()

    # One GPU's share of the step under an 8-way split: each call alone, then
    # the shard calls captured together as one step (not the metric).
    shard = None
    shard_calls = [] if args.no_shards else build_shards(q4, torch, dev)
    if shard_calls:
        log("one GPU's share of each call under an 8-way split")
        shard_rows = {}
        for c in shard_calls:
            us, r = time_call(torch, c)
            shard_rows[c.name] = {"us_per_call": round(us, 3), "GBps": round(c.nbytes / us / 1e3, 1),
                                  "pct_peak": round(100 * c.nbytes / us / 1e3 / PEAK_GBS, 1),
                                  "alg_bytes": c.nbytes, "rotating_copies": r}
            tag = "[1/8 share]" if getattr(c, "in_step", True) else "[1/8 share, not in the share step]"
            log(f"{c.name:28s} {us:9.2f} us  {c.nbytes / us / 1e3:8.1f} GB/s  "
                f"({100 * c.nbytes / us / 1e3 / PEAK_GBS:5.1f}% of 8 TB/s)  {tag}")
        shard_calls = [c for c in shard_calls if getattr(c, "in_step", True)]
        shard_sets = [c.sets_fn(1)[0] for c in shard_calls]
        shard_graph = capture(torch, lambda: [c.fn(s) for c, s in zip(shard_calls, shard_sets)])
        for _ in range(3):
            shard_graph.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(50):
            shard_graph.replay()
        e1.record()
        torch.cuda.synchronize()
        shard_us = e0.elapsed_time(e1) * 1e3 / 50
        shard_bytes = sum(c.nbytes for c in shard_calls)
        log(f"1/8 share of the step: {shard_us:.1f} us, {shard_bytes / 1e6:.1f} MB")
        shard = {"shards": 8, "split": "columns for split4 (each range in eighths), gate/up, the LM head "
                                       "and the lanes; K for down (its partial y needs one 16 KB "
                                       "all-reduce across GPUs, not built: one GPU only)",
                 "step_us": round(shard_us, 2), "step_alg_bytes": shard_bytes,
                 "step_GBps": round(shard_bytes / shard_us / 1e3, 1), "per_call": shard_rows}
        del shard_graph, shard_sets, shard_calls
        torch.cuda.empty_cache()

    # The step graph.
    sets = [c.sets_fn(1)[0] for c in calls]
    step = capture(torch, lambda: [c.fn(s) for c, s in zip(calls, sets)])
    # Graph replays must reproduce the eager result bit for bit.
    y_graph_ref = keep["y4"].clone()
    for _ in range(args.warmup):
        step.replay()
    torch.cuda.synchronize()
    assert torch.equal(keep["y4"], y_graph_ref), "graph replay differs from the eager call"

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    log(f"step: {ms_per_step * 1e3:.1f} us, {step_bytes / 1e6:.1f} MB, wall {wall:.3f}s")
    assert torch.equal(keep["y4"], y_graph_ref), "graph replay differs from the eager call"

    dom = per_call["norm LM head 151936x4096"]
    traffic = read_traffic()
    roofline = {"bound": "hbm", "achieved": round(dom["alg_bytes"] / dom["us_per_call"] / 1e3, 1),
                "peak": PEAK_GBS, "unit": "GB/s",
                "frac": round(dom["alg_bytes"] / dom["us_per_call"] / 1e3 / PEAK_GBS, 4),
                "traffic": traffic, "kernel": "gemv_reg_kernel<M=1,NCOL=4,kNorm> (int4_matvec_norm)",
                "alg_bytes_per_launch": dom["alg_bytes"], "us_per_launch": dom["us_per_call"]}

    # The streaming-read ceiling at every call's size, and each call's share of it.
    # (Not for the GEMM, bound by the matrix cores, nor for the host-table
    # gather, whose bytes cross the host link.)
    def hbm_row(name, v):
        return "TFLOPs" not in v and "host table" not in name
    ceiling = stream_read_ceiling(q4, torch, dev, [v["alg_bytes"] for v in per_call.values()]
                                  + [v["alg_bytes"] for k, v in next_rows.items() if hbm_row(k, v)],
                                  props.multi_processor_count)
    for rows in (per_call, next_rows):
        for k, v in rows.items():
            if v["alg_bytes"] in ceiling and hbm_row(k, v):
                v["stream_read_us"] = ceiling[v["alg_bytes"]]["us"]
                v["pct_of_stream_read"] = round(100 * ceiling[v["alg_bytes"]]["us"] / v["us_per_call"], 1)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline()

    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 (lanes M=2,4,8: f32 activations split into fp16 hi + lo, fp32 accumulation)",
        "data": "synthetic",
        "config": {"workload": ("decode step: split4 6656x4096 + gated MLP 2x14336x4096 + "
                                "down 4096x14336 + norm LM head 151936x4096 (gs 128) + "
                                "lanes M=1,2,4,8 25600x5120 (gs 64)"),
                   "alg_bytes_per_step": step_bytes, "pct_of_8TBps": round(100 * value / PEAK_GBS, 1),
                   "weights": "int4 codes + fp32 scale/zero per group, N(0,0.02) seeded"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "per_call": per_call,
        "next_rows": next_rows,
        "one_gpu_share_of_8": shard,
        "stream_read_ceiling": {str(k): v for k, v in ceiling.items()},
        "quantize_pack": {"elements": quant["elements"], "seconds": round(quant["seconds"], 5),
                          "GBps_fp32_in": round(4 * quant["elements"] / quant["seconds"] / 1e9, 1),
                          "GBps_alg": round((4.5 * quant["elements"] + 8 * quant["groups"])
                                            / quant["seconds"] / 1e9, 1),
                          "timing": "HIP events around each matrix's launch (after a one-row warm-up)"},
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", None),
                   "cus": props.multi_processor_count, "hip": torch.version.hip},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

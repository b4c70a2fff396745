#!/usr/bin/env python3
"""Benchmark of the MI355X scaled linear layer with a fused epilogue.

Headline workload (one "step"): the FP8-dynamic decode linear, A[M,4096] e4m3
against a B[6144,4096] e4m3 weight with per-token x per-channel scales and a
bias, at every token count M in {1, 2, 4, 8, 16, 24, 32}; at each M the step
runs one call per weight copy of a 16-copy rotation (16 distinct weight
buffers, 384 MiB in all, so the 256 MB MALL cannot serve repeated reads --
as 16 layers of a model would).  value = algorithmic HBM bytes of the step /
its time, in TB/s.

Timing follows the graph-replay discipline of the vLLM linear-backend
write-up: each M's calls are captured once into a HIP graph and replayed, so
kernels run back to back without host launch gaps; HIP events on the launch
stream bracket every replay.  The per-shape table covers all five workloads
(TFLOP/s, TB/s and their roofline fractions) and the unfused three-kernel
prefill path.  The CPU oracle is timed on a bounded sample for the
cpu_baseline field.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-shapes]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12                                     # bytes/s
# Dense MFMA peaks per operand dtype.  mxfp4 pairs 4-bit weights with bf16
# activations: no fp4 x fp4 instruction applies, the contraction is bf16.
MFMA_PEAK = {"bf16": 2.5e15, "fp16": 2.5e15, "fp8_dynamic": 5.0e15, "block_fp8": 5.0e15,
             "w8a8_int8": 5.0e15, "mxfp4": 2.5e15}
RIDGE = {q: MFMA_PEAK[q] / HBM_PEAK for q in MFMA_PEAK}
E4M3_WIDENED = ("fp8_dynamic", "block_fp8")            # contracted by the bf16 MFMA
HEAD_CFG = 2
NCOPY_TARGET_BYTES = 384 << 20                        # rotation footprint > 256 MB MALL
METRIC = "TFLOP/s & HBM TB/s (fraction of roofline) per shape, M∈{1..32} and M=4096"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-shapes", action="store_true", help="skip the per-shape table")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--reps", type=int, default=20, help="graph replays per shape in the table")
    ap.add_argument("--counters", action="store_true",
                    help="short run for rocprofv3 --pmc passes: the headline graphs for two "
                         "steps, then a plain 256 MiB device copy that calibrates the counters")
    ap.add_argument("--counters-shapes", default=None, metavar="CFG:M[,M...][;CFG:M...]",
                    help="counter run: three calls of each listed workload shape (two weight "
                         "copies), then the 256 MiB copy; e.g. 4:512,2048;2:1,32")
    ap.add_argument("--counters-prefill", action="store_true",
                    help="short run for rocprofv3 --pmc passes on the 4096^3 bf16 prefill: two "
                         "fused calls, two unfused three-kernel calls, then the 256 MiB copy")
    return ap.parse_args()


def counters_copy(torch):
    """A plain 256 MiB device-to-device copy whose counter readings calibrate
    FETCH_SIZE / WRITE_SIZE (bytes moved are known)."""
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()


def counters_prefill(torch, h):
    import synth
    c = synth.WORKLOADS[5]
    wl = Workload(torch, 5, c["Ms"], ncopy=2)
    M = c["Ms"][0]
    d = wl.dev[M]
    T = torch.empty_like(d["C"])
    U = torch.empty_like(d["C"])
    for r in range(2):
        wl.call(h, M, r)
    torch.cuda.synchronize()
    for r in range(2):
        h.run_unfused(d["A"], wl.B[r], d["C"], T, U, quant=wl.quant, act=wl.act,
                      alpha=d["alpha"], bias=wl.bias, residual=d["residual"])
    torch.cuda.synchronize()
    counters_copy(torch)
    print(json.dumps({"counters_run": "prefill", "copy_bytes": 256 << 20,
                      "fused_algorithmic_bytes": wl.bytes(M),
                      "tensor_bytes": 2 * M * wl.N, "M": M, "N": wl.N, "K": wl.K}), flush=True)


def counters_shapes(torch, h, spec):
    """Three calls of each workload shape in `spec` ("cfg:M,M;cfg:M") over two
    weight copies, then the calibration copy; for rocprofv3 counter passes."""
    import synth
    out = []
    for part in spec.split(";"):
        cfg, ms = part.split(":")
        cfg, ms = int(cfg), [int(m) for m in ms.split(",")]
        wl = Workload(torch, cfg, ms, ncopy=2)
        for M in ms:
            for r in range(3):
                wl.call(h, M, r)
            torch.cuda.synchronize()
            out.append(dict(cfg=cfg, M=M, N=wl.N, K=wl.K, variant=h.describe(wl.quant, M, wl.N, wl.K),
                            algorithmic_bytes=wl.bytes(M), flops=wl.flops(M)))
        del wl
        torch.cuda.empty_cache()
    counters_copy(torch)
    print(json.dumps({"counters_run": "shapes", "copy_bytes": 256 << 20, "shapes": out}),
          flush=True)


def source_digest():
    """Hash of the kernel sources, .hip and .hpp (to tell whether stored
    counters still apply; the variant table and host code do not change a
    kernel's traffic)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "epilogue_scaled_gemm_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if not name.endswith((".hip", ".hpp")):
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


class Workload:
    """Device operands of one workload, with a rotation of weight copies."""

    def __init__(self, torch, cfg, Ms, quant=None, ncopy=None):
        import synth
        self.torch = torch
        self.cfg = cfg
        self.Ms = list(Ms)
        self.probs = {M: synth.make(cfg, M, quant) for M in self.Ms}
        p0 = self.probs[self.Ms[0]]
        self.quant, self.act, self.N, self.K = p0.quant, p0.act, p0.N, p0.K
        wbytes = p0.B.nbytes
        self.ncopy = ncopy or max(2, min(32, -(-NCOPY_TARGET_BYTES // wbytes)))
        B0 = self._dev(p0.B)
        self.B = [B0] + [B0.clone() for _ in range(self.ncopy - 1)]
        self.sb = self._dev(p0.sb)
        self.bias = self._dev(p0.bias)
        self.dev = {}
        for M, p in self.probs.items():
            self.dev[M] = dict(A=self._dev(p.A), sa=self._dev(p.sa), residual=self._dev(p.residual),
                               C=torch.empty((M, p.N), dtype=torch.int16, device="cuda"),
                               alpha=p.alpha)

    def _dev(self, a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return self.torch.from_numpy(np.ascontiguousarray(a)).cuda()

    def call(self, h, M, copy):
        d = self.dev[M]
        h.run(d["A"], self.B[copy % self.ncopy], d["C"], quant=self.quant, act=self.act,
              sa=d["sa"], sb=self.sb, alpha=d["alpha"], bias=self.bias, residual=d["residual"])

    def bytes(self, M):
        import synth
        p = self.probs[M]
        return synth.algorithmic_bytes(self.quant, M, self.N, self.K, p.bias is not None,
                                       p.residual is not None)

    def flops(self, M):
        return 2 * M * self.N * self.K

    def graph(self, h, M, reps, offset=0):
        """A HIP graph of `reps` calls at token count M over rotating copies."""
        torch = self.torch
        self.call(h, M, offset)               # warm (workspace allocation)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(reps):
                self.call(h, M, offset + r)
        return g


def time_graphs(torch, graphs, reps):
    """Median time (s) of one replay of each graph over `reps` rounds of
    replays, the graphs interleaved within a round so they see the same
    clock and power state; HIP events bracket every replay."""
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in graphs] for _ in range(reps)]
    for r in range(reps):
        for g, (s, e) in zip(graphs, ev[r]):
            s.record()
            g.replay()
            e.record()
    torch.cuda.synchronize()
    return [float(np.median([ev[r][i][0].elapsed_time(ev[r][i][1]) for r in range(reps)])) / 1e3
            for i in range(len(graphs))]


def shape_row(name, quant, M, N, K, t, nbytes, flops, variant, kernel_calls=1):
    ai = flops / nbytes
    bound = "mfma" if ai > RIDGE[quant] else "hbm"
    tbs, tfs = nbytes / t, flops / t
    row = dict(shape=name, quant=quant, M=M, N=N, K=K, variant=variant, us=round(t * 1e6, 3),
               TBps=round(tbs / 1e12, 4), TFLOPs=round(tfs / 1e12, 3),
               hbm_frac=round(tbs / HBM_PEAK, 4), mfma_frac=round(tfs / MFMA_PEAK[quant], 4),
               bound=bound, kernels_per_call=kernel_calls,
               roof_frac=round((tbs / HBM_PEAK) if bound == "hbm" else (tfs / MFMA_PEAK[quant]), 4))
    if quant in E4M3_WIDENED:
        # e4m3 operands are widened exactly to bf16 and multiplied by the
        # bf16 MFMA: the rate the kernels can reach is the bf16 one.
        row["mfma_frac_bf16_rate"] = round(tfs / MFMA_PEAK["bf16"], 4)
    return row


CEILING_MIB = (12, 24, 48, 96)                       # the decode workloads' weight sizes
CEILING_LAUNCH = [(g, u) for g in (512, 1024, 2048, 4096) for u in (4, 8, 16)]


def stream_ceiling(torch, h, reps):
    """Measured HBM read ceiling: lin_gemm_stream_read (a kernel that only
    reads) over the same kind of rotation as the decode rows (copies of the
    buffer totalling >= 384 MiB, one call per copy per graph replay), for
    each weight size of the decode workloads and a few launch shapes; the
    fastest launch shape is the ceiling for that byte count."""
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    out = []
    for mib in CEILING_MIB:
        nb = mib << 20
        ncopy = max(2, min(32, -(-NCOPY_TARGET_BYTES // nb)))
        bufs = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(ncopy)]
        for b in bufs:
            b.fill_(1)
        graphs = []
        for grid, unroll in CEILING_LAUNCH:
            h.stream_read(bufs[0], sink, grid, unroll)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for b in bufs:
                    h.stream_read(b, sink, grid, unroll)
            graphs.append(g)
        ts = [t / ncopy for t in time_graphs(torch, graphs, max(5, reps))]
        i = int(np.argmin(ts))
        row = dict(MiB=mib, bytes=nb, copies=ncopy, us=round(ts[i] * 1e6, 3),
                   TBps=round(nb / ts[i] / 1e12, 4), hbm_frac=round(nb / ts[i] / HBM_PEAK, 4),
                   grid=CEILING_LAUNCH[i][0], unroll=CEILING_LAUNCH[i][1],
                   all_us={f"{g}x{u}": round(t * 1e6, 3) for (g, u), t in zip(CEILING_LAUNCH, ts)})
        out.append(row)
        print(f"[ceiling] {row}", file=sys.stderr, flush=True)
        del graphs, bufs
    torch.cuda.empty_cache()
    return out


def ceiling_us(ceiling, weight_bytes):
    """The measured read time of the ceiling entry for exactly this byte
    count, else None."""
    for c in ceiling or []:
        if c["bytes"] == weight_bytes:
            return c["us"]
    return None


def per_shape_table(torch, h, reps):
    import synth
    rows = []
    for cfg in (1, 2, 3, 4, 5, 6, 7, 8):
        c = synth.WORKLOADS[cfg]
        wl = Workload(torch, cfg, c["Ms"])
        for M in c["Ms"]:
            R = wl.ncopy
            graphs = [wl.graph(h, M, R)]
            keep = None
            if cfg == 5:
                gu, keep = unfused_graph(torch, h, wl, M)
                graphs.append(gu)
            ts = time_graphs(torch, graphs, max(3, reps // (1 if M < 512 else 4)))
            rows.append(shape_row(c["name"], wl.quant, M, wl.N, wl.K, ts[0] / R, wl.bytes(M),
                                  wl.flops(M), h.describe(wl.quant, M, wl.N, wl.K)))
            print(f"[shape] {rows[-1]}", file=sys.stderr, flush=True)
            if cfg == 5:
                # compulsory bytes: the fused traffic plus a write and a read of T and of U
                nbytes = wl.bytes(M) + 2 * 2 * (2 * M * wl.N)
                rows.append(shape_row("prefill_bf16_unfused_3kernel", wl.quant, M, wl.N, wl.K,
                                      ts[1] / R, nbytes, wl.flops(M),
                                      "gemm + bias_act + scale_residual", kernel_calls=3))
                print(f"[shape] {rows[-1]}", file=sys.stderr, flush=True)
            del graphs, keep
        del wl
        torch.cuda.empty_cache()
    return rows


def dynamic_quant_rows(torch, h, reps):
    """The dynamic activation quantization: the kernel alone (per-token e4m3
    and int8, 1x128-block e4m3) over a rotation of activation copies, and the
    FP8 decode with quantization in front (lin_gemm_run_dynamic) beside the
    same decode on pre-quantized activations.  HBM-bound: the compulsory
    bytes of the kernel are 2 per value read, 1 per code written and 4 per
    scale."""
    import synth
    rows = []
    kinds = [("fp8_token", "fp8_dynamic", 1, 4096), ("fp8_token", "fp8_dynamic", 32, 4096),
             ("fp8_token", "fp8_dynamic", 4096, 4096), ("int8_token", "w8a8_int8", 4096, 4096),
             ("fp8_block", "block_fp8", 4096, 12288)]
    for kind, quant, M, K in kinds:
        X = synth.activations16(M, K, seed=M + K)
        xb = 2 * M * K
        ncopy = max(2, min(16, -(-NCOPY_TARGET_BYTES // xb)))
        Xs = [torch.from_numpy(X.view(np.int16)).cuda() for _ in range(ncopy)]
        Q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
        nsc = M * (K // 128) if kind == "fp8_block" else M
        S = torch.empty(nsc, dtype=torch.float32, device="cuda")
        h.quantize(Xs[0], Q, S, kind)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for x in Xs:
                h.quantize(x, Q, S, kind)
        t = time_graphs(torch, [g], max(3, reps))[0] / ncopy
        rows.append(shape_row(f"dynamic_quant_{kind}", quant, M, 0, K, t, 3 * M * K + 4 * nsc,
                              0, "quantize"))
        print(f"[shape] {rows[-1]}", file=sys.stderr, flush=True)
        del g, Xs, Q, S
    # The headline decode with the quantization in front (a separate kernel,
    # or the decode kernel's own prologue where the table asks for it),
    # interleaved with the pre-quantized call.
    wl = Workload(torch, HEAD_CFG, [1, 2, 8, 32])
    for M in (1, 2, 8, 32):
        R = wl.ncopy
        X = torch.from_numpy(synth.activations16(M, wl.K, seed=M).view(np.int16)).cuda()
        d = wl.dev[M]

        def call(copy):
            h.run_dynamic(X, wl.B[copy % R], d["C"], quant=wl.quant, act=wl.act, sb=wl.sb,
                          alpha=d["alpha"], bias=wl.bias, residual=d["residual"])
        call(0)
        torch.cuda.synchronize()
        gd = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gd):
            for r in range(R):
                call(r)
        gq = wl.graph(h, M, R)
        td, tq = time_graphs(torch, [gd, gq], max(3, reps))
        v = h.describe(wl.quant, M, wl.N, wl.K)
        dyn_variant = (v + " (quantization prologue)") if "dq=1" in v else ("quantize + " + v)
        # compulsory bytes: the layer's, with A read as 16-bit activations
        nbytes = wl.bytes(M) - M * wl.K + 2 * M * wl.K
        rows.append(shape_row("fp8_dynamic_decode_quantize_in_front", wl.quant, M, wl.N, wl.K,
                              td / R, nbytes, wl.flops(M),
                              dyn_variant, kernel_calls=1 if "dq=1" in dyn_variant else 2))
        rows[-1]["us_prequantized"] = round(tq / R * 1e6, 3)
        print(f"[shape] {rows[-1]}", file=sys.stderr, flush=True)
        del gd, gq
    del wl
    torch.cuda.empty_cache()
    return rows


def moe_rows(torch, h, reps, ncopy=16):
    """Mixture-of-experts layer (synth.MOE): one grouped call per routing,
    beside the same routing run as one lin_gemm_run per expert with rows.
    Each of the `ncopy` replays of a graph uses its own routing and its own
    copy of the expert weights, so no replay finds its experts in the
    last-level cache.  The row bound passed is the token count (experts are
    distinct per token, so no expert gets more rows than there are tokens).  Eight distinct expert weights are drawn and repeated
    over the 128 experts (the bytes streamed, not their values, set the
    time)."""
    import synth
    c = synth.MOE
    E, N, K, quant = c["E"], c["N"], c["K"], c["quant"]
    g8 = synth.make_grouped(quant, c["act"], [0] * 8, N, K, seed=77, bias=False)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    B8, sb8 = dev(np.stack(g8["Bs"])), dev(np.stack(g8["sbs"]))
    Bs = [B8.repeat(E // 8, 1, 1).contiguous() for _ in range(ncopy)]
    sbs = [sb8.repeat(E // 8, 1).contiguous() for _ in range(ncopy)]
    rows = []
    for T in c["Ts"]:
        M = T * c["topk"]
        routes = []
        for r in range(ncopy):
            sizes = synth.moe_routing(T, E, c["topk"], seed=1000 * T + r)
            off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
            rng = np.random.Generator(np.random.PCG64(r))
            A, sa = synth.encode(quant, rng.standard_normal((M, K), dtype=np.float32), "a")
            d = dict(sizes=sizes, off=off, offd=dev(off), A=dev(A), sa=dev(sa),
                     C=torch.empty((M, N), dtype=torch.int16, device="cuda"))
            # per-expert scale slices in their own (aligned) buffers
            d["sa_seg"] = {x: dev(sa[off[x]:off[x + 1]]) for x in range(E) if sizes[x]}
            routes.append(d)

        def grouped(r):
            d = routes[r]
            h.run_grouped(d["A"], Bs[r], d["C"], d["offd"], quant=quant, act=c["act"],
                          sa=d["sa"], sb=sbs[r], max_rows=T)

        def loop(r):
            d = routes[r]
            for x, sa_x in d["sa_seg"].items():
                m0, m1 = int(d["off"][x]), int(d["off"][x + 1])
                h.run(d["A"][m0:m1], Bs[r][x], d["C"][m0:m1], quant=quant, act=c["act"],
                      sa=sa_x, sb=sbs[r][x])

        graphs = []
        for fn in (grouped, loop):
            for r in range(ncopy):
                fn(r)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for r in range(ncopy):
                    fn(r)
            graphs.append(g)
        tg, tl = time_graphs(torch, graphs, max(3, reps))
        nbytes = int(np.mean([synth.moe_bytes(quant, d["sizes"], N, K) for d in routes]))
        active = float(np.mean([np.count_nonzero(d["sizes"]) for d in routes]))
        row = shape_row(f"{c['name']}_{'decode' if T <= 32 else 'prefill'}", quant, M, N, K,
                        tg / ncopy, nbytes, 2 * M * N * K,
                        f"grouped, {E} experts top-{c['topk']}")
        row.update(tokens=T, active_experts=active, us_per_expert_loop=round(tl / ncopy * 1e6, 3),
                   loop_kernels_per_call=active)
        rows.append(row)
        print(f"[shape] {row}", file=sys.stderr, flush=True)
        del graphs, routes
    del Bs, sbs
    torch.cuda.empty_cache()
    return rows


def vendor_rows(torch, reps):
    """Context, not a target: the same shapes through torch's own bf16 GEMM
    (hipBLASLt / rocBLAS behind torch.mm / torch.addmm), timed the same
    way (graph replay over rotating weight copies).  Prefill: the plain GEMM
    and the GEMM followed by torch's bias / tanh-GELU / x0.5 / residual ops;
    decode: the bf16 6144 x 4096 layer at M = 1, 8, 32."""
    import torch.nn.functional as F
    rows = []
    gen = torch.Generator(device="cuda").manual_seed(5)

    def timed(fn, ncopy, M, N, K, name, variant, nbytes):
        fn(0)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(ncopy):
                fn(r)
        t = time_graphs(torch, [g], max(3, reps))[0] / ncopy
        row = shape_row(name, "bf16", M, N, K, t, nbytes, 2 * M * N * K, variant)
        print(f"[shape] {row}", file=sys.stderr, flush=True)
        del g
        return row

    M = N = K = 4096
    A = torch.randn(M, K, device="cuda", generator=gen).to(torch.bfloat16)
    Bw = [torch.randn(N, K, device="cuda", generator=gen).mul_(0.02).to(torch.bfloat16)
          for _ in range(2)]
    bias = torch.rand(N, device="cuda", generator=gen).sub_(0.5).to(torch.bfloat16)
    res = torch.randn(M, N, device="cuda", generator=gen).to(torch.bfloat16)
    out = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
    rows.append(timed(lambda r: torch.mm(A, Bw[r % 2].t(), out=out), 2, M, N, K,
                      "vendor_bf16_gemm_4096", "torch.mm", 2 * (M * K + N * K + M * N)))
    rows.append(timed(lambda r: F.gelu(torch.addmm(bias, A, Bw[r % 2].t(), out=out),
                                       approximate="tanh").mul_(0.5).add_(res), 2, M, N, K,
                      "vendor_bf16_prefill_epilogue_4096", "torch.addmm + gelu + mul_ + add_",
                      2 * (M * K + N * K + N + 2 * M * N)))
    del A, Bw, res, out
    N, K, ncopy = 6144, 4096, 8
    Bw = [torch.randn(N, K, device="cuda", generator=gen).mul_(0.02).to(torch.bfloat16)
          for _ in range(ncopy)]
    bias = torch.rand(N, device="cuda", generator=gen).sub_(0.5).to(torch.bfloat16)
    for M in (1, 8, 32):
        A = torch.randn(M, K, device="cuda", generator=gen).to(torch.bfloat16)
        out = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
        rows.append(timed(lambda r: torch.addmm(bias, A, Bw[r].t(), out=out), ncopy, M, N, K,
                          "vendor_bf16_decode", "torch.addmm",
                          2 * (M * K + N * K + N + M * N)))
    del Bw
    torch.cuda.empty_cache()
    return rows


def unfused_graph(torch, h, wl, M):
    """A HIP graph of the three-kernel path on the prefill problem (GEMM -> T,
    bias+GELU -> U, 0.5*U + residual -> C) over the weight rotation."""
    d = wl.dev[M]
    T = torch.empty_like(d["C"])
    U = torch.empty_like(d["C"])

    def call(copy):
        h.run_unfused(d["A"], wl.B[copy % wl.ncopy], d["C"], T, U, quant=wl.quant, act=wl.act,
                      alpha=d["alpha"], bias=wl.bias, residual=d["residual"])

    call(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for r in range(wl.ncopy):
            call(r)
    return g, (T, U)


def cpu_baseline(target_s):
    """The oracle, as it stands, on a bounded sample of the headline workload:
    whole passes of the M sweep, repeated until ~target_s of oracle time."""
    import oracle
    import synth
    c = synth.WORKLOADS[HEAD_CFG]
    probs = [synth.make(HEAD_CFG, M) for M in c["Ms"]]
    ncols = c["N"]
    done_bytes, elapsed, passes = 0.0, 0.0, 0
    while elapsed < target_s and passes < 50:
        for p in probs:
            t0 = time.perf_counter()
            oracle.linear(p.quant, p.act, p.A, p.B[:ncols], p.sa, p.sb[:ncols], p.bias[:ncols],
                          None, p.alpha)
            elapsed += time.perf_counter() - t0
            done_bytes += synth.algorithmic_bytes(p.quant, p.M, ncols, p.K, True, False)
        passes += 1
    return dict(value=done_bytes / elapsed / 1e12, unit="TB/s", cores=oracle.num_threads(),
                kind="oracle",
                sample=f"fp8_dynamic decode, the full M sweep {list(c['Ms'])} at N={ncols}, "
                       f"K={c['K']}, repeated {passes} times ({elapsed:.1f} s of oracle time)")


def load_traffic(kernel, digest):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    k = t.get("kernels", {}).get(kernel)
    if not k or t.get("source_digest") != digest:
        return None
    return k.get("bytes_per_launch")


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no collectives or multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import epilogue_scaled_gemm_amd as lg

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.init()
    h = lg.Handle()
    if args.counters_prefill:
        counters_prefill(torch, h)
        h.close()
        return
    if args.counters_shapes:
        counters_shapes(torch, h, args.counters_shapes)
        h.close()
        return
    c = synth.WORKLOADS[HEAD_CFG]
    Ms = list(c["Ms"])
    wl = Workload(torch, HEAD_CFG, Ms)
    R = wl.ncopy
    # Largest M first so the split-K workspace is sized before any capture.
    graphs = {M: wl.graph(h, M, R) for M in sorted(Ms, reverse=True)}
    torch.cuda.synchronize()
    print(f"[bench] workload {c['name']} N={wl.N} K={wl.K} Ms={Ms} copies={R} "
          f"({R * wl.B[0].numel() / 2**20:.0f} MiB of weights)", file=sys.stderr, flush=True)

    if args.counters:
        for _ in range(2):
            for M in Ms:
                graphs[M].replay()
        torch.cuda.synchronize()
        counters_copy(torch)
        print(json.dumps({"counters_run": True, "copy_bytes": 256 << 20,
                          "kernel_bytes": {M: wl.bytes(M) for M in Ms}}), flush=True)
        return

    for _ in range(args.warmup):
        for M in Ms:
            graphs[M].replay()
    torch.cuda.synchronize()

    ev = [(M, torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps) for M in Ms]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()                            # barrier: one rank
    t_start.record()
    i = 0
    for _ in range(args.steps):
        for M in Ms:
            ev[i][1].record()
            graphs[M].replay()
            ev[i][2].record()
            i += 1
    t_end.record()
    torch.cuda.synchronize()
    total_s = t_start.elapsed_time(t_end) / 1e3
    per_M = {M: 0.0 for M in Ms}
    for M, s, e in ev:
        per_M[M] += s.elapsed_time(e) / 1e3
    step_bytes = sum(wl.bytes(M) for M in Ms) * R
    value = step_bytes * args.steps / total_s / 1e12

    # Dominant kernel: the decode instantiation with the most time.  The
    # template arguments are quant kind (2 = e4m3), token tiles (one 16-token
    # tile up to M = 16, two up to 32), swap-AB, waves, unroll, 16-row weight
    # tiles per workgroup (1 up to 16 rows, 2 up to 32, else 4) and the
    # activation mode (0: every lane loads its e4m3 activations itself; 2:
    # staged through LDS, "xs=1" in the variant; 3..6: widened once per wave
    # into LDS, "xs=2", with 1, 2, 4 or 8 chunks of 16 bytes per lane: the
    # smallest that holds M tokens x the wave's slice, whose steps of 128
    # bytes are rounded up to a power of two of at least max(unroll, 2)).
    def kernel_name(M):
        v = dict(kv.split("=") for kv in h.describe(wl.quant, M, wl.N, wl.K).split()[1:])
        rows = int(v["rows"])
        rt = 1 if rows <= 16 else (2 if rows <= 32 else 4)
        am = 2 if v.get("xs") == "1" else 0
        if v.get("xs") == "2":
            steps = -(-wl.K // 128)
            per = -(-steps // int(v["waves"]))
            wst = max(int(v["unroll"]), 2)
            while wst < per:
                wst *= 2
            rounds = -(-M * wst * 8 // 64)
            am = 3 + next(i for i, r in enumerate((1, 2, 4, 8)) if rounds <= r)
        return (f"decode_kernel<2, {1 if M <= 16 else 2}, {'true' if v['swap'] == '1' else 'false'}"
                f", {v['waves']}, {v['unroll']}, {rt}, {am}>")
    groups = {}
    for M in Ms:
        groups.setdefault(kernel_name(M), []).append(M)
    kname, kms = max(groups.items(), key=lambda kv: sum(per_M[M] for M in kv[1]))
    launches = args.steps * R * len(kms)
    ktime = sum(per_M[M] for M in kms)
    avg_dur = ktime / launches
    avg_bytes = sum(wl.bytes(M) for M in kms) / len(kms)
    achieved = avg_bytes / avg_dur
    digest = source_digest()
    traffic = load_traffic(kname, digest)
    roofline = dict(bound="hbm", achieved=round(achieved / 1e9, 1), peak=HBM_PEAK / 1e9,
                    unit="GB/s", frac=round(achieved / HBM_PEAK, 4), traffic=traffic,
                    kernel=kname, avg_launch_us=round(avg_dur * 1e6, 3),
                    algorithmic_bytes_per_launch=int(avg_bytes),
                    variant=h.describe(wl.quant, kms[0], wl.N, wl.K))
    per_m_rows = [dict(M=M, us_per_call=round(per_M[M] / (args.steps * R) * 1e6, 3),
                       TBps=round(wl.bytes(M) * R * args.steps / per_M[M] / 1e12, 4),
                       hbm_frac=round(wl.bytes(M) * R * args.steps / per_M[M] / HBM_PEAK, 4),
                       variant=h.describe(wl.quant, M, wl.N, wl.K)) for M in Ms]
    wbytes = wl.B[0].numel() * wl.B[0].element_size()
    del graphs, wl
    torch.cuda.empty_cache()

    ceiling = stream_ceiling(torch, h, args.reps)
    head_ceil = ceiling_us(ceiling, wbytes)
    if head_ceil:
        roofline["stream_ceiling_us"] = head_ceil
        roofline["of_stream_ceiling"] = round(head_ceil / roofline["avg_launch_us"], 4)
        for r in per_m_rows:
            r["of_stream_ceiling"] = round(head_ceil / r["us_per_call"], 4)

    shapes = None
    if not args.no_shapes:
        shapes = (per_shape_table(torch, h, args.reps) + dynamic_quant_rows(torch, h, args.reps)
                  + moe_rows(torch, h, args.reps) + vendor_rows(torch, args.reps))
        for r in shapes:
            if r.get("bound") == "hbm" and r.get("N") and r.get("M", 0) <= 32:
                wb = r["N"] * (r["K"] // 2 if r["quant"] == "mxfp4" else
                               r["K"] * (2 if r["quant"] in ("bf16", "fp16") else 1))
                cu = ceiling_us(ceiling, wb)
                if cu and r["shape"].startswith(("fp8", "w8a8", "block", "mxfp4", "bf16")):
                    r["of_stream_ceiling"] = round(cu / r["us"], 4)
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_s / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3",
        "data": "synthetic",
        "config": {"workload": f"{c['name']}: A[M,{c['K']}] e4m3 x B[{c['N']},{c['K']}] e4m3, "
                               f"per-token x per-channel fp32 scales, bf16 bias and output; "
                               f"M in {Ms}; {R} weight copies per M per step",
                   "M": Ms, "N": c["N"], "K": c["K"], "weight_copies": R,
                   "calls_per_step": R * len(Ms), "parallelism": "single GPU"},
        "roofline": roofline,
        "per_M": per_m_rows,
        "cpu_baseline": cpu,
        "hbm_stream_ceiling": ceiling,
        "shapes": shapes,
        "source_digest": digest,
    }
    print(json.dumps(out), flush=True)
    h.close()


if __name__ == "__main__":
    main()

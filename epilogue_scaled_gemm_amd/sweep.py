"""Offline sweep: time candidate variants per shape on the GPU and write the
shape-keyed variant table (a text table for lin_gemm_create / LIN_GEMM_CONFIG
with --out, and the built-in csrc/table_mi355x.inc with --emit-inc).

The per-shape search of the vLLM linear-backend write-up (sections "Одно
ядро вместо трёх вариантов" and "Как автотюнер ищет конфиги") benchmarks
configurations the way they run in production -- replayed from a graph --
and keeps the best per shape.  Here the space is small and enumerated
(swap-AB, split-K factor and reduction, waves, unroll for M <= 32; tile
shapes otherwise); each candidate is timed as a HIP-graph replay of calls
over a rotation of weight copies larger than the 256 MB MALL.

    python -m epilogue_scaled_gemm_amd.sweep [--out PATH] [--workloads 2,3,4]
        [--all-m] [--dynamic] [--emit-inc PATH]

--all-m sweeps every token count 1..32 of the decode workloads (not only the
workloads' own list); --ms sweeps a given token list instead (each swept count
then covers the counts above the previous one up to itself); --merge with
--emit-inc cuts the existing include's entries of the same shape around the
new token ranges and keeps the rest; --dynamic also times lin_gemm_run_dynamic with the
winning decode variant with and without the quantization prologue (dq=1)
and keeps the prologue where it is faster; --emit-inc writes the measured
entries as the C++ include that the library compiles in as its built-in
table (csrc/table_mi355x.inc).  Consecutive token counts with the same
winner are merged into one ranged entry.
"""
import argparse
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

ROTATION_BYTES = 384 << 20

# (waves, unroll, rows per workgroup)
DECODE_SHAPES = [(8, 1, 16), (8, 2, 16), (4, 4, 16), (16, 1, 16), (8, 1, 8), (8, 1, 12),
                 (16, 1, 12), (16, 1, 8), (8, 2, 8), (8, 1, 32), (4, 2, 32), (8, 2, 32),
                 (8, 1, 24), (4, 1, 64), (8, 1, 64), (8, 4, 12), (8, 4, 24), (12, 1, 12), (12, 1, 16),
                 (16, 1, 24), (16, 1, 32), (16, 2, 24)]
DECODE_CANDIDATES = [
    f"decode swap=1 split={sp} reduce=twopass waves={w} unroll={u} rows={r}"
    for sp in (1, 2) for w, u, r in DECODE_SHAPES
] + ["decode swap=0 split=1 reduce=twopass waves=8 unroll=2",
     "decode swap=1 split=2 reduce=lastwg waves=8 unroll=1 rows=32",
     "decode swap=1 split=2 reduce=atomic waves=8 unroll=1 rows=32"]
# Staged activations (xs=1), compiled for some shapes per weight format
# (a shape without it runs unstaged and simply times the same).
XS_SHAPES = [(8, 1, 12), (8, 1, 16), (8, 2, 16), (8, 4, 12), (8, 4, 24), (12, 1, 16),
             (8, 1, 24), (8, 2, 12), (4, 4, 16), (16, 1, 16), (4, 2, 32), (8, 1, 32),
             (8, 2, 32), (16, 1, 24), (16, 1, 32), (16, 2, 24), (16, 2, 32), (16, 2, 16),
             (12, 2, 16)]
XS_CANDIDATES = [f"decode swap=1 split=1 reduce=twopass waves={w} unroll={u} rows={r} xs=1"
                 for w, u, r in XS_SHAPES]
# Staged activations with K split across workgroups: 64-row workgroups
# read a quarter of the tokens' activation bytes each, which pays where K
# is long (block e4m3 at K = 12288, 17-32 tokens); swept where K >= 8192.
XS_SPLIT_CANDIDATES = [f"decode swap=1 split={sp} reduce=twopass waves={w} unroll={u} rows={r} xs=1"
                       for sp in (2, 4) for w, u, r in ((8, 1, 64), (16, 1, 32), (8, 1, 32))]
# Widened e4m3 activations (xs=2; up to 16 tokens; elsewhere the same
# variant falls back to staging).
WD_SHAPES = [(8, 1, 12), (8, 2, 12), (8, 4, 12), (8, 1, 16), (8, 2, 16), (12, 1, 12),
             (12, 1, 16), (16, 1, 16), (8, 1, 24), (8, 1, 32), (4, 4, 16), (16, 1, 24), (16, 2, 24)]
WD_CANDIDATES = [f"decode swap=1 split=1 reduce=twopass waves={w} unroll={u} rows={r} xs=2"
                 for w, u, r in WD_SHAPES]

TILE_CANDIDATES = ["tile bm=256 bn=256 wm=2 wn=2", "tile bm=128 bn=256 wm=2 wn=2",
                   "tile bm=256 bn=128 wm=2 wn=2", "tile bm=128 bn=128 wm=2 wn=2",
                   "tile bm=64 bn=128 wm=1 wn=4", "tile bm=64 bn=64 wm=2 wn=2",
                   "tile bm=256 bn=256 wm=2 wn=4", "tile bm=256 bn=128 wm=2 wn=4",
                   "tile bm=128 bn=128 wm=2 wn=4", "pp split=1 group=4", "pp split=2 group=4",
                   "pp split=4 group=4", "pp split=8 group=4"]
# Stream-K tile variants (sk = persistent workgroups per CU).
SK_CANDIDATES = [f"tile bm={bm} bn={bn} wm={wm} wn={wn} sk={sk}"
                 for bm, bn, wm, wn in ((128, 128, 2, 2), (64, 128, 1, 4), (128, 128, 2, 4),
                                        (256, 128, 2, 4), (256, 256, 2, 4))
                 for sk in (1, 2)]


def _dev(torch, a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def capture_variant(torch, h, p, ops, Bs, spec):
    """A HIP graph of one call of `spec` per weight copy (rotating B), and its
    output buffer.  Keep the output and every operand (ops, Bs) alive while
    the graph is replayed: entering another capture empties the allocator
    cache, which would hand their memory back to the driver, and a replay
    would then access freed memory.  Raises LinGemmError if the variant does
    not apply."""
    h.set_force(spec)
    try:
        C = torch.empty((p.M, p.N), dtype=torch.int16, device="cuda")

        def call(i):
            h.run(ops["A"], Bs[i % len(Bs)], C, quant=p.quant, act=p.act, sa=ops["sa"],
                  sb=ops["sb"], alpha=p.alpha, bias=ops["bias"], residual=ops["residual"])

        call(0)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(len(Bs)):
                call(i)
    finally:
        h.set_force(None)
    return g, C


def time_interleaved(torch, graphs, rounds):
    """Median seconds per replay of each graph.  Every round replays all the
    graphs once, so the candidates see the same clock and power state."""
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in graphs] for _ in range(rounds)]
    for r in range(rounds):
        for g, (s, e) in zip(graphs, ev[r]):
            s.record()
            g.replay()
            e.record()
    torch.cuda.synchronize()
    return [float(np.median([ev[r][i][0].elapsed_time(ev[r][i][1]) for r in range(rounds)])) / 1e3
            for i in range(len(graphs))]


def time_variant(torch, h, p, ops, Bs, spec, reps=10):
    """Seconds per call of one variant (graph replay, rotating B)."""
    g, C = capture_variant(torch, h, p, ops, Bs, spec)  # C: the graph writes it
    return time_interleaved(torch, [g], reps)[0] / len(Bs)


def capture_dynamic(torch, h, p, ops, Bs, X, spec):
    """A HIP graph of lin_gemm_run_dynamic calls (rotating B) under `spec`, and
    its output buffer (keep it while the graph is replayed: entering another
    capture empties the allocator cache, which would release it)."""
    h.set_force(spec)
    try:
        C = torch.empty((p.M, p.N), dtype=torch.int16, device="cuda")

        def call(i):
            h.run_dynamic(X, Bs[i % len(Bs)], C, quant=p.quant, act=p.act, sb=ops["sb"],
                          alpha=p.alpha, bias=ops["bias"], residual=ops["residual"])

        call(0)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(len(Bs)):
                call(i)
    finally:
        h.set_force(None)
    return g, C


def merge_ranges(entries):
    """Consecutive token counts (same quant, N, K) with the same winner ->
    one (quant, m_lo, m_hi, N, K, spec, [times]) entry."""
    out = []
    for q, M, N, K, spec, t in entries:
        last = out[-1] if out else None
        if last and last[0] == q and last[3] == N and last[4] == K and last[5] == spec \
                and last[2] == M - 1:
            out[-1] = (q, last[1], M, N, K, spec, last[6] + [t])
        else:
            out.append((q, M, M, N, K, spec, [t]))
    return out


def sparse_ranges(entries):
    """Entries of a sweep over a sparse token list (e.g. 64, 128, ... 2048 above
    the decode range): each swept count M covers the counts above the
    previous swept one up to M (the first from 33, or from itself at or below
    32); counts above the largest keep the table's other entries."""
    out = []
    by = {}
    for q, M, N, K, spec, t in entries:
        by.setdefault((q, N, K), []).append((M, spec, t))
    for (q, N, K), rows in by.items():
        rows.sort()
        prev = None
        for i, (M, spec, t) in enumerate(rows):
            lo = (prev + 1) if prev is not None else (33 if M > 32 else M)
            hi = M
            out.append((q, lo, hi, N, K, spec, [t]))
            prev = M
    return out


def merge_lines(old, new_lines):
    """Table lines after merging: an existing entry of the same (quant, N, K)
    keeps the token counts no new entry covers (its range is cut, or split in
    two, around the new ranges, so coverage never shrinks); the new entries
    follow the kept ones."""
    def key(line):
        f = line.split("#", 1)[0].split()
        if len(f) < 6:
            return None
        hi = 1 << 40 if f[2] == "*" else int(f[2])
        return f[0], int(f[1]), hi, f[3], f[4], f

    new_keys = [key(l) for l in new_lines]
    kept = []
    for l in old:
        k = key(l)
        if not k:
            kept.append(l)
            continue
        pieces = [(k[1], k[2])]
        for n in new_keys:
            if not n or (n[0], n[3], n[4]) != (k[0], k[3], k[4]):
                continue
            cut = []
            for lo, hi in pieces:
                if n[2] < lo or n[1] > hi:
                    cut.append((lo, hi))
                    continue
                if lo < n[1]:
                    cut.append((lo, n[1] - 1))
                if n[2] < hi:
                    cut.append((n[2] + 1, hi))
            pieces = cut
        f = k[5]
        rest = l.split("#", 1)
        spec = " ".join(f[5:])
        note = ("   #" + rest[1]) if len(rest) > 1 else ""
        for lo, hi in pieces:
            if (lo, hi) == (k[1], k[2]):
                kept.append(l)
            else:
                hs = "*" if hi == 1 << 40 else str(hi)
                kept.append(f"{f[0]:<12} {lo:<5} {hs:<5} {f[3]:<6} {f[4]:<6} {spec}{note}")
    return kept + list(new_lines)


def merge_inc(path, new_lines, log=print):
    """Rewrite the table include at `path` with `merge_lines` of its entries
    and the new ones."""
    text = open(path).read() if os.path.exists(path) else ""
    body = text.split('R"TABLE(', 1)[1].split(')TABLE"', 1)[0] if 'R"TABLE(' in text else ""
    old = [l for l in body.splitlines() if l.strip() and not l.lstrip().startswith("#")]
    lines = merge_lines(old, new_lines)
    with open(path, "w") as f:
        f.write("// Measured entries of the built-in variant table, written by\n"
                "// epilogue_scaled_gemm_amd.sweep (graph replay over rotating weight\n"
                "// copies on an MI355X); microseconds per call in the comments.\n"
                "R\"TABLE(\n# quant        m_lo  m_hi  N      K      variant\n"
                + "\n".join(lines) + "\n)TABLE\"\n")
    log(f"merged {len(new_lines)} entries into {path} ({len(lines) - len(new_lines)} kept or cut)")


def sweep(workloads, out_path, reps, log=print, max_m=None, all_m=False, dynamic=False,
          emit_inc=None, quant=None, ms=None, merge=False, min_m=None):
    import torch
    import synth
    import epilogue_scaled_gemm_amd as lg

    h = lg.Handle()
    entries = []
    # Context: a plain device copy (read + write) of 256 MiB and of 24 MiB.
    for mib in (256, 24):
        src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(20):
            dst.copy_(src)
        e.record()
        e.synchronize()
        t = s.elapsed_time(e) / 1e3 / 20
        log(f"copy {mib} MiB: {t * 1e6:.1f} us, {2 * (mib << 20) / t / 1e12:.2f} TB/s (read+write)")
        del src, dst
    for cfg in workloads:
        c = synth.WORKLOADS[cfg]
        ms_w = list(c["Ms"]) if not ms else list(ms)
        if all_m and min(ms_w) <= 32:
            ms_w = sorted(set(ms_w) | set(range(1, 33)))
        for M in ms_w:
            if (max_m is not None and M > max_m) or (min_m is not None and M < min_m):
                continue
            p = synth.make(cfg, M, quant)
            ops = {k: _dev(torch, v) for k, v in p.operands().items() if k != "alpha"}
            ncopy = max(2, min(32, -(-ROTATION_BYTES // p.B.nbytes)))
            Bs = [ops["B"]] + [ops["B"].clone() for _ in range(ncopy - 1)]
            cands = DECODE_CANDIDATES if M <= 32 else TILE_CANDIDATES + SK_CANDIDATES
            if p.quant in ("fp8_dynamic", "mxfp4", "w8a8_int8", "block_fp8", "bf16", "fp16"):
                cands = cands + XS_CANDIDATES
                if p.K >= 8192:
                    cands = cands + XS_SPLIT_CANDIDATES
            if p.quant in ("fp8_dynamic", "block_fp8") and M <= 16:
                cands = cands + WD_CANDIDATES
            # Warm every candidate first (the handle's split-K workspace only
            # grows, so it reaches its final size before any graph is
            # captured), then time them in interleaved rounds.
            ok = []
            for spec in cands:
                if p.quant == "block_fp8" and "rows=" in spec and \
                        128 % int(spec.split("rows=")[1].split()[0]):
                    continue
                h.set_force(spec)
                try:
                    C = torch.empty((p.M, p.N), dtype=torch.int16, device="cuda")
                    h.run(ops["A"], Bs[0], C, quant=p.quant, act=p.act, sa=ops["sa"],
                          sb=ops["sb"], alpha=p.alpha, bias=ops["bias"], residual=ops["residual"])
                    ok.append(spec)
                except lg.LinGemmError as ex:
                    log(f"  skip {spec}: {ex}")
                finally:
                    h.set_force(None)
            torch.cuda.synchronize()
            caps = [capture_variant(torch, h, p, ops, Bs, spec) for spec in ok]
            ts = time_interleaved(torch, [g for g, _ in caps], reps if M <= 32 else max(3, reps // 2))
            best = None
            for spec, t in zip(ok, ts):
                t /= len(Bs)
                log(f"{c['name']} M={M}: {t * 1e6:9.2f} us  {spec}")
                if best is None or t < best[0]:
                    best = (t, spec)
            del caps
            log(f"BEST {c['name']} M={M}: {best[0] * 1e6:.2f} us  {best[1]}")
            spec = best[1]
            if dynamic and M <= 16 and spec.startswith("decode") and \
                    p.quant in ("fp8_dynamic", "w8a8_int8", "block_fp8"):
                X = torch.from_numpy(synth.activations16(M, p.K, seed=M).view(np.int16)).cuda()
                try:
                    gd = [capture_dynamic(torch, h, p, ops, Bs, X, spec),
                          capture_dynamic(torch, h, p, ops, Bs, X, spec + " dq=1")]
                    t0, t1 = (t / len(Bs) for t in
                              time_interleaved(torch, [g for g, _ in gd], reps))
                    log(f"DYNAMIC {c['name']} M={M}: separate kernel {t0 * 1e6:.2f} us, "
                        f"prologue {t1 * 1e6:.2f} us")
                    if t1 < 0.98 * t0:
                        spec += " dq=1"
                    del gd
                except lg.LinGemmError as ex:
                    log(f"  no prologue for {spec}: {ex}")
            entries.append((p.quant, M, p.N, p.K, spec, best[0]))
            del Bs, ops
            torch.cuda.empty_cache()
    h.close()
    merged = sparse_ranges(entries) if ms else merge_ranges(entries)
    measured = [f"{q:<12} {lo:<5} {hi:<5} {N:<6} {K:<6} {spec}   # "
                + ", ".join(f"{t * 1e6:.2f}" for t in ts) + " us"
                for q, lo, hi, N, K, spec, ts in merged]
    if emit_inc and merge:
        merge_inc(emit_inc, measured, log)
    elif emit_inc:
        with open(emit_inc, "w") as f:
            f.write("// Measured entries of the built-in variant table, written by\n"
                    "// epilogue_scaled_gemm_amd.sweep (graph replay over rotating weight\n"
                    "// copies on an MI355X); microseconds per call in the comments.\n"
                    "R\"TABLE(\n# quant        m_lo  m_hi  N      K      variant\n"
                    + "\n".join(measured) + "\n)TABLE\"\n")
        log(f"wrote {emit_inc}")
    lines = ["# Variant table for MI355X (gfx950), written by epilogue_scaled_gemm_amd.sweep.",
             "# <quant> <m_lo> <m_hi> <N> <K> <variant>   (first match wins; the",
             "# built-in defaults follow the measured entries)",
             "# measured us per call in the trailing comment"] + measured
    lines += ["*            1     32    *      *      decode swap=1 split=1 reduce=twopass waves=8 unroll=2 rows=16",
              "block_fp8    257   *     *      *      pp split=0 group=4",
              "block_fp8    33    *     *      *      tile bm=128 bn=128 wm=2 wn=2 group=4",
              "*            33    256   *      *      tile bm=64 bn=128 wm=1 wn=4 group=4",
              "*            257   1024  *      *      tile bm=128 bn=128 wm=2 wn=4 group=4",
              "bf16         1025  *     *      *      pp group=4",
              "fp16         1025  *     *      *      pp group=4",
              "w8a8_int8    1025  *     *      *      pp group=4",
              "*            1025  *     *      *      tile bm=256 bn=256 wm=2 wn=4 group=4"]
    if out_path:
        os.makedirs(os.path.dirname(out_path), exist_ok=True)
        with open(out_path, "w") as f:
            f.write("\n".join(lines) + "\n")
        log(f"wrote {out_path}")
    return entries


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--out", default=None)
    ap.add_argument("--workloads", default="1,2,3,4,5")
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--max-m", type=int, default=None, help="only token counts up to this")
    ap.add_argument("--min-m", type=int, default=None, help="only token counts from this")
    ap.add_argument("--all-m", action="store_true", help="every token count 1..32 (decode)")
    ap.add_argument("--dynamic", action="store_true",
                    help="choose the quantization prologue (dq=1) where it is faster")
    ap.add_argument("--emit-inc", default=None, help="write the measured entries as C++ include")
    ap.add_argument("--quant", default=None,
                    help="run the workloads in this quant mode (same draws), e.g. fp16")
    ap.add_argument("--merge", action="store_true",
                    help="with --emit-inc: cut the existing include's entries of the same shape "
                         "around the new token ranges, keep the rest")
    ap.add_argument("--ms", default=None,
                    help="token counts to sweep instead of each workload's own list, e.g. "
                         "64,128,256,512,1024,2048")
    a = ap.parse_args()
    sweep([int(x) for x in a.workloads.split(",")], a.out, a.reps,
          log=lambda s: print(s, flush=True), max_m=a.max_m, all_m=a.all_m, dynamic=a.dynamic,
          emit_inc=a.emit_inc, quant=a.quant,
          ms=[int(x) for x in a.ms.split(",")] if a.ms else None, merge=a.merge, min_m=a.min_m)


if __name__ == "__main__":
    main()

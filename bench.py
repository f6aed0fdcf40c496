#!/usr/bin/env python3
"""Benchmark of the W4A8 linear layer on one MI355X; prints one JSON line.

A step is one pass of the per-token hot path over one batch of synthetic input through
w4a8_linear: the activation prepass and the linear (one fused kernel at one row when the head is
small enough, where every GEMV workgroup quantizes the row itself; the prepass kernel then the
GEMV or GEMM otherwise).  The default workload is the largest one-row configuration, the decode
GEMV of a vocabulary head: M=1, K=1536, N=262144, symmetric 4-bit weights in 64-groups with fp16
scales (215 MB per step), X ~ N(0,1) with 15 outlier channels x15.  The same line carries a
`secondary` record for the prefill GEMM half of the metric, timed in the same process: by
default the 128-row gate|up prompt tile M=128, K=5120, N=34816 with affine 4-bit weights, priced
in int8 TOPS against the dense int8 MFMA peak.  The weights are packed once (load time, not in a
step).

Timing.  Weights are replicated into a pool of distinct packed buffers totalling >= 512 MiB (twice
the 256 MiB last-level cache) and the steps walk through the pool, so every step streams its
weights from HBM, as a decode does across layers.  The K timed steps are captured once into a HIP
graph (launch gaps of a Python loop would otherwise dominate microsecond kernels) and replayed
between stream synchronizations; W warmup steps run first (by default 1000, a few tens of
milliseconds, so that the GPU's clocks have settled: after 20 the timed graph's replay ran 4%
slow on the decode head, the first replays of a run ramping from 35 to 33 us per step).  The
dominant kernel's average duration is timed the same way from a graph of launches of that kernel
alone over the same pool (at one row the fused kernel is the whole step), bracketed by HIP events
on the capturing stream.

value      = weight bytes (nibbles + scales [+ bias] [+ codebook]) per step / step time (GB/s)
roofline   = algorithmic bytes of one launch of the dominant kernel (weights + xq + xs + xsum + y,
             plus the fp32 row when the prepass is fused in) / its average duration, against
             the 8 TB/s HBM peak (or int8 ops against the 5.0 POP/s dense MFMA peak for a GEMM
             whose MFMA floor is above its HBM floor).  The duration is the median over
             --batches batches (default 7) that alternate between the line's kernels (and the
             HBM read probe), each batch a graph of --steps launches between two HIP events on
             the launching stream; the best batch is reported beside it.
             pct_hbm_probe (one-row workloads): the kernel's byte rate over that of a plain read
             of the same packed buffers (libw4a8_probe.so, 16-byte loads), the achievable rate.
             pct_valu_ceiling (GEMMs): the time the VALU needs for the epilogue alone (an int32
             convert and one FMA per output element and group, 2*M*N*K/G lane operations at
             39.3 T lane-ops/s: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz) over the kernel's time.
             pct_roofline (GEMMs): achieved TOPS over min(peak, arithmetic intensity x 8 TB/s).
sclk_mhz   = the shader clock the driver reports during the run, where it can be read
cpu_baseline = the CPU oracle (plain C, OpenMP) on the primary workload (a column sample of it
             when large), repeated for about 10 s

--glu ACT times the gated variant instead (w4a8_linear_glu): the config's weights read as a
[gate; up] pair (n = 2F), and the output is act(gate) * up, fp32 [m][F].

--a16 times the fp16-activation path instead (w4a8_linear_a16: the prepass writing X as half
and its fp32 group sums, then the GEMV / GEMM with f16 MFMA); its dominant kernel is the GEMV /
GEMM alone (w4a8_gemm_a16), priced against the 2.5 PFLOP/s dense fp16 MFMA peak when that floor
is above the HBM floor.

--attn A1|A2 times the int8 prefill attention over a cached segment instead (w4a8_attn_prefill
on a cache packed once by w4a8_attn_pack_kv): A1 a global layer, A2 a 512-wide sliding window
over a rolled ring with 4 sinks; 8 query heads on 2 key/value heads, head_dim 256, 256 queries
against 1024 cached slots.  value = int8 operations of the two products over the visible
(query, slot) pairs per second, against the 5.0 POP/s dense int8 MFMA peak.

--argmax CAP times the greedy tail of a vocabulary head instead (one row; w4a8_lm_head_argmax:
the GEMV that also soft-caps the logits with CAP (0: no cap) and stores each 64-row panel's
largest key, with the prepass fused into it where w4a8_linear fuses it, else a prepass kernel
before it, and a one-workgroup reduction of those keys into the token).  The timed "kernel" is
the GEMV and the reduction together (with the prepass where it is fused in, else
w4a8_gemv_argmax on prepared activations), with the GEMV's algorithmic bytes plus the keys
(written and read) and the token.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W4A8 linear: weight GB/s at M=1 and int8 TOPS at M≥128 (% of roofline)"
HBM_PEAK_GBPS = 8000.0
# weight formats 3-6 (int8, and the 2-, 1- and 3-bit codebooks) have their own GEMV / GEMM
BYTE_DECODED = (3, 4, 5, 6)
INT8_PEAK_TOPS = 5000.0
VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9          # fp32 lane operations per second, no packed math
F16_PEAK_TFLOPS = 2500.0
POOL_BYTES = 512 << 20

# HBM bytes per launch of the dominant kernel, read from two rocprofv3 --pmc passes (FETCH_SIZE,
# WRITE_SIZE in KiB per dispatch) and scaled by what the same counters read for a plain 256 MiB
# device copy (FETCH_SIZE reads half of the copy's bytes on this chip, WRITE_SIZE all of them).
# Each entry holds the SHA-256 prefix of the kernel's sources when the counters were taken: once
# the kernel changes, the figure no longer describes it and `traffic` is reported as null.
KERNEL_SOURCES = {
    "gemv": ["gemv.hip", "w4a8_kernels.h"],
    "gemm": ["gemm.hip", "w4a8_kernels.h"],
}
TRAFFIC = {
    "C5a": dict(kernel="gemv", source_sha="9e7fcf52161c7224", fetch_kib=104509.38,
                write_kib=1025.6885, fetch_factor=1.99980, write_factor=1.0),
    "C3a": dict(kernel="gemm", source_sha="38de9063a4a389a3", fetch_kib=53272.42,
                write_kib=17408.0000, fetch_factor=1.99980, write_factor=1.0),
}


def w8_gemv_workgroups(cfg):
    """Workgroups of the one-row GEMV of the int8 and CQ1-CQ3 formats, as the library picks them:
    8 wavefronts per 64-row panel, halved while a wavefront would get fewer than 4 groups (128-k
    chunks for CQ1 / CQ3) and the grid keeps at least 1024 workgroups."""
    units = -(-cfg.k // 128) if cfg.fmt in (5, 6) else cfg.k // cfg.group
    panels = -(-cfg.n // 64)
    wpp = 8
    while wpp > 1 and units < 4 * wpp and -(-panels // (8 // (wpp // 2))) >= 1024:
        wpp //= 2
    return -(-panels // (8 // wpp))


def fused_one_row(cfg):
    """Whether w4a8_linear runs this workload as one kernel (the prepass fused into the GEMV),
    as the library decides it: one row, k <= 16384, and at most 4096 panels (2048 with the
    128-block rotation) for the 4-bit formats, 1024 GEMV workgroups for the byte-decoded ones."""
    if cfg.m != 1 or cfg.k > 16384:
        return False
    if cfg.fmt in BYTE_DECODED:
        return w8_gemv_workgroups(cfg) <= 1024
    return -(-cfg.n // 64) <= (2048 if cfg.hadamard else 4096)


def kernel_source_sha(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "bit_group_quantized_act_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(cfg_name, kernel):
    t = TRAFFIC.get(cfg_name)
    if t is None or t["kernel"] != kernel or t["source_sha"] != kernel_source_sha(kernel):
        return None
    return int(round((t["fetch_kib"] * t["fetch_factor"] + t["write_kib"] * t["write_factor"])
                     * 1024))


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--config", default="C5a",
                    help="workload (C1, C2a, C2b, C3a, C3b, C4, C5a, C5b, C5o); default C5a")
    ap.add_argument("--secondary", default="C3a",
                    help="a second workload timed in the same process and reported as the line's "
                         "`secondary` record (its plain linear); 'none' disables it; default C3a")
    ap.add_argument("--batches", type=int, default=7,
                    help="alternating timing batches of the line's kernels (median and best)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="time budget of the CPU oracle baseline (0 disables it)")
    ap.add_argument("--glu", choices=["silu", "gelu_tanh", "gelu_erf"], default=None,
                    help="time w4a8_linear_glu (the weights as a [gate; up] pair) instead")
    ap.add_argument("--argmax", type=float, default=None, metavar="CAP",
                    help="time w4a8_lm_head_argmax (soft cap CAP, 0 for none) on a one-row "
                         "workload instead")
    ap.add_argument("--w8", action="store_true",
                    help="the config's shape with int8 weights (format 3, W8A8) instead")
    ap.add_argument("--cq2", action="store_true",
                    help="the config's shape with 2-bit codebook weights (format 4, CQ2) instead")
    ap.add_argument("--cq1", action="store_true",
                    help="the config's shape with 1-bit codebook weights (format 5, CQ1) instead")
    ap.add_argument("--cq3", action="store_true",
                    help="the config's shape with 3-bit codebook weights (format 6, CQ3) instead")
    ap.add_argument("--a16", action="store_true",
                    help="time the fp16-activation path (w4a8_linear_a16) instead")
    ap.add_argument("--attn", choices=["A1", "A2"], default=None,
                    help="time the int8 prefill attention over a cached segment instead")
    ap.add_argument("--hot", action="store_true",
                    help="reuse one weight buffer (measures cache, not HBM; labelled)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="instead of the benchmark, run a plain device copy of this many MiB a "
                         "few times (the known-size kernel that scales HBM byte counters)")
    return ap.parse_args()


def copy_calibration(mib):
    """A plain copy of `mib` MiB, eight times over distinct buffers: a kernel that reads and
    writes exactly `mib` MiB per launch, for scaling FETCH_SIZE / WRITE_SIZE counter readings."""
    import torch
    dev = torch.device("cuda:0")
    n = mib << 20
    srcs = [torch.full((n,), i, dtype=torch.uint8, device=dev) for i in range(2)]
    dsts = [torch.empty((n,), dtype=torch.uint8, device=dev) for _ in range(2)]
    torch.cuda.synchronize()
    for i in range(8):
        dsts[i % 2].copy_(srcs[(i // 2) % 2])
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 8}), flush=True)


def attention_bench(args):
    """The int8 prefill attention: one JSON line in the same format."""
    import numpy as np
    import torch
    from bit_group_quantized_act_amd import synth, w4a8
    w4a8.load()
    dev = torch.device("cuda:0")
    A = synth.make_attn(args.attn)
    c = A["cfg"]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    AL, packed = w4a8.attn_pack_kv(t(A["k8"]), t(A["ks"]), t(A["v8"]), t(A["vs"]), t(A["kvpos"]))
    q = t(A["q"])
    nh, nq, d = c.nh, c.nq, c.d
    out = (torch.empty((nh, nq, d), dtype=torch.float32, device=dev),
           torch.empty((nh, nq), dtype=torch.float32, device=dev),
           torch.empty((nh, nq), dtype=torch.float32, device=dev),
           torch.empty((nh, nq, d), dtype=torch.int8, device=dev),
           torch.empty((nh, nq), dtype=torch.float32, device=dev))
    need = w4a8.load().w4a8_attn_work_bytes(__import__("ctypes").byref(AL), nh, nq)
    work = torch.empty(max(1, need // 4), dtype=torch.float32, device=dev)
    # visible (query, slot) pairs, from the positions (the same rule the kernel applies)
    tq = A["pos0"] + np.arange(nq)[:, None]
    p = A["kvpos"][None, :].astype(np.int64)
    vis = (p >= 0) & (p <= tq)
    if c.window > 0:
        vis &= (p < c.sink) | (tq - p < c.window)
    ops = 4 * nh * d * int(vis.sum())            # QK and AV: 2 ops per multiply-add each
    stream = torch.cuda.Stream()

    def call():
        w4a8.attn_prefill(AL, packed, q, A["pos0"], c.window, c.sink, A["scale"], out=out,
                          work=work)

    def graph(count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            call()
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=stream):
                for _ in range(count):
                    call()
        torch.cuda.synchronize()
        return g

    def timed(g):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    if args.warmup > 0:
        timed(graph(args.warmup))
    g = graph(args.steps)
    timed(g)
    ms = timed(g) / args.steps
    tops = ops / (ms * 1e-3) / 1e12
    cpu = None
    if args.cpu_seconds > 0:
        import oracle                      # the CPU baseline leg (test infrastructure)
        hq = c.nh // c.nkvh                # one key/value head and its query heads
        reps, t0 = 0, time.perf_counter()
        while True:
            q8, sq = oracle.attn_quant_q(A["q"][:hq])
            kq, sk = oracle.attn_requant_k(A["k8"][:1], A["ks"][:1])
            oracle.attn_int8(q8, sq, kq, sk, A["v8"][:1], A["vs"][:1], A["kvpos"], A["pos0"],
                             c.window, c.sink, A["scale"])
            reps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        cpu = dict(value=round(ops * hq / nh * reps / el / 1e12, 5), unit="TOPS",
                   cores=oracle.num_threads(), kind="oracle",
                   sample=f"{hq} of the {nh} query heads (one key/value head) of {c.name}, "
                          f"repeated {reps}x in {el:.1f} s")
    line = {
        "metric": "int8 prefill attention over a cached segment: int8 TOPS of QK and AV",
        "value": round(tops, 3), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": f"{c.name}: {nh} query heads on {c.nkvh} key/value heads, "
                               f"head_dim {d}, {nq} queries against {c.nkv} cached int8 slots"
                               + (f", window {c.window} with {c.sink} sinks over a rolled ring"
                                  if c.window else ", global layer"),
                   "visible_pairs_per_head": int(vis.sum()), "parallelism": "single GPU"},
        "roofline": dict(bound="mfma", achieved=round(tops, 3), peak=INT8_PEAK_TOPS,
                         unit="TOPS", frac=round(tops / INT8_PEAK_TOPS, 5), traffic=None,
                         kernel="attn_kernel (+ attn_merge)", kernel_us=round(ms * 1000, 3),
                         int_ops_per_launch=ops),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def workload_name(cfg, glu=None, cap=None, a16=False):
    from bit_group_quantized_act_amd import synth
    kind = "decode GEMV" if cfg.m == 1 else "prefill GEMM"
    rot = ", 128-block WHT" if cfg.hadamard else ""
    if cfg.extra.get("row_scale"):
        rot += f", one scale per row seen as K/{cfg.group} groups"
    fused = fused_one_row(cfg)
    if a16:
        one = cfg.m == 1 and cfg.k <= 16384 and -(-cfg.n // 64) <= 2048
        return (f"{cfg.name} {kind}: M={cfg.m} K={cfg.k} N={cfg.n} G={cfg.group} "
                f"{synth.FORMAT_NAMES[cfg.fmt]} 4-bit weights x fp16 activations ("
                + ("prepass (X as half, fp32 group sums) fused into the GEMV" if one else
                   f"prepass writing X as half and its fp32 group sums + "
                   f"{'GEMV' if cfg.m == 1 else 'GEMM'}") + " per step)")
    how = ("prepass fused into the GEMV" if fused else
           "prepass + GEMV" if cfg.m == 1 else "prepass + GEMM")
    gated = "" if glu is None else f", gated output {glu}(gate)*up with F={cfg.n // 2}"
    tail = "" if cap is None else (f", greedy tail: logits soft-capped at {cap:g} and their "
                                   f"first maximum" if cap > 0 else
                                   ", greedy tail: the first maximum of the logits")
    wdesc = {synth.FMT_INT8: "int8", synth.FMT_CQ2: "2-bit codebook (CQ2)",
             synth.FMT_CQ1: "1-bit codebook (CQ1)", synth.FMT_CQ3: "3-bit codebook (CQ3)"}.get(
        cfg.fmt, f"{synth.FORMAT_NAMES[cfg.fmt]} 4-bit")
    return (f"{cfg.name} {kind}: M={cfg.m} K={cfg.k} N={cfg.n} G={cfg.group} "
            f"{wdesc} weights{rot}{gated}{tail} ({how} per step)")


def read_sclk_mhz():
    """The current shader clock from the driver's sysfs table (the entry marked '*'), else from
    rocm-smi; None if neither can be read."""
    import glob
    import re
    import subprocess
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as fh:
                for line in fh:
                    if "*" in line:
                        m = re.search(r"(\d+)\s*Mhz", line, re.I)
                        if m:
                            return int(m.group(1))
        except OSError:
            continue
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True,
                           timeout=20)
        m = re.search(r"sclk.*?\((\d+)\s*Mhz\)", r.stdout, re.I)
        if m:
            return int(m.group(1))
    except (OSError, subprocess.SubprocessError):
        pass
    return None


class LayerBench:
    """One workload's buffers, its step (w4a8_linear or the chosen variant) and its dominant
    kernel alone, over a pool of weight copies that defeats the last-level cache."""

    def __init__(self, args, name, variants=True):
        import numpy as np
        import torch
        from bit_group_quantized_act_amd import synth, w4a8
        self.w4a8, self.synth = w4a8, synth
        dev = self.dev = torch.device("cuda:0")
        chosen = [f for f, on in ((synth.FMT_INT8, args.w8), (synth.FMT_CQ2, args.cq2),
                                  (synth.FMT_CQ1, args.cq1), (synth.FMT_CQ3, args.cq3))
                  if on and variants]
        over = {"fmt": chosen[0]} if chosen else {}
        layer = self.layer = synth.make(name, **over)
        cfg = self.cfg = layer["cfg"]
        self.byte_decoded = cfg.fmt in BYTE_DECODED
        t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        if "row_scales" in layer:      # one scale per row, packed through the row-scale view
            lay, packed0 = w4a8.pack_row_scale(t(layer["codes"]), t(layer["row_scales"]),
                                               cfg.fmt, cfg.group, row_bias=t(layer["row_bias"]),
                                               codebook=t(layer["codebook"]))
        else:
            lay, packed0 = w4a8.pack(t(layer["codes"]), t(layer["scales"]), cfg.fmt, cfg.group,
                                     bias=t(layer["bias"]), codebook=t(layer["codebook"]))
        self.lay = lay
        self.wbytes = synth.weight_bytes(cfg)
        fused = fused_one_row(cfg)                          # w4a8_linear's one-kernel path
        self.cap = cap = args.argmax if variants else None
        self.a16 = a16 = args.a16 and variants
        self.glu = args.glu if variants else None
        alg_bytes = synth.algorithmic_bytes(cfg, fused_prep=fused)
        # fp16 activations at one row (k <= 16384, at most 2048 panels): w4a8_linear_a16 is one
        # kernel with the prepass fused in
        self.fused_a16 = fused_a16 = a16 and cfg.m == 1 and cfg.k <= 16384 and \
            -(-cfg.n // 64) <= 2048
        if a16:      # weights + xh (2 bytes per input) + fp32 group sums + y, no xq / xs / xsum
            alg_bytes = synth.weight_bytes(cfg) + 2 * cfg.m * cfg.k + 4 * cfg.m * (cfg.k // 64) \
                + 4 * cfg.m * cfg.n
            if fused_a16:                                  # + the fp32 row read
                alg_bytes += 4 * cfg.k
        if cap is not None:                                # keys written and read, token, logit
            alg_bytes += 2 * w4a8.argmax_work_bytes(cfg.n) + 8
        act = None
        if self.glu is not None:
            act = {"silu": w4a8.ACT_SILU, "gelu_tanh": w4a8.ACT_GELU_TANH,
                   "gelu_erf": w4a8.ACT_GELU_ERF}[self.glu]
            alg_bytes -= 4 * cfg.m * (cfg.n // 2)         # the output is [m][F], not [m][n]
        self.act, self.fused, self.alg_bytes = act, fused, alg_bytes
        self.ops = synth.int_ops(cfg)
        pool_n = self.pool_n = 1 if args.hot else max(2, -(-POOL_BYTES // lay.bytes))
        self.pool = [packed0] + [packed0.clone() for _ in range(pool_n - 1)]
        self.x = t(layer["x"])
        ng = cfg.k // cfg.group
        self.xq = torch.empty((cfg.m, cfg.k), dtype=torch.int8, device=dev)
        self.xs = torch.empty((ng, cfg.m), dtype=torch.float32, device=dev)     # group-major
        self.xsum = torch.empty((ng, cfg.m), dtype=torch.int32, device=dev)
        self.y = torch.empty((cfg.m, cfg.n if act is None else cfg.n // 2), dtype=torch.float32,
                             device=dev)
        self.token = torch.empty(1, dtype=torch.int32, device=dev)
        self.tval = torch.empty(1, dtype=torch.float32, device=dev)
        self.work = w4a8.argmax_work(lay, dev)
        self.xh16, self.xsf16 = w4a8.a16_buffers(cfg.m, cfg.k, dev) if a16 else (None, None)
        torch.cuda.synchronize()

    def kernel(self, i):
        """The dominant kernel alone: the fused prepass + GEMV at one row (the plain GEMV for a
        vocabulary-sized row), the GEMM above."""
        w, lay, pk = self.w4a8, self.lay, self.pool[i % self.pool_n]
        x, y, xq, xs, xsum = self.x, self.y, self.xq, self.xs, self.xsum
        if self.fused_a16:
            w.linear_a16(lay, pk, x, out=y, prep_out=(self.xh16, self.xsf16))
        elif self.a16:
            w.gemm_a16(lay, pk, self.xh16, self.xsf16, out=y)
        elif self.cap is not None and self.fused:
            w.lm_head_argmax(lay, pk, x, self.cap, self.cfg.hadamard,
                             out=(y[0], self.token, self.tval), work=self.work,
                             prep_out=(xq, xs, xsum))
        elif self.cap is not None:
            w.gemv_argmax(lay, pk, xq, xs, xsum, self.cap, out=(y[0], self.token, self.tval),
                          work=self.work)
        elif self.act is not None:
            if self.fused:
                w.linear_glu(lay, pk, x, self.act, self.cfg.hadamard, out=y,
                             prep_out=(xq, xs, xsum))
            else:
                w.gemm_glu(lay, pk, xq, xs, xsum, self.act, out=y)
        elif self.fused:
            w.linear(lay, pk, x, self.cfg.hadamard, out=y, prep_out=(xq, xs, xsum))
        elif self.cfg.m == 1:
            w.gemv(lay, pk, xq[0], xs, xsum, out=y[0])
        else:
            w.gemm(lay, pk, xq, xs, xsum, out=y)

    def step(self, i):
        """One pass of the hot path: the prepass and the linear (or the chosen variant)."""
        w, lay, pk = self.w4a8, self.lay, self.pool[i % self.pool_n]
        x, y, prep = self.x, self.y, (self.xq, self.xs, self.xsum)
        if self.a16:
            w.linear_a16(lay, pk, x, out=y, prep_out=(self.xh16, self.xsf16))
        elif self.cap is not None:
            w.lm_head_argmax(lay, pk, x, self.cap, self.cfg.hadamard,
                             out=(y[0], self.token, self.tval), work=self.work, prep_out=prep)
        elif self.act is not None:
            w.linear_glu(lay, pk, x, self.act, self.cfg.hadamard, out=y, prep_out=prep)
        else:
            w.linear(lay, pk, x, self.cfg.hadamard, out=y, prep_out=prep)

    def kernel_name(self):
        kname = "gemv" if self.cfg.m == 1 else "gemm"  # the fused kernel lives in gemv.hip
        if self.cap is not None:
            return ("lm_head_argmax (prepass fused into the GEMV with the tail + key reduction)"
                    if self.fused else "gemv_argmax (GEMV with the tail + key reduction)")
        return f"{kname}_a16" if self.a16 else f"{kname}_w8" if self.byte_decoded else kname

    def traffic(self):
        kname = "gemv" if self.cfg.m == 1 else "gemm"
        variant = ("glu" if self.act is not None else "argmax" if self.cap is not None else
                   "a16" if self.a16 else
                   self.synth.FORMAT_NAMES[self.cfg.fmt] if self.byte_decoded else None)
        key = self.cfg.name if variant is None else f"{self.cfg.name}-{variant}"
        return measured_traffic(key, kname)

    def roofline(self, us_median, us_best, probe_gbps=None):
        """The dominant kernel against its bound: HBM bytes, or int8 / fp16 MFMA operations for
        a GEMM whose MFMA floor is above its HBM floor."""
        cfg = self.cfg
        hbm_floor = self.alg_bytes / (HBM_PEAK_GBPS * 1e9)
        peak_mfma = F16_PEAK_TFLOPS if self.a16 else INT8_PEAK_TOPS
        mfma_floor = self.ops / (peak_mfma * 1e12)
        tops = self.ops / (us_median * 1e-6) / 1e12
        if cfg.m > 1 and mfma_floor > hbm_floor:
            roof = dict(bound="mfma", achieved=round(tops, 2), peak=peak_mfma,
                        unit="TFLOP/s", frac=round(tops / peak_mfma, 4))
        else:
            achieved = self.alg_bytes / (us_median * 1e-6) / 1e9
            roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBPS,
                        unit="GB/s", frac=round(achieved / HBM_PEAK_GBPS, 4))
        roof.update(traffic=self.traffic(), kernel=self.kernel_name(),
                    kernel_us=round(us_median, 3), kernel_us_best=round(us_best, 3),
                    alg_bytes_per_launch=self.alg_bytes, int_ops_per_launch=self.ops,
                    tops=round(tops, 2))
        if probe_gbps is not None:
            roof["probe_GBps"] = round(probe_gbps, 1)
            roof["pct_hbm_probe"] = round(self.alg_bytes / (us_median * 1e-6) / 1e9 /
                                          probe_gbps, 4)
        if cfg.m > 1:
            roof["pct_mfma_peak"] = round(tops / peak_mfma, 4)
            roof["pct_hbm_peak"] = round(self.alg_bytes / (us_median * 1e-6) / 1e9 /
                                         HBM_PEAK_GBPS, 4)
            valu_us = 2.0 * cfg.m * cfg.n * (cfg.k // cfg.group) / VALU_LANE_OPS * 1e6
            roof["valu_epilogue_floor_us"] = round(valu_us, 3)
            roof["pct_valu_ceiling"] = round(valu_us / us_median, 4)
            ceiling = min(peak_mfma, self.ops / self.alg_bytes * HBM_PEAK_GBPS / 1000.0)
            roof["pct_roofline"] = round(tops / ceiling, 4)
        return roof


class StreamProbe:
    """A plain read of the packed weight buffers of a workload (its pool, so every launch
    streams from HBM), in one of a few launch shapes: the achievable read rate for that byte
    count is the best shape's."""

    SHAPES = [(wg, u) for wg in (1024, 2048, 4096, 8192) for u in (4, 8)]

    def __init__(self, lb):
        import ctypes
        import torch
        path = os.path.join(ROOT, "bit_group_quantized_act_amd", "libw4a8_probe.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built: run __graft_entry__.build()")
        self.lib = ctypes.CDLL(path)
        self.lib.stream_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                               ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
        self.lib.stream_probe_read.restype = ctypes.c_int
        self.lb = lb
        self.bytes = lb.lay.bytes // 16 * 16
        self.sink = torch.empty(max(wg for wg, _ in self.SHAPES), dtype=torch.int32,
                                device=lb.dev)

    def kernel(self, shape):
        import ctypes
        import torch
        wg, unroll = shape

        def call(i):
            pk = self.lb.pool[i % self.lb.pool_n]
            rc = self.lib.stream_probe_read(
                ctypes.c_void_p(pk.data_ptr()), self.bytes, ctypes.c_void_p(self.sink.data_ptr()),
                wg, unroll, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if rc != 0:
                raise RuntimeError(f"stream_probe_read failed: hipError {rc}")
        return call


def cpu_baseline(lb, seconds):
    """The CPU oracle (test infrastructure) on a bounded sample of the workload: all rows,
    `cols` weight rows (all of them when the layer is small; matched gate and up rows for the
    gated output), at most ~2e9 multiply-adds per repetition, repeated for `seconds`."""
    import numpy as np
    import oracle
    cfg, layer, act, cap, a16 = lb.cfg, lb.layer, lb.act, lb.cap, lb.a16
    cols = cfg.n if cfg.m * cfg.n * cfg.k <= 2e9 else \
        max(64, int(2e9 / (cfg.m * cfg.k)) // 64 * 64)
    rows = np.arange(cols)
    if act is not None:               # matched gate and up rows: cols / 2 outputs
        half = max(1, cols // 2)
        rows = np.concatenate([np.arange(half), cfg.n // 2 + np.arange(half)])
    sub = lambda a: None if a is None else np.ascontiguousarray(a[rows])
    codes, scales, bias, cb = (sub(layer[key]) for key in ("codes", "scales", "bias",
                                                            "codebook"))
    sample_wbytes = lb.wbytes * rows.size / cfg.n
    reps, t0 = 0, time.perf_counter()
    while True:
        if a16:
            oh, osf = oracle.prep_a16(layer["x"])
            yo = oracle.linear_a16(cfg.fmt, codes, scales, oh, osf, cfg.group, bias_f16=bias,
                                   with_terms=False)
        else:
            oq, os_, osum = oracle.prep(layer["x"], cfg.group, cfg.hadamard)
            yo = oracle.linear(cfg.fmt, codes, scales, oq, os_, osum, cfg.group,
                               bias_f16=bias, codebook=cb, with_terms=False)
        if act is not None:
            oracle.glu(act, yo)
        if cap is not None:
            oracle.softcap_argmax(yo, cap)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    what = ("the whole workload" if rows.size == cfg.n else
            f"all {cfg.m} rows x {rows.size} of the {cfg.n} weight rows")
    return dict(value=round(sample_wbytes * reps / el / 1e9, 3), unit="GB/s",
                cores=oracle.num_threads(), kind="oracle",
                sample=f"{what} of {cfg.name} ({'fp16-activation ' if a16 else ''}prep + linear"
                       f"{' + gated output' if act is not None else ''}"
                       f"{' + soft cap and argmax' if cap is not None else ''}), repeated "
                       f"{reps}x in {el:.1f} s ({1e3 * el / reps:.2f} ms each)")


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the layer would "
              "shard by output columns, one slice of the packed panels per GPU); run with "
              "--gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_group_quantized_act_amd import synth, w4a8

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration_mib > 0:
        copy_calibration(args.copy_calibration_mib)
        return
    if args.attn is not None:
        attention_bench(args)
        return
    w4a8.load()   # fails loudly if the HIP library is not built
    torch.cuda.set_device(torch.device("cuda:0"))

    if sum(bool(v) for v in (args.w8, args.cq2, args.cq1, args.cq3)) > 1:
        print("give at most one of --w8 / --cq2 / --cq1 / --cq3", file=sys.stderr)
        sys.exit(2)
    cfg0 = synth.config(args.config)
    variant = args.a16 or args.argmax is not None or args.glu is not None
    if variant and (args.w8 or args.cq2 or args.cq1 or args.cq3):
        print("--w8 / --cq1 / --cq2 / --cq3 time the plain linear only", file=sys.stderr)
        sys.exit(2)
    if args.a16 and (args.argmax is not None or args.glu is not None or cfg0.group != 64 or
                     cfg0.fmt == synth.FMT_CODEBOOK):
        print("--a16 needs a symmetric or affine 64-group workload and no --glu / --argmax",
              file=sys.stderr)
        sys.exit(2)
    if args.argmax is not None and (cfg0.m != 1 or args.glu is not None or
                                    not args.argmax >= 0):
        print("--argmax needs a one-row workload, no --glu and a cap >= 0", file=sys.stderr)
        sys.exit(2)
    if args.glu is not None and cfg0.n % 128 != 0:
        print(f"--glu needs n = 2F with F a multiple of 64 ({cfg0.name} has n = {cfg0.n})",
              file=sys.stderr)
        sys.exit(2)

    primary = LayerBench(args, args.config)
    cfg = primary.cfg
    secondary = None
    if args.secondary.lower() != "none" and args.secondary != args.config:
        secondary = LayerBench(args, args.secondary, variants=False)
    probe = StreamProbe(primary) if cfg.m == 1 else None
    stream = torch.cuda.Stream()

    def capture(fn, count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            fn(0)                      # one eager call on the capture stream before capturing
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=stream):
                for i in range(count):
                    fn(i)
        torch.cuda.synchronize()
        return g

    def timed(g):
        # HIP events recorded on the stream the graph's kernels run on
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    # the steps: warmup, then exactly `steps` steps of the primary workload in one graph
    if args.warmup > 0:
        timed(capture(primary.step, args.warmup))
    g_steps = capture(primary.step, args.steps)
    ms_per_step = timed(g_steps) / args.steps
    sec_ms_per_step = None
    if secondary is not None:
        g_sec_steps = capture(secondary.step, args.steps)
        timed(g_sec_steps)
        sec_ms_per_step = timed(g_sec_steps) / args.steps

    # the dominant kernels alone, in alternating batches
    graphs = [("primary", capture(primary.kernel, args.steps))]
    if secondary is not None:
        graphs.append(("secondary", capture(secondary.kernel, args.steps)))
    if probe is not None:
        for shape in probe.SHAPES:
            graphs.append((("probe",) + shape, capture(probe.kernel(shape), args.steps)))
    for _, g in graphs:
        timed(g)                                    # warm each graph
    us = {name: [] for name, _ in graphs}
    for _ in range(max(1, args.batches)):
        for name, g in graphs:
            us[name].append(timed(g) * 1000.0 / args.steps)
    med = {k: float(sorted(v)[len(v) // 2]) for k, v in us.items()}
    best = {k: float(min(v)) for k, v in us.items()}
    sclk = read_sclk_mhz()

    probe_gbps = None
    if probe is not None:
        pkey = min((k for k in med if k[0] == "probe"), key=lambda k: med[k])
        probe_gbps = probe.bytes / (med[pkey] * 1e-6) / 1e9
    roof = primary.roofline(med["primary"], best["primary"], probe_gbps)
    if probe is not None:
        roof["probe_us"] = round(med[pkey], 3)
        roof["probe_shape"] = f"{pkey[1]} workgroups x 256 lanes, {pkey[2]} loads in flight"
    value = primary.wbytes / (ms_per_step * 1e-3) / 1e9

    sec = None
    if secondary is not None:
        sc = secondary.cfg
        sec = {"workload": workload_name(sc), "m": sc.m, "k": sc.k, "n": sc.n,
               "group": sc.group, "format": synth.FORMAT_NAMES[sc.fmt],
               "weight_pool_buffers": secondary.pool_n,
               "metric": "int8 TOPS (2*M*N*K per second)" if sc.m > 1 else "weight GB/s",
               "ms_per_step": round(sec_ms_per_step, 6),
               "step_value": round(secondary.ops / (sec_ms_per_step * 1e-3) / 1e12, 2)
               if sc.m > 1 else round(secondary.wbytes / (sec_ms_per_step * 1e-3) / 1e9, 2),
               "roofline": secondary.roofline(med["secondary"], best["secondary"])}

    cpu = cpu_baseline(primary, args.cpu_seconds) if args.cpu_seconds > 0 else None

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if primary.a16 else "int8",
        "data": "synthetic",
        "config": {"workload": workload_name(cfg, primary.glu, primary.cap, primary.a16),
                   "m": cfg.m, "k": cfg.k, "n": cfg.n, "group": cfg.group,
                   "format": synth.FORMAT_NAMES[cfg.fmt], "weight_pool_buffers": primary.pool_n,
                   "hot_cache": bool(args.hot), "parallelism": "single GPU",
                   "batches": max(1, args.batches)},
        "roofline": roof,
        "secondary": sec,
        "sclk_mhz": sclk,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the two-level sparse-attention decode step on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c3_128k_gqa]

A step is one whole decode step over one batch: block selection (summary
GEMM + top-Kb), token selection (INT4 label scores + top-Kt) and attention over
the kept tokens, for every (batch, kv head) pair, with inputs resident in HBM.
The default workload is the 128k-context GQA decode (batch 8, 64 query heads on
8 kv heads, head dim 128, block 64, Kb=128, Kt=4096, 16 INT4 label channels).

Cold measurement: R copies of the cache live at distinct device addresses and
the steps rotate over them, so no step finds its bytes in the 256 MB Infinity
Cache left there by the previous step (R * touched bytes >= 1 GiB). Each timed
step replays a HIP graph captured from the step's library calls (no host
launch cost in the timed region; --no-graph launches them one by one).

Prints one JSON line: queries/sec (= batch / step time); the HBM roofline of
the whole step (algorithmic bytes per step / step time), with the dominant
kernel (attention; the library records HIP events around each of its launches
on the stream it runs on) as a labelled sub-field, against HBM for the GQA
kernels and against the bf16 MFMA peak for the latent-attention kernel; the
index build (summaries and INT4 label cache, once per cache, outside the step)
timed on its own; and the fp64 oracle timed on host cores over a bounded
sample of pairs as the CPU baseline.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

import workload as W  # noqa: E402

METRIC = "sparse-attn decode queries/sec at 32k/128k ctx; achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


def algorithmic_bytes(s, dense=False):
    """Bytes the selection must touch per step (summaries, label cache of the
    candidates, gathered K/V rows, q, out) and the attention kernel's share.
    dense: attention over every token, nothing selected."""
    kb = min(s.Kb, s.NB)
    kt = min(s.Kt, kb * s.bs)
    summ = 0 if dense else s.pairs * s.NB * 2 * s.D * 2
    label = 0 if dense else s.pairs * kb * s.bs * (s.r // 2 + 4)
    rows = s.pairs * kt * s.row * 2
    q = s.B * s.Hq * s.D * 2
    out = s.B * s.Hq * s.DV * 4
    return dict(summaries=summ, label=label, kv_rows=rows, q=q, out=out, total=summ + label + rows + q + out,
                attention=rows + q + out + s.B * s.Hq * 4)


def attention_kernel(s):
    """Name of the attention kernel tls_sparse_decode launches for this shape."""
    if s.D == 576 and s.DV == 512 and s.v_is_k_prefix and s.G > 16:
        return "k_attend_mla"
    if s.D == 128 and s.DV == 128 and not s.v_is_k_prefix:
        return "k_attend_pv"
    return "k_attend_gqa" if s.D <= 128 else "k_attend"


def source_code(text):
    """C/C++ source text without its comments, every run of white space
    shown as one blank (string and character literals otherwise kept): what
    a counter summary depends on."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_sha():
    """Digest of every kernel source (the .hip files, their device headers and
    the launch header), comments and layout aside: a counter summary is valid
    only for the code it was taken with."""
    import hashlib
    h = hashlib.sha256()
    csrc = ROOT / "two_level_sparse_amd" / "csrc"
    files = list(csrc.glob("*.hip")) + list(csrc.glob("*_dev.h")) + [csrc / "tls_dev.h", csrc / "tls_launch.h"]
    for f in sorted(set(files)):
        h.update(f.name.encode())
        h.update(source_code(f.read_text()).encode())
    return h.hexdigest()[:16]


def measured_traffic(config, key):
    """HBM bytes (counters FETCH_SIZE + WRITE_SIZE, calibrated) per step
    (key "step_traffic_bytes") or per attention launch ("attention_traffic_bytes")
    from the committed counter summary, or None when a kernel source changed
    since the counters were taken."""
    prof = ROOT / "profiles" / f"traffic_{config}.txt"
    if not prof.exists():
        return None
    sha = kernel_source_sha()
    for line in prof.read_text().splitlines():
        if line.startswith(key + "="):
            kv = dict(tok.split("=") for tok in line.split())
            if kv.get("source_sha256_prefix") == sha:
                return int(kv[key])
    return None


def attention_flops(s):
    """Multiply-adds x 2 of the attention over the kept tokens: q.K (D) and P.V (DV) per head and token."""
    kt = min(s.Kt, min(s.Kb, s.NB) * s.bs)
    return 2.0 * s.pairs * s.G * kt * (s.D + s.DV)


class TimingEvent:
    """A HIP event created for timing only (hipEventDisableSystemFence): when
    it completes, the runtime does not add a system-scope memory fence, so the
    interval between two of them spans the kernel between them and not also a
    write-back of caches to the host, which no launch inside the timed graph
    pays. Created through the HIP runtime this process already uses (the one
    torch loaded). Read only after a device synchronisation."""
    _hip = None

    def __init__(self):
        import ctypes as C
        if TimingEvent._hip is None:
            path = next(l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l)
            TimingEvent._hip = C.CDLL(path)
        h = C.c_void_p()
        rc = TimingEvent._hip.hipEventCreateWithFlags(C.byref(h), C.c_uint(0x20000000))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.cuda_event = h.value  # the handle tls_profile_events passes on

    def elapsed_time(self, end) -> float:
        import ctypes as C
        ms = C.c_float()
        rc = TimingEvent._hip.hipEventElapsedTime(C.byref(ms), C.c_void_p(self.cuda_event),
                                                   C.c_void_p(end.cuda_event))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if TimingEvent._hip is not None and self.cuda_event:
            import ctypes as C
            TimingEvent._hip.hipEventDestroy(C.c_void_p(self.cuda_event))


def block_scorer_mfma(s, dec, qs, caches, stream, reps=20):
    """The block-score GEMM [G x 2D] . [2D x NB] per pair, timed alone with the
    library's events: cold (rotating over the cache copies) and warm (one
    copy, its summaries left in the Infinity Cache by the previous call)."""
    import torch
    import two_level_sparse_amd as T
    flops = 2.0 * s.G * s.NB * 2 * s.D * s.pairs
    summ_bytes = s.pairs * s.NB * 2 * s.D * 2
    # the GEMM's roofline: with its operands (summaries, q) and scores moved
    # through HBM at the peak rate, the products keep MFMA busy at most
    # (flop per byte) / (peak flop/s / peak byte/s) of the launch
    per_byte = flops / (summ_bytes + s.B * s.Hq * s.D * 2 + s.pairs * s.NB * 4)
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    out = {"kernel": "k_score_blocks_lds" if s.G > 48 else "k_score_blocks", "flops": flops,
           "bytes": summ_bytes, "mfma_peak_tflops": MFMA_BF16_PEAK_TFLOPS, "flop_per_byte": round(per_byte, 1),
           "mfma_util_bound_at_hbm_peak": round(min(1.0, per_byte / ridge), 4)}
    for mode in ("cold", "warm"):
        evs = [(TimingEvent(), TimingEvent()) for _ in range(reps)]
        torch.cuda._sleep(int(2e7))  # the host queues every call before the GPU starts them
        for i in range(reps + 2):
            r = i % len(caches) if mode == "cold" else 0
            if i >= 2:
                T.tls_profile_events(T.TLS_PROFILE_BLOCK_SCORES, *evs[i - 2])
            dec.select_blocks(qs[r], caches[r])
            T.tls_profile_events(T.TLS_PROFILE_BLOCK_SCORES)
        torch.cuda.synchronize()
        us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
        out[mode] = {"us": round(us, 2), "tflops": round(flops / us / 1e6, 1),
                     "mfma_util": round(flops / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4),
                     "GBps": round(summ_bytes / us / 1e3, 1)}
    return out


def build_time(s, cache, reps=5):
    """The index build (tls_build_summaries: key max/min per block and the INT4
    label cache, once per cache, outside the decode step) timed on its own with
    events: bytes = every key row read once + summaries, codes and scales written."""
    import torch
    kb = s.pairs * s.N * s.D * 2  # the K half of every row (the label pass reads only label channels of it)
    written = s.pairs * (s.NB * 2 * s.D * 2 + s.N * (s.r // 2) + s.N * 4)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cache.build()
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        cache.build()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / reps * 1e3
    return {"kernel": "k_build", "us": round(us, 1), "bytes": kb + written,
            "GBps": round((kb + written) / us / 1e3, 1), "frac": round((kb + written) / us / 1e3 / HBM_PEAK_GBS, 4),
            "note": "once per cache, excluded from the per-step rate"}


class DenseDecoder:
    """Attention over every cached token through the same library call (the
    baseline the pages compare against: dense decode at the same shape)."""

    def __init__(self, s):
        import torch
        from two_level_sparse_amd.runtime import Decoder
        self.dec = Decoder(s)
        self.idx = torch.arange(s.N, dtype=torch.int32, device="cuda").expand(s.B, s.Hkv, s.N).contiguous()

    def decode(self, q, kv, **kw):
        self.dec.decode(q, kv, token_idx=self.idx, **kw)

    def step(self, q, cache, stream=None):
        self.dec.decode(q, cache.kv, stream, token_idx=self.idx)
        return self.dec.out


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(s, q, kv, lab, budget_s=15.0):
    """The fp64 oracle (O3..O9 of one step; summaries/label cache prebuilt,
    untimed) on a bounded sample of pairs, scaled to queries/sec of a full step."""
    import oracle
    nth = oracle.num_threads()
    n = min(s.pairs, max(1, nth))
    pairs = np.arange(n, dtype=np.int32)
    built = oracle.decode(s, q, kv, lab, pairs=pairs)
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.decode(s, q, kv, lab, pairs=pairs, built=built)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or el / reps * (reps + 1) > 2 * budget_s:
            break
    per_sample = el / reps
    step_s = per_sample * s.pairs / n
    return {"value": s.B / step_s, "unit": "queries/s", "cores": nth, "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{n} of {s.pairs} (batch, kv-head) pairs of one step, {reps} repetitions, "
                      f"{per_sample * 1e3:.1f} ms each, scaled by {s.pairs}/{n}; summaries and label cache "
                      f"prebuilt (untimed); fp64 C oracle with OpenMP over pairs"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c3_128k_gqa", choices=list(W.CONFIGS))
    ap.add_argument("--rotate", type=int, default=0, help="cache copies to rotate over (0 = enough for 1 GiB)")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="launch the timed steps one call at a time instead of replaying a captured HIP graph per step")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one plain 256 MiB device copy before timing (counter calibration for profiles)")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-mode", default=None, choices=["device", "gather", "memcpy", "full"],
                    help="offloaded workload: where the transfer is planned and how blocks move (default: library's; "
                         "full = every selected block every step, the baseline without reuse)")
    ap.add_argument("--no-stagger", action="store_true",
                    help="offloaded workload: the baseline without staggering (select, transfer, attend in order)")
    ap.add_argument("--layers", type=int, default=1,
                    help="offloaded workload: layers stepped as one model, each its own offloaded cache and queries "
                         "(layer l's transfer runs under the attention of the layers after it)")
    ap.add_argument("--mode", default="tls", choices=["tls", "quest", "ds", "dense"],
                    help="tls: the two-level step; quest: block stage only (every token of the kept blocks); "
                         "ds: token stage only (Kt tokens selected over the whole cache); "
                         "dense: attention over every cached token, no selection (baselines at the same shape)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (this operator is built and "
              f"timed on a single MI355X; see the design notes for how it would shard).", file=sys.stderr)
        sys.exit(2)

    import torch

    import two_level_sparse_amd as T
    from two_level_sparse_amd.runtime import Cache, Decoder, bf16

    T.load_library()
    s = W.CONFIGS[args.config]
    if s.steps:
        if args.layers > 1:
            return bench_offload_layers(args, s)
        return bench_offload(args, s)
    s_data = s  # the cache and queries; s below is the shape the calls run with
    if args.mode == "quest":
        s = s.with_(Kt=min(s.Kb, s.NB) * s.bs)
    elif args.mode == "ds":
        s = s.with_(Kb=s.NB)
    elif args.mode == "dense":
        s = s.with_(Kb=s.NB, Kt=s.N)
    ab = algorithmic_bytes(s, dense=args.mode == "dense")
    touched = ab["total"]
    R = args.rotate or max(1, min(64, math.ceil((1 << 30) / touched)))
    log(f"[bench] {s.name} ({args.mode}): generating inputs (rotation over {R} cache copies)")
    q0 = W.gen_q(s_data)
    kv = W.gen_kv(s_data)
    lab = W.label_channels(s_data, kv[0])
    base = Cache(s_data, kv, lab).build()
    torch.cuda.synchronize()
    caches = [base]
    for r in range(1, R):
        c = Cache.__new__(Cache)
        c.s, c.shape = s, base.shape
        c.kv = base.kv.clone()
        c.label_ch = base.label_ch
        c.summ, c.codes, c.scale = base.summ.clone(), base.codes.clone(), base.scale.clone()
        caches.append(c)
    qs = [bf16(q0)] + [bf16(W.gen_q(s.with_(seed=s.seed + 100 * r))) for r in range(1, R)]
    if args.mode == "dense":
        dec = DenseDecoder(s)
    else:
        dec = Decoder(s)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    graphs = None
    if args.graph:
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(side):
                dec.step(qs[r], caches[r])  # warm the allocator/kernels outside capture
                with torch.cuda.graph(g, stream=side):
                    dec.step(qs[r], caches[r])
            graphs.append(g)
        stream.wait_stream(side)
        torch.cuda.synchronize()

    def one_step(i, ev=None, eager=False):
        r = i % R
        if graphs is not None and not eager:
            graphs[r].replay()
            return
        if args.mode != "dense":
            dec.select(qs[r], caches[r])
        if ev is not None:  # the library records these around its attention kernel
            T.tls_profile_events(T.TLS_PROFILE_ATTENTION, ev[0], ev[1])
        dec.decode(qs[r], caches[r].kv)
        if ev is not None:
            T.tls_profile_events(T.TLS_PROFILE_ATTENTION)

    for i in range(args.warmup):
        one_step(i)
    torch.cuda.synchronize()
    if args.calibrate_copy:  # a copy kernel of known size: 256 MiB read + 256 MiB written
        src = torch.empty(64 << 20, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    K = args.steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {K} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    # five windows of the timed steps, for the median rate
    bounds = sorted({K * w // 5 for w in range(1, 5)})
    wev = {b: torch.cuda.Event(enable_timing=True) for b in bounds}
    start.record(stream)
    for i in range(K):
        if i in wev:
            wev[i].record(stream)
        one_step(i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / K
    step_s = ms_step / 1e3
    marks = [(0, start)] + [(b, wev[b]) for b in bounds] + [(K, end)]
    win = [a[1].elapsed_time(b[1]) / (b[0] - a[0]) for a, b in zip(marks, marks[1:]) if b[0] > a[0]]
    ms_median = float(np.median(win))

    # The attention kernel alone, timed with the events the library records
    # around it on its stream, over further steps launched one call at a time
    # on the same rotating caches. A spin kernel first lets the host queue all
    # of them, so the GPU runs them back to back as in the timed replays.
    scorer = None
    P = max(20, 2 * R) if args.mode != "dense" else 5
    evs = [(TimingEvent(), TimingEvent()) for _ in range(P)]
    torch.cuda._sleep(int(2e7))
    for i in range(P):
        one_step(i, evs[i], eager=True)
    torch.cuda.synchronize()
    dec_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    how = ("timing-only HIP events (no system-scope fence) recorded by the library around each attention "
           "launch, steps queued behind a spin kernel")
    if args.mode != "dense":
        scorer = block_scorer_mfma(s, dec, qs, caches, stream)

    # the whole step against HBM: algorithmic bytes per step / step time
    ach_step = ab["total"] / step_s / 1e9
    roof = {"bound": "hbm", "kernel": "whole step (every kernel of one step, replayed as one graph)",
            "achieved": round(ach_step, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach_step / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(s.name, "step_traffic_bytes") if args.mode == "tls" else None,
            "bytes_per_step": ab["total"], "step_us": round(step_s * 1e6, 2),
            "timing": "events around the timed graph replays (inter-kernel gaps included)"}
    if dec_ms:  # the dominant kernel, attention
        kname = attention_kernel(s)
        dk = {"kernel": f"{kname} (attention of tls_sparse_decode)", "launch_us": round(dec_ms * 1e3, 2),
              "bytes_per_launch": ab["attention"], "timing": how}
        gbs = ab["attention"] / (dec_ms / 1e3) / 1e9
        if kname == "k_attend_mla":
            # both products on MFMA, 128 heads on one latent row: bound by the matrix cores
            tfl = attention_flops(s) / (dec_ms / 1e3) / 1e12
            dk.update({"bound": "mfma", "achieved": round(tfl, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                       "unit": "TFLOP/s", "frac": round(tfl / MFMA_BF16_PEAK_TFLOPS, 4),
                       "flops_per_launch": attention_flops(s),
                       "hbm": {"achieved": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}})
        else:
            dk.update({"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(gbs / HBM_PEAK_GBS, 4)})
        dk["traffic"] = measured_traffic(s.name, "attention_traffic_bytes") if args.mode == "tls" else None
        roof["dominant_kernel"] = dk

    res = {
        "metric": METRIC,
        "value": round(s.B / step_s, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{s.name}: batch {s.B}, {s.Hq} q heads / {s.Hkv} kv heads, head dim {s.D}/{s.DV}, "
                               f"context {s.N}, block {s.bs}, Kb={s.Kb}, Kt={s.Kt}, {s.r} INT4 label channels",
                   "batch": s.B, "ctx_len": s.N, "rotation": R, "graph": bool(graphs),
                   "mode": args.mode},
        "hbm": {"algorithmic_bytes_per_step": ab["total"],
                "achieved_GBps": round(ab["total"] / step_s / 1e9, 1),
                "frac_of_peak": round(ab["total"] / step_s / 1e9 / HBM_PEAK_GBS, 4)},
        "roofline": roof,
        "ms_per_step_median_of_5_windows": round(ms_median, 5),
        "block_scorer": scorer,
        "index_build": build_time(s_data, base) if args.mode != "dense" else None,
        "wall_s": round(wall, 3),
    }
    if not args.calibrate_copy:  # (a counter run keeps its calibration copy the last copy)
        res["peaks_measured"] = measured_peaks()
    if not args.no_cpu and args.mode == "tls":
        log("[bench] oracle CPU baseline")
        res["cpu_baseline"] = cpu_baseline(s, q0, kv, lab, args.cpu_budget)
    print(json.dumps(res), flush=True)


def measured_peaks():
    """What this GPU reaches on plain work, beside the published peaks that the
    roofline fractions use: a 1 GiB device-to-device copy (2 GiB of HBM
    traffic, torch's copy kernel) and an 8192^3 bf16 GEMM (hipBLASLt through
    torch), best of six each."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best_ms(fn):
        t = []
        for _ in range(6):
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            t.append(a.elapsed_time(b))
        return min(t)

    src = torch.empty(256 << 20, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    copy_ms = best_ms(lambda: dst.copy_(src))
    copy_gbs = 2 * src.numel() * 4 / (copy_ms / 1e3) / 1e9
    del src, dst
    n = 8192
    x = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
    y = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
    gemm_ms = best_ms(lambda: torch.mm(x, y))
    tflops = 2.0 * n ** 3 / (gemm_ms / 1e3) / 1e12
    del x, y
    torch.cuda.empty_cache()
    return {"hbm_copy_GBps": round(copy_gbs, 1), "hbm_copy_frac_of_peak": round(copy_gbs / HBM_PEAK_GBS, 4),
            "bf16_gemm_TFLOPs": round(tflops, 1), "bf16_gemm_frac_of_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "how": "best of 6: a 1 GiB device-to-device copy (read + write) and an 8192^3 bf16 torch.mm, "
                   "after the timed region"}


PCIE5_X16_GBS = 64.0  # PCIe 5.0 x16, one direction: 32 GT/s x 16 lanes, 128b/130b coding


def cpu_baseline_staggered(s, qs, kv, lab, budget_s):
    """The fp64 oracle's staggered schedule (O10: token stage, attention, next
    selection, delta and evictions for every pair) over the first k drift
    steps, k grown until the budget is used; scaled to queries/sec."""
    import oracle
    nth = oracle.num_threads()
    built = oracle.decode(s, qs[0], kv, lab)
    k, el = 1, 0.0
    while True:
        t0 = time.perf_counter()
        oracle.staggered(s, qs[:k], kv, lab, built)
        el = time.perf_counter() - t0
        if k >= qs.shape[0] or el * 2 > budget_s:
            break
        k = min(qs.shape[0], 2 * k)
    return {"value": s.B * k / el, "unit": "queries/s", "cores": nth, "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"the first {k} of {qs.shape[0]} staggered steps, all {s.pairs} pairs, {el:.2f} s; summaries, "
                      f"label cache and the prologue selection prebuilt (untimed); fp64 C oracle with OpenMP over "
                      f"pairs"}


def bench_offload(args, s):
    """Staggered decode with the full cache in pinned host memory: only the
    block summaries, the label cache and 2*Kb resident blocks per pair live in
    HBM. A step = token stage + attention on M_{t-1} (main stream) overlapped
    with stage 1 for M_t (stage stream) and the delta prefetch (copy stream).
    Each timed repetition starts a fresh decoder (prologue untimed), captures
    the drift steps into one HIP graph and times its replay; the value is the
    median over the repetitions."""
    import torch

    import two_level_sparse_amd as T
    from two_level_sparse_amd.runtime import Cache, StaggeredDecoder, bf16

    log(f"[bench] {s.name}: generating inputs")
    q0 = W.gen_q(s)
    kv = W.gen_kv(s)
    lab = W.label_channels(s, kv[0])
    cache = Cache(s, kv, lab).build()
    torch.cuda.synchronize()
    cache.kv = None  # the full cache stays on the host; HBM keeps only the indices
    torch.cuda.empty_cache()
    host = torch.from_numpy(kv.view(np.int16)).view(torch.bfloat16).pin_memory()
    steps = s.steps
    qs = W.drift_queries(s, q0, steps)
    qd = [bf16(qs[t]) for t in range(steps)]
    block_bytes = s.bs * s.row * 2
    kb = min(s.Kb, s.NB)
    modes = {"gather": 0, "memcpy": 1, "device": 2, "full": 3}
    mode = modes[args.copy_mode] if args.copy_mode else None
    stream = torch.cuda.current_stream()

    def run(n, graph):
        sd = StaggeredDecoder(s, cache, host, qd[0], copy_mode=mode, stagger=not args.no_stagger)
        g = sd.capture(qd[:n]) if graph and sd.device_planned else None
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        if g is not None:
            g.replay()
        else:
            for t in range(n):
                sd.step(qd[t])
        end.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(end)
        moved = sd.total_copied()
        used = {v: k for k, v in modes.items()}[sd.copy_mode]
        graphed = g is not None
        sd.close()
        del g
        return ms, moved, used, graphed

    reps = 3
    log("[bench] warmup")
    run(min(8, steps), args.graph)
    log(f"[bench] timing {reps} x {steps} staggered steps")
    t0 = time.perf_counter()
    runs = [run(steps, args.graph) for _ in range(reps)]
    wall = time.perf_counter() - t0
    per = sorted(r[0] / steps for r in runs)
    ms_step = per[len(per) // 2]
    moved, used, graphed = runs[0][1], runs[0][2], runs[0][3]

    # The host-copy kernel alone: events the library records around it, over
    # the drift steps launched one call at a time behind a spin kernel (the
    # host queues them all first, so the GPU runs them back to back).
    log("[bench] host-copy kernel events")
    sd = StaggeredDecoder(s, cache, host, qd[0], copy_mode=mode, stagger=not args.no_stagger)
    torch.cuda.synchronize()
    evs = [(TimingEvent(), TimingEvent()) for _ in range(steps)]
    torch.cuda._sleep(int(6e7))
    for t in range(steps):
        T.tls_profile_events(T.TLS_PROFILE_HOST_COPY, evs[t][0], evs[t][1])
        sd.step(qd[t])
    T.tls_profile_events(T.TLS_PROFILE_HOST_COPY)
    torch.cuda.synchronize()
    copy_ms = [a.elapsed_time(b) for a, b in evs] if used != "memcpy" else []
    sd.close()

    # the host link's large-copy rate, for scale: 64 MiB pinned -> device by the DMA engines
    big = torch.empty(64 << 20, dtype=torch.uint8).pin_memory()
    dst = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        dst.copy_(big, non_blocking=True)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(5):
        dst.copy_(big, non_blocking=True)
    b.record(stream)
    torch.cuda.synchronize()
    link_GBps = 5 * (64 << 20) / (a.elapsed_time(b) / 1e3) / 1e9
    del big, dst

    ab = algorithmic_bytes(s)
    hbm_step = ab["summaries"] + ab["label"] + ab["kv_rows"] + ab["q"] + ab["out"]
    h2d_step = moved * block_bytes / steps
    roof = None
    if copy_ms:
        cus = float(np.mean(copy_ms)) * 1e3
        ach = h2d_step / cus / 1e3
        roof = {"bound": "pcie", "kernel": "k_copy_listed (host->device block copy of tls_prefetch_delta)"
                if used in ("device", "full") else "k_gather_blocks (host->device block copy of tls_prefetch_delta)",
                "achieved": round(ach, 2), "peak": PCIE5_X16_GBS, "unit": "GB/s", "frac": round(ach / PCIE5_X16_GBS, 4),
                "traffic": None, "launch_us": round(cus, 2), "bytes_per_launch": int(h2d_step),
                "measured_link_GBps": round(link_GBps, 2),
                "timing": "timing-only HIP events (no system-scope fence) recorded by the library around each copy launch, steps queued behind a spin "
                          "kernel; peak = PCIe 5.0 x16 per direction; measured_link_GBps = 64 MiB pinned copies"}
    res = {
        "metric": METRIC,
        "value": round(s.B / (ms_step / 1e3), 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": min(8, steps),
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{s.name}: batch {s.B}, {s.Hq} q heads / {s.Hkv} kv heads, head dim {s.D}, context "
                               f"{s.N}, block {s.bs}, Kb={s.Kb}, Kt={s.Kt}, {s.r} INT4 label channels, full KV in "
                               f"pinned host memory, {steps} {'in-order' if args.no_stagger else 'staggered'} steps "
                               f"with query drift 0.1",
                   "batch": s.B, "ctx_len": s.N, "offload": True, "graph": graphed,
                   "repetitions": reps},
        "ms_per_step_each_repetition": [round(x, 5) for x in per],
        "offload": {"planning": {"device": "device", "full": "device, every selected block (no reuse)"}.get(
                        used, f"host ({used} copies)"),
                    "staggered": not args.no_stagger,
                    "blocks_copied_per_step": round(moved / steps, 1),
                    "delta_fraction": round(moved / (steps * s.pairs * kb), 4),
                    "h2d_bytes_per_step": int(h2d_step),
                    "h2d_GBps_over_the_step": round(h2d_step / (ms_step / 1e3) / 1e9, 2),
                    "h2d_bound_ms_per_step": round(h2d_step / (link_GBps * 1e9) * 1e3, 5),
                    "hbm_algorithmic_bytes_per_step": hbm_step},
        "roofline": roof,
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu and not args.no_stagger and used != "full":
        log("[bench] oracle CPU baseline")
        res["cpu_baseline"] = cpu_baseline_staggered(s, qs, kv, lab, args.cpu_budget)
    print(json.dumps(res), flush=True)


def bench_offload_layers(args, s):
    """L layers of the offloaded workload stepped as one model (LayeredDecoder):
    layer l's token stage and attention run after layer l-1's, its stage 1 and
    transfer on the shared side streams, so a layer's transfer runs under the
    attention of the layers after it. Every layer has its own device index
    (summaries, label cache), resident cache and query sequence (its own
    seed); the layers share one pinned host cache, whose contents only set the
    selections (host reads are never cached on the device). A step = step t of
    every layer; timed as one graph replay of all steps (device planning),
    staggered and, for comparison, in order (select, transfer, attend per
    layer); the host-copy kernels are timed alone with the library's events."""
    import torch

    import two_level_sparse_amd as T
    from two_level_sparse_amd.runtime import Cache, LayeredDecoder, bf16

    L, steps = args.layers, s.steps
    log(f"[bench] {s.name} x {L} layers: generating inputs")
    kv = W.gen_kv(s)
    lab = W.label_channels(s, kv[0])
    base = Cache(s, kv, lab).build()
    torch.cuda.synchronize()
    base.kv = None
    caches = [base]
    for _ in range(1, L):
        c = Cache.__new__(Cache)
        c.s, c.shape, c.kv, c.label_ch = s, base.shape, None, base.label_ch
        c.summ, c.codes, c.scale = base.summ.clone(), base.codes.clone(), base.scale.clone()
        caches.append(c)
    torch.cuda.empty_cache()
    host = torch.from_numpy(kv.view(np.int16)).view(torch.bfloat16).pin_memory()
    del kv
    q0s = [W.gen_q(s.with_(seed=s.seed + 101 * l)) for l in range(L)]
    qd = [[bf16(q) for q in W.drift_queries(s, q0s[l], steps)] for l in range(L)]
    stream = torch.cuda.current_stream()

    def run(stagger):
        ld = LayeredDecoder(s, caches, [host] * L, [qd[l][0] for l in range(L)], stagger=stagger)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            main = torch.cuda.current_stream()
            for t in range(steps):
                ld.step([qd[l][t] for l in range(L)])
            main.wait_stream(ld.stage)
            main.wait_stream(ld.side)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        moved = ld.total_copied()
        ld.close()
        del g
        return a.elapsed_time(b) / steps, moved

    log("[bench] warmup")
    run(True)
    reps = 3
    log(f"[bench] timing {reps} x {steps} steps of {L} layers, staggered and in order")
    t0 = time.perf_counter()
    pipe = sorted(run(True)[0] for _ in range(reps))
    serial = sorted(run(False)[0] for _ in range(reps))
    wall = time.perf_counter() - t0
    ms_pipe, ms_serial = pipe[len(pipe) // 2], serial[len(serial) // 2]
    moved = run(True)[1]

    # the host-copy kernels alone (events around each launch, eager steps behind a spin kernel)
    ld = LayeredDecoder(s, caches, [host] * L, [qd[l][0] for l in range(L)])
    torch.cuda.synchronize()
    n_ev = min(steps, 16)
    evs = [(TimingEvent(), TimingEvent()) for _ in range(n_ev * L)]
    torch.cuda._sleep(int(6e7))
    for t in range(n_ev):
        for l, d in enumerate(ld.layers):
            T.tls_profile_events(T.TLS_PROFILE_HOST_COPY, *evs[t * L + l])
            d.step(qd[l][t], helper=False)
    T.tls_profile_events(T.TLS_PROFILE_HOST_COPY)
    torch.cuda.synchronize()
    copy_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    ld.close()

    block_bytes = s.bs * s.row * 2
    h2d_step = moved * block_bytes / steps
    hidden = (ms_serial - ms_pipe) / (L * copy_ms) if copy_ms > 0 else None
    res = {
        "metric": METRIC,
        "value": round(s.B / (ms_pipe / 1e3), 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": steps,
        "ms_per_step": round(ms_pipe, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{s.name} x {L} layers: batch {s.B}, {s.Hq} q heads / {s.Hkv} kv heads, head dim "
                               f"{s.D}, context {s.N} per layer, block {s.bs}, Kb={s.Kb}, Kt={s.Kt}, full KV in pinned "
                               f"host memory, {steps} staggered steps of every layer with query drift 0.1",
                   "batch": s.B, "ctx_len": s.N, "layers": L, "offload": True, "graph": True, "repetitions": reps},
        "layers": {"ms_per_step_staggered": round(ms_pipe, 5), "ms_per_step_in_order": round(ms_serial, 5),
                   "ms_per_layer_step_staggered": round(ms_pipe / L, 5),
                   "copy_kernel_ms_per_layer_step": round(copy_ms, 5),
                   "copy_time_hidden_fraction": None if hidden is None else round(min(max(hidden, 0.0), 1.0), 4),
                   "blocks_copied_per_step": round(moved / steps, 1), "h2d_bytes_per_step": int(h2d_step),
                   "note": "hidden fraction = (in-order - staggered step time) / (L x copy-kernel time)"},
        "roofline": None,
        "wall_s": round(wall, 3),
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the fused attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of the forward pass over the whole workload (inputs already
resident in HBM).  The default workload is the long-context causal one
(B=1, H=32, N=16384, d=128, fp16), the largest head-dim-128 configuration.
Prints ONE JSON line on stdout; progress goes to stderr.

Metric: forward TFLOP/s with FLOP = 4*B*H*N^2*d, halved under a causal mask.
``roofline`` relates the kernel's average launch time (HIP events on the launch
stream) to the dense fp16/bf16 MFMA peak of MI355X (2.5 PFLOP/s at 2.4 GHz) and
to that peak scaled to the engine clock measured over the timed steps
(``clock_ghz``, ``frac_at_measured_clock``; fa2_clock_sample before and after).
``cpu_baseline`` times the fp64 CPU oracle on a bounded, strided sample of the
same workload's query rows on all host cores and scales it to TFLOP/s.

The default forward run also times the other named workloads (``workloads``:
each with its rate, roofline fractions, clock and a short oracle sample) and
forward plus gradients on the two 2048-token workloads (``fwd_bwd``, next to
the pages' A100 figures for those shapes); ``--headline-only`` skips them.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, published
PEAK_CLOCK_GHZ = 2.4       # engine clock the published MFMA peak assumes (256 CUs x 4096 FLOP/clk)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E bandwidth, published
PEAK_FP8_MFMA_TFLOPS = 5000.0  # MI355X dense fp8 MFMA, published
# The fp8 forward runs half its products (Q K^T) at the fp8 peak and half (P V)
# at the 16-bit peak: its ceiling is the time-weighted mix of the two.
PEAK_FP8_QK_TFLOPS = 2.0 / (1.0 / PEAK_FP8_MFMA_TFLOPS + 1.0 / PEAK_MFMA_TFLOPS)
DEFAULT_DECODE_WORKLOAD = "decode_b8h32_m1_n16384_d128"
DEFAULT_WORKLOAD = "b1h32_n16384_d128_causal"
PROFILES = os.path.join(ROOT, "profiles")
# The sources that define the kernels of each pass (a recorded profile applies
# while their digest is unchanged).
KERNEL_SOURCES = [os.path.join(ROOT, "exact_attention_11_amd", "csrc", f)
                  for f in ("fa2_common.h", "fa2_fwd_8wave.h", "fa2_fwd_pair.h", "fa2_fwd_w64.h")]
BWD_KERNEL_SOURCES = [os.path.join(ROOT, "exact_attention_11_amd", "csrc", f)
                      for f in ("fa2_common.h", "fa2_bwd.h")]
DECODE_KERNEL_SOURCES = [os.path.join(ROOT, "exact_attention_11_amd", "csrc", f)
                         for f in ("fa2_common.h", "fa2_decode.h")]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def flop_count(B: int, H: int, N: int, d: int, causal: bool) -> float:
    f = 4.0 * B * H * N * N * d
    return f / 2.0 if causal else f


def visible_pairs(N: int, causal: bool, window=None, prefix: int = 0, doc_len: int = 0) -> float:
    """Number of (query, key) pairs a general mask leaves visible: the window
    [r - wl, r + wr] (causal: wr = 0) and the prefix [0, prefix), each cut to
    the row's document when contiguous documents of doc_len rows are given."""
    import numpy as np

    wl, wr = window if window is not None else (-1, -1)
    if causal:
        wr = 0
    r = np.arange(N, dtype=np.int64)
    ds = (r // doc_len) * doc_len if doc_len else np.zeros(N, dtype=np.int64)
    de = np.minimum(ds + doc_len, N) - 1 if doc_len else np.full(N, N - 1, dtype=np.int64)
    lo = np.maximum(ds, r - wl) if wl >= 0 else ds
    hi = np.minimum(de, r + wr) if wr >= 0 else de
    pl, ph = ds, np.minimum(de, prefix - 1)

    def size(a, b):
        return np.maximum(0, b - a + 1)

    both = size(np.maximum(lo, pl), np.minimum(hi, ph))
    return float(np.sum(size(lo, hi) + size(pl, ph) - both))


_TOKEN = re.compile(r'"(?:\\.|[^"\\\n])*"|//[^\n]*|/\*.*?\*/', re.S)


def code_text(src: str) -> str:
    """C++ source with comments removed and whitespace runs collapsed: what a
    compiler sees, so that editing a comment does not void a recorded profile."""
    text = _TOKEN.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", src)
    return " ".join(text.split())


def kernel_source_digest(sources=None) -> str:
    h = hashlib.sha256()
    for p in sources or KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, summary: str | None = None, sources=None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(PROFILES, summary or f"fa2_fwd_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"kernel_source_digest:\s*(\w+)", text)
    m_val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_src or not m_val or m_src.group(1) != kernel_source_digest(sources):
        return None
    return float(m_val.group(1))


def host_threads() -> int:
    """Threads for the CPU oracle: the process's CPU share (OMP_NUM_THREADS when
    set, else the affinity mask)."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(w, q, k, v, target_s: float = 12.0):
    """Time the fp64 oracle on a strided sample of the workload's query rows.

    Rows are strided over the whole sequence, so the mix of causal row lengths
    matches the full workload.  A first (untimed) run on one head sizes the rows
    per head; whole heads are then timed in order until the sample has taken
    about ``target_s`` seconds (or the heads run out).
    """
    import numpy as np

    import oracle

    threads = host_threads()
    scale = float(np.float32(w.scale))
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]

    def run_head(i: int, rows_per_head: int):
        stride = max(1, w.N // rows_per_head)
        b, h = heads[i]
        qq, kk, vv = (t[b, h].double().numpy() for t in (q, k, v))
        rows = np.arange(i % stride, w.N, stride, dtype=np.int64)[:rows_per_head]
        t0 = time.perf_counter()
        oracle.attention_rows_f64(qq, kk, vv, rows, w.causal, scale, nthreads=threads)
        secs = time.perf_counter() - t0
        keys = float((rows + 1).sum()) if w.causal else float(len(rows)) * w.N
        return 4.0 * w.d * keys, secs

    # Calibrate on enough rows to give every thread work (the oracle hands out
    # rows in blocks of 64); this run also warms the thread pool and is not
    # counted.
    cal_rows = min(w.N, 64 * threads)
    f_cal, t_cal = run_head(0, cal_rows)
    rate = f_cal / max(t_cal, 1e-6)                       # FLOP/s of the oracle
    flop_per_row = f_cal / cal_rows
    rows_per_head = min(w.N, max(cal_rows, int(rate * target_s / flop_per_row)))
    flop, secs, n_heads = 0.0, 0.0, 0
    while n_heads < len(heads) and secs < target_s:
        f, t = run_head(n_heads, rows_per_head)
        flop += f
        secs += t
        n_heads += 1
    return {
        "value": flop / secs / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{n_heads} head(s) x {rows_per_head} strided query rows of {w.name}: "
                  f"{flop / 1e9:.1f} GFLOP in {secs:.1f} s (fp64 three-stage oracle)",
    }


def cpu_baseline_bwd(w, q, k, v, dout, target_s: float = 12.0):
    """Time the fp64 gradient oracle on whole heads of the workload, a batch of
    one head per host thread at a time (the oracle works a head per thread),
    until the sample has taken about ``target_s`` seconds (at least one batch)."""
    import numpy as np

    import oracle

    threads = host_threads()
    scale = float(np.float32(w.scale))
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    flop_head = 2.5 * flop_count(1, 1, w.N, w.d, w.causal)
    secs, n, used = 0.0, 0, 1
    while n < len(heads) and secs < target_s:
        batch = heads[n:n + threads]
        args = [np.stack([t[b, h].double().numpy() for (b, h) in batch])[None] for t in (q, k, v, dout)]
        t0 = time.perf_counter()
        oracle.attention_bwd_f64(*args, w.causal, scale, nthreads=threads)
        secs += time.perf_counter() - t0
        n += len(batch)
        used = max(used, len(batch))
    return {
        "value": n * flop_head / secs / 1e12,
        "unit": "TFLOP/s",
        "cores": used,
        "kind": "oracle",
        "sample": f"{n} whole head(s) of {w.name}: {n * flop_head / 1e9:.1f} GFLOP in {secs:.1f} s "
                  f"(fp64 gradient oracle)",
    }


def decode_bytes(w, lens) -> float:
    """Compulsory HBM bytes of one decode call: every visible cache row of K and
    V read once (the last new row of a sequence sees all of its len_b rows), Q
    read once, O and L written once."""
    rows = float(sum(int(x) for x in lens))
    kv = 2.0 * rows * w.H * w.d * 2
    qo = 2.0 * w.B * w.H * w.Mq * w.d * 2
    return kv + qo + w.B * w.H * w.Mq * 4


def cpu_baseline_masked(w, q, k, v, window, prefix, seg, pairs_per_head, target_s: float = 12.0, dout=None):
    """Time the fp64 general-mask oracle (with ``dout``: the masked gradient
    oracle) on whole heads of the workload, one head per host thread per call,
    until about ``target_s`` seconds have passed; the rate counts 4 d FLOP per
    visible (query, key) pair for the forward and 2.5 times that for the
    gradients, like the GPU line."""
    import numpy as np

    import oracle

    threads = host_threads()
    scale = float(np.float32(w.scale))
    wl, wr = window if window is not None else (-1, -1)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done, flop, secs = 0, 0.0, 0.0
    while done < len(heads) and secs < target_s:
        batch = heads[done:done + threads]
        # one batch entry per head, each with its batch's segment ids
        qs = np.stack([q[b, h].double().numpy() for b, h in batch])[:, None]
        ks = np.stack([k[b, h].double().numpy() for b, h in batch])[:, None]
        vs = np.stack([v[b, h].double().numpy() for b, h in batch])[:, None]
        segs = None if seg is None else np.stack([seg[b] for b, _ in batch])
        t0 = time.perf_counter()
        if dout is None:
            oracle.attention_masked_f64(qs, ks, vs, scale, window_left=wl, window_right=wr, prefix=prefix,
                                        segment_ids=segs, causal=w.causal, nthreads=threads)
        else:
            gs = np.stack([dout[b, h].double().numpy() for b, h in batch])[:, None]
            oracle.attention_bwd_masked_f64(qs, ks, vs, gs, scale, window_left=wl, window_right=wr, prefix=prefix,
                                            segment_ids=segs, causal=w.causal, nthreads=threads)
        secs += time.perf_counter() - t0
        flop += (4.0 if dout is None else 10.0) * w.d * pairs_per_head * len(batch)
        done += len(batch)
    kind = "general-mask oracle" if dout is None else "masked gradient oracle"
    return {
        "value": flop / secs / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} whole head(s) of {w.name} under the mask: {flop / 1e9:.1f} GFLOP of visible pairs in "
                  f"{secs:.1f} s (fp64 {kind})",
    }


def cpu_baseline_decode(w, q, k, v, lens, target_s: float = 12.0):
    """Time the fp64 decode oracle on whole (batch, head) pairs, one pair per host
    thread per call (the oracle works a (batch, head) pair per thread), until
    about ``target_s`` seconds have passed."""
    import numpy as np

    import oracle

    threads = host_threads()
    scale = float(np.float32(w.scale))
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)]
    done, nbytes, secs = 0, 0.0, 0.0
    while done < len(pairs) and secs < target_s:
        batch = pairs[done:done + threads]
        # the pairs as a batch of single-head sequences with their own lengths
        qs = np.stack([q[b, h].double().numpy() for b, h in batch])[:, None]
        ks = np.stack([k[b, h].double().numpy() for b, h in batch])[:, None]
        vs = np.stack([v[b, h].double().numpy() for b, h in batch])[:, None]
        lens_b = [int(lens[b]) for b, _ in batch]
        t0 = time.perf_counter()
        oracle.attention_decode_f64(qs, ks, vs, scale, seqlens=lens_b, causal=w.causal, nthreads=threads)
        secs += time.perf_counter() - t0
        nbytes += 2.0 * sum(lens_b) * w.d * 2
        done += len(batch)
    return {
        "value": nbytes / secs / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} (batch, head) pair(s) of {w.name}: {nbytes / 1e9:.2f} GB of fp16/bf16 cache rows in "
                  f"{secs:.1f} s (fp64 decode oracle)",
    }


class Timing:
    """What time_steps measured: ms_per_step (first event to last over the
    steps), avg/min/median launch ms (per-step event pairs), wall ms per step,
    the extra warm-up steps, and the engine clock over the timed steps (per XCD
    the average clock of its busiest CU; clock_ghz is their mean)."""

    def __init__(self, **kw):
        self.__dict__.update(kw)


def time_steps(step, stream, args, steps=None, min_warmup_ms=None):
    """Warm up (args.warmup calls, then until min_warmup_ms has passed), then
    time ``steps`` calls with HIP events on ``stream``.  A clock sample
    (fa2_clock_sample) is enqueued on the same stream right before the first
    timed call and right after the last, so the engine clock over the timed
    steps comes out per XCD."""
    import statistics

    import torch

    import exact_attention_11_amd as fa

    steps = args.steps if steps is None else steps
    min_warmup_ms = args.min_warmup_ms if min_warmup_ms is None else min_warmup_ms
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    extra = 0
    t_w0 = time.perf_counter()
    while (time.perf_counter() - t_w0) * 1e3 < min_warmup_ms:
        for _ in range(5):
            step()
        extra += 5
        torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    clk = [torch.zeros(4 * fa.CLOCK_BLOCKS, dtype=torch.int64, device="cuda") for _ in range(2)]
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    fa.clock_sample(clk[0], stream)
    for i in range(steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    fa.clock_sample(clk[1], stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall0
    launch_ms = [s_.elapsed_time(e) for s_, e in zip(starts, ends)]
    total_ms = starts[0].elapsed_time(ends[-1])
    per_cu = fa.clock_ghz(clk[0].cpu().tolist(), clk[1].cpu().tolist())
    per_xcd = fa.xcd_clocks(per_cu)
    ghz = sum(per_xcd.values()) / len(per_xcd) if per_xcd else None
    return Timing(ms_per_step=total_ms / steps, avg_ms=sum(launch_ms) / len(launch_ms), min_ms=min(launch_ms),
                  median_ms=statistics.median(launch_ms), wall_ms=wall_s * 1e3 / steps, extra=extra, steps=steps,
                  clock_ghz=ghz, clock_ghz_min=min(per_xcd.values()) if per_xcd else None,
                  clock_ghz_max=max(per_xcd.values()) if per_xcd else None, clock_xcds=len(per_xcd),
                  clock_cus=len(per_cu))


def clock_fields(t: "Timing", achieved: float, peak: float, unit_peak_at: float = PEAK_CLOCK_GHZ) -> dict:
    """The measured engine clock and the fraction of the peak scaled to it
    (the published peak assumes unit_peak_at GHz)."""
    if not t.clock_ghz:
        return {"clock_ghz": None, "frac_at_measured_clock": None}
    return {"clock_ghz": round(t.clock_ghz, 4),
            "clock_ghz_xcd_range": [round(t.clock_ghz_min, 4), round(t.clock_ghz_max, 4)],
            "peak_at_measured_clock": round(peak * t.clock_ghz / unit_peak_at, 1),
            "frac_at_measured_clock": round(achieved / (peak * t.clock_ghz / unit_peak_at), 4)}


def run_decode(args) -> int:
    import torch

    import exact_attention_11_amd as fa
    from exact_attention_11_amd.inputs import DECODE_WORKLOADS, decode_workload_inputs

    name = args.workload if args.workload in DECODE_WORKLOADS else DEFAULT_DECODE_WORKLOAD
    w = DECODE_WORKLOADS[name]
    log(f"workload {w.name}: {w.what} (decode)")
    q, k, v, lens = decode_workload_inputs(w, seed=0)
    dq, dk, dv, dl = q.cuda(), k.cuda(), v.cuda(), lens.cuda()
    o = torch.empty_like(dq)
    lse = torch.empty((w.B, w.H, w.Mq), dtype=torch.float32, device="cuda")
    need = fa.fa2_decode_workspace_bytes(w.B, w.H, w.Mq, w.Nk, w.d)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        fa.decode(dq, dk, dv, seqlens=dl, causal=w.causal, scale=w.scale, out=o, lse=lse, stream=stream,
                  workspace=ws)

    nbytes = decode_bytes(w, lens.tolist())
    t = time_steps(step, stream, args)
    ms_per_step, avg_ms, extra = t.ms_per_step, t.avg_ms, t.extra
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (avg_ms * 1e-3) / 1e9
    log(f"{args.steps} steps: {ms_per_step:.4f} ms/step (events), launch avg {avg_ms:.4f} ms, min {t.min_ms:.4f} ms, "
        f"wall {t.wall_ms:.4f} ms/step -> {value:.1f} GB/s, clock {t.clock_ghz} GHz")
    result = {
        "metric": "decode GB/s of compulsory HBM traffic (cache rows, Q, O, L), % of MI355X 8 TB/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_warmup_steps": extra,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "pass": "decode", "B": w.B, "H": w.H, "Mq": w.Mq, "Nk": w.Nk, "d": w.d,
                   "causal": w.causal, "lengths": w.lengths, "bytes_per_step": nbytes, "workspace_bytes": need,
                   "kernel_source_digest": kernel_source_digest(DECODE_KERNEL_SOURCES)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": recorded_traffic(w.name, f"fa2_decode_{w.name[len('decode_'):]}_kernel_stats.md",
                                                 DECODE_KERNEL_SOURCES),
                     "clock_ghz": round(t.clock_ghz, 4) if t.clock_ghz else None},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample of the workload ...")
        result["cpu_baseline"] = cpu_baseline_decode(w, q, k, v, lens.tolist(), args.cpu_seconds)
        log(f"cpu baseline: {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--min-warmup-ms", type=float, default=300.0,
                    help="extra untimed steps until the warm-up has lasted this long (clock ramp-up)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--window", type=int, nargs=2, default=None, metavar=("LEFT", "RIGHT"),
                    help="forward or gradient pass under a sliding window (-1: no bound on that side)")
    ap.add_argument("--prefix", type=int, default=0, help="forward or gradient pass: keys below this are visible to every query")
    ap.add_argument("--documents", type=int, default=0,
                    help="forward or gradient pass: split each sequence into this many equal contiguous documents")
    ap.add_argument("--fp8", action="store_true",
                    help="forward pass with Q and K in fp8 (e4m3, per-head scales) and V, O in the workload's "
                         "16-bit type (head dims 64, 128, 256; with or without a mask)")
    ap.add_argument("--pass", dest="pass_", choices=("fwd", "bwd", "decode"), default="fwd",
                    help="time the forward pass (the headline), the gradient pass of the workload, or decode "
                         "against a key/value cache (a decode workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing (profiling runs)")
    ap.add_argument("--headline-only", action="store_true",
                    help="forward pass: time only --workload, not the other workloads and fwd+bwd lines")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target wall time of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the attention forward pass here runs on a single MI355X, "
              "so --gpus must be 1.", file=sys.stderr)
        return 2

    import torch

    if not torch.cuda.is_available():
        log("no GPU visible")
        return 1

    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n // 2, dtype=torch.float16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {n} bytes 5 times")
        return 0

    if args.pass_ == "decode" and (args.window is not None or args.prefix > 0 or args.documents > 0):
        log("masks other than causal apply to the forward and gradient passes only")
        return 2
    if args.pass_ != "fwd" and args.fp8:
        log("fp8 inputs apply to the forward pass only")
        return 2
    if args.pass_ == "decode":
        return run_decode(args)

    import exact_attention_11_amd as fa
    from exact_attention_11_amd.inputs import WORKLOADS, workload_inputs

    w = WORKLOADS[args.workload]
    log(f"workload {w.name}: {w.what} ({args.pass_} pass)")
    q, k, v = workload_inputs(w, seed=0)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    o = torch.empty_like(dq)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    masked = args.window is not None or args.prefix > 0 or args.documents > 0
    mask_cfg = None
    peak = PEAK_MFMA_TFLOPS
    if masked:
        # contiguous documents of equal length; the same ids for every batch
        doc_len = -(-w.N // args.documents) if args.documents > 0 else 0
        seg = None
        seg_host = None
        if doc_len:
            seg_host = (torch.arange(w.N, dtype=torch.int32) // doc_len).repeat(w.B, 1).contiguous()
            seg = seg_host.cuda()
        window = tuple(args.window) if args.window is not None else None
        pairs = visible_pairs(w.N, w.causal, window, args.prefix, doc_len)
        mask_cfg = {"window": list(window) if window else None, "prefix": args.prefix, "documents": args.documents,
                    "visible_pairs_per_head": pairs}
        mask_kw = dict(window=window, prefix=args.prefix, segment_ids=seg)
    else:
        mask_kw = {}
    if args.fp8:
        if w.d not in (64, 128, 256):
            log("the fp8 forward pass serves head dims 64, 128 and 256")
            return 2
        from exact_attention_11_amd.inputs import make_qkv_fp8
        q8, k8, v16, dsq, dsk = make_qkv_fp8(w.B, w.H, w.N, w.d, q.dtype, w.dist, seed=0)
        dq8, dk8, dv16, ddq, ddk = q8.cuda(), k8.cuda(), v16.cuda(), dsq.cuda(), dsk.cuda()
        del dq, dk, dv

        def step():
            fa.forward_fp8(dq8, dk8, dv16, ddq, ddk, causal=w.causal, scale=w.scale, out=o, lse=lse, stream=stream,
                           **mask_kw)
        flop = 4.0 * w.B * w.H * w.d * pairs if masked else flop_count(w.B, w.H, w.N, w.d, w.causal)
        metric = ("attention fwd TFLOP/s with fp8 (e4m3) Q, K and 16-bit V" +
                  (" over visible pairs (general mask)" if masked else "") +
                  ", % of the MI355X MFMA ceiling for half fp8, half fp16/bf16 products")
        peak = PEAK_FP8_QK_TFLOPS
        # the oracle timing below runs on the real (descaled) inputs
        q = q8.to(torch.float64) * dsq.to(torch.float64).reshape(w.B, w.H, 1, 1)
        k = k8.to(torch.float64) * dsk.to(torch.float64).reshape(w.B, w.H, 1, 1)
        v = v16
    elif args.pass_ == "fwd" and masked:
        def step():
            fa.forward(dq, dk, dv, causal=w.causal, scale=w.scale, out=o, lse=lse, stream=stream, **mask_kw)
        flop = 4.0 * w.B * w.H * w.d * pairs
        metric = "attention fwd TFLOP/s over visible pairs (general mask), % of MI355X FP16/BF16 MFMA peak"
    elif args.pass_ == "fwd":
        def step():
            fa.forward(dq, dk, dv, causal=w.causal, scale=w.scale, out=o, lse=lse, stream=stream)
        flop = flop_count(w.B, w.H, w.N, w.d, w.causal)
        metric = "attention fwd TFLOP/s and % of MI355X FP16/BF16 MFMA peak, hd128 seq 2k-16k"
    else:
        # The gradient pass of the same problem: its inputs are the forward's O and
        # L and a seeded dO.
        fa.forward(dq, dk, dv, causal=w.causal, scale=w.scale, out=o, lse=lse, stream=stream, **mask_kw)
        g = torch.Generator().manual_seed(1)
        dout_h = torch.randn((w.B, w.H, w.N, w.d), generator=g).to(q.dtype)
        dout = dout_h.cuda()
        delta = torch.empty_like(lse)
        gq, gk, gv = torch.empty_like(dq), torch.empty_like(dq), torch.empty_like(dq)

        def step():
            fa.backward(dq, dk, dv, o, dout, lse, causal=w.causal, scale=w.scale, stream=stream, delta=delta,
                        dq=gq, dk=gk, dv=gv, **mask_kw)
        # Conventional count: five N x N x d products per (query, key) pair (S, dP,
        # dV, dQ, dK), 2.5x the forward's; under a general mask over the visible
        # pairs.
        if masked:
            flop = 2.5 * 4.0 * w.B * w.H * w.d * pairs
            metric = ("attention bwd TFLOP/s over visible pairs (general mask, 5 products per pair), % of MI355X "
                      "FP16/BF16 MFMA peak")
        else:
            flop = 2.5 * flop_count(w.B, w.H, w.N, w.d, w.causal)
            metric = "attention bwd TFLOP/s (5 products per pair) and % of MI355X FP16/BF16 MFMA peak"

    # The engine clock ramps up over the first tens of milliseconds of MFMA load;
    # time_steps keeps running untimed steps until the warm-up has lasted
    # min_warmup_ms so the timed steps see the steady clock (the count is
    # reported in the JSON line).
    t = time_steps(step, stream, args)
    ms_per_step, avg_launch_ms, extra = t.ms_per_step, t.avg_ms, t.extra
    value = flop / (ms_per_step * 1e-3) / 1e12
    achieved = flop / (avg_launch_ms * 1e-3) / 1e12
    log(f"{args.steps} steps: {ms_per_step:.4f} ms/step (events), launch avg {avg_launch_ms:.4f} ms, "
        f"min {t.min_ms:.4f} ms, wall {t.wall_ms:.4f} ms/step -> {value:.1f} TFLOP/s; engine clock "
        f"{t.clock_ghz} GHz over {t.clock_xcds} XCDs")

    traffic = recorded_traffic(w.name) if args.pass_ == "fwd" and not masked and not args.fp8 else None
    result = {
        "metric": metric,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_warmup_steps": extra,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"fp8-e4m3 QK, {w.dtype} PV" if args.fp8 else w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "pass": args.pass_, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "fp8": args.fp8,
                   "causal": w.causal, "mask": mask_cfg, "inputs": w.dist, "flop_per_step": flop,
                   "kernel_source_digest": kernel_source_digest(
                       KERNEL_SOURCES if args.pass_ == "fwd" else BWD_KERNEL_SOURCES)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": round(peak, 1),
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic, **clock_fields(t, achieved, peak)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample of the workload ...")
        if masked:
            result["cpu_baseline"] = cpu_baseline_masked(w, q, k, v, window, args.prefix,
                                                         None if seg_host is None else seg_host.numpy(),
                                                         pairs, args.cpu_seconds,
                                                         dout=dout_h if args.pass_ == "bwd" else None)
        elif args.pass_ == "fwd":
            result["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_seconds)
        else:
            result["cpu_baseline"] = cpu_baseline_bwd(w, q, k, v, dout_h, args.cpu_seconds)
        log(f"cpu baseline: {result['cpu_baseline']}")
    if args.pass_ == "fwd" and not masked and not args.fp8 and not args.headline_only:
        del q, k, v, dq, dk, dv, o, lse
        torch.cuda.empty_cache()
        result["workloads"] = [measure_forward(WORKLOADS[n], args)
                               for n in WORKLOADS if n != w.name]
        result["fwd_bwd"] = [measure_fwd_bwd(WORKLOADS[n], args) for n in FWD_BWD_WORKLOADS]
    print(json.dumps(result), flush=True)
    return 0


# The pages' A100 fwd+bwd context ("FlashAttention-2: Where the Second 2x
# Actually Comes From", Benchmarks): about 190 TFLOP/s at head dim 64, sequence
# 2k, no mask, and about 160 at head dim 128, sequence 2k, causal (FP16, read
# from plots).  The two 2048-token workloads have those shapes.
FWD_BWD_WORKLOADS = {"b8h16_n2048_d64": 190.0, "b8h16_n2048_d128_causal": 160.0}


def measure_forward(w, args) -> dict:
    """One forward workload other than the headline: a few timed steps (the
    tiny one: many, reported by the median launch), its rate against the MFMA
    peak at 2.4 GHz and at the measured clock, and a short oracle sample on
    the host cores."""
    import torch

    import exact_attention_11_amd as fa
    from exact_attention_11_amd.inputs import workload_inputs

    log(f"workload {w.name}: {w.what} (fwd pass)")
    q, k, v = workload_inputs(w, seed=0)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    o = torch.empty_like(dq)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        fa.forward(dq, dk, dv, causal=w.causal, scale=w.scale, out=o, lse=lse, stream=stream)

    tiny = w.N * w.B * w.H <= 4096
    t = time_steps(step, stream, args, steps=200 if tiny else max(args.steps, 20), min_warmup_ms=150.0)
    flop = flop_count(w.B, w.H, w.N, w.d, w.causal)
    ms = t.median_ms if tiny else t.ms_per_step
    achieved = flop / ((t.median_ms if tiny else t.avg_ms) * 1e-3) / 1e12
    value = flop / (ms * 1e-3) / 1e12
    log(f"  {t.steps} steps: {t.ms_per_step:.4f} ms/step, launch avg {t.avg_ms:.4f} median {t.median_ms:.4f} ms "
        f"-> {value:.1f} TFLOP/s, clock {t.clock_ghz} GHz")
    out = {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "dtype": w.dtype, "causal": w.causal,
           "inputs": w.dist, "flop_per_step": flop, "steps": t.steps,
           "ms_per_step": round(ms, 5), "timing": "median launch" if tiny else "events over the steps",
           "value": round(value, 3), "unit": "TFLOP/s",
           "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_MFMA_TFLOPS,
                        "frac": round(achieved / PEAK_MFMA_TFLOPS, 4), "traffic": recorded_traffic(w.name),
                        **clock_fields(t, achieved, PEAK_MFMA_TFLOPS)},
           "cpu_baseline": None}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, q, k, v, min(args.cpu_seconds, 3.0))
        log(f"  cpu baseline: {out['cpu_baseline']['value']:.4f} TFLOP/s on {out['cpu_baseline']['cores']} threads")
    return out


def measure_fwd_bwd(w, args) -> dict:
    """Forward plus gradient pass of a workload per step, counted as 3.5x the
    forward's FLOP (the forward's two products plus five in the gradients),
    next to the pages' A100 figure for that shape."""
    import torch

    import exact_attention_11_amd as fa
    from exact_attention_11_amd.inputs import workload_inputs

    log(f"workload {w.name}: forward + gradients")
    q, k, v = (t_.cuda() for t_ in workload_inputs(w, seed=0))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    dout = torch.randn((w.B, w.H, w.N, w.d), generator=torch.Generator().manual_seed(1)).to(q.dtype).cuda()
    delta = torch.empty_like(lse)
    gq, gk, gv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def step():
        fa.forward(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, stream=stream)
        fa.backward(q, k, v, o, dout, lse, causal=w.causal, scale=w.scale, stream=stream, delta=delta,
                    dq=gq, dk=gk, dv=gv)

    t = time_steps(step, stream, args, steps=max(args.steps, 20), min_warmup_ms=150.0)
    flop = 3.5 * flop_count(w.B, w.H, w.N, w.d, w.causal)
    value = flop / (t.ms_per_step * 1e-3) / 1e12
    log(f"  {t.steps} steps: {t.ms_per_step:.4f} ms/step -> {value:.1f} TFLOP/s fwd+bwd, clock {t.clock_ghz} GHz")
    return {"workload": w.name, "pass": "fwd+bwd", "flop_per_step": flop, "steps": t.steps,
            "ms_per_step": round(t.ms_per_step, 5), "value": round(value, 3), "unit": "TFLOP/s",
            "frac": round(value / PEAK_MFMA_TFLOPS, 4), "clock_ghz": round(t.clock_ghz, 4) if t.clock_ghz else None,
            "pages_a100_context_tflops": FWD_BWD_WORKLOADS[w.name]}


if __name__ == "__main__":
    sys.exit(main())

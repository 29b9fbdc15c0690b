#!/usr/bin/env python3
"""Benchmark of the fp8 MQA indexer hot path (logits + top-k) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = the whole hot path over one synthetic batch: the fused C entry
(indexer_logits_topk_ragged, or indexer_logits_topk_paged for the decode
workload), which per row chunk launches the fp8 MQA logits into its workspace
and then the per-row top-k.  The default workload is the largest one, the
long prefix of the chunking page's `warm_long_150K+60K` scenario: 7500 query
rows over 210000 keys under the 2e9-byte logits cap (4 chunks of 2380, 2380,
2380 and 360 rows).  Inputs are resident in HBM before timing starts.  Rank 0
prints one JSON line.

Two timed regions run back to back, each after its own warm-up and each
bracketed by synchronisations:
  1. K steps of the fused entry: `value` and `ms_per_step` (the calls alone
     between two synchronisations), then K more steps each bracketed by HIP
     events for the per-step distribution;
  2. K steps of the same launches made one call at a time (the logits entry
     into the same chunk buffer, then the top-k entry), with HIP events on the
     launch stream between them: the per-launch durations behind `roofline`
     (`split_ms_per_step` shows that both regions do the same work).
Under `rocprofv3 --selected-regions` only these two regions are traced
(roctxProfilerResume / Pause around them).

Extra modes (used to collect counters and cross-checks):
  --no-cpu-baseline    skip the oracle timing (profiling runs)
  --copy-calibration   only run a plain device copy of known size (for
                       scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters)
  --core-probe N       only run the logits-core probe (the logits kernels'
                       per-fragment code on register operands) N times at the
                       ragged kernel's occupancy (for its SQ counters)
  --all-workloads PATH time every workload, with the oracle beside each,
                       and write a JSON list to PATH
  --trace-summary CSV  (no GPU) summarise a rocprofv3 kernel_trace.csv or
                       counter_collection.csv of a run of this script made
                       with the same --steps / --warmup: per kernel, only the
                       dispatches of the timed steps of both regions
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_FP8_PEAK = 5.0e15     # MI355X dense fp8 MFMA, FLOP/s
HBM_PEAK = 8.0e12          # MI355X HBM3E, bytes/s
H, D = 32, 128
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_counters.json")
KERNEL_SOURCES = ["fp8_mqa_logits_amd/csrc/logits_ragged.hip", "fp8_mqa_logits_amd/csrc/mqa_core.hpp",
                  "fp8_mqa_logits_amd/csrc/device_common.hpp", "fp8_mqa_logits_amd/csrc/logits_paged.hip",
                  "fp8_mqa_logits_amd/csrc/topk.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_prefix_210k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the on-box MFMA and copy peak probes")
    ap.add_argument("--cold", action="store_true",
                    help="read a 512 MiB scratch buffer before each timed step (cold, clean caches)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--core-probe", type=int, default=0, metavar="LAUNCHES",
                    help="only run the logits-core probe at the ragged kernel's occupancy, LAUNCHES times")
    ap.add_argument("--trace-summary", default="", metavar="CSV")
    ap.add_argument("--all-workloads", default="")
    ap.add_argument("--overlap", action="store_true", help="time the fused loop serial vs overlapped")
    ap.add_argument("--cap-sweep", action="store_true",
                    help="the chunking page's experiment: fused step per logits cap (0 = one shot), serial and "
                         "overlapped, on the page's four scenarios")
    ap.add_argument("--prep", action="store_true", help="time index preparation at the PR page's shapes")
    ap.add_argument("--quant", action="store_true", help="time the fp8 quantiser on the path's kv and q shapes")
    ap.add_argument("--sparse-mla", action="store_true",
                    help="time the sparse MLA attention over top-k slots (the step after the indexer)")
    return ap.parse_args()


def _dev(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# ---------------------------------------------------------------------------
# ragged prefill workload
# ---------------------------------------------------------------------------

class RaggedStep:
    def __init__(self, inp):
        import torch
        import fp8_mqa_logits_amd as F
        self.F = F
        self.inp = inp
        self.q, self.kv, self.sc, self.w, self.ks, self.ke = (
            _dev(inp.q), _dev(inp.kv), _dev(inp.kv_scale), _dev(inp.weights), _dev(inp.ks), _dev(inp.ke))
        m, n, k = inp.m, inp.n, inp.k
        self.cap = inp.cap_bytes
        # the fused entry's chunks: ceil(m / the cap-derived size), rows spread evenly over them
        cmax = F.fp8idx_rows_per_chunk(self.cap, n, m)
        nch = -(-m // cmax)
        self.rpc = -(-m // nch)
        self.ld = (n + 3) // 4 * 4
        self.logits = torch.empty((self.rpc, self.ld), dtype=torch.float32, device="cuda")
        tk = F.fp8idx_workspace_bytes(F.OP_TOPK, self.rpc, n, k, 0)
        self.ws_topk = torch.empty(max(tk, 1) + 256, dtype=torch.uint8, device="cuda")
        self.ws_logits = torch.empty(512, dtype=torch.uint8, device="cuda")
        self.out = torch.empty((m, k), dtype=torch.int32, device="cuda")
        fws = F.fp8idx_workspace_bytes(F.OP_LOGITS_TOPK_RAGGED, m, n, k, self.cap)
        self.fused_ws = torch.empty(fws + 256, dtype=torch.uint8, device="cuda")
        self.events = []
        import numpy as np
        pairs = np.maximum(inp.ke.astype(np.int64) - inp.ks, 0)
        # algorithmic flops of each chunk's logits launch: 2 * H * D per valid (row, key) pair
        self.chunk_flops = [2.0 * H * D * float(pairs[s:s + self.rpc].sum()) for s in range(0, m, self.rpc)]
        self.entry = "indexer_logits_topk_ragged"

    def run(self, record=False):
        """One pass of the hot path: per chunk, logits launch then top-k launch."""
        import torch
        F, inp = self.F, self.inp
        for s in range(0, inp.m, self.rpc):
            e = min(inp.m, s + self.rpc)
            lg = self.logits[: e - s, : inp.n] if self.ld == inp.n else self.logits[: e - s]
            if record:
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                ev[0].record()
            F.indexer_logits_ragged(self.q[s:e], self.kv, self.sc, self.w[s:e], self.ks[s:e], self.ke[s:e],
                                    clean=False, logits=self.logits[: e - s], workspace=self.ws_logits)
            if record:
                ev[1].record()
            F.indexer_topk(self.logits[: e - s], self.ke[s:e], inp.k, ks=self.ks[s:e], width=inp.n, row0=s,
                           out=self.out[s:e], workspace=self.ws_topk)
            if record:
                ev[2].record()
                self.events.append((ev, e - s))

    def run_fused(self):
        self.F.indexer_logits_topk_ragged(self.q, self.kv, self.sc, self.w, self.ks, self.ke, self.inp.k,
                                          logits_cap_bytes=self.cap, out=self.out, workspace=self.fused_ws)

    def run_overlap(self):
        """The fused loop with chunk N - 1's top-k on a side stream while chunk N's logits run."""
        import torch
        if getattr(self, "overlap_ws", None) is None:
            need = self.F.fp8idx_workspace_bytes(self.F.OP_LOGITS_TOPK_RAGGED_OVERLAP, self.inp.m, self.inp.n,
                                                 self.inp.k, self.cap)
            self.overlap_ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
            self.side = torch.cuda.Stream()
        self.F.indexer_logits_topk_ragged_overlap(self.q, self.kv, self.sc, self.w, self.ks, self.ke, self.inp.k,
                                                  side_stream=self.side, logits_cap_bytes=self.cap,
                                                  out=self.out, workspace=self.overlap_ws)

    def kernel_times(self):
        """Mean logits and top-k launch durations (ms) over the recorded launches, and their count."""
        lt = [ev[0].elapsed_time(ev[1]) for ev, _ in self.events]
        tt = [ev[1].elapsed_time(ev[2]) for ev, _ in self.events]
        return sum(lt) / len(lt), sum(tt) / len(tt), len(lt)

    def logits_flops_per_launch(self):
        """Mean algorithmic flops of one logits launch (the chunks' mean)."""
        return sum(self.chunk_flops) / len(self.chunk_flops)

    def flops(self):
        return 2.0 * H * D * self.inp.valid_pairs

    def topk_bytes(self):
        # read each row's window once (fp32) and write k int32 indices per row
        return 4.0 * self.inp.valid_pairs + 4.0 * self.inp.m * self.inp.k


class PagedStep:
    def __init__(self, inp):
        import torch
        import fp8_mqa_logits_amd as F
        self.F = F
        self.inp = inp
        self.args = [_dev(a) for a in (inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len,
                                       inp.block_table)]
        self.width = inp.max_pages * 64
        self.ld = (self.width + 3) // 4 * 4
        self.logits = torch.empty((inp.rows, self.ld), dtype=torch.float32, device="cuda")
        tk = F.fp8idx_workspace_bytes(F.OP_TOPK, inp.rows, self.width, inp.k, 0)
        self.ws_topk = torch.empty(max(tk, 1) + 256, dtype=torch.uint8, device="cuda")
        self.out = torch.empty((inp.rows, inp.k), dtype=torch.int32, device="cuda")
        m = F.TopkMap(kind=F.MAP_BLOCK_TABLE, table=self.args[5], rows_per_req=inp.next_n, page_size=64,
                      num_pages=inp.kv_pool.shape[0])
        self.map = m
        fws = F.fp8idx_workspace_bytes_paged(inp.B, inp.next_n, self.width, inp.k, 0)
        self.fused_ws = torch.empty(fws + 256, dtype=torch.uint8, device="cuda")
        self.events = []
        self.entry = "indexer_logits_topk_paged"

    def run(self, record=False):
        import torch
        F, inp = self.F, self.inp
        if record:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            ev[0].record()
        F.indexer_logits_paged(*self.args, width=self.width, clean=False, logits=self.logits)
        if record:
            ev[1].record()
        F.indexer_topk(self.logits, self.args[4], inp.k, width=self.width, map=self.map, out=self.out,
                       workspace=self.ws_topk)
        if record:
            ev[2].record()
            self.events.append((ev, inp.rows))

    def run_fused(self):
        self.F.indexer_logits_topk_paged(*self.args, self.inp.k, width=self.width, out=self.out,
                                         workspace=self.fused_ws)

    kernel_times = RaggedStep.kernel_times

    def flops(self):
        return 2.0 * H * D * self.inp.valid_pairs

    def kv_bytes(self):
        inp = self.inp
        q = inp.rows * H * D
        w = inp.rows * H * 4
        bt = int(((inp.ctx.astype("int64") + 63) // 64).sum()) * 4
        return float(inp.kv_bytes + q + w + bt + 4.0 * inp.valid_pairs)

    def topk_bytes(self):
        return 4.0 * self.inp.valid_pairs + 4.0 * self.inp.rows * self.inp.k


class Roctx:
    """roctxProfilerResume / roctxProfilerPause (rocprofiler-sdk), so that a run under
    `rocprofv3 --selected-regions` traces the timed regions only.  Without the profiler the calls do
    nothing; without the library they are skipped."""

    def __init__(self):
        import ctypes
        self.lib = None
        for name in ("librocprofiler-sdk-roctx.so.1", "librocprofiler-sdk-roctx.so"):
            try:
                self.lib = ctypes.CDLL(name)
                break
            except OSError:
                continue
        if self.lib is not None:
            for fn in ("roctxProfilerPause", "roctxProfilerResume"):
                getattr(self.lib, fn).argtypes = [ctypes.c_uint64]
                getattr(self.lib, fn).restype = ctypes.c_int

    def pause(self):
        if self.lib is not None:
            self.lib.roctxProfilerPause(0)

    def resume(self):
        if self.lib is not None:
            self.lib.roctxProfilerResume(0)


ROCTX = None


def _roctx():
    global ROCTX
    if ROCTX is None:
        ROCTX = Roctx()
    return ROCTX


def _scratch():
    """512 MiB of device memory for evicting the caches (twice the 256 MB Infinity Cache)."""
    import torch
    x = torch.zeros((512 << 20) // 4, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    return x


def _evict(scratch):
    """Evict the caches by reading the scratch buffer: the lines it leaves are clean, so the step
    that follows pays no write-backs for them (rewriting the buffer instead would leave up to 256 MB
    of dirty lines whose write-backs land inside the step)."""
    scratch.sum()


def _time_steps(step, steps, warmup, record, cold=False):
    """Wall ms per step over `steps` timed steps of the launches made one call at a time; with
    record, per-launch and per-step HIP events (on the launch stream) are kept on the step for the
    kernel times and the step distribution.

    cold: before every step a 512 MiB scratch buffer is read (more than the 256 MB Infinity Cache),
    so each step starts with caches holding none of its data (see _evict); the flush lies outside
    the step events, and the returned ms per step is then the mean of the step events instead of the
    wall time."""
    import torch
    scratch = _scratch() if cold else None
    for _ in range(warmup):
        step.run()
    torch.cuda.synchronize()
    step.events = []
    step.step_events = []
    _roctx().resume()
    t0 = time.perf_counter()
    for i in range(steps):
        if cold:
            _evict(scratch)
        if record:
            se = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            se[0].record()
        step.run(record=record)
        if record:
            se[1].record()
            step.step_events.append(se)
    torch.cuda.synchronize()
    t = time.perf_counter() - t0
    _roctx().pause()
    if cold and record:
        return sum(e[0].elapsed_time(e[1]) for e in step.step_events) / steps
    return t * 1e3 / steps


def _median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def _distribution(step, fused_events):
    """Median and min of the fused step times and of the per-launch kernel times (ms)."""
    st = [e[0].elapsed_time(e[1]) for e in fused_events]
    lt = [ev[0].elapsed_time(ev[1]) for ev, _ in step.events]
    tt = [ev[1].elapsed_time(ev[2]) for ev, _ in step.events]
    return {"step_ms_median": round(_median(st), 4), "step_ms_min": round(min(st), 4),
            "logits_launch_ms_median": round(_median(lt), 4), "logits_launch_ms_min": round(min(lt), 4),
            "topk_launch_ms_median": round(_median(tt), 4), "topk_launch_ms_min": round(min(tt), 4)}


def measured_peaks():
    """On-box peaks next to the published ones.

    mfma: the library's fp8 MFMA throughput probe (2 and 4 workgroups of 256 threads per CU, each wave
    4 x 4096 back-to-back 16x16x128 fp8 MFMAs on four accumulators), HIP events around 5 launches;
    the faster of the two.
    copy: a device-to-device copy of 1 GiB (torch copy_), read plus written bytes, 5 copies.
    """
    import torch
    import fp8_mqa_logits_amd as F
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    iters, reps = 4096, 5
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    mfma_tflops, best = 0.0, 0
    for per_cu in (2, 4):
        blocks = per_cu * cus
        out, flops = F.fp8idx_probe_mfma_fp8(blocks, iters)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            F.fp8idx_probe_mfma_fp8(blocks, iters, out=out)
        e1.record()
        torch.cuda.synchronize()
        t = flops / (e0.elapsed_time(e1) / reps * 1e-3) / 1e12
        if t > mfma_tflops:
            mfma_tflops, best = t, blocks
    core = core_probe(cus, (2, 3, 4), iters=2048, reps=reps)
    nbytes = 1 << 30
    x = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").uniform_()
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 2.0 * nbytes / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
    del x, y, out
    torch.cuda.empty_cache()
    return {"mfma_fp8_tflops": round(mfma_tflops, 1), "copy_gbps": round(copy_gbps, 1),
            "logits_core_tflops": {str(k): round(v, 1) for k, v in core.items()},
            "mfma_probe": f"{best} x 256 threads, 4 x {iters} fp8 16x16x128 MFMAs per wave, {reps} launches",
            "logits_core_probe": (f"2, 3 and 4 x {cus} workgroups of 256 threads, 2048 logits-core fragments "
                                  f"(8 fp8 16x16x128 MFMAs + exact epilogue) per wave, {reps} launches"),
            "copy_probe": f"1 GiB device copy, read + written bytes, {reps} copies"}


# Workgroups of the ragged logits kernel resident per CU (4 waves each, 168 VGPRs: 3 waves per SIMD).
RAGGED_WGS_PER_CU = 3


def core_probe(cus, per_cu_list, iters, reps):
    """TFLOP/s of the logits-core probe (the logits kernels' per-fragment MFMA + exact-epilogue code on
    register operands, no memory traffic) at each number of 256-thread workgroups per CU."""
    import torch
    import fp8_mqa_logits_amd as F
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {}
    for per_cu in per_cu_list:
        blocks = per_cu * cus
        out, flops = F.fp8idx_probe_logits_core(blocks, iters)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            F.fp8idx_probe_logits_core(blocks, iters, out=out)
        e1.record()
        torch.cuda.synchronize()
        res[per_cu] = flops / (e0.elapsed_time(e1) / reps * 1e-3) / 1e12
    return res


def _time_fused(step, steps, warmup, overlap=False, cold=False):
    """(ms per step, per-step event pairs) over `steps` calls of the fused entry (or the overlapped
    one).  The timed loop holds the calls alone, between two synchronisations: a timing event pair
    recorded inside every step costs GPU time of its own (about 13 us per step, 7% of a decode step).
    The per-step distribution comes from a second loop of `steps` calls, each bracketed by events.
    With `cold`, a scratch read between steps evicts the caches and the step times are those events."""
    import torch
    run = step.run_overlap if overlap else step.run_fused
    scratch = _scratch() if cold else None
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    t = None
    if not cold:
        _roctx().resume()
        t0 = time.perf_counter()
        for _ in range(steps):
            run()
        torch.cuda.synchronize()
        t = time.perf_counter() - t0
        _roctx().pause()
    evs = []
    for i in range(steps):
        if cold:
            _evict(scratch)
        e = [torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
        e[0].record()
        run()
        e[1].record()
        evs.append(e)
    torch.cuda.synchronize()
    if cold:
        return sum(a.elapsed_time(b) for a, b in evs) / steps, evs
    return t * 1e3 / steps, evs


def _traffic(workload, kernel_key):
    """HBM bytes per launch of a kernel on a workload from the committed counter runs, if they were
    taken on these kernel sources."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_hash") != kernel_source_hash():
        return None
    k = c.get("workloads", {}).get(workload, {}).get(kernel_key)
    if not k:
        return None
    return k.get("hbm_bytes_per_launch")


def _cpu_info():
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return int(threads), cpu_model


def _cpu_baseline(inp, budget_s):
    """Time the float64 oracle (logits + top-k) on an evenly spaced row sample of the workload,
    scaled to the whole workload (TFLOP/s and the ms/layer it implies)."""
    import numpy as np
    from oracle import mqa_logits, paged_mqa_logits, topk_indices
    paged = hasattr(inp, "kv_pool")
    rows_total = inp.rows if paged else inp.m
    lens = inp.row_len.astype(np.int64) if paged else np.maximum(inp.ke.astype(np.int64) - inp.ks, 0)
    order = np.linspace(0, rows_total - 1, num=min(rows_total, 4096)).astype(np.int64)
    order = np.unique(order)
    width = inp.max_pages * inp.page_size if paged else None
    done, valid, t_total = 0, 0, 0.0
    block = 8
    while done < order.size and (t_total < budget_s or done < 8):
        rows = order[done:done + block]
        t0 = time.perf_counter()
        if paged:
            L = paged_mqa_logits(inp.q, inp.kv_pool, inp.scale_pool, inp.weights, inp.row_len, inp.block_table,
                                 inp.page_size, width=width, rows=rows)
            topk_indices(L, np.zeros(rows.size, np.int64), inp.row_len[rows], inp.k)
        else:
            L = mqa_logits(inp.q[rows], inp.kv, inp.kv_scale, inp.weights[rows], inp.ks[rows], inp.ke[rows])
            topk_indices(L, inp.ks[rows], inp.ke[rows], inp.k)
        t_total += time.perf_counter() - t0
        valid += int(lens[rows].sum())
        done += rows.size
    tflops = 2.0 * H * D * valid / t_total / 1e12
    threads, cpu_model = _cpu_info()
    ms_layer = t_total * 1e3 * inp.valid_pairs / max(valid, 1)
    return {"value": round(tflops, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model, "ms_per_layer_equivalent": round(ms_layer, 1),
            "sample": f"{done} evenly spaced rows of {rows_total} ({valid} valid (row, key) pairs), "
                      f"float64 logits + top-k, {t_total:.1f} s, scaled to all "
                      f"{inp.valid_pairs} pairs"}


def run_workload(name, steps, warmup, cold=False, overlap=False):
    """Both timed regions on one workload: the fused entry (step time), then the same launches one
    call at a time with per-launch events (kernel times)."""
    import torch
    from workloads.generate import config_inputs
    inp = config_inputs(name)
    paged = hasattr(inp, "kv_pool")
    step = PagedStep(inp) if paged else RaggedStep(inp)
    torch.cuda.synchronize()
    fused_ms, fused_events = _time_fused(step, steps, warmup, cold=cold)
    split_ms = _time_steps(step, steps, warmup, record=True, cold=cold)
    logit_ms, topk_ms, launches = step.kernel_times()
    per_step = launches // steps
    res = {"workload": inp.name, "entry": step.entry, "ms_per_step": fused_ms, "split_ms_per_step": split_ms,
           "logits_ms": logit_ms * per_step, "topk_ms": topk_ms * per_step, "logits_ms_per_launch": logit_ms,
           "topk_ms_per_launch": topk_ms, "launches_per_step": per_step, "flops": step.flops(),
           "fused_events": fused_events, "inp": inp, "step": step}
    if overlap and not paged and step.rpc < inp.m:
        res["overlap_ms_per_step"], _ = _time_fused(step, steps, warmup, overlap=True)
    return res


# Logits caps of the chunking page's experiment (bytes; 0 = one shot, the whole rows x keys buffer).
CAP_SWEEP = (0, 8_000_000_000, 4_000_000_000, 2_000_000_000, 1_000_000_000, 500_000_000)


def cap_sweep(steps, warmup):
    """The fused logits + top-k step per logits cap, serial and with chunk N - 1's top-k overlapped
    (the chunking page's `main`: ms per layer per cap against the one-shot run).  Every cap's selection
    is compared with the one-shot selection: the per-(row, key) arithmetic does not depend on the
    chunking, so the selected sets must be equal."""
    import dataclasses
    import numpy as np
    import torch
    from workloads.generate import config_inputs
    out = []
    for name in ("prefill_64k", "tail_80k", "warm_154k", "long_prefix_210k"):
        base = config_inputs(name)
        one_shot, ref = None, None
        for cap in CAP_SWEEP:
            inp = dataclasses.replace(base, cap_bytes=cap)
            step = RaggedStep(inp)
            chunks = -(-inp.m // step.rpc)
            serial, _ = _time_fused(step, steps, warmup)
            sel = np.sort(step.out.cpu().numpy(), axis=1)
            if ref is None:
                ref, one_shot = sel, serial
            r = {"workload": base.name.split("_cap")[0], "cap_gb": cap / 1e9, "chunks": chunks,
                 "rows_per_chunk": step.rpc, "peak_logits_mb": round(step.rpc * step.ld * 4 / 1e6, 1),
                 "serial_ms": round(serial, 4), "vs_one_shot": round(serial / one_shot - 1, 4),
                 "selection_equal_one_shot": bool(np.array_equal(sel, ref))}
            if chunks > 1:
                over, _ = _time_fused(step, steps, warmup, overlap=True)
                r["overlap_ms"] = round(over, 4)
                r["overlap_selection_equal_one_shot"] = bool(
                    np.array_equal(np.sort(step.out.cpu().numpy(), axis=1), ref))
            out.append(r)
            del step
            torch.cuda.empty_cache()
    return out


QUANT_SHAPES = (
    ("kv_n65536_d128", 65536, 128),          # the 65536-key prefill's kv (per-token scales)
    ("q_m8192_h32_d128", 8192 * 32, 128),    # its q, one row per (query row, head)
    ("kv_n210000_d128", 210000, 128),        # the long-prefix workload's kv
)


def quant_workloads(steps, warmup):
    """Time indexer_quant_fp8 on the path's kv and q shapes: HBM bytes = 4 read + 1 written per
    element plus 4 per row (the scale), HIP events on the launch stream around each launch."""
    import torch
    import fp8_mqa_logits_amd as F
    from workloads.generate import quant_inputs
    out = []
    for name, rows, D in QUANT_SHAPES:
        x = torch.from_numpy(quant_inputs(rows, D, seed=rows)).cuda()
        codes = torch.empty((rows, D), dtype=torch.uint8, device="cuda")
        scale = torch.empty(rows, dtype=torch.float32, device="cuda")
        for _ in range(warmup):
            F.indexer_quant_fp8(x, codes=codes, scale=scale)
        torch.cuda.synchronize()
        evs = []
        for _ in range(steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            F.indexer_quant_fp8(x, codes=codes, scale=scale)
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
        nbytes = rows * D * 5 + rows * 4
        out.append({"workload": f"quant_{name}", "rows": rows, "D": D, "ms": ms, "hbm_bytes": nbytes,
                    "gbps": nbytes / (ms * 1e-3) / 1e9, "hbm_frac": nbytes / (ms * 1e-3) / HBM_PEAK})
        del x, codes, scale
        torch.cuda.empty_cache()
    return out


# Sparse MLA attention over the top-k slots (the step after the indexer).  The pool holds one MLA
# row per indexer token slot: 64 requests x E[ctx] = 69632 tokens for the decode workload.
MLA_SHAPES = (
    ("decode_t256_h64", 256, 64, 2048, 64 * 69632),     # 64 requests x 4 rows, 64 heads per rank
    ("decode_t256_h16", 256, 16, 2048, 64 * 69632),     # the same with heads sliced across ranks
    ("decode_t4_h64_split", 4, 64, 2048, 64 * 69632),   # one request: split-K partials + combine
    ("prefill_t2048_h64", 2048, 64, 2048, 8 * 65536),   # a prefill batch of 2048 query tokens
)
BF16_PEAK = 2.5e15


def _mla_device_inputs(T, H, topk, S, seed):
    """Seeded synthetic sparse MLA inputs drawn on the device (the recipe of
    workloads.generate.sparse_mla_inputs at pool sizes too large to draw on the host): q randn
    clamped to [-2, 2] in bf16, kv randn clamped and cast to e4m3fn, kv_scale U[0.5, 1.5), and
    uniform random slot ids."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    q = torch.randn((T, H, 576), generator=g, device="cuda").clamp_(-2, 2).to(torch.bfloat16)
    kv = torch.empty((S, 576), dtype=torch.uint8, device="cuda")
    for s0 in range(0, S, 262144):
        e = min(S, s0 + 262144)
        x = torch.randn((e - s0, 576), generator=g, device="cuda").clamp_(-2, 2)
        kv[s0:e] = x.to(torch.float8_e4m3fn).view(torch.uint8)
        del x
    sc = torch.rand(S, generator=g, device="cuda") + 0.5
    idx = torch.randint(0, S, (T, topk), generator=g, device="cuda", dtype=torch.int32)
    return q, kv, sc, idx


def sparse_mla_workloads(steps, warmup, cpu_tokens=0):
    """Time indexer_sparse_mla: flops 2 T H topk (576 + 512); HBM bytes = the gathered rows
    (576 code bytes + a 4-byte scale per listed slot) + q + indices + outputs."""
    import torch
    import fp8_mqa_logits_amd as F
    out = []
    for name, T, Hh, topk, S in MLA_SHAPES:
        q, kv, sc, idx = _mla_device_inputs(T, Hh, topk, S, seed=T + Hh)
        o = torch.empty((T, Hh, 512), dtype=torch.float32, device="cuda")
        lse = torch.empty((T, Hh), dtype=torch.float32, device="cuda")
        need = F.fp8idx_sparse_mla_workspace_bytes(T, Hh, topk)
        ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda") if need else None
        scale = 576 ** -0.5
        ms = _event_ms(lambda: F.indexer_sparse_mla(q, kv, sc, idx, scale, out=o, lse=lse, workspace=ws),
                       steps, warmup)
        flops = 2.0 * T * Hh * topk * (576 + 512)
        nbytes = T * topk * (576 + 4) + T * Hh * 576 * 2 + T * topk * 4 + T * Hh * (512 + 1) * 4
        r = {"workload": f"sparse_mla_{name}", "T": T, "H": Hh, "topk": topk, "slots": S, "ms": ms,
             "tflops": flops / (ms * 1e-3) / 1e12, "bf16_frac": flops / (ms * 1e-3) / BF16_PEAK,
             "hbm_bytes": nbytes, "gbps": nbytes / (ms * 1e-3) / 1e9, "hbm_frac": nbytes / (ms * 1e-3) / HBM_PEAK,
             "splits": 1 if need == 0 else None}
        if cpu_tokens > 0 and name == MLA_SHAPES[0][0]:
            from oracle import sparse_mla
            import numpy as np
            toks = list(range(cpu_tokens))
            sel = idx[:cpu_tokens].cpu().numpy()
            uniq, inv = np.unique(sel, return_inverse=True)
            kv_s = kv[torch.from_numpy(uniq).cuda().long()].cpu().numpy()
            sc_s = sc[torch.from_numpy(uniq).cuda().long()].cpu().numpy()
            q_s = q[:cpu_tokens].view(torch.int16).cpu().numpy().view(np.uint16)
            t0 = time.perf_counter()
            sparse_mla(q_s, kv_s, sc_s, inv.reshape(sel.shape).astype(np.int32), scale, tokens=toks)
            cpu_s = time.perf_counter() - t0
            r["cpu_oracle_ms_per_token"] = cpu_s * 1e3 / cpu_tokens
            r["cpu_oracle_sample"] = f"{cpu_tokens} tokens of {T}, all {Hh} heads, float64 numpy"
        out.append(r)
        del q, kv, sc, idx, o, lse, ws
        torch.cuda.empty_cache()
    return out


def _event_ms(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / len(evs)


def _graph_ms(fn, calls=20, replays=10):
    """Per-call device time of fn from a graph of `calls` captured calls, replayed (the PR page
    times its index kernels from CUDA-graph samples, without host launch cost)."""
    import torch
    s = torch.cuda.Stream()
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(calls):
                fn(stream=s)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (calls * replays)


def prep_workloads(steps, warmup):
    """Index preparation at the shape of the PR page's index benchmark: 8 requests x 1M tokens
    (16 queries per request for prefill; 1 and 4 rows per request for decode and MTP, page 64).
    Per-call device time from graph replays; `steps` and `warmup` are unused here."""
    import torch
    import fp8_mqa_logits_amd as F
    B, S = 8, 1 << 20
    g = torch.Generator(device="cpu").manual_seed(21)
    table = torch.randint(0, 1 << 30, (B, S), generator=g, dtype=torch.int32).cuda()
    seq = torch.full((B,), S, dtype=torch.int32, device="cuda")
    req = torch.randperm(B, generator=g).to(torch.int32).cuda()
    q16 = torch.full((B,), 16, dtype=torch.int32, device="cuda")
    r2p = torch.randint(0, 1 << 20, (B, S // 64), generator=g, dtype=torch.int32).cuda()
    out = []
    ms = _graph_ms(lambda stream=None: F.indexer_prepare_ragged(seq, q16, req, table, max_q=B * 16,
                                                                max_keys=B * S, stream=stream))
    nbytes = B * S * 8
    out.append({"workload": "prep_prefill_8x1M_q16_with_ragged_copy", "ms": ms, "hbm_bytes": nbytes,
                "gbps": nbytes / (ms * 1e-3) / 1e9})
    ms = _graph_ms(lambda stream=None: F.indexer_prepare_ragged(seq, q16, req, table, max_q=B * 16, max_keys=0,
                                                                ragged_mem=False, stream=stream))
    out.append({"workload": "prep_prefill_8x1M_q16_windows_only", "ms": ms})
    for nn in (1, 4):
        ms = _graph_ms(lambda stream=None: F.indexer_prepare_decode(seq, req, r2p, nn, stream=stream))
        out.append({"workload": f"prep_decode_8x1M_next_n{nn}", "ms": ms, "hbm_bytes": B * (S // 64) * 8})
    del table, r2p
    torch.cuda.empty_cache()
    return out


def copy_calibration():
    import torch
    nbytes = 1 << 30
    x = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").uniform_()
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "launches": 3}), flush=True)


def _timed_dispatches(n, steps, warmup):
    """Positions of the timed dispatches among a kernel's n dispatches in one run of this script.

    The fused region runs `warmup` steps, `steps` timed steps and `steps` steps with per-step events;
    the call-by-call region runs `warmup` steps, then `steps` timed steps.  A kernel launched c times
    per step in both regions has n = (2 * warmup + 3 * steps) * c dispatches; one that only the fused
    entry launches (the paged top-k that reads the logits kernel's fragment maxima) has
    (warmup + 2 * steps) * c, and one only the call-by-call region launches (warmup + steps) * c.
    The warm-up dispatches are dropped.  Returns None when n fits none of these (a kernel outside the
    timed regions)."""
    if n == 0:
        return None
    both, fused, split = 2 * warmup + 3 * steps, warmup + 2 * steps, warmup + steps
    if n % both == 0:
        c = n // both
        return (list(range(warmup * c, (warmup + 2 * steps) * c)) +
                list(range((2 * warmup + 2 * steps) * c, (2 * warmup + 3 * steps) * c)))
    if n % fused == 0:
        c = n // fused
        return list(range(warmup * c, (warmup + 2 * steps) * c))
    if n % split == 0:
        c = n // split
        return list(range(warmup * c, (warmup + steps) * c))
    return None


def trace_summary(path, steps, warmup):
    """Markdown summary of a rocprofv3 per-dispatch CSV restricted to the timed dispatches."""
    import csv
    from collections import OrderedDict
    with open(path, newline="") as f:
        rows = list(csv.DictReader(f))
    out = []
    if rows and "Counter_Name" in rows[0]:
        # counter_collection.csv: one row per (dispatch, counter)
        by = OrderedDict()
        for r in rows:
            by.setdefault(r["Kernel_Name"], OrderedDict()).setdefault(int(r["Dispatch_Id"]), {})[
                r["Counter_Name"]] = float(r["Counter_Value"])
        out.append("| kernel | dispatches (timed / all) | counter | mean per timed dispatch |")
        out.append("|---|---|---|---|")
        for name, disp in by.items():
            ids = sorted(disp)
            sel = _timed_dispatches(len(ids), steps, warmup)
            if sel is None:
                continue
            counters = sorted({c for d in disp.values() for c in d})
            for cn in counters:
                vals = [disp[ids[i]].get(cn, 0.0) for i in sel]
                out.append(f"| `{name}` | {len(sel)} / {len(ids)} | {cn} | {sum(vals) / len(vals):.6g} |")
        return "\n".join(out)
    by = OrderedDict()
    for r in rows:
        by.setdefault(r["Kernel_Name"], []).append(
            (int(r["Dispatch_Id"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    out.append("| kernel | timed dispatches | mean us | median us | min us | max us | all dispatches | mean us (all) |")
    out.append("|---|---|---|---|---|---|---|---|")
    for name, ds in by.items():
        ds.sort()
        durs = [d for _, d in ds]
        sel = _timed_dispatches(len(durs), steps, warmup)
        allm = sum(durs) / len(durs) / 1e3
        if sel is None:
            out.append(f"| `{name}` | outside the timed regions | | | | | {len(durs)} | {allm:.2f} |")
            continue
        t = sorted(durs[i] for i in sel)
        out.append(f"| `{name}` | {len(t)} | {sum(t) / len(t) / 1e3:.2f} | {_median(t) / 1e3:.2f} | "
                   f"{t[0] / 1e3:.2f} | {t[-1] / 1e3:.2f} | {len(durs)} | {allm:.2f} |")
    return "\n".join(out)


def main():
    a = _args()
    if a.trace_summary:
        print(trace_summary(a.trace_summary, a.steps, a.warmup))
        return
    _roctx()   # load the marker library before the GPU runtime starts
    if a.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {a.gpus}); "
              "the indexer path is rank-local: every rank runs this same single-GPU path on its own rows", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    import fp8_mqa_logits_amd as F
    F.load_library()
    if a.copy_calibration:
        copy_calibration()
        return
    if a.core_probe:
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        t = core_probe(cus, (RAGGED_WGS_PER_CU,), iters=4096, reps=a.core_probe)[RAGGED_WGS_PER_CU]
        print(json.dumps({"probe": "logits_core", "wgs_per_cu": RAGGED_WGS_PER_CU, "launches": a.core_probe,
                          "tflops": round(t, 1)}), flush=True)
        return
    if a.all_workloads:
        rows = []
        for name in ("tiny", "prefill_64k", "prefill_35k", "paged_decode", "long_prefix_210k"):
            r = run_workload(name, a.steps, a.warmup, overlap=True)
            inp, step = r.pop("inp"), r.pop("step")
            r.pop("fused_events")
            r["logits_tflops"] = r["flops"] / (r["logits_ms"] * 1e-3) / 1e12
            r["logits_mfma_frac"] = r["logits_tflops"] * 1e12 / MFMA_FP8_PEAK
            r["topk_gbps"] = step.topk_bytes() / (r["topk_ms"] * 1e-3) / 1e9
            r["topk_hbm_frac"] = r["topk_gbps"] * 1e9 / HBM_PEAK
            if hasattr(step, "kv_bytes"):
                r["logits_hbm_gbps"] = step.kv_bytes() / (r["logits_ms"] * 1e-3) / 1e9
                r["logits_hbm_frac"] = r["logits_hbm_gbps"] * 1e9 / HBM_PEAK
            if not a.no_cpu_baseline:
                r["cpu_baseline"] = _cpu_baseline(inp, a.cpu_seconds)
            rows.append(r)
            print(json.dumps(r), file=sys.stderr, flush=True)
            del inp, step
            torch.cuda.empty_cache()
        for q in (quant_workloads(a.steps, a.warmup) + prep_workloads(a.steps, a.warmup) +
                  sparse_mla_workloads(a.steps, a.warmup, cpu_tokens=2)):
            rows.append(q)
            print(json.dumps(q), file=sys.stderr, flush=True)
        with open(a.all_workloads, "w") as f:
            json.dump(rows, f, indent=1)
        return
    if a.overlap:
        from workloads.generate import config_inputs
        for name, cap in (("prefill_64k", 2_000_000_000), ("long_prefix_210k", None)):
            inp = config_inputs(name)
            if cap is not None:
                inp.cap_bytes = cap
                inp.name = f"{inp.name}_cap2GB"
            step = RaggedStep(inp)
            serial, _ = _time_fused(step, a.steps, a.warmup)
            over, _ = _time_fused(step, a.steps, a.warmup, overlap=True)
            print(json.dumps({"workload": inp.name, "chunks": -(-inp.m // step.rpc), "rows_per_chunk": step.rpc,
                              "fused_serial_ms": round(serial, 4), "fused_overlap_ms": round(over, 4),
                              "overlap_gain": round(serial / over - 1, 4)}), flush=True)
            del step, inp
            torch.cuda.empty_cache()
        return
    if a.cap_sweep:
        for r in cap_sweep(a.steps, a.warmup):
            print(json.dumps(r), flush=True)
        return
    if a.prep:
        for q in prep_workloads(a.steps, a.warmup):
            print(json.dumps(q), flush=True)
        return
    if a.quant:
        for q in quant_workloads(a.steps, a.warmup):
            print(json.dumps(q), flush=True)
        return
    if a.sparse_mla:
        for q in sparse_mla_workloads(a.steps, a.warmup, cpu_tokens=0 if a.no_cpu_baseline else 2):
            print(json.dumps(q), flush=True)
        return

    r = run_workload(a.workload, a.steps, a.warmup, cold=a.cold)
    inp, step = r["inp"], r["step"]
    flops = r["flops"]
    paged = hasattr(inp, "kv_pool")
    if paged:
        # HBM bound: kv + scales of every referenced key, q, weights, block-table entries and the
        # logits written, over the logits launch
        achieved = step.kv_bytes() / (r["logits_ms_per_launch"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                "frac": round(achieved * 1e9 / HBM_PEAK, 4), "traffic": _traffic(inp.name, "logits_paged")}
        metric_value, unit = step.kv_bytes() / (r["ms_per_step"] * 1e-3) / 1e9, "GB/s"
    else:
        # MFMA bound: 2 * H * D flops per valid (row, key) pair; the mean logits launch of a step
        # (chunks of unequal size) against the mean launch duration
        achieved = step.logits_flops_per_launch() / (r["logits_ms_per_launch"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_FP8_PEAK / 1e12,
                "unit": "TFLOP/s", "frac": round(achieved * 1e12 / MFMA_FP8_PEAK, 4),
                "traffic": _traffic(inp.name, "logits_ragged")}
        metric_value, unit = flops / (r["ms_per_step"] * 1e-3) / 1e12, "TFLOP/s"
    out = {
        "metric": "indexer logits+top-k ms/layer & TFLOP/s (prefill), GB/s (decode), % roofline",
        "value": round(metric_value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": inp.name, "entry": r["entry"], "caches": "cold" if a.cold else "warm"},
        "roofline": roof,
        "logits_ms": round(r["logits_ms"], 4),
        "topk_ms": round(r["topk_ms"], 4),
        "split_ms_per_step": round(r["split_ms_per_step"], 4),
        "launches_per_step": r["launches_per_step"],
        "logits_ms_per_launch": round(r["logits_ms_per_launch"], 4),
        "topk_gbps": round(step.topk_bytes() / (r["topk_ms"] * 1e-3) / 1e9, 1),
        "kernel_source_hash": kernel_source_hash(),
    }
    if paged:
        out["config"].update({"requests": inp.B, "rows_per_request": inp.next_n, "page_size": inp.page_size,
                              "k": inp.k, "width": step.width, "valid_pairs": inp.valid_pairs})
        out["logits_hbm_bytes_per_launch"] = step.kv_bytes()
    else:
        out["config"].update({"m": inp.m, "n": inp.n, "H": H, "D": D, "k": inp.k,
                              "logits_cap_bytes": inp.cap_bytes, "rows_per_chunk": step.rpc,
                              "chunks": len(step.chunk_flops), "valid_pairs": inp.valid_pairs})
        out["logits_flops_per_launch"] = step.logits_flops_per_launch()
    out.update(_distribution(step, r["fused_events"]))
    if not a.no_peaks:
        pk = measured_peaks()
        if paged:
            pk["logits_frac_of_copy"] = round(roof["achieved"] / pk["copy_gbps"], 4)
        else:
            pk["logits_frac_of_mfma_probe"] = round(roof["achieved"] / pk["mfma_fp8_tflops"], 4)
            pk["logits_frac_of_core_probe"] = round(
                roof["achieved"] / pk["logits_core_tflops"][str(RAGGED_WGS_PER_CU)], 4)
        out["measured_peaks"] = pk
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = _cpu_baseline(inp, a.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

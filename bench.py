"""Benchmark of the paged-attention read path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only C2,C3,...]
                    [--no-cpu-baseline] [--no-flush] [--no-warm] [--no-clocks]

Prints ONE JSON line.  The headline ``value`` is the decode workload "GQA
decode, bf16, B=64, H_q=32, H_kv=8, D=128, page_size=16, contexts U[128,4096]"
(seed 2): algorithmic K/V bytes of one step (every visible K and V element
once) divided by the mean HIP-event time of the step (pa_decode +
pa_split_reduce), with the inputs resident in HBM and the 256 MB last-level
cache flushed before every step.  ``roofline`` is for the dominant kernel
(the decode kernel alone, timed by its own event pair).  Secondary sections
report the same decode with fp8 (E4M3) pages, the chunked prefill (bf16
and fp8 pages),
long-context decode, mixed batch and a long-prompt prefill sweep, each with
its own roofline (``traffic`` is the HBM bytes per launch from the committed
rocprofv3 counter summary of that section while its kernel source is
unchanged), small-batch decode latencies and the K/V write (bf16 and into an
fp8 pool).  ``cpu_baseline`` times the fp32 CPU oracle on the host on the
full decode workload and once on the chunked prefill.  ``clocks`` holds the
per-XCD gfx clocks and the memory clock that amd-smi reads while the decode
and the long-prompt prefill run back to back (outside the timed regions).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
FLUSH_BYTES = 1 << 30          # > 256 MB last-level cache


# --------------------------------------------------------------------- work
def decode_kv_bytes(x, unique: bool = False) -> int:
    """K+V bytes a decode call must read: every visible key and value of
    every kv head once (unique=True counts shared physical pages once)."""
    per_tok = x.kv_token_bytes()
    if not unique:
        return int(x.context_lens.astype(np.int64).sum()) * per_tok
    seen = {}
    for b in range(x.B):
        n = int(x.context_lens[b])
        for lp in range((n + x.page_size - 1) // x.page_size):
            p = int(x.block_table[b, lp])
            seen[p] = max(seen.get(p, 0), min(x.page_size, n - lp * x.page_size))
    return int(sum(seen.values())) * per_tok


def prefill_flops(x) -> float:
    """4 * D * H_q * (number of visible (query, key) pairs): QK^T and PV,
    two flops per multiply-add, causal-visible pairs only."""
    pairs = 0
    rows = x.rows_valid()
    for b in range(x.B):
        ctx, lb = int(x.context_lens[b]), int(rows[b])
        if x.causal:
            pairs += sum(ctx - lb + i + 1 for i in range(lb))
        else:
            pairs += lb * ctx
    return 4.0 * x.D * x.H_q * pairs


# ------------------------------------------------------------------- timing
class Runner:
    def __init__(self, torch, api, flush: bool):
        self.torch = torch
        self.api = api
        self.flush_buf = None
        if flush:
            self.flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")

    def flush(self):
        """Evict the last-level cache by reading 1 GiB: the cache then holds
        clean lines of another buffer, so the timed call pays its own cold
        misses and no write-back of someone else's dirty lines."""
        if self.flush_buf is not None:
            self.flush_sink = self.flush_buf.sum()

    def to_device(self, x, pages=None):
        from tests._gpu import DeviceInputs
        return DeviceInputs(x, pages=pages)

    def time_decode(self, d, steps, warmup, partition_tokens=0, num_cus=0, fused=True):
        """Times `steps` decode steps (pa_decode + pa_split_reduce, one event
        pair around both), then `steps` launches of pa_decode alone (its own
        event pair) for the kernel figure; the last-level cache is flushed
        before each."""
        torch, api = self.torch, self.api
        x = d.x
        out = torch.empty_like(d.q)
        from tests._gpu import kv_scales
        args = api.make_args(d.q, d.kp, d.vp, d.bt, d.cl, out, scale=x.scale, mask=d.mask,
                             query_lens=d.ql, **kv_scales(x))
        plan = api.pa_decode_plan(args, partition_tokens=partition_tokens, num_cus=num_cus)
        S, P = plan.num_splits, plan.partition_tokens
        ws = api.Workspace.for_plan(plan, d.q, fused=fused)

        def step():
            api.pa_decode(args, ws)
            if S > 1:
                api.pa_split_reduce(args, ws)

        for _ in range(warmup):
            self.flush()
            step()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            self.flush()
            ev[k][0].record()
            step()
            ev[k][1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        step_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
        kev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for k in range(steps):
            self.flush()
            kev[k][0].record()
            api.pa_decode(args, ws)
            kev[k][1].record()
        if S > 1:
            api.pa_split_reduce(args, ws)  # leave `out` complete
        torch.cuda.synchronize()
        dec = np.array([e[0].elapsed_time(e[1]) for e in kev])
        sched = "balanced" if plan.schedule == api.SCHEDULE_BALANCED else "partitions"
        return {"S": S, "P": P, "schedule": sched, "fused": bool(ws.counters is not None),
                "decode_ms": dec, "step_ms": step_ms, "wall_s": wall, "out": out}

    def time_append(self, a, steps, warmup):
        """Times pa_append of the write workload `a` (K/V rows and slots on the
        device); the pool is the same every call (rows land in the same
        slots), the last-level cache is flushed before each call."""
        torch, api = self.torch, self.api
        from tests._gpu import dev
        p = a.paged
        kp, vp = dev(p.key_pages), dev(p.value_pages)
        k, v, sm = dev(a.key), dev(a.value), dev(a.slot_mapping)
        sc = dict(k_scale=p.k_scale, v_scale=p.v_scale) if p.kv_dtype else {}
        for _ in range(warmup):
            self.flush()
            api.pa_append(k, v, sm, kp, vp, **sc)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        torch.cuda.synchronize()
        for e in ev:
            self.flush()
            e[0].record()
            api.pa_append(k, v, sm, kp, vp, **sc)
            e[1].record()
        torch.cuda.synchronize()
        return {"ms": np.array([e[0].elapsed_time(e[1]) for e in ev])}

    def time_ragged_ab(self, m, steps, warmup):
        """Times ONE pa_attention call over the packed rows of the mixed
        workload `m` (decode kernel for its one-row requests, prefill kernel
        for the rest, on one stream) and the same requests as two calls back
        to back (pa_decode, then pa_prefill, on one stream), alternating call
        by call so that both see the same clocks; one event pair around each,
        workspaces set up outside the timed regions, the last-level cache
        flushed before each.  Returns (one-call ms, two-call ms, route)."""
        torch, api = self.torch, self.api
        import workloads as W
        from tests._gpu import DeviceInputs, dev
        r = W.pack_ragged(m)
        dd = DeviceInputs(m.decode)
        dp = DeviceInputs(m.prefill, pages=(dd.kp, dd.vp))
        outd, outp = torch.empty_like(dd.q), torch.empty_like(dp.q)
        ad = api.make_args(dd.q, dd.kp, dd.vp, dd.bt, dd.cl, outd, scale=m.decode.scale,
                           mask=dd.mask)
        wd = api.Workspace.for_plan(api.pa_decode_plan(ad), dd.q, fused=True)
        apf = api.make_args(dp.q, dp.kp, dp.vp, dp.bt, dp.cl, outp, scale=m.prefill.scale,
                            mask=dp.mask, query_lens=dp.ql)
        wp = api.PrefillWorkspace.for_args(apf, dp.q.device)
        qd = dev(r.query)
        out = torch.empty_like(qd)
        args = api.make_args(qd, dd.kp, dd.vp, dev(r.block_table), dev(r.context_lens), out,
                             scale=r.scale, mask="causal" if r.causal else "none",
                             query_start_loc=dev(r.query_start_loc),
                             max_query_len=r.max_query_len)
        ap = api.pa_attention_plan(args)
        ws = api.attention_workspace(ap, args, qd)

        def two():
            api.pa_decode(ad, wd)
            api.pa_prefill(apf, wp)

        calls = (lambda: api.pa_attention(args, ws), two)
        for _ in range(warmup):
            for fn in calls:
                self.flush()
                fn()
        ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(2)]
              for _ in range(steps)]
        torch.cuda.synchronize()
        for k in range(steps):
            for i, fn in enumerate(calls):
                self.flush()
                ev[k][i][0].record()
                fn()
                ev[k][i][1].record()
        torch.cuda.synchronize()
        ms = np.array([[e[i][0].elapsed_time(e[i][1]) for i in range(2)] for e in ev])
        return ms[:, 0], ms[:, 1], ap.route

    def time_shared_ab(self, d, groups, steps, warmup):
        """Times pa_decode_shared over device inputs `d` with the request
        groups `groups` (the prefix launch and the decode launch, one event
        pair around both) and pa_decode over the same inputs, alternating
        call by call so that both see the same clocks; workspaces and groups
        set up outside the timed regions, the last-level cache flushed
        before each call.  Returns (shared ms, unshared ms)."""
        torch, api = self.torch, self.api
        from tests._gpu import dev
        x = d.x
        out = torch.empty_like(d.q)
        args = api.make_args(d.q, d.kp, d.vp, d.bt, d.cl, out, scale=x.scale, mask=d.mask,
                             query_lens=d.ql)
        gs, pl = dev(groups.group_start), dev(groups.prefix_lens)
        g = api.PrefixGroups(gs, pl, groups.max_group_size)
        plan = api.pa_decode_shared_plan(args, g)
        ws = api.SharedWorkspace(plan, args, d.q.device)
        dplan = api.pa_decode_plan(args)
        dws = api.Workspace.for_plan(dplan, d.q, fused=True)
        calls = (lambda: api.pa_decode_shared(args, g, ws), lambda: api.pa_decode(args, dws))
        for _ in range(warmup):
            for fn in calls:
                self.flush()
                fn()
        ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(2)]
              for _ in range(steps)]
        torch.cuda.synchronize()
        for k in range(steps):
            for i, fn in enumerate(calls):
                self.flush()
                ev[k][i][0].record()
                fn()
                ev[k][i][1].record()
        torch.cuda.synchronize()
        ms = np.array([[e[i][0].elapsed_time(e[i][1]) for i in range(2)] for e in ev])
        return ms[:, 0], ms[:, 1]

    def time_prefill(self, d, steps, warmup, flush=False, split=True):
        """Times pa_prefill; `split` passes the key-split workspace of the
        library's plan (allocated outside the timed region)."""
        torch, api = self.torch, self.api
        x = d.x
        out = torch.empty_like(d.q)
        fp8 = getattr(x, "kv_dtype", None) == "fp8_e4m3"
        args = api.make_args(d.q, d.kp, d.vp, d.bt, d.cl, out, scale=x.scale, mask=d.mask,
                             query_lens=d.ql,
                             **(dict(k_scale=x.k_scale, v_scale=x.v_scale) if fp8 else {}))
        ws = api.PrefillWorkspace.for_args(args, d.q.device) if split else None
        for _ in range(warmup):
            if flush:
                self.flush()
            api.pa_prefill(args, ws)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        torch.cuda.synchronize()
        for k in range(steps):
            if flush:
                self.flush()
            ev[k][0].record()
            api.pa_prefill(args, ws)
            ev[k][1].record()
        torch.cuda.synchronize()
        return {"ms": np.array([e[0].elapsed_time(e[1]) for e in ev]), "out": out}


def _stats(ms):
    return {"mean_ms": float(np.mean(ms)), "median_ms": float(np.median(ms)),
            "p10_ms": float(np.percentile(ms, 10)), "p90_ms": float(np.percentile(ms, 90))}


def _source_sha(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "paged_kv_cache_96_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _counters(name, sha):
    """HBM traffic per launch from committed rocprofv3 counter summaries, or
    None when the kernel source changed since they were taken."""
    path = os.path.join(ROOT, "profiles", f"{name}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("kernel_source_sha") != sha:
        return None
    return c.get("hbm_bytes_per_launch")


# ------------------------------------------------------------------- clocks
def _amd_smi_clocks(exe, busy, timeout_s):
    """One `amd-smi metric -c --json` run as a child process while `busy()`
    keeps the GPU working; (gfx MHz per XCD, memory MHz, seconds) or None."""
    import subprocess
    try:
        proc = subprocess.Popen([exe, "metric", "-c", "--json"], stdout=subprocess.PIPE,
                                stderr=subprocess.DEVNULL)
    except OSError:
        return None
    t0 = time.perf_counter()
    while proc.poll() is None and time.perf_counter() - t0 < timeout_s:
        busy()
    try:
        raw, _ = proc.communicate(timeout=5.0)
    except subprocess.TimeoutExpired:
        proc.kill()
        proc.communicate()
        return None
    try:
        d = json.loads(raw)
        gpus = d["gpu_data"] if isinstance(d, dict) else d
        if len(gpus) != 1:
            return None
        c = gpus[0]["clock"]
        gfx = sorted((int(k.split("_")[1]), v["clk"]["value"]) for k, v in c.items()
                     if k.startswith("gfx_") and isinstance(v, dict))
        mem = c.get("mem_0", {}).get("clk", {}).get("value")
    except (ValueError, KeyError, TypeError, AttributeError, IndexError):
        return None
    return [v for _, v in gfx], mem, round(time.perf_counter() - t0, 3)


def sample_clocks(busy, samples=3, timeout_s=30.0, gap_s=1.0):
    """Clocks of the GPU while it runs a workload: keeps calling `busy()`
    (which enqueues work and synchronises) throughout, and reads the clocks
    with amd-smi `samples` times, each after `gap_s` more seconds of work
    (the tool reports a snapshot that the amdgpu kernel driver refreshes; readings taken
    back to back repeat it).  Each reading is the gfx clock of every XCD and
    the memory clock in MHz.  None where amd-smi is missing or fails, or
    under a profiler (the child would be profiled too)."""
    import shutil
    if any(k.startswith("ROCPROF") for k in os.environ):
        return None
    exe = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    if not os.path.exists(exe):
        return None
    out = []
    for _ in range(samples):
        t_gap = time.perf_counter()
        while time.perf_counter() - t_gap < gap_s:
            busy()
        r = _amd_smi_clocks(exe, busy, timeout_s)
        if r is None:
            return None
        out.append({"gfx_mhz_per_xcd": r[0], "mem_mhz": r[1], "sample_s": r[2]})
    return out


# --------------------------------------------------------------- cpu oracle
def host_cpu_model() -> str:
    """The host CPU's model name (first "model name" of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x, kv_bytes, x3=None, flops3=None, min_seconds=10.0, max_runs=2000):
    """The CPU oracle (fp32 two-pass build, OpenMP over (request, kv head))
    timed on the host: the full decode workload repeatedly for ~min_seconds
    on all host cores, a few runs on one core, and one run of the chunked
    prefill workload `x3` on all cores."""
    import oracle
    oracle.load(oracle.lib_for("f32"))
    times, threads = [], 0
    t_all = time.perf_counter()
    while len(times) < max_runs and (time.perf_counter() - t_all) < min_seconds:
        t0 = time.perf_counter()
        _, threads = oracle.attention_of(x, return_threads=True)
        times.append(time.perf_counter() - t0)
    t = float(np.mean(times))
    # the same oracle on one host core, a few runs
    t1s = []
    t_one = time.perf_counter()
    while len(t1s) < 3 and (time.perf_counter() - t_one) < min_seconds / 2:
        t0 = time.perf_counter()
        oracle.attention_of(x, nthreads=1)
        t1s.append(time.perf_counter() - t0)
    t1 = float(np.mean(t1s))
    res = {"value": kv_bytes / t / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
           "host_cpu": host_cpu_model(),
           "sample": f"the full decode workload ({x.B} requests, {int(x.context_lens.sum())} "
                     f"keys), fp32 C oracle, mean of {len(times)} run(s) of {t:.2f} s",
           "single_core": {"value": kv_bytes / t1 / 1e9, "unit": "GB/s", "cores": 1,
                           "sample": f"mean of {len(t1s)} run(s) of {t1:.2f} s"}}
    if x3 is not None:
        t0 = time.perf_counter()
        _, th3 = oracle.attention_of(x3, return_threads=True)
        t3 = time.perf_counter() - t0
        res["prefill_C3"] = {"value": flops3 / t3 / 1e12, "unit": "TFLOP/s", "cores": int(th3),
                             "sample": f"the chunked prefill workload, one run of {t3:.2f} s"}
    return res


def decode_busy(run, d, n=20):
    """Back-to-back decode steps (the timed configuration, cache flushed
    before each) for the clock sample."""
    torch, api = run.torch, run.api
    x = d.x
    out = torch.empty_like(d.q)
    args = api.make_args(d.q, d.kp, d.vp, d.bt, d.cl, out, scale=x.scale, mask=d.mask,
                         query_lens=d.ql)
    plan = api.pa_decode_plan(args)
    ws = api.Workspace.for_plan(plan, d.q, fused=True)

    def busy():
        for _ in range(n):
            run.flush()
            api.pa_decode(args, ws)
            if plan.num_splits > 1:
                api.pa_split_reduce(args, ws)
        torch.cuda.synchronize()
    return busy


def prefill_busy(run, d, n=2):
    """Back-to-back prefill calls (with the key-split workspace) for the
    clock sample."""
    torch, api = run.torch, run.api
    x = d.x
    out = torch.empty_like(d.q)
    args = api.make_args(d.q, d.kp, d.vp, d.bt, d.cl, out, scale=x.scale, mask=d.mask,
                         query_lens=d.ql)
    ws = api.PrefillWorkspace.for_args(args, d.q.device)

    def busy():
        for _ in range(n):
            api.pa_prefill(args, ws)
        torch.cuda.synchronize()
    return busy


# --------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", default="C2,C2fp8,C3,C3fp8,C4,C5,shared,long,small,append",
                    help="sections to run (C2 is the headline; leaving it out leaves `value` "
                         "null, for profiling runs): C2, C2fp8, C3, C3fp8, C4, C5, shared (the "
                         "shared-prefix decode alone), long (= long4096, "
                         "long16384), small, threshold, append (all write shapes), "
                         "append_long, append_fp8")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the unflushed C2 decode steps (profiling runs)")
    ap.add_argument("--no-clocks", action="store_true",
                    help="skip the amd-smi clock samples (profiling runs)")
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (3 times): the known "
                         "byte count that scales the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        n = (1 << 30) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": 1 << 30, "bytes_written": 1 << 30}))
        return

    from paged_kv_cache_96_amd import api
    import workloads as W

    only = set(args.only.split(","))
    if "long" in only:
        only |= {"long4096", "long16384"}
    run = Runner(torch, api, flush=not args.no_flush)
    log = lambda *a: print(*a, file=sys.stderr, flush=True)  # noqa: E731
    sha_dec = _source_sha("pa_decode.hip", "pa_common.hpp", "pa_merge.hpp", "pa_internal.h")
    sha_pre = _source_sha("pa_prefill.hip", "pa_common.hpp", "pa_merge.hpp", "pa_internal.h")
    sha_app = _source_sha("pa_append.hip", "pa_write.h")
    sha_shared = _source_sha("pa_decode.hip", "pa_prefill.hip", "pa_common.hpp", "pa_merge.hpp",
                             "pa_internal.h")

    def hbm_roofline(kernel, nbytes, ms, counters, sha):
        gbs = nbytes / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                "traffic": _counters(counters, sha), "algorithmic_bytes_per_launch": nbytes,
                "mean_launch_us": round(ms * 1e3, 2), "source_sha": sha}

    def mfma_roofline(flops, ms, counters):
        tf = flops / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "kernel": "prefill_kernel", "achieved": round(tf, 2),
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                "traffic": _counters(counters, sha_pre), "algorithmic_flops_per_launch": flops,
                "mean_launch_us": round(ms * 1e3, 2), "source_sha": sha_pre}

    result = {
        "metric": "decode K/V HBM GB/s (% of peak) + prefill TFLOP/s (% MFMA peak), 1 MI355X",
        "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "GQA decode bf16 B64 Hq32 Hkv8 D128 L1 page16 ctx U[128,4096] seed2"},
        "roofline": None,
    }
    clocks = {"source": "amd-smi metric -c, three readings one second apart while the "
                        "workload runs back to back (outside the timed regions); amdgpu "
                        "driver snapshots, context only"}

    # ---- headline: C2 GQA decode
    x2 = W.make_c2()
    kv2 = decode_kv_bytes(x2)
    if "C2" in only:
        d2 = run.to_device(x2)
        log(f"[bench] decode C2: {kv2 / 1e6:.1f} MB of K/V per step")
        r2 = run.time_decode(d2, args.steps, args.warmup, args.partition_tokens)
        step_ms = float(np.mean(r2["step_ms"]))
        dec_ms = float(np.mean(r2["decode_ms"]))
        value = kv2 / (step_ms * 1e-3) / 1e9
        log(f"[bench] decode C2: step {step_ms * 1e3:.1f} us (decode {dec_ms * 1e3:.1f} us), "
            f"{value:.0f} GB/s, {r2['schedule']} S={r2['S']} P={r2['P']}")
        result.update({
            "value": round(value, 2), "ms_per_step": round(step_ms, 5),
            "config": {"workload": "GQA decode bf16 B64 Hq32 Hkv8 D128 L1 page16 ctx U[128,4096] seed2",
                       "B": x2.B, "H_q": x2.H_q, "H_kv": x2.H_kv, "D": x2.D, "page_size": 16,
                       "schedule": r2["schedule"], "num_splits": r2["S"],
                       "partition_tokens": r2["P"], "llc_flushed": not args.no_flush,
                       "kv_bytes_per_step": kv2},
            "roofline": hbm_roofline("decode_kernel", kv2, dec_ms, "decode_c2", sha_dec),
            "step_stats": _stats(r2["step_ms"]),
            "warm": None,
            "merge": "fused into pa_decode" if r2["fused"] else "pa_split_reduce kernel",
            "wall_s_timed_region": round(r2["wall_s"], 4),
        })
        del r2
        if not args.no_clocks:
            clocks["decode_C2"] = sample_clocks(decode_busy(run, d2))
            log(f"[bench] clocks under C2 decode: {clocks['decode_C2']}")
        if not args.no_flush and not args.no_warm:
            # the same steps without the cache flush between them (K/V partly in
            # the 256 MB last-level cache): context only, never `value`
            rw = Runner(torch, api, flush=False).time_decode(d2, args.steps, args.warmup,
                                                             args.partition_tokens)
            wm = float(np.mean(rw["step_ms"]))
            result["warm"] = {"ms_per_step": round(wm, 5),
                              "gbs": round(kv2 / (wm * 1e-3) / 1e9, 2),
                              "decode_ms": round(float(np.mean(rw["decode_ms"])), 5)}
            log(f"[bench] decode C2 warm (no flush): step {wm * 1e3:.1f} us")
            del rw
        del d2

    sections = {}
    if "C2fp8" in only:
        # the same decode with fp8 (E4M3) pages: half the K/V bytes per token
        x8 = W.make_c2_fp8()
        d8 = run.to_device(x8)
        kv8 = decode_kv_bytes(x8)
        r8 = run.time_decode(d8, args.steps, args.warmup)
        sm = float(np.mean(r8["step_ms"]))
        dm = float(np.mean(r8["decode_ms"]))
        log(f"[bench] decode C2 fp8: step {sm * 1e3:.1f} us (decode {dm * 1e3:.1f} us), "
            f"{kv8 / sm / 1e6:.0f} GB/s of fp8 K/V, S={r8['S']}")
        sections["decode_C2_fp8"] = {
            "workload": "GQA decode bf16 query, fp8 e4m3 K/V pages (k/v scale 0.5), B64 Hq32 Hkv8 "
                        "D128 page16 ctx U[128,4096] seed2",
            "kv_bytes": kv8, "gbs_step": round(kv8 / sm / 1e6, 2), "schedule": r8["schedule"],
            "num_splits": r8["S"], **_stats(r8["step_ms"]),
            "roofline": hbm_roofline("decode_kernel", kv8, dm, "decode_c2_fp8", sha_dec)}
        del d8, r8, x8
    x3 = fl3 = None
    if "C3" in only or not args.no_cpu_baseline:
        x3 = W.make_c3()
        fl3 = prefill_flops(x3)
    if "C3" in only:
        d3 = run.to_device(x3)
        r3 = run.time_prefill(d3, args.steps, args.warmup, flush=True)
        ms = float(np.mean(r3["ms"]))
        log(f"[bench] prefill C3: {ms * 1e3:.1f} us, {fl3 / ms / 1e9:.1f} TFLOP/s")
        sections["prefill_C3"] = {
            "workload": "chunked causal prefill bf16 B4 Hq28 Hkv4 D128 L512 prefix U[0,2048] page16 seed3",
            "flops": fl3, "tflops": round(fl3 / ms / 1e9, 2), **_stats(r3["ms"]),
            "roofline": mfma_roofline(fl3, ms, "prefill_c3")}
        del d3, r3
    if "C3fp8" in only:
        # the same chunked prefill over fp8 (E4M3) pages: the codes are
        # widened to bf16 on their way into LDS, so the flops are the same
        x3f = W.make_c3_fp8()
        fl3f = prefill_flops(x3f)
        d3f = run.to_device(x3f)
        r3f = run.time_prefill(d3f, args.steps, args.warmup, flush=True)
        ms = float(np.mean(r3f["ms"]))
        log(f"[bench] prefill C3 fp8: {ms * 1e3:.1f} us, {fl3f / ms / 1e9:.1f} TFLOP/s")
        sections["prefill_C3_fp8"] = {
            "workload": "chunked causal prefill bf16 query, fp8 e4m3 K/V pages (k/v scale 0.5) "
                        "B4 Hq28 Hkv4 D128 L512 prefix U[0,2048] page16 seed3",
            "flops": fl3f, "tflops": round(fl3f / ms / 1e9, 2), **_stats(r3f["ms"]),
            "roofline": mfma_roofline(fl3f, ms, "prefill_c3_fp8")}
        del d3f, r3f, x3f
    long = []
    for L in (4096, 16384):
        if f"long{L}" not in only:
            continue
        xl = W.make_random(100 + L, B=1, H_q=28, H_kv=4, L=L, D=128, page_size=16, ctx=[L],
                           dtype="bf16", causal=True, extra_free_pages=16)
        dl = run.to_device(xl)
        fl = prefill_flops(xl)
        rl = run.time_prefill(dl, max(5, args.steps // 6), 2, flush=True)
        ms = float(np.mean(rl["ms"]))
        tf = fl / (ms * 1e-3) / 1e12
        log(f"[bench] long prefill L={L}: {ms * 1e3:.1f} us, {tf:.1f} TFLOP/s")
        long.append({"workload": f"long-prompt causal prefill bf16 B1 Hq28 Hkv4 D128 L{L} prefix0 page16",
                     "flops": fl, "tflops": round(tf, 2), **_stats(rl["ms"]),
                     "roofline": mfma_roofline(fl, ms, f"prefill_long{L}")})
        if L == 16384 and not args.no_clocks:
            clocks["prefill_L16384"] = sample_clocks(prefill_busy(run, dl))
            log(f"[bench] clocks under L={L} prefill: {clocks['prefill_L16384']}")
        del dl, rl
    if long:
        sections["prefill_long_prompt"] = long
    if "C4" in only:
        x4 = W.make_c4()
        d4 = run.to_device(x4)
        kv4 = decode_kv_bytes(x4)
        r4 = run.time_decode(d4, max(10, args.steps // 3), args.warmup)
        sm = float(np.mean(r4["step_ms"]))
        dm = float(np.mean(r4["decode_ms"]))
        log(f"[bench] decode C4: {sm * 1e3:.1f} us, {kv4 / sm / 1e6:.0f} GB/s, S={r4['S']}")
        sections["decode_C4"] = {
            "workload": "long-context decode bf16 B8 Hq32 Hkv8 D128 page16 ctx U[32768,131072] seed4",
            "kv_bytes": kv4, "gbs_step": round(kv4 / sm / 1e6, 2), "schedule": r4["schedule"],
            "num_splits": r4["S"], "partition_tokens": r4["P"], **_stats(r4["step_ms"]),
            "roofline": hbm_roofline("decode_kernel", kv4, dm, "decode_c4", sha_dec)}
        del d4, r4, x4
    if "C5" in only:
        m = W.make_c5()
        dd = run.to_device(m.decode)
        dp = run.to_device(m.prefill, pages=(dd.kp, dd.vp))
        rd = run.time_decode(dd, max(10, args.steps // 3), args.warmup)
        rp = run.time_prefill(dp, max(10, args.steps // 3), args.warmup, flush=True)
        logical = decode_kv_bytes(m.decode)
        unique = decode_kv_bytes(m.decode, unique=True)
        sm = float(np.mean(rd["step_ms"]))
        dm = float(np.mean(rd["decode_ms"]))
        pm = float(np.mean(rp["ms"]))
        fl = prefill_flops(m.prefill)
        log(f"[bench] mixed C5: decode {sm * 1e3:.1f} us ({unique / sm / 1e6:.0f} GB/s unique), "
            f"prefill {pm * 1e3:.1f} us ({fl / pm / 1e9:.1f} TFLOP/s)")
        sections["mixed_C5"] = {
            "workload": "mixed ragged batch bf16 48 decode + 8 prefill Hq32 Hkv8 D128 page128, "
                        "25% share a 2048-token prefix, seed5",
            "decode_unique_kv_bytes": unique, "decode_logical_kv_bytes": logical,
            "decode_gbs_unique": round(unique / sm / 1e6, 2),
            "decode_gbs_logical": round(logical / sm / 1e6, 2), "decode_mean_ms": sm,
            "prefill_flops": fl, "prefill_tflops": round(fl / pm / 1e9, 2), "prefill_mean_ms": pm,
            "combined_ms": round(sm + pm, 5),
            "roofline_decode": hbm_roofline("decode_kernel", unique, dm, "decode_c5", sha_dec),
            "roofline_prefill": mfma_roofline(fl, pm, "prefill_c5")}
        sections["mixed_C5"]["roofline_decode"]["note"] = \
            "achieved on unique K/V bytes (shared prefix pages counted once)"
        del dd, dp, rd, rp
        # the same 56 requests as ONE call over packed query rows, against the
        # two calls back to back, interleaved call by call
        one, two, _ = run.time_ragged_ab(m, max(10, args.steps // 3), args.warmup)
        om, tm = float(np.mean(one)), float(np.mean(two))
        log(f"[bench] mixed C5 as one ragged call: {om * 1e3:.1f} us "
            f"(two calls back to back {tm * 1e3:.1f} us)")
        sections["mixed_C5"]["one_call"] = {
            "what": "one pa_attention call over packed rows (query_start_loc): the decode "
                    "kernel for the 48 one-row requests, the prefill kernel for the 8 others; "
                    "timed alternately with pa_decode + pa_prefill back to back on one "
                    "stream (each flushed once)",
            **_stats(one), "two_calls_back_to_back": _stats(two)}
    if "shared" in only:
        # shared-prefix decode (pa_decode_shared: one prefix launch reads each
        # group's shared pages once, then the decode launch walks the rest and
        # merges), against pa_decode on the same requests, interleaved call by
        # call: the decode part of C5 (11 of 48 requests share 16 pages of
        # 128 keys, moved to the front as one group) and a prefix-heavy batch
        # (64 requests sharing a 16384-key prefix, own suffixes U[128,4096])
        m5 = W.make_c5()
        xg, g5, _ = W.c5_decode_grouped(m5)
        xh, gh = W.make_shared(31, H_q=32, H_kv=8, L=1, D=128, page_size=16, group_sizes=[64],
                               prefix_pages=[1024], suffix=(128, 4096))
        n = max(10, args.steps // 3)
        sh = []
        for name, key, xx, gg in (
                ("C5 decode part: 48 requests bf16 Hq32 Hkv8 D128 page128, 11 share a "
                 "2048-key prefix (one group)", "decode_c5_shared", xg, g5),
                ("prefix-heavy decode: 64 requests bf16 Hq32 Hkv8 D128 page16 sharing a "
                 "16384-key prefix, own suffixes U[128,4096] seed31", "decode_prefix64_shared",
                 xh, gh)):
            dx = run.to_device(xx)
            unique, logical = decode_kv_bytes(xx, unique=True), decode_kv_bytes(xx)
            rs, ru = run.time_shared_ab(dx, gg, n, args.warmup)
            shm, um = float(np.mean(rs)), float(np.mean(ru))
            log(f"[bench] shared-prefix decode, {name.split(':')[0]}: shared {shm * 1e3:.1f} us "
                f"({unique / shm / 1e6:.0f} GB/s unique), unshared {um * 1e3:.1f} us "
                f"({unique / um / 1e6:.0f} GB/s unique)")
            sh.append({
                "workload": name, "groups": gg.num_groups,
                "sharers": int(gg.group_start[-1]), "unique_kv_bytes": unique,
                "logical_kv_bytes": logical, "gbs_unique": round(unique / shm / 1e6, 2),
                **_stats(rs),
                "unshared": {"gbs_unique": round(unique / um / 1e6, 2), **_stats(ru)},
                "speedup": round(um / shm, 3),
                "roofline": hbm_roofline("prefill_kernel (prefix launch) + decode_kernel, one "
                                         "call", unique, shm, key, sha_shared)})
            del dx
        sections["decode_shared_prefix"] = sh
    if "small" in only:
        # latency-bound decode: one to four requests over long contexts
        # (H 32/8, D 128, page 16), where the merge of many pieces per row
        # block is part of the step
        sb = []
        for B, ctx in ((1, 4096), (1, 16384), (1, 32768), (2, 4096), (4, 4096)):
            xs = W.make_random(800 + B, B=B, H_q=32, H_kv=8, L=1, D=128, page_size=16,
                               ctx=[ctx] * B, dtype="bf16", causal=True, extra_free_pages=16)
            ds = run.to_device(xs)
            kvs = decode_kv_bytes(xs)
            rs = run.time_decode(ds, max(10, args.steps // 3), args.warmup)
            sm = float(np.mean(rs["step_ms"]))
            log(f"[bench] small-batch decode B={B} ctx={ctx}: {sm * 1e3:.1f} us, "
                f"{kvs / sm / 1e6:.0f} GB/s, S={rs['S']}")
            sb.append({"workload": f"decode bf16 B{B} Hq32 Hkv8 D128 page16 ctx {ctx}",
                       "kv_bytes": kvs, "gbs_step": round(kvs / sm / 1e6, 2),
                       "schedule": rs["schedule"], "num_splits": rs["S"], **_stats(rs["step_ms"])})
            del ds, rs, xs
        sections["decode_small_batch"] = sb
    if "threshold" in only:
        # decode vs prefill around the router's threshold (not in the default
        # run): 64 requests, ctx U[128,4096], H 32/8, D 128, bf16
        th = []
        for L in (1, 2, 4, 8, 16, 32):
            xt = W.make_random(700 + L, B=64, H_q=32, H_kv=8, L=L, D=128, page_size=16,
                               ctx=(128, 4096), dtype="bf16", causal=True, extra_free_pages=64)
            dt = run.to_device(xt)
            row = {"L": L, "rows_per_kv_head": 4 * L}
            if L <= 8:
                row["decode_step_us"] = round(float(np.mean(
                    run.time_decode(dt, 20, 3)["step_ms"])) * 1e3, 2)
            row["prefill_us"] = round(float(np.mean(
                run.time_prefill(dt, 20, 3, flush=True)["ms"])) * 1e3, 2)
            log(f"[bench] threshold L={L}: {row}")
            th.append(row)
            del dt, xt
        sections["route_threshold"] = th
    shapes = []
    if "append" in only:
        shapes += [
            ("C2 decode step: 64 requests x 1 token, H_kv 8, D 128, page 16", None,
             dict(seed=2, B=64, H_kv=8, D=128, page_size=16, ctx_old=(127, 4095), n_new=[1] * 64)),
            ("C3 chunks: 4 requests x 512 tokens after prefixes U[0,2048], H_kv 4, D 128, page 16",
             None, dict(seed=3, B=4, H_kv=4, D=128, page_size=16, ctx_old=(0, 2048),
                        n_new=[512] * 4))]
    if "append" in only or "append_long" in only:
        shapes.append(("long chunk: 1 request x 16384 tokens, H_kv 8, D 128, page 16", "append_long",
                       dict(seed=9, B=1, H_kv=8, D=128, page_size=16, ctx_old=[0], n_new=[16384])))
    if "append" in only or "append_fp8" in only:
        shapes.append(("long chunk into an fp8 e4m3 pool (bf16 rows quantised, k/v scale 0.5): "
                       "1 request x 16384 tokens, H_kv 8, D 128, page 16", "append_fp8_long",
                       dict(seed=9, B=1, H_kv=8, D=128, page_size=16, ctx_old=[0], n_new=[16384],
                            kv_dtype="fp8_e4m3")))
    if shapes:
        # the K/V write that precedes attention (pa_append), timed on its own
        wr = []
        for name, counters, kw in shapes:
            a = W.make_append(dtype="bf16", **kw)
            ra = run.time_append(a, max(10, args.steps // 3), args.warmup)
            ms = float(np.mean(ra["ms"]))
            gbs = a.moved_bytes() / (ms * 1e-3) / 1e9
            log(f"[bench] append {name.split(':')[0]}: {ms * 1e3:.2f} us, {gbs:.0f} GB/s")
            wr.append({"workload": f"K/V write bf16, {name}", "tokens": a.num_tokens,
                       "moved_bytes": a.moved_bytes(), "gbs": round(gbs, 2), **_stats(ra["ms"]),
                       "roofline": hbm_roofline("append_kernel", a.moved_bytes(), ms,
                                                counters or "none", sha_app)})
            del a
        sections["append"] = wr
    result["sections"] = sections
    result["clocks"] = clocks

    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline on the decode and chunked-prefill workloads")
        result["cpu_baseline"] = cpu_baseline(x2, kv2, x3, fl3)
    print(json.dumps(result), flush=True)

if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the MI355X tree-verify attention (split-KV flash-decode over an MLA paged KV cache).

Prints ONE JSON line. A step is one verify call: the partial kernel plus the combine kernel over
one batch of seeded synthetic inputs already resident in HBM. The default workload is the ragged
B=4 batch with prefixes 4096/32768/120000/185000, q_len 16, H 64, scattered slots in a 2M-row
pool, under the balanced schedule with a budget of one workgroup per CU (units = CUs / 128-row
tiles = 32 on MI355X); --schedule per-request --nsplit 64 runs nsplit splits per request instead.

Timing: parity of the run's inputs is checked against the oracle first; then each of the `steps`
timed steps reads a 1 GiB scrub buffer (evicting L2 and the MALL, outside the events) and replays
the partial and the combine graphs between HIP events on one stream. `value` is the effective KV
bandwidth (sum of L_b * 1152 bytes per step / median step time), `ms_per_step` the median step. The
one-graph step is also replayed 50 times cold (scrub before each) and 50 times hot, reported as
median/p10/p90.

The roofline object covers the dominant kernel (the partial kernel): its algorithmic flops (or
bytes, when the workload sits below the MFMA ridge) per launch over its mean duration in the timed
steps. cpu_baseline runs the fp64 CPU oracle over the whole step once on all host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verify-attn µs/step + effective KV GB/s (% HBM/MFMA roofline) at 16k/65k/185k"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
RIDGE = MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)  # flop per byte


def algorithmic(inp):
    """Algorithmic bytes and flops of one step: every KV row once, 4 index bytes and q_len mask bytes
    per column, the queries once, out and lse once; flops = q_len * H * L * (576 + 512) * 2."""
    lengths = [p + inp.q_len for p in inp.prefixes]
    total_L = sum(lengths)
    rows = inp.B * inp.q_len * inp.H
    kv = total_L * 1152
    partial_bytes = kv + total_L * 4 + inp.q_len * total_L + rows * 576 * 2
    step_bytes = partial_bytes + rows * 512 * 2 + rows * 4
    flops = inp.q_len * inp.H * total_L * (576 + 512) * 2
    return dict(total_L=total_L, kv_bytes=kv, partial_bytes=partial_bytes, step_bytes=step_bytes, flops=flops)


class Workload:
    """Device buffers of one configuration and the library calls on them."""

    def __init__(self, wl, layout, nsplit, dev, balanced=False):
        import numpy as np
        import torch

        import speculative_decoding_mla_split_amd as pkg
        import workloads as W

        self.pkg, self.torch, self.np, self.W = pkg, torch, np, W
        self.wl, self.layout, self.nsplit, self.balanced = wl, layout, nsplit, balanced
        self.inp = W.make_inputs(wl, layout=layout)
        inp = self.inp
        self.dev = dev

        def t(a, bf16=False):
            a = np.ascontiguousarray(a)
            if bf16:
                return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
            return torch.from_numpy(a).to(dev)

        pool = torch.full((inp.N, 576), W.BF16_NAN, dtype=torch.int16, device=dev)
        pool[torch.from_numpy(inp.ref_slots.astype(np.int64)).to(dev)] = torch.from_numpy(
            inp.ref_rows.view(np.int16)).to(dev)
        self.pool = pool.view(torch.bfloat16)
        self.q_nope, self.q_rope = t(inp.q_nope, True), t(inp.q_rope, True)
        self.kv_indptr, self.kv_indices = t(inp.kv_indptr), t(inp.kv_indices)
        self.out_cache_loc, self.custom_mask, self.mask_indptr = t(inp.out_cache_loc), t(inp.custom_mask), t(
            inp.mask_indptr)
        size = pkg.balanced_workspace_size if balanced else pkg.workspace_size
        self.ws_bytes = size(inp.B, inp.q_len, inp.H, nsplit)
        assert self.ws_bytes > 0
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.out = torch.empty((inp.B, inp.q_len, inp.H, 512), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((inp.B, inp.q_len, inp.H), dtype=torch.float32, device=dev)
        self.alg = algorithmic(inp)

    def partial(self, stream):
        inp = self.inp
        call = self.pkg.balanced_partial_raw if self.balanced else self.pkg.partial_raw
        rc = call(self.q_nope.data_ptr(), self.q_rope.data_ptr(), self.pool.data_ptr(), inp.N,
                  self.kv_indptr.data_ptr(), self.kv_indices.data_ptr(), self.out_cache_loc.data_ptr(),
                  self.custom_mask.data_ptr(), self.mask_indptr.data_ptr(), inp.B, inp.q_len, inp.H,
                  inp.scale, self.nsplit, self.ws.data_ptr(), self.ws_bytes, stream.cuda_stream)
        assert rc == 0, self.pkg.status_string(rc)

    def combine(self, stream):
        inp = self.inp
        call = self.pkg.balanced_combine_raw if self.balanced else self.pkg.combine_raw
        rc = call(self.ws.data_ptr(), self.ws_bytes, self.pool.data_ptr(), inp.N, inp.B, inp.q_len, inp.H, self.nsplit,
                  self.out.data_ptr(), self.lse.data_ptr(), stream.cuda_stream)
        assert rc == 0, self.pkg.status_string(rc)

    def step(self, stream):
        self.partial(stream)
        self.combine(stream)

    def capture(self, stream):
        """Three graphs on `stream`: the whole step (partial + combine), the partial alone and the
        combine alone (the last two let events bracket each kernel inside a timed step)."""
        torch = self.torch
        with torch.cuda.stream(stream):
            self.step(stream)  # first launches outside capture (lazy module loading)
        torch.cuda.synchronize()
        self.g_step, self.g_part, self.g_comb = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        for g, fn in ((self.g_step, self.step), (self.g_part, self.partial), (self.g_comb, self.combine)):
            with torch.cuda.graph(g, stream=stream):
                fn(stream)
        torch.cuda.synchronize()

    def _replay(self, g, stream):
        with self.torch.cuda.stream(stream):
            g.replay()

    def kernel_split(self, stream, n, scrub):
        """n eager steps, each a scrub then the partial and combine kernels with HIP events on `stream`
        around each (an eager launch puts ~5 us less between its events than a graph launch does, so
        these give the kernels' own durations); per-step times (us): step, partial, combine."""
        torch = self.torch
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
        torch.cuda.synchronize()
        for k in range(n):
            scrub_l2(torch, scrub, stream)
            evs[k][0].record(stream)
            self.partial(stream)
            evs[k][1].record(stream)
            self.combine(stream)
            evs[k][2].record(stream)
        torch.cuda.synchronize()
        stepu = [evs[k][0].elapsed_time(evs[k][2]) * 1e3 for k in range(n)]
        part = [evs[k][0].elapsed_time(evs[k][1]) * 1e3 for k in range(n)]
        comb = [evs[k][1].elapsed_time(evs[k][2]) * 1e3 for k in range(n)]
        return stepu, part, comb

    def graph_replays(self, stream, n, scrub=None, warmup=10):
        """The step graph replayed n times between HIP events: cold (a scrub before each replay,
        outside the events) or hot (back to back) when scrub is None; per-replay times (us)."""
        torch = self.torch
        for _ in range(warmup):
            if scrub is not None:
                scrub_l2(torch, scrub, stream)
            self._replay(self.g_step, stream)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
        torch.cuda.synchronize()
        for k in range(n):
            if scrub is not None:
                scrub_l2(torch, scrub, stream)
            evs[k][0].record(stream)
            self._replay(self.g_step, stream)
            evs[k][1].record(stream)
        torch.cuda.synchronize()
        return [evs[k][0].elapsed_time(evs[k][1]) * 1e3 for k in range(n)]

    def parity(self, nrows, seed=0):
        """Sampled rows (corners + random) of the last step against the fp64 oracle."""
        import oracle
        np, W, torch = self.np, self.W, self.torch
        torch.cuda.synchronize()
        inp = self.inp
        rng = np.random.default_rng(seed)
        rows = {(b, i, h) for b in range(inp.B) for i in (0, inp.q_len - 1) for h in (0, inp.H - 1)}
        while len(rows) < nrows:
            rows.add((int(rng.integers(inp.B)), int(rng.integers(inp.q_len)), int(rng.integers(inp.H))))
        rows = np.array(sorted(rows), np.int32)
        pool, ki, oc = W.compact_inputs(inp)
        ref_out, ref_lse = oracle.attn_rows(*oracle.inputs_args(inp, pool, ki, oc), rows=rows)
        got = self.out.float().cpu().numpy().astype(np.float64)[rows[:, 0], rows[:, 1], rows[:, 2]]
        got_lse = self.lse.cpu().numpy().astype(np.float64)[rows[:, 0], rows[:, 1], rows[:, 2]]
        err = float(np.abs(got - ref_out).max())
        rel = float(np.linalg.norm(got - ref_out) / np.linalg.norm(ref_out))
        lerr = float(np.abs(got_lse - ref_lse).max())
        ok = err <= 1e-2 and rel <= 5e-3 and lerr <= 1e-3
        return dict(rows=int(len(rows)), max_abs=err, rel_l2=rel, lse_abs=lerr, ok=bool(ok))


def scrub_l2(torch, scrub, stream):
    """Evict L2 and the MALL with a 1 GiB read on the bench stream itself. A read, not a write: a fill
    leaves dirty lines whose write-back would land inside the next timed step, and a fill on another
    stream would overlap it."""
    with torch.cuda.stream(stream):
        scrub.view(torch.int64).sum()


def settle(wk, stream, scrub, replays=30, seconds=0.04):
    """Untimed step replays (each after a scrub) until at least `replays` of them and `seconds` have
    passed. Power management holds the GPU clock low for the first few dozen launches of this
    MFMA-heavy step after an idle period: rocprofv3 counters of the partial kernel show the same
    GRBM_GUI_ACTIVE cycles per dispatch throughout, at ~1.85 GHz effective for the first launches
    and ~2.05 GHz from about the 30th on. Other busy work beforehand does not help: memory-bound work
    does not raise the clock, and a burst of bf16 GEMMs leaves it lower for a while."""
    torch = wk.torch
    torch.cuda.synchronize()
    t0, n = time.perf_counter(), 0
    while n < replays or time.perf_counter() - t0 < seconds:
        scrub_l2(torch, scrub, stream)
        wk._replay(wk.g_step, stream)
        n += 1
        if n % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def hbm_probe(torch, dev, stream, gib=2.0, reps=10):
    """Stream probe for context: a plain device copy (read + write) and a read-only reduction of
    `gib` GiB, best of `reps`, in GB/s (bytes moved / event time)."""
    n = int(gib * (1 << 30))
    a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    res = {}
    for name, fn, nbytes in (("copy_GBs", lambda: b.copy_(a), 2 * n),
                             ("read_GBs", lambda: a.view(torch.int64).sum(), n)):
        best = None
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                e0.record(stream)
                fn()
                e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3
            best = us if best is None else min(best, us)
        res[name] = nbytes / (best * 1e-6) / 1e9
    del a, b
    torch.cuda.empty_cache()
    res["bytes"] = n
    res["note"] = "plain torch copy_ and int64 sum, best of %d; context for the 8 TB/s nominal peak" % reps
    return res


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_seconds(inp, nthreads):
    """Wall time of one full fp64 oracle run (every row of the step) on `nthreads` host threads."""
    import oracle
    import workloads as W
    pool, ki, oc = W.compact_inputs(inp)
    args = oracle.inputs_args(inp, pool, ki, oc)
    t0 = time.perf_counter()
    oracle.attn(*args, nthreads=nthreads)
    return time.perf_counter() - t0


def cpu_baseline(inp, alg, wl_name):
    """The fp64 CPU oracle over the whole step (every (b, i, h) row), once, on all host cores."""
    cores = len(os.sched_getaffinity(0))
    t = oracle_seconds(inp, cores)
    return dict(value=alg["kv_bytes"] / t / 1e9, unit="GB/s", cores=cores, kind="oracle",
                sample=f"the whole {wl_name} step (all {inp.B * inp.q_len * inp.H} query rows), one run of "
                       f"{t:.1f} s on {cores} threads ({cpu_model()})", us_per_step=t * 1e6, seconds=t)


def oracle_timings(names):
    """Full oracle runs of the smaller configurations: median of 3 on all host cores, and one
    1-thread run for the three smallest."""
    import workloads as W
    cores = len(os.sched_getaffinity(0))
    out = {}
    for k, name in enumerate(names):
        wl = W.CONFIGS[name]
        inp = W.make_inputs(wl, layout=wl.layout)
        runs = sorted(oracle_seconds(inp, cores) for _ in range(3))
        rec = {"seconds_all_cores": runs[1], "cores": cores,
               "kv_GBs_all_cores": algorithmic(inp)["kv_bytes"] / runs[1] / 1e9}
        if k < 3:
            rec["seconds_1_thread"] = oracle_seconds(inp, 1)
        out[name] = rec
    out["cpu_model"] = cpu_model()
    return out


def stats(xs):
    xs = sorted(xs)
    n = len(xs)
    return dict(median=xs[n // 2], p10=xs[max(0, int(n * 0.1))], p90=xs[min(n - 1, int(n * 0.9))],
                mean=sum(xs) / n)


def roofline_for(wk, part_us):
    alg = wk.alg
    ai = alg["flops"] / alg["partial_bytes"]
    t = part_us * 1e-6
    if ai > RIDGE:
        ach = alg["flops"] / t / 1e12
        return dict(bound="mfma", achieved=ach, peak=MFMA_BF16_PEAK_TFS, unit="TFLOP/s", frac=ach / MFMA_BF16_PEAK_TFS,
                    traffic=None, algorithmic_flops=alg["flops"], algorithmic_bytes=alg["partial_bytes"],
                    arithmetic_intensity=ai)
    ach = alg["partial_bytes"] / t / 1e9
    return dict(bound="hbm", achieved=ach, peak=HBM_PEAK_GBS, unit="GB/s", frac=ach / HBM_PEAK_GBS, traffic=None,
                algorithmic_flops=alg["flops"], algorithmic_bytes=alg["partial_bytes"], arithmetic_intensity=ai)


KERNEL_SRC = os.path.join(ROOT, "speculative_decoding_mla_split_amd", "csrc", "mla_verify.hip")


def kernel_source_sha():
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()


def measured_traffic(workload, split_tag):
    """HBM bytes per partial-kernel launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary,
    scaled by the same counters' reading for a plain copy of known size; None when there is no
    summary for this workload or the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_verify_partial_{workload}_{split_tag}.json")
    if not os.path.exists(path):
        return None, "no counter summary"
    t = json.load(open(path))
    if t.get("source_sha256") != kernel_source_sha():
        return None, "kernel changed since the counters were taken"
    fetch = t["fetch_kib_per_dispatch"] * 1024 / t["copy_fetch_factor"]
    write = t["write_kib_per_dispatch"] * 1024 / t["copy_write_factor"]
    return fetch + write, os.path.relpath(path, ROOT)


def copy_calibration(gib: float, reps: int):
    """A plain device copy of a known size (for scaling the FETCH_SIZE / WRITE_SIZE counters)."""
    import torch
    n = int(gib * (1 << 30))
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": reps}))


def _event_mean_us(stream, fn, reps, warmup=3):
    """Mean duration of fn() over reps back-to-back launches, timed with HIP events on `stream`."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def _graph_mean_us(stream, fn, per_graph, replays=5):
    """Mean device time of fn() with the host out of the loop: per_graph calls captured into one graph,
    replayed `replays` times between HIP events on `stream`."""
    import torch
    with torch.cuda.stream(stream):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(per_graph):
            fn()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(replays):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (replays * per_graph)


def measure_tree_mask(inp, stream, dev, reps=50):
    """Device tree -> mask builder on the workload's trees: time per call, bytes written, parity."""
    import numpy as np
    import torch

    import speculative_decoding_mla_split_amd as pkg
    parents = torch.from_numpy(np.stack(inp.parents).astype(np.int32)).to(dev)
    kv_indptr = torch.from_numpy(inp.kv_indptr).to(dev)
    total = int(inp.mask_indptr[-1])
    mask = torch.empty(total, dtype=torch.uint8, device=dev)
    indptr = torch.empty(inp.B + 1, dtype=torch.int32, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    call = lambda: pkg.build_tree_mask(parents, kv_indptr, mask, indptr, status, stream=stream)  # noqa: E731
    eager_us = _event_mean_us(stream, call, reps)
    us = _graph_mean_us(stream, call, reps)
    exact = bool(np.array_equal(mask.cpu().numpy(), inp.custom_mask)
                 and np.array_equal(indptr.cpu().numpy(), inp.mask_indptr) and int(status.item()) == 0)
    nbytes = total + 4 * (inp.B + 1) + 4 * parents.numel() + 4 * (inp.B + 1)
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"us_per_call": us, "timing": "graph of back-to-back calls, HIP events", "eager_us_per_call": eager_us,
            "mask_bytes": total, "algorithmic_bytes": nbytes, "achieved_GBs": gbs,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS},
            "launches_per_call": 1, "bit_exact_vs_generator": exact, "reps": reps}


def measure_kv_compact(inp, wl, stream, dev, partial_us_scattered, nsplit, balanced, reps=10):
    """KV compaction of every prefix row into runs past the pool's used rows: time, bandwidth, and the
    partial kernel's time on the compacted indices next to the scattered ones."""
    import numpy as np
    import torch

    import speculative_decoding_mla_split_amd as pkg
    import workloads as W
    tot = int(inp.kv_indptr[-1])
    N = wl.N + tot
    pool = torch.full((N, 576), W.BF16_NAN, dtype=torch.int16, device=dev)
    pool[torch.from_numpy(inp.ref_slots.astype(np.int64)).to(dev)] = torch.from_numpy(inp.ref_rows.view(np.int16)).to(dev)
    pool = pool.view(torch.bfloat16)
    kv_indptr = torch.from_numpy(inp.kv_indptr).to(dev)
    kv_indices = torch.from_numpy(inp.kv_indices).to(dev)
    starts = torch.from_numpy((wl.N + inp.kv_indptr[:-1]).astype(np.int32)).to(dev)
    new_idx = torch.empty(tot, dtype=torch.int32, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    us = _event_mean_us(stream, lambda: pkg.compact_kv(pool, kv_indptr, kv_indices, starts, new_idx, status,
                                                        stream=stream), reps, warmup=1)
    ok = int(status.item()) == 0 and bool(np.array_equal(
        new_idx.cpu().numpy(), np.concatenate([wl.N + inp.kv_indptr[b] + np.arange(inp.prefixes[b])
                                               for b in range(inp.B)])))
    nbytes = 2 * tot * 1152 + 8 * tot
    gbs = nbytes / (us * 1e-6) / 1e9
    # a plain contiguous device copy of the same byte count, as the practical ceiling of read + write
    csrc = torch.empty(tot * 1152, dtype=torch.uint8, device=dev).fill_(1)
    cdst = torch.empty_like(csrc)

    def plain_copy():
        with torch.cuda.stream(stream):
            cdst.copy_(csrc)
    copy_us = _event_mean_us(stream, plain_copy, reps, warmup=1)
    del csrc, cdst
    # the partial kernel over the compacted prefix rows (draft rows stay where they are)
    size = pkg.balanced_workspace_size if balanced else pkg.workspace_size
    ws = torch.empty(size(inp.B, inp.q_len, inp.H, nsplit), dtype=torch.uint8, device=dev)
    q_nope = torch.from_numpy(inp.q_nope.view(np.int16)).to(dev).view(torch.bfloat16)
    q_rope = torch.from_numpy(inp.q_rope.view(np.int16)).to(dev).view(torch.bfloat16)
    occ = torch.from_numpy(inp.out_cache_loc).to(dev)
    cmask = torch.from_numpy(inp.custom_mask).to(dev)
    mip = torch.from_numpy(inp.mask_indptr).to(dev)

    def part(indices):
        call = pkg.balanced_partial_raw if balanced else pkg.partial_raw
        rc = call(q_nope.data_ptr(), q_rope.data_ptr(), pool.data_ptr(), N, kv_indptr.data_ptr(),
                  indices.data_ptr(), occ.data_ptr(), cmask.data_ptr(), mip.data_ptr(), inp.B, inp.q_len,
                  inp.H, inp.scale, nsplit, ws.data_ptr(), ws.numel(), stream.cuda_stream)
        assert rc == 0
    # the same pool read through the original (scattered) and the compacted indices, timed alike and
    # alternately (the headline's steady-state figure is reported beside them)
    t_sc, t_co = [], []
    for _ in range(2):
        t_sc.append(_event_mean_us(stream, lambda: part(kv_indices), 20, warmup=20))
        t_co.append(_event_mean_us(stream, lambda: part(new_idx), 20, warmup=20))
    sc_us, part_us = sum(t_sc) / len(t_sc), sum(t_co) / len(t_co)
    return {"us_per_call": us, "rows_moved": tot, "algorithmic_bytes": nbytes, "achieved_GBs": gbs,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS},
            "plain_copy_GBs": 2 * tot * 1152 / (copy_us * 1e-6) / 1e9, "vs_plain_copy": copy_us / us,
            "indices_exact": ok, "partial_us_scattered": sc_us, "partial_us_compacted": part_us,
            "partial_us_headline": partial_us_scattered,
            "break_even_steps": (us / (sc_us - part_us)) if sc_us > part_us else None,
            "reps": reps}


def measure_check(wk, stream, strides=(1024, 64)):
    """Validate mode: the device reference check (mla_verify_attn_check) of the last step's output at
    a few sample strides: time per check and the report it wrote."""
    import math

    import torch
    pkg, inp = wk.pkg, wk.inp
    rep = torch.zeros(pkg.REPORT_WORDS, dtype=torch.float32, device=wk.dev)
    res = []
    for stride in strides:
        cws = torch.empty(pkg.check_workspace_size(inp.B, inp.q_len, inp.H, stride), dtype=torch.uint8,
                          device=wk.dev)

        def chk():
            rc = pkg.check_raw(wk.q_nope.data_ptr(), wk.q_rope.data_ptr(), wk.pool.data_ptr(), inp.N,
                               wk.kv_indptr.data_ptr(), wk.kv_indices.data_ptr(), wk.out_cache_loc.data_ptr(),
                               wk.custom_mask.data_ptr(), wk.mask_indptr.data_ptr(), inp.B, inp.q_len, inp.H, inp.scale,
                               wk.out.data_ptr(), wk.lse.data_ptr(), stride, cws.data_ptr(), cws.numel(),
                               rep.data_ptr(), stream.cuda_stream)
            assert rc == 0
        us = _event_mean_us(stream, chk, 3, warmup=1)
        r = rep.cpu().tolist()
        rows = math.ceil(inp.B * inp.q_len * inp.H / stride)
        cols = sum(inp.prefixes[(k // (inp.q_len * inp.H))] + inp.q_len
                   for k in range(0, inp.B * inp.q_len * inp.H, stride))
        res.append({"sample_stride": stride, "rows_checked": rows, "us_per_check": us,
                    "reference_kv_bytes_read": 3 * 1152 * cols,
                    "report": {"max_abs_out": r[0], "max_abs_lse": r[1], "rows": r[2], "bad_rows": r[3]}})
    return res


def step_floor_us(alg):
    return max(alg["step_bytes"] / (HBM_PEAK_GBS * 1e9), alg["flops"] / (MFMA_BF16_PEAK_TFS * 1e12)) * 1e6


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="ragged4_185k_h64")
    ap.add_argument("--layout", default=None)
    ap.add_argument("--nsplit", type=int, default=None,
                    help="per-request schedule: splits per request (default: the workload's largest)")
    ap.add_argument("--schedule", choices=("balanced", "per-request"), default="balanced",
                    help="balanced: one split budget for the batch (mla_verify_attn_balanced); "
                         "per-request: nsplit splits per request (mla_verify_attn)")
    ap.add_argument("--units", type=int, default=None,
                    help="balanced schedule: split budget (default: CUs / 128-row tiles, one workgroup per CU)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true", help="skip the 16k/65k configuration sweep")
    ap.add_argument("--parity-rows", type=int, default=48)
    ap.add_argument("--no-next", action="store_true", help="skip the tree-mask and KV-compaction measurements")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration under rocprofv3 --pmc)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the verify attention is a single-GPU "
                                   "kernel here (multi-GPU sharding is a design note, not built)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(1.0, 4)
        return

    import torch

    import workloads as W

    dev = torch.device("cuda:0")
    wl = W.CONFIGS[args.config]
    layout = args.layout or wl.layout
    balanced = args.schedule == "balanced"
    n_rt = -(-wl.q_len * wl.H // 128)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    units = args.units or max(wl.B, cus // n_rt)
    nsplit = units if balanced else (args.nsplit or wl.nsplits[-1])
    stream = torch.cuda.Stream(device=dev)
    print(f"[bench] {wl.name} layout={layout} schedule={args.schedule} "
          f"{'units' if balanced else 'nsplit'}={nsplit}", file=sys.stderr, flush=True)
    wk = Workload(wl, layout, nsplit, dev, balanced=balanced)
    scrub = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    # parity of this run's inputs before any timing
    with torch.cuda.stream(stream):
        wk.step(stream)
    parity = wk.parity(args.parity_rows)
    print(f"[bench] parity on {parity['rows']} sampled rows: ok={parity['ok']}", file=sys.stderr, flush=True)
    wk.capture(stream)
    settled = settle(wk, stream, scrub)
    for _ in range(args.warmup):
        scrub_l2(torch, scrub, stream)
        wk._replay(wk.g_step, stream)
    # the timed region: exactly `steps` steps, each a scrub (outside the events) then one replay of the
    # step graph between HIP events
    t0 = time.perf_counter()
    timed = wk.graph_replays(stream, args.steps, scrub=scrub, warmup=0)
    wall = time.perf_counter() - t0
    step_s = stats(timed)
    print(f"[bench] timed {args.steps} steps: median {step_s['median']:.1f} us/step", file=sys.stderr, flush=True)
    # the kernels' own durations (eager launches, same scrub), and the protocol's 50-replay distributions
    e_step, part, comb = wk.kernel_split(stream, max(args.steps, 20), scrub)
    part_s, comb_s, eager_s = stats(part), stats(comb), stats(e_step)
    cold = stats(wk.graph_replays(stream, 50, scrub=scrub, warmup=0))
    hot = stats(wk.graph_replays(stream, 50))
    check = None if args.no_next else measure_check(wk, stream)
    alg = wk.alg
    med = step_s["median"]
    value = alg["kv_bytes"] / (med * 1e-6) / 1e9
    floor = step_floor_us(alg)
    roof = roofline_for(wk, part_s["mean"])
    traffic, traffic_src = measured_traffic(wl.name, ("u" if balanced else "ns") + str(nsplit))
    roof["traffic"] = traffic
    roof["traffic_source"] = traffic_src
    roof["duration_us"] = part_s["mean"]
    roof["duration_source"] = ("mean of HIP events around eager launches of the partial kernel, each after "
                               "a 1 GiB scrub")
    result = {
        "metric": METRIC, "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": med / 1e3, "us_per_step": med, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "prefixes": list(wl.prefixes), "q_len": wl.q_len, "H": wl.H,
                   "pool_rows": wl.N, "layout": layout, "schedule": args.schedule,
                   ("units" if balanced else "nsplit"): nsplit, "seed": wl.seed,
                   "scale": "1/sqrt(192)", "parallelism": "single GPU"},
        "timing": ("each timed step: a 1 GiB scrub read (outside the events), then one replay of the captured "
                   "step graph (partial + combine) between HIP events on one stream; value and ms_per_step use "
                   "the median step. kernels_us: eager launches with events around each kernel, same scrub"),
        "timed_region_wall_s": wall,
        "settle_replays": settled,
        "settle": ("untimed step replays before the warmup steps (at least 30 and 40 ms): the GPU clock ramps "
                   "from ~1.85 to ~2.05 GHz over the first few dozen launches of the step"),
        "roofline": roof,
        "step_us": step_s,
        "kernels_us": {"partial": part_s, "combine": comb_s, "eager_step": eager_s},
        "graph_step_cold_us": cold, "graph_step_hot_us": hot,
        "graph_protocol": "one-graph step: 10 warm-up replays, then 50 replays between HIP events, each after a "
                          "1 GiB scrub (cold); hot = 50 back-to-back replays",
        "step_floor_us": floor, "step_roofline_frac": floor / med,
        "algorithmic_GBs": alg["step_bytes"] / (med * 1e-6) / 1e9,
        "algorithmic_frac_hbm": alg["step_bytes"] / (med * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "tflops_step": alg["flops"] / (med * 1e-6) / 1e12,
        "tflops_frac_mfma": alg["flops"] / (med * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFS,
        "parity_sampled": parity,
    }
    if check is not None:
        result["validate_check"] = check
    main_inp = wk.inp
    del wk
    torch.cuda.empty_cache()
    result["hbm_probe"] = hbm_probe(torch, dev, stream)

    if not args.no_next:
        print("[bench] tree mask builder", file=sys.stderr, flush=True)
        nxt = {"tree_mask": measure_tree_mask(main_inp, stream, dev)}
        print("[bench] kv compaction", file=sys.stderr, flush=True)
        nxt["kv_compact"] = measure_kv_compact(main_inp, wl, stream, dev, part_s["mean"], nsplit, balanced)
        result["next_rows"] = nxt
        torch.cuda.empty_cache()

    if not args.no_others:
        def auto_units(w):  # one workgroup per CU: the balanced schedule's default budget
            return max(w.B, cus // -(-w.q_len * w.H // 128))

        sweep = [(n, lay, "balanced", auto_units(W.CONFIGS[n])) for n, lay in
                 (("16k_h64", "scattered"), ("16k_h64", "contiguous"), ("65k_h8", "scattered"),
                  ("4k_h64", "scattered"), ("tiny_256_h8", "scattered"))]
        sweep += [(wl.name, layout, "per-request", 64), (wl.name, layout, "balanced", 64),
                  ("16k_h64", "scattered", "per-request", 16), ("16k_h64", "scattered", "per-request", 32),
                  ("16k_h64", "scattered", "per-request", 64), ("16k_h64", "contiguous", "per-request", 16),
                  ("65k_h8", "scattered", "per-request", 16), ("65k_h8", "scattered", "per-request", 64),
                  ("4k_h64", "scattered", "per-request", 16), ("tiny_256_h8", "scattered", "per-request", 4)]
        others = []
        for name, lay, sched, ns in sweep:
            print(f"[bench] config {name} {lay} {sched} {ns}", file=sys.stderr, flush=True)
            ow = Workload(W.CONFIGS[name], lay, ns, dev, balanced=sched == "balanced")
            ow.capture(stream)
            settle(ow, stream, scrub, replays=10, seconds=0.02)
            cold_o = stats(ow.graph_replays(stream, 50, scrub=scrub))
            hot_o = stats(ow.graph_replays(stream, 50))
            _, pcl, ccl = ow.kernel_split(stream, 25, scrub)
            pc, cc = stats(pcl), stats(ccl)
            a = ow.alg
            fl = step_floor_us(a)
            t = cold_o["median"]
            tr, tr_src = measured_traffic(name, ("u" if sched == "balanced" else "ns") + str(ns))
            pr = roofline_for(ow, pc["mean"])
            pr["traffic"], pr["traffic_source"] = tr, tr_src
            others.append({
                "workload": name, "layout": lay, "schedule": sched, ("units" if sched == "balanced" else "nsplit"): ns,
                "step_us_cold": cold_o, "step_us_hot": hot_o, "partial_us_cold": pc, "combine_us_cold": cc,
                "kv_GBs_cold": a["kv_bytes"] / (t * 1e-6) / 1e9,
                "algorithmic_GBs_cold": a["step_bytes"] / (t * 1e-6) / 1e9,
                "algorithmic_frac_hbm": a["step_bytes"] / (t * 1e-6) / 1e9 / HBM_PEAK_GBS,
                "tflops_cold": a["flops"] / (t * 1e-6) / 1e12,
                "tflops_frac_mfma": a["flops"] / (t * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFS,
                "step_floor_us": fl, "roofline_frac_cold": fl / t, "roofline_frac_hot": fl / hot_o["median"],
                "partial_roofline": pr,
            })
            del ow
            torch.cuda.empty_cache()
        result["other_configs"] = others
    del scrub
    torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        print("[bench] cpu baseline: the full oracle step", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(main_inp, alg, wl.name)
        if not args.no_others:
            print("[bench] oracle timings of the smaller configurations", file=sys.stderr, flush=True)
            result["oracle_timings"] = oracle_timings(["tiny_256_h8", "4k_h64", "16k_h64", "65k_h8"])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

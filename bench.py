"""Benchmark of the deterministic attention backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

One step = one whole backward (dash_attn_bwd_prepare then dash_attn_bwd_run,
which together are exactly dash_attn_bwd: preprocess, persistent backward, and
for the atomic reference the finalize pass) over one batch of synthetic bf16
input already resident in HBM.  Each schedule is timed separately: W untimed
steps, then K steps between two device synchronisations, with HIP events
recorded on the call's stream before the preprocess, between the phases and
after the persistent kernel.  Prints one JSON line.  Outside the timed
region each schedule's output is checked for run-to-run bit identity at this
size (the first warm-up output against the last timed step and five more
steps on rotating streams behind a random amount of unrelated work), and the
last timed step's turn waits are read from the workspace: `wait_fraction` is
the time waves spent waiting for an earlier dQ contribution, as a share of
the persistent grid's wave time (the schedule's bubbles).

The `table` row is the library's searched task table for the workload
(dash_schedule_search over the family of walks on the device's grid, with the
automatic selector's weights: a task costs 1, a causal diagonal task 1, the
exposed hand-off 0.1), run as dash_attn_bwd_prepare then
dash_attn_bwd_table_run with the same events.  When the search returns exactly
the table of a closed form that splits no query heads it is not timed twice:
the line names that closed form instead.

The headline value is the whole-step throughput of the fastest deterministic
schedule in TFLOP/s with FLOPs = 10*B*Hq*S^2*D (halved for a causal mask).  The
roofline object prices the persistent backward kernel alone (events around
dash_attn_bwd_run).  Its bound is the one the kernel's algorithmic intensity
selects: algorithmic FLOPs over algorithmic bytes (per (KV tile, Q tile) task
the Q and dO tiles, the two per-row values, and the fp32 dQ partial sum read
by every contributor but the first and written by every contributor but the
last; per (batch, KV head, KV tile) K, V, dK and dV; the bf16 dQ) against the
ridge point 2.5 PFLOP/s / 8 TB/s.  `achieved` is the algorithmic bytes (HBM
bound) or FLOPs (MFMA bound) of one launch over the kernel's mean duration; the
fraction of the other peak is reported beside it.  The traffic figure is the
calibrated FETCH_SIZE + WRITE_SIZE of that kernel read from the committed
rocprofv3 summary, reported only while that summary's kernel-source hash
matches the current source.  The cpu_baseline object times the float64 oracle
on a bounded sample of the same workload on the host cores.

The headline workload is the largest configuration, the 16k full-mask layer
(B=1 S=16384 Hq=Hkv=32 D=128).  Unless --config or --headline-only is given,
the line also carries "workloads": the same per-schedule measurements, the
roofline of the best schedule and det/atomic for each other configuration.
"""

import argparse
import hashlib
import json
import os
import re
import struct
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
# the sources the persistent kernel is compiled from
KERNEL_SOURCES = [os.path.join(ROOT, "scheduling_persistent_attn_amd", "csrc", f)
                  for f in ("bwd.hip", "bwd_wide.hip", "bwd_wide64.hip", "bwd_common.h", "lds_layout.h", "schedule.h",
                            "kernels.h")]


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published

CONFIGS = {
    "llama8b_causal": dict(B=4, S=4096, Hq=32, Hkv=8, D=128, causal=True,
                           desc="causal attention backward shaped like an 8B Llama-style "
                                "layer: B=4 S=4096 Hq=32 Hkv=8 (GQA 4) D=128"),
    "small_full": dict(B=1, S=256, Hq=2, Hkv=2, D=64, causal=False,
                       desc="full-mask attention backward B=1 S=256 Hq=Hkv=2 D=64"),
    "dit_full": dict(B=2, S=4096, Hq=24, Hkv=24, D=64, causal=False,
                     desc="full-mask attention backward shaped like a diffusion/vision "
                          "block: B=2 S=4096 Hq=Hkv=24 D=64"),
    "long_full": dict(B=1, S=16384, Hq=32, Hkv=32, D=128, causal=False,
                      desc="long-sequence full-mask attention backward B=1 S=16384 "
                           "Hq=Hkv=32 D=128"),
    "qwen7b_causal": dict(B=1, S=16384, Hq=28, Hkv=4, D=128, causal=True,
                          desc="long-sequence causal attention backward shaped like a 7B "
                               "Qwen-style layer: B=1 S=16384 Hq=28 Hkv=4 (GQA 7) D=128"),
}
# the headline workload: the largest of the five configurations (the 16k
# full-mask layer, 1.1e13 FLOPs per step); every other one is summarised in
# the same line under "workloads"
DEFAULT_CONFIG = "long_full"
OTHER_WORKLOADS = ("small_full", "llama8b_causal", "dit_full", "qwen7b_causal")

# kv heads of the float64 oracle's timed sample per workload (whole key/value
# groups, so that dK/dV of those heads are complete): the first and last
# groups of batch 0, about 10-20 s of host work on a 16-thread host
CPU_SAMPLE_KV_HEADS = {"long_full": (0, 1, 2, 29, 30, 31), "qwen7b_causal": (0, 3)}


def flops(cfg):
    f = 10.0 * cfg["B"] * cfg["Hq"] * cfg["S"] ** 2 * cfg["D"]
    return f / 2 if cfg["causal"] else f


def algorithmic_bytes(cfg, T, parts=1):
    """Bytes one backward launch must move between HBM and the chip under
    this design (whole tiles; see the module docstring).  With the query heads
    split into `parts`, every part loads K and V itself and writes fp32 dK/dV
    sums that the final pass reads back."""
    B, S, Hq, Hkv, D = cfg["B"], cfg["S"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    N = (S + T - 1) // T
    tiles = B * Hq * N                                     # dQ tiles
    tasks = B * Hq * (N * (N + 1) // 2 if cfg["causal"] else N * N)
    per_task = 2 * T * D * 2 + 2 * T * 4                   # Q, dO tiles; -lse/scale, -Dl
    handoff = 2 * (tasks - tiles) * T * D * 4              # fp32 partial sum: load + store
    dq_out = tiles * T * D * 2
    kv_tiles = B * Hkv * N
    kv = kv_tiles * (parts * 2 * T * D * 2 + 2 * T * D * 2)  # K, V in (per part); dK, dV out
    if parts > 1:
        kv += kv_tiles * parts * 2 * T * D * 4 * 2           # fp32 part sums: store + load
    return tasks * per_task + handoff + dq_out + kv


def dq_partial_adds(cfg, T):
    """fp32 element additions into the dQ accumulator per launch: every task
    adds its T x D contribution (whole tiles)."""
    B, S, Hq, D = cfg["B"], cfg["S"], cfg["Hq"], cfg["D"]
    N = (S + T - 1) // T
    tasks = B * Hq * (N * (N + 1) // 2 if cfg["causal"] else N * N)
    return tasks * T * D


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# weights of the table search: those of the library's automatic selector
SEARCH_WEIGHTS = (1.0, 1.0, 0.1)


def searched_table(dash, cfg):
    """The library's searched table for the workload on the device grid:
    {"offs", "tasks", "family", "items", "per_head", "makespan", "same_as"}."""
    B, S, Hq, Hkv, D = cfg["B"], cfg["S"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    mask = 1 if cfg["causal"] else 0
    T = dash.dash_attn_tile_size(S, D)
    N = (S + T - 1) // T
    G = Hq // Hkv
    grid = dash.dash_attn_bwd_grid_size(S, D, mask)
    res = dash.dash_schedule_search(S, D, mask, G, B * Hkv, grid, *SEARCH_WEIGHTS)
    offs = [int(v) for v in res["item_offsets"]]
    tasks = [tuple(int(v) for v in t) for t in res["tasks"].tolist()]
    raw = dash.dash_schedule_table_pack(S, D, mask, G, offs, tasks)
    per_head = (struct.unpack_from("<I", raw, 12)[0] & 0x100) != 0
    same_as = None
    names = {v: k for k, v in dash.SCHEDULES.items()}
    for s in (dash.NAIVE, dash.DESCENDING_Q, dash.SHIFT, dash.SYMMETRIC_SHIFT):
        if s == dash.SYMMETRIC_SHIFT and (not mask or N % 2):
            continue
        if dash.dash_attn_bwd_head_parts(B, Hq, Hkv, S, D, mask, s) != 1:
            continue
        co, ct = dash.dash_schedule_table_closed_form(mask, s, N, G)
        if [int(v) for v in co] == offs and [tuple(int(v) for v in t) for t in ct.tolist()] == tasks:
            same_as = names[s]
            break
    return {"offs": offs, "tasks": tasks, "family": list(res["family"]), "items": len(offs) - 1,
            "per_head": per_head, "makespan": res["report"]["makespan"], "same_as": same_as}


def time_schedule(dash, x, o, lse, cfg, sched, steps, warmup, table=None):
    """Times one schedule; `table` (from searched_table) runs the TABLE
    schedule under that table."""
    import torch
    mask = 1 if cfg["causal"] else 0
    if table is not None:
        sched = dash.TABLE
        tdev, titems = dash.upload_table(x["q"], x["k"], cfg["causal"], table["offs"], table["tasks"])
    ws = dash.new_workspace(x["q"], x["k"], mask, sched)
    dq = torch.empty_like(x["q"])
    dk = torch.empty_like(x["k"])
    dv = torch.empty_like(x["v"])
    stream = torch.cuda.current_stream()
    Hkv = x["k"].shape[2]

    # events on the stream the kernels are launched on
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]

    def step(e=None, s=None):
        s = stream if s is None else s
        if e:
            e[0].record(s)
        dash.dash_attn_bwd_prepare(o, x["do"], lse, tuple(x["q"].shape), Hkv, mask, sched,
                                   ws, s)
        if e:
            e[1].record(s)
        if table is not None:
            dash.dash_attn_bwd_table_run(x["q"], x["k"], x["v"], x["do"], dq, dk, dv, mask, tdev,
                                         titems, 0, ws, s)
        else:
            dash.dash_attn_bwd_run(x["q"], x["k"], x["v"], x["do"], dq, dk, dv, mask, sched,
                                   ws, s)
        if e:
            e[2].record(s)

    def bits():
        return [t.view(torch.int16).clone() for t in (dq, dk, dv)]

    for n in range(warmup):
        step()
        if n == 0:
            ref = bits()  # the reference for the run-to-run check below
    dash.dash_attn_bwd_check(ws, stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for n in range(steps):
        step(ev[n])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dash.dash_attn_bwd_check(ws, stream)
    per = sorted(e[0].elapsed_time(e[2]) for e in ev)
    kern = [e[1].elapsed_time(e[2]) for e in ev]
    out = {"ms_mean": sum(per) / len(per), "ms_median": per[len(per) // 2],
           "ms_p10": per[len(per) // 10],
           "ms_p90": per[min(len(per) - 1, (9 * len(per)) // 10)],
           "kernel_ms_mean": sum(kern) / len(kern),
           "wall_ms_per_step": 1e3 * wall / steps}
    # the last timed step's bubbles: time its waves spent waiting for a turn,
    # as a share of the time all waves of the persistent grid were resident
    wst = dash.dash_attn_bwd_wait_stats(ws, stream)
    S, D = x["q"].shape[1], x["q"].shape[3]
    waves = dash.dash_attn_bwd_grid_size(S, D, mask) * dash.dash_attn_tile_size(S, D) // 32
    out["turn_waits"] = wst["waits"]
    # the shader clock of the last timed launch: workgroup 0's s_memtime and
    # 100 MHz s_memrealtime stamps at the kernel's start and exit (control
    # words 8-15 of the workspace)
    st = ws[32:64].view(torch.int64).cpu().tolist()
    if st[3] > st[1] and st[2] > st[0]:
        out["sclk_mhz"] = round(100.0 * (st[2] - st[0]) / (st[3] - st[1]), 1)
    if table is not None:
        # a per-head table writes one partial per query head; a whole-tile
        # table none
        out["head_parts"] = x["q"].shape[2] // Hkv if table["per_head"] else 1
    else:
        out["head_parts"] = dash.dash_attn_bwd_head_parts(x["q"].shape[0], x["q"].shape[2], Hkv,
                                                          S, D, mask, sched)
    out["wait_fraction"] = wst["wait_seconds"] / (waves * kern[-1] * 1e-3)
    if warmup > 0:
        out["repro"] = reproducibility(dash, step, bits, ref, ws)
    return out


def reproducibility(dash, step, bits, ref, ws, extra=5):
    """Outside the timed region: the outputs of the last timed step and of
    `extra` more steps, each on one of three streams behind a seeded random
    amount of unrelated work, compared bit for bit with the first warm-up
    step's.  Returns the number of runs compared and how many differed."""
    import random
    import torch
    differ = int(any(not torch.equal(a, b) for a, b in zip(ref, bits())))
    streams = [torch.cuda.Stream() for _ in range(3)]
    filler = torch.ones(1 << 22, device=ref[0].device)
    rng = random.Random(1234)
    for n in range(extra):
        s = streams[n % 3]
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for _ in range(rng.randint(0, 6)):
                filler.mul_(1.0001)
            step(s=s)
            dash.dash_attn_bwd_check(ws, s)
            differ += int(any(not torch.equal(a, b) for a, b in zip(ref, bits())))
        torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return {"runs": extra + 1, "differ": differ}


def time_forward(dash, x, cfg, steps, warmup):
    """Mean event-timed duration of dash_attn_fwd (O and LSE) on this input,
    outputs allocated once outside the timed region."""
    import torch
    o, lse = dash.forward(x["q"], x["k"], x["v"], cfg["causal"])
    mask = dash.MASK_CAUSAL if cfg["causal"] else dash.MASK_FULL
    for _ in range(warmup):
        dash.dash_attn_fwd(x["q"], x["k"], x["v"], o, lse, mask)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dash.dash_attn_fwd(x["q"], x["k"], x["v"], o, lse, mask)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def committed_traffic(config, schedule):
    """Calibrated HBM bytes per launch of the persistent kernel, from the
    committed rocprofv3 summary; None if there is none or it was taken on a
    different kernel source."""
    path = os.path.join(ROOT, "profiles", "bwd_main_%s.md" % config)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    if not m:
        return None
    if kernel_source_hash() != m.group(1):
        return None
    m = re.search(r"traffic_bytes_per_launch\[%s\]:\s*([0-9.eE+]+)" % re.escape(schedule), text)
    return float(m.group(1)) if m else None


def cpu_baseline(name, cfg, budget_s=20.0):
    """Time the float64 oracle (forward + backward) on whole (batch, kv head)
    groups of the workload and report the rate in TFLOP/s of the same FLOP
    formula.  Workloads listed in CPU_SAMPLE_KV_HEADS time exactly those kv
    heads of batch 0; the others take groups in order until the budget is
    used or every group is done (batch 0's inputs stand in for every batch:
    the oracle's work does not depend on the values)."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import attention as oa
    from scheduling_persistent_attn_amd.inputs import as_float64, make_inputs

    B, S, Hq, Hkv, D = cfg["B"], cfg["S"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    G = Hq // Hkv
    x = make_inputs(1, S, Hq, Hkv, D, seed=1000)
    h = {k: as_float64(v) for k, v in x.items()}
    fixed = CPU_SAMPLE_KV_HEADS.get(name)
    done = []
    t0 = time.perf_counter()
    while True:
        kv = fixed[len(done)] if fixed else len(done) % Hkv
        hs = list(range(kv * G, (kv + 1) * G))
        oa.attention_backward(h["q"][:, :, hs], h["k"][:, :, kv:kv + 1],
                              h["v"][:, :, kv:kv + 1], h["do"][:, :, hs], cfg["causal"])
        done.append(kv)
        if fixed:
            if len(done) == len(fixed):
                break
        elif time.perf_counter() - t0 >= budget_s or len(done) >= B * Hkv:
            break
    dt = time.perf_counter() - t0
    fl = flops(dict(cfg, B=1, Hq=G * len(done)))
    threads = 0
    for info in threadpool_info():
        if info.get("user_api") == "blas":
            threads = max(threads, info.get("num_threads", 0))
    heads = sorted(g for kv in set(done) for g in range(kv * G, (kv + 1) * G))
    if fixed:
        what = ("the fixed sample of kv heads %s of batch 0 (query heads %s), %d of the "
                "workload's %d (batch, kv head) groups"
                % (list(fixed), _ranges(heads), len(done), B * Hkv))
    else:
        what = ("%d of %d (batch, kv head) groups (%d query heads; batch 0's inputs for every "
                "batch)" % (len(done), B * Hkv, G * len(done)))
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": threads or os.cpu_count(),
            "kind": "oracle",
            "sample": "float64 oracle forward+backward of %s at S=%d D=%d, %.1f s; the rate "
                      "extrapolates linearly to the whole workload (heads are independent); "
                      "includes the oracle's own float64 forward" % (what, S, D, dt)}


def _ranges(xs):
    out, i = [], 0
    while i < len(xs):
        j = i
        while j + 1 < len(xs) and xs[j + 1] == xs[j] + 1:
            j += 1
        out.append(str(xs[i]) if i == j else "%d-%d" % (xs[i], xs[j]))
        i = j + 1
    return ",".join(out)


def roofline(cfg, T, fl, kernel_ms, schedule, traffic, parts=1):
    """The persistent kernel against the peak its algorithmic intensity
    selects (ridge = PEAK_BF16 / PEAK_HBM FLOP per byte)."""
    nbytes = algorithmic_bytes(cfg, T, parts)
    gbs = nbytes / (kernel_ms * 1e-3) / 1e9
    tflops = fl / (kernel_ms * 1e-3) / 1e12
    intensity = fl / nbytes
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    r = {"kernel": "bwd_main (%s)" % schedule,
         "algorithmic_bytes": nbytes, "algorithmic_flops": fl,
         "intensity_flop_per_byte": round(intensity, 2), "ridge_flop_per_byte": round(ridge, 2)}
    if intensity < ridge:
        r.update(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                 frac=round(gbs / PEAK_HBM_GBS, 4),
                 mfma_frac=round(tflops / PEAK_BF16_TFLOPS, 4))
    else:
        r.update(bound="mfma", achieved=round(tflops, 3), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                 frac=round(tflops / PEAK_BF16_TFLOPS, 4),
                 hbm_frac=round(gbs / PEAK_HBM_GBS, 4))
    # calibrated FETCH_SIZE + WRITE_SIZE bytes per launch (None when the
    # committed profile predates the kernel source)
    r["traffic"] = traffic
    return r


def sim_report():
    """Critical path, efficiency and Lemma 1 check of every schedule on every
    large workload, from the library's simulator: P = 256 workers (the
    compute units of an MI355X) and 132 (the SM count of the H800 the pages
    measure on), dynamic dispatch, c = c_diag = 1, r/c in {0, 0.1, 0.25}.
    Each schedule runs with the query-head split the library gives it (a
    split group simulates as `parts` groups of G / parts heads, in the same
    dispatch order).  A last row per case is the searched table
    (dash_schedule_search with the same weights; schedule "table", with its
    family and whether it is in the per-head form).  One line of JSON per
    case."""
    import scheduling_persistent_attn_amd as dash
    names = {v: k for k, v in dash.SCHEDULES.items()}
    for name in ("llama8b_causal", "dit_full", "long_full", "qwen7b_causal"):
        cfg = CONFIGS[name]
        T = dash.dash_attn_tile_size(cfg["S"], cfg["D"])
        N = (cfg["S"] + T - 1) // T
        G = cfg["Hq"] // cfg["Hkv"]
        groups = cfg["B"] * cfg["Hkv"]
        mask = 1 if cfg["causal"] else 0
        for P in (256, 132):
            for r in (0.0, 0.1, 0.25):
                for sched in (dash.NAIVE, dash.DESCENDING_Q, dash.SHIFT, dash.SYMMETRIC_SHIFT):
                    if sched == dash.SYMMETRIC_SHIFT and (not mask or N % 2):
                        continue
                    parts = dash.dash_attn_bwd_head_parts(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["S"],
                                                          cfg["D"], mask, sched)
                    res = dash.dash_sim_run(mask, sched, N, G // parts, groups * parts, P, 1, 1.0, 1.0, r)
                    print(json.dumps({"workload": name, "N": N, "G": G, "groups": groups,
                                      "head_parts": parts,
                                      "P": P, "r_over_c": r, "schedule": names[sched],
                                      "critical_path": res["makespan"],
                                      "efficiency": res["efficiency"],
                                      "lemma1_violations": res["violations"],
                                      "order_edges": res["order_edges"],
                                      "deadlock": bool(res["deadlock"])}), flush=True)
                tab = dash.dash_schedule_search(cfg["S"], cfg["D"], mask, G, groups, P, 1.0, 1.0, r)
                raw = dash.dash_schedule_table_pack(cfg["S"], cfg["D"], mask, G, tab["item_offsets"],
                                                    tab["tasks"])
                rep = tab["report"]
                print(json.dumps({"workload": name, "N": N, "G": G, "groups": groups,
                                  "P": P, "r_over_c": r, "schedule": "table",
                                  "family": list(tab["family"]),
                                  "per_head": bool(struct.unpack_from("<I", raw, 12)[0] & 0x100),
                                  "critical_path": rep["makespan"],
                                  "efficiency": rep["efficiency"],
                                  "lemma1_violations": rep["violations"],
                                  "order_edges": rep["order_edges"],
                                  "deadlock": bool(rep["deadlock"])}), flush=True)


def trace_report(dash, name):
    """Per-task timelines from the debug build's trace beside the simulator.

    Runs every deterministic schedule of a workload once with the traced
    library and prints one JSON line each: the measured makespan (first task
    start to last task end), the mean task time, the wave time spent outside
    tasks (idle or between items) as a share of the grid's time, and the
    simulator's critical path for the same shape and grid with r/c = 0.1,
    priced at one task cost for every schedule (the smallest median task time
    among them: a task that waited for a turn is slower by its wait)."""
    import ctypes
    import numpy as np
    import torch
    from scheduling_persistent_attn_amd.inputs import make_inputs

    L = dash.trace_lib()
    cfg = CONFIGS[name]
    B, S, Hq, Hkv, D = cfg["B"], cfg["S"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    mask = 1 if cfg["causal"] else 0
    T = dash.dash_attn_tile_size(S, D)
    N = (S + T - 1) // T
    G = Hq // Hkv
    x = make_inputs(B, S, Hq, Hkv, D, seed=1000, device="cuda")
    o, lse = dash.forward(x["q"], x["k"], x["v"], cfg["causal"])
    dq, dk, dv = (torch.empty_like(x[k]) for k in ("q", "k", "v"))
    P = dash.dash_attn_bwd_grid_size(S, D, mask)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    names = {v: k for k, v in dash.SCHEDULES.items()}
    rows = []
    for sched in (dash.NAIVE, dash.DESCENDING_Q, dash.SHIFT, dash.SYMMETRIC_SHIFT):
        if sched == dash.SYMMETRIC_SHIFT and (not mask or N % 2):
            continue
        n = L.dash_attn_bwd_workspace_size(B, Hq, Hkv, S, D, mask, sched)
        ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
        for _ in range(2):  # the second run is the one read
            ws.zero_()
            st = L.dash_attn_bwd(ptr(x["q"]), ptr(x["k"]), ptr(x["v"]), ptr(o), ptr(x["do"]), ptr(lse),
                                 ptr(dq), ptr(dk), ptr(dv), B, Hq, Hkv, S, D, mask, sched, ptr(ws), n, s)
            assert st == 0 and L.dash_attn_bwd_check(ptr(ws), s) == 0
        parts = dash.dash_attn_bwd_head_parts(B, Hq, Hkv, S, D, mask, sched)
        Gp = G // parts
        paired = sched == dash.SYMMETRIC_SHIFT
        tlen = Gp * (N + 1 if paired else N)
        items = B * Hkv * parts * dash.dash_schedule_num_items(mask, sched, N)
        nrec = items * tlen
        region = (nrec * 64 + 255) // 256 * 256
        start = (n - region) // 8
        rec = ws.view(torch.int64)[start:start + nrec * 8].cpu().numpy().reshape(nrec, 8)
        rec = rec[rec[:, 3] != 0]
        t0, t1 = rec[:, 3].astype(float), rec[:, 4].astype(float)
        dur = (t1 - t0) / 100.0  # microseconds (100 MHz clock)
        span = (t1.max() - t0.min()) / 100.0
        sim = dash.dash_sim_run(mask, sched, N, Gp, B * Hkv * parts, P, 1, 1.0, 1.0, 0.1)
        rows.append({"workload": name, "schedule": names[sched], "tile": T, "head_parts": parts,
                     "tasks": int(len(rec)), "grid": P,
                     "measured_makespan_us": round(span, 1),
                     "mean_task_us": round(float(dur.mean()), 2),
                     "median_task_us": round(float(np.median(dur)), 2),
                     "outside_tasks_fraction": round(1.0 - float(dur.sum()) / (P * span), 4),
                     "simulated_critical_path_tasks": round(sim["makespan"], 2),
                     "simulated_efficiency": round(sim["efficiency"], 4)})
        del ws
    # one task cost for every schedule: the smallest median task time (tasks
    # that waited for a turn are in the tail of their schedule's distribution)
    c = min(r["median_task_us"] for r in rows)
    for r in rows:
        r["task_cost_us"] = c
        r["simulated_makespan_us"] = round(r["simulated_critical_path_tasks"] * c, 1)
        r["measured_over_simulated"] = round(r["measured_makespan_us"] / r["simulated_makespan_us"], 4)
        print(json.dumps(r), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=DEFAULT_CONFIG, choices=sorted(CONFIGS))
    ap.add_argument("--schedules", default="naive,descending_q,shift,symmetric_shift,table,atomic")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline workload, not the summary of the others")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (reference "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters to bytes)")
    ap.add_argument("--trace-report", action="store_true",
                    help="only run the traced debug build once per deterministic schedule of "
                         "--config and compare the measured task timelines with the simulator")
    ap.add_argument("--sim-report", action="store_true",
                    help="only print the schedule simulator's critical paths for every "
                         "workload and schedule (CPU; no GPU needed)")
    args = ap.parse_args()
    if args.sim_report:
        sim_report()
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import scheduling_persistent_attn_amd as dash

    if args.trace_report:
        trace_report(dash, args.config)
        return

    if args.copy_calibration:
        n = 1 << 30
        a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        # and the rate of the same copy, for scale (bytes read + written)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 10
        print(json.dumps({"copy_calibration_bytes": n, "copies": 3,
                          "copy_ms": round(ms, 4), "copy_read_write_TBps": round(2 * n / ms / 1e9, 3)}),
              flush=True)
        return

    head = measure(dash, args.config, args, headline=True)
    line = head
    if not args.headline_only and args.config == DEFAULT_CONFIG:
        # every other workload in the same line: per-schedule whole-step and
        # kernel rates, the roofline of its best schedule and det/atomic
        line["workloads"] = {}
        for name in OTHER_WORKLOADS:
            w = measure(dash, name, args, headline=False)
            line["workloads"][name] = w
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.config, CONFIGS[args.config], args.cpu_budget)
        line["cpu_baseline"]["value"] = round(line["cpu_baseline"]["value"], 6)
    print(json.dumps(line), flush=True)


def measure(dash, name, args, headline):
    """Times every schedule of one workload.  headline=True returns the
    benchmark line's fields; otherwise a summary of the workload."""
    import torch
    from scheduling_persistent_attn_amd.inputs import make_inputs

    cfg = CONFIGS[name]
    B, S, Hq, Hkv, D = cfg["B"], cfg["S"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    T = dash.dash_attn_tile_size(S, D)
    N = (S + T - 1) // T
    log("workload %s: %s" % (name, cfg["desc"]))
    x = make_inputs(B, S, Hq, Hkv, D, seed=1000, device="cuda")
    o, lse = dash.forward(x["q"], x["k"], x["v"], cfg["causal"])
    torch.cuda.synchronize()
    fl = flops(cfg)

    results = {}
    tinfo = None
    for sname in args.schedules.split(","):
        if sname == "table":
            tinfo = searched_table(dash, cfg)
            log("  searched table: family %s, %d items per group%s, simulated %.1f%s" % (
                tinfo["family"], tinfo["items"], " (per-head form)" if tinfo["per_head"] else "",
                tinfo["makespan"], ", same as %s" % tinfo["same_as"] if tinfo["same_as"] else ""))
            if tinfo["same_as"]:
                continue
            r = time_schedule(dash, x, o, lse, cfg, None, args.steps, args.warmup, table=tinfo)
        else:
            sched = dash.SCHEDULES[sname]
            if sched == dash.SYMMETRIC_SHIFT and (not cfg["causal"] or N % 2):
                continue
            r = time_schedule(dash, x, o, lse, cfg, sched, args.steps, args.warmup)
        r["tflops"] = fl / (r["ms_mean"] * 1e-3) / 1e12
        r["kernel_tflops"] = fl / (r["kernel_ms_mean"] * 1e-3) / 1e12
        r["pct_peak"] = 100.0 * r["tflops"] / PEAK_BF16_TFLOPS
        results[sname] = r
        rep = r.get("repro")
        log("  %-16s %8.3f ms  %7.1f TFLOP/s  %5.1f%% of peak  (kernel %.3f ms)  waiting %4.1f%%%s"
            % (sname, r["ms_mean"], r["tflops"], r["pct_peak"], r["kernel_ms_mean"],
               100.0 * r["wait_fraction"],
               "  %d of %d runs differ from the first" % (rep["differ"], rep["runs"]) if rep else ""))
    det = {k: v for k, v in results.items() if k != "atomic"}
    best = max(det, key=lambda k: det[k]["tflops"])
    atomic = results.get("atomic")
    for k, v in results.items():
        v["det_over_atomic"] = (v["tflops"] / atomic["tflops"]) if atomic else None
    bestr = det[best]
    sched_out = {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                 for k, v in results.items()}
    mask = 1 if cfg["causal"] else 0
    parts = bestr["head_parts"]
    roof = roofline(cfg, T, fl, bestr["kernel_ms_mean"], best, committed_traffic(name, best), parts)
    table_out = None
    if tinfo is not None:
        table_out = {k: tinfo[k] for k in ("family", "items", "per_head", "makespan", "same_as")}
    bit_identical = (all(v["repro"]["differ"] == 0 for v in det.values())
                     if all("repro" in v for v in det.values()) else None)
    names = {v: k for k, v in dash.SCHEDULES.items()}
    names[dash.TABLE] = "table"   # AUTO may resolve to the searched table
    auto = names[dash.dash_attn_bwd_auto_schedule(B, Hq, Hkv, S, D, 1 if cfg["causal"] else 0)]
    shape = {"B": B, "S": S, "Hq": Hq, "Hkv": Hkv, "D": D,
             "mask": "causal" if cfg["causal"] else "full", "tile": T, "head_parts": parts}
    if not headline:
        del x, o, lse
        torch.cuda.empty_cache()
        return dict(shape, workload=cfg["desc"], best_schedule=best,
                    value=round(bestr["tflops"], 3), ms_per_step=round(bestr["ms_mean"], 4),
                    pct_peak=round(bestr["pct_peak"], 2),
                    det_over_atomic=round(bestr["det_over_atomic"], 4) if atomic else None,
                    schedules=sched_out, roofline=roof,
                    deterministic_bit_identical=bit_identical,
                    auto_schedule=auto, auto_is_measured_best=auto == best,
                    searched_table=table_out)

    line = {
        "metric": "deterministic attn-bwd TFLOP/s on 1 MI355X; % bf16 MFMA peak; ratio vs atomic dQ",
        "value": round(bestr["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(bestr["ms_mean"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: N(0,1) fp32 cast to bf16, seeds 1000-1003; O and LSE from dash_attn_fwd",
        "config": dict({"workload": cfg["desc"]}, **shape, best_schedule=best),
        "pct_peak": round(bestr["pct_peak"], 2),
        "det_over_atomic": round(bestr["det_over_atomic"], 4) if atomic else None,
        "schedules": sched_out,
        "roofline": roof,
        "searched_table": table_out,
    }
    # run-to-run bit identity at this size, in this launch configuration:
    # every deterministic schedule must reproduce its first output exactly
    # (the atomic reference's count of differing runs is the positive control)
    if bit_identical is not None:
        line["deterministic_bit_identical"] = bit_identical
    # the shader clock the persistent kernel ran at (measured inside the last
    # timed launch of the best schedule), beside the peak fraction, which is
    # priced at the published 2.4 GHz
    clk = bestr.get("sclk_mhz")
    if clk:
        line["sclk_mhz"] = clk
        line["pct_peak_at_measured_clock"] = round(bestr["pct_peak"] * 2400.0 / clk, 2)
    # the whole attention layer: forward (O, LSE) then the backward step
    # above; forward FLOPs are 4*B*Hq*S^2*D (halved for a causal mask)
    fwd_ms = time_forward(dash, x, cfg, args.steps, args.warmup)
    layer_ms = fwd_ms + bestr["ms_mean"]
    line["layer"] = {"fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bestr["ms_mean"], 4),
                     "ms": round(layer_ms, 4),
                     "tflops": round(1.4 * fl / (layer_ms * 1e-3) / 1e12, 3),
                     "fwd_tflops": round(0.4 * fl / (fwd_ms * 1e-3) / 1e12, 3)}
    # the schedule the simulator picks for this shape on this device (AUTO)
    line["auto_schedule"] = auto
    line["auto_is_measured_best"] = auto == best
    del x, o, lse
    torch.cuda.empty_cache()
    return line


if __name__ == "__main__":
    main()

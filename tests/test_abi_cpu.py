"""Host-side tests of libdash_attn.so (no GPU needed).

* every symbol declared in include/dash_attn.h is exported;
* argument validation returns its documented status before any device call;
* the library's closed-form schedules equal the oracle's task lists and
  lockstep ranks;
* the library's C++ DAG simulator equals the oracle simulator.
"""

import ctypes
import os
import re
import sys

import pytest

import scheduling_persistent_attn_amd as dash
from oracle import dag
from oracle import schedule as sch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dash_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dash_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = declared_functions()
    assert len(names) >= 10
    L = dash.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(dash.SYMBOLS)


def test_watchdog_setting_validation():
    # out-of-range limits are refused and leave the setting alone; the
    # setter touches no device
    for bad in (-1.0, float("nan"), float("inf"), 3600.5):
        with pytest.raises(dash.DashError) as e:
            dash.dash_attn_set_watchdog(bad)
        assert e.value.status == dash.DASH_ERR_SHAPE
    for ok in (0.0, 1e-6, 3600.0, 2.0):
        dash.dash_attn_set_watchdog(ok)


def test_wait_stats_needs_a_workspace():
    # both refusals happen before any device access
    n = ctypes.c_longlong()
    L = dash.lib()
    assert L.dash_attn_bwd_wait_stats(None, 1 << 20, None, ctypes.byref(n), None, None) \
        == dash.DASH_ERR_NULL
    buf = ctypes.create_string_buffer(256)
    assert L.dash_attn_bwd_wait_stats(ctypes.cast(buf, ctypes.c_void_p), 256, None,
                                      ctypes.byref(n), None, None) == dash.DASH_ERR_WORKSPACE


def test_status_strings():
    for s in range(10):
        assert dash.dash_status_string(s)
    assert "unknown" in dash.dash_status_string(99)


def test_tile_and_workspace_size():
    assert dash.dash_attn_tile_size(256, 64) == 64
    assert dash.dash_attn_tile_size(4096, 64) == 256
    assert dash.dash_attn_tile_size(513, 64) == 256
    assert dash.dash_attn_tile_size(512, 128) == 128
    assert dash.dash_attn_tile_size(513, 128) == 256
    assert dash.dash_attn_tile_size(4096, 128) == 256
    assert dash.dash_attn_tile_size(100, 96) == 0
    # one turn counter per slice a wave reduces per pass: 32 x 32 for tiles of
    # 64 and 128, 32 x 16 for 256 (both head dims)
    for (B, Hq, Hkv, S, D, T, per_tile) in ((4, 32, 8, 4096, 128, 256, 256 * 128 // 512),
                                            (2, 8, 4, 512, 128, 128, 128 * 128 // 1024),
                                            (2, 24, 24, 4096, 64, 256, 256 * 64 // 512)):
        N = (S + T - 1) // T
        n = dash.dash_attn_bwd_workspace_size(B, Hq, Hkv, S, D, 1, 2)
        rows = B * Hq * N * T
        # control words, wait counters (4096 x 4 uint64), turn counters, the two
        # per-row arrays and the fp32 dQ partial sums
        want = 256 + 4096 * 32 + B * Hq * N * per_tile * 4 + 2 * rows * 4 + rows * D * 4
        assert want <= n <= want + 5 * 256, (S, D)
    # ragged S rounds up to whole tiles
    assert dash.dash_attn_bwd_workspace_size(1, 2, 2, 300, 64, 0, 0) > 0
    # invalid
    assert dash.dash_attn_bwd_workspace_size(1, 3, 2, 256, 64, 0, 0) == 0
    assert dash.dash_attn_bwd_workspace_size(1, 2, 2, 256, 80, 0, 0) == 0
    assert dash.dash_attn_bwd_workspace_size(1, 2, 2, 256, 64, 2, 0) == 0
    assert dash.dash_attn_bwd_workspace_size(1, 2, 2, 256, 64, 0, 9) == 0


def _bwd(**kw):
    args = dict(q=1 << 12, k=1 << 12, v=1 << 12, o=1 << 12, do=1 << 12, lse=1 << 12,
                dq=1 << 12, dk=1 << 12, dv=1 << 12, B=1, Hq=2, Hkv=2, S=256, D=64,
                mask=0, sched=0, ws=1 << 12, wsb=1 << 30)
    args.update(kw)
    p = ctypes.c_void_p
    return dash.lib().dash_attn_bwd(
        p(args["q"]), p(args["k"]), p(args["v"]), p(args["o"]), p(args["do"]),
        p(args["lse"]), p(args["dq"]), p(args["dk"]), p(args["dv"]),
        args["B"], args["Hq"], args["Hkv"], args["S"], args["D"], args["mask"],
        args["sched"], p(args["ws"]), args["wsb"], None)


def test_bwd_validation_before_device():
    assert _bwd(q=None) == dash.DASH_ERR_NULL
    assert _bwd(dv=None) == dash.DASH_ERR_NULL
    assert _bwd(Hq=3, Hkv=2) == dash.DASH_ERR_SHAPE
    assert _bwd(B=-1) == dash.DASH_ERR_SHAPE
    assert _bwd(D=96) == dash.DASH_ERR_UNSUPPORTED
    assert _bwd(mask=3) == dash.DASH_ERR_SCHEDULE_MASK
    assert _bwd(sched=7) == dash.DASH_ERR_SCHEDULE_MASK
    # symmetric shift needs a causal mask and an even tile count
    assert _bwd(sched=3, mask=0) == dash.DASH_ERR_SCHEDULE_MASK
    assert _bwd(sched=3, mask=1, S=192) == dash.DASH_ERR_SCHEDULE_MASK   # N = 3
    assert _bwd(q=(1 << 12) + 2) == dash.DASH_ERR_SHAPE                  # misaligned
    assert _bwd(ws=None) == dash.DASH_ERR_WORKSPACE
    assert _bwd(wsb=16) == dash.DASH_ERR_WORKSPACE
    assert _bwd(ws=(1 << 12) + 64) == dash.DASH_ERR_WORKSPACE            # misaligned
    # sizes whose element offsets do not fit 32 bits are refused
    assert _bwd(B=64, S=65536, Hq=8, Hkv=8, D=128) == dash.DASH_ERR_UNSUPPORTED
    # empty problems are a no-op
    assert _bwd(S=0, q=None, ws=None) == dash.DASH_OK
    assert _bwd(B=0, q=None, ws=None) == dash.DASH_OK


def test_fwd_validation_before_device():
    p = ctypes.c_void_p
    f = dash.lib().dash_attn_fwd
    a = p(1 << 12)
    assert f(None, a, a, a, a, 1, 2, 2, 256, 64, 0, None) == dash.DASH_ERR_NULL
    assert f(a, a, a, a, a, 1, 3, 2, 256, 64, 0, None) == dash.DASH_ERR_SHAPE
    assert f(a, a, a, a, a, 1, 2, 2, 256, 72, 0, None) == dash.DASH_ERR_UNSUPPORTED
    assert f(a, a, a, a, a, 1, 2, 2, 256, 64, 5, None) == dash.DASH_ERR_SCHEDULE_MASK
    assert f(None, None, None, None, None, 1, 2, 2, 0, 64, 0, None) == dash.DASH_OK
    # 32-bit element offsets and the batch grid dimension bound the problem
    assert f(a, a, a, a, a, 1, 128, 8, 1 << 17, 128, 1, None) == dash.DASH_ERR_UNSUPPORTED
    assert f(a, a, a, a, a, 65536, 1, 1, 1, 64, 0, None) == dash.DASH_ERR_UNSUPPORTED


COMBOS = [(s, m) for s in (sch.NAIVE, sch.DESCENDING_Q, sch.SHIFT, sch.ATOMIC)
          for m in (sch.FULL, sch.CAUSAL)] + [(sch.SYMMETRIC_SHIFT, sch.CAUSAL)]


@pytest.mark.parametrize("s,m", COMBOS)
@pytest.mark.parametrize("N", [1, 2, 3, 4, 7, 8, 32])
@pytest.mark.parametrize("G", [1, 2, 7])
def test_library_schedule_equals_oracle(s, m, N, G):
    if s == sch.SYMMETRIC_SHIFT and N % 2:
        assert dash.dash_schedule_num_items(m, s, N) == -1
        return
    its = sch.items(s, m, N, G)
    rk = sch.ranks(s, m, N, G)
    assert dash.dash_schedule_num_items(m, s, N) == len(its)
    for n, it in enumerate(its):
        assert dash.dash_schedule_item_len(m, s, N, G, n) == len(it)
        for step, (g, i, j) in enumerate(it):
            got = dash.dash_schedule_task(m, s, N, G, n, step)
            assert got == (g, i, j, rk[(g, i, j)]), (n, step)


def test_schedule_out_of_range():
    assert dash.dash_schedule_num_items(0, 3, 4) == -1
    assert dash.dash_schedule_item_len(1, 0, 4, 1, 4) == -1
    with pytest.raises(ValueError):
        dash.dash_schedule_task(1, 0, 4, 1, 0, 4)


SIM_CASES = [
    (sch.NAIVE, sch.FULL), (sch.DESCENDING_Q, sch.FULL), (sch.SHIFT, sch.FULL),
    (sch.NAIVE, sch.CAUSAL), (sch.DESCENDING_Q, sch.CAUSAL), (sch.SHIFT, sch.CAUSAL),
    (sch.SYMMETRIC_SHIFT, sch.CAUSAL),
]


@pytest.mark.parametrize("s,m", SIM_CASES)
@pytest.mark.parametrize("N,G,groups,P", [(4, 1, 1, 4), (4, 2, 3, 5), (6, 3, 2, 8),
                                          (8, 1, 4, 6), (2, 4, 5, 3)])
@pytest.mark.parametrize("dispatch", [0, 1])
def test_library_simulator_equals_oracle(s, m, N, G, groups, P, dispatch):
    c, cd, r = 5.0, 3.0, 1.0
    ref = dag.simulate(s, m, N, G=G, groups=groups, P=P,
                       dispatch="dynamic" if dispatch else "static",
                       c=c, c_diag=cd, r=r)
    got = dash.dash_sim_run(m, s, N, G, groups, P, dispatch, c, cd, r)
    assert bool(got["deadlock"]) == ref["deadlock"]
    assert got["order_edges"] == ref["order_edges"]
    assert got["total_work"] == ref["total_work"]
    assert got["base_makespan"] == ref["base_makespan"]
    if not ref["deadlock"]:
        assert got["makespan"] == ref["makespan"]
        assert got["violations"] == ref["violations"]
        assert got["max_deficit"] == ref["max_deficit"]
        assert abs(got["efficiency"] - ref["efficiency"]) < 1e-12


def test_simulator_closed_forms_large():
    # one group, one worker per item: the hand-derived critical paths
    N, c, r = 128, 4.0, 1.0
    got = dash.dash_sim_run(sch.FULL, sch.SHIFT, N, 1, 1, N, 0, c, c, r)
    assert got["makespan"] == N * (c + r) and got["violations"] == 0
    got = dash.dash_sim_run(sch.FULL, sch.NAIVE, N, 1, 1, N, 0, c, c, r)
    assert got["makespan"] == N * (c + r) + (N - 1) * r
    assert got["violations"] == N * (N - 1)
    got = dash.dash_sim_run(sch.CAUSAL, sch.SYMMETRIC_SHIFT, N, 1, 1, N // 2, 0, c, c, r)
    assert got["makespan"] == (N + 1) * (c + r) and got["violations"] == 0
    got = dash.dash_sim_run(sch.CAUSAL, sch.DESCENDING_Q, N, 1, 1, N, 0, c, c, r)
    assert got["makespan"] == N * (c + r) and got["max_deficit"] == r


def test_simulator_rejects():
    with pytest.raises(dash.DashError):
        dash.dash_sim_run(sch.FULL, sch.SYMMETRIC_SHIFT, 4)
    with pytest.raises(dash.DashError):
        dash.dash_sim_run(sch.FULL, sch.SHIFT, 0)


def test_phase_validation_before_device():
    p = ctypes.c_void_p
    L = dash.lib()
    a = p(1 << 12)
    # prepare: o, dout, lse are required; q/k/v/dq/dk/dv are not read
    assert L.dash_attn_bwd_prepare(None, a, a, 1, 2, 2, 256, 64, 0, 0, a, 1 << 30,
                                   None) == dash.DASH_ERR_NULL
    assert L.dash_attn_bwd_prepare(a, a, a, 1, 3, 2, 256, 64, 0, 0, a, 1 << 30,
                                   None) == dash.DASH_ERR_SHAPE
    assert L.dash_attn_bwd_prepare(a, a, a, 1, 2, 2, 256, 64, 0, 0, a, 16,
                                   None) == dash.DASH_ERR_WORKSPACE
    assert L.dash_attn_bwd_prepare(a, a, a, 1, 2, 2, 256, 64, 0, 3, a, 1 << 30,
                                   None) == dash.DASH_ERR_SCHEDULE_MASK
    assert L.dash_attn_bwd_prepare(None, None, None, 1, 2, 2, 0, 64, 0, 0, None, 0,
                                   None) == dash.DASH_OK
    # run: q, k, v, dout, dq, dk, dv are required; o and lse are not read
    args = [a] * 7 + [1, 2, 2, 256, 64, 0, 0, a, 1 << 30, None]
    for n in range(7):
        bad = list(args)
        bad[n] = None
        assert L.dash_attn_bwd_run(*bad) == dash.DASH_ERR_NULL, n
    bad = list(args)
    bad[11] = 80
    assert L.dash_attn_bwd_run(*bad) == dash.DASH_ERR_UNSUPPORTED
    bad = list(args)
    bad[14] = None
    assert L.dash_attn_bwd_run(*bad) == dash.DASH_ERR_WORKSPACE


SELECT_CASES = [
    # mask, N, G, groups, P, dispatch, c, c_diag, r
    (sch.FULL, 4, 1, 1, 4, 0, 4.0, 4.0, 1.0),
    (sch.FULL, 4, 1, 2, 3, 1, 4.0, 4.0, 1.0),     # shift cannot keep a group resident
    (sch.FULL, 6, 2, 2, 12, 1, 5.0, 5.0, 0.5),
    (sch.CAUSAL, 4, 1, 1, 2, 0, 4.0, 2.0, 1.0),
    (sch.CAUSAL, 6, 3, 2, 8, 1, 5.0, 3.0, 1.0),
    (sch.CAUSAL, 5, 2, 3, 6, 1, 1.0, 1.0, 0.1),  # odd N: no symmetric shift
    (sch.CAUSAL, 8, 1, 4, 3, 1, 1.0, 1.0, 0.1),
    (sch.CAUSAL, 8, 4, 2, 16, 1, 1.0, 1.0, 0.1),
]


@pytest.mark.parametrize("case", SELECT_CASES)
def test_library_selection_equals_oracle(case):
    m, N, G, groups, P, disp, c, cd, r = case
    ref = dag.select(m, N, G=G, groups=groups, P=P, dispatch="dynamic" if disp else "static",
                     c=c, c_diag=cd, r=r)
    if ref is None:
        with pytest.raises(dash.DashError):
            dash.dash_sim_select(m, N, G, groups, P, disp, c, cd, r)
        return
    sched, res = dash.dash_sim_select(m, N, G, groups, P, disp, c, cd, r)
    assert sched == ref[0]
    assert res["makespan"] == ref[1]["makespan"]


def test_selection_closed_forms():
    # one group, one worker per chain, full mask: shift reaches N(c + r), the
    # naive order pays (N - 1) r more (the critical paths pinned above)
    N, c, r = 16, 4.0, 1.0
    sched, res = dash.dash_sim_select(sch.FULL, N, 1, 1, N, 0, c, c, r)
    assert sched == sch.SHIFT and res["makespan"] == N * (c + r)
    # causal, even N, N/2 workers: the symmetric pairs finish in (N + 1)(c + r),
    # against N (c + r) + (N - 1) r at least for one-chain-per-worker orders
    sched, res = dash.dash_sim_select(sch.CAUSAL, N, 1, 1, N // 2, 0, c, c, r)
    assert sched == sch.SYMMETRIC_SHIFT and res["makespan"] == (N + 1) * (c + r)
    # fewer workers than a group's chains: the shift family deadlocks and is
    # never chosen
    sched, _ = dash.dash_sim_select(sch.FULL, N, 1, 1, N // 2, 1, c, c, r)
    assert sched in (sch.NAIVE, sch.DESCENDING_Q)


def test_auto_schedule_arguments():
    L = dash.lib()
    # AUTO: the closed forms' workspace and room for the largest table of the
    # shape (N = 4 tiles of 64 keys, G = 1: 8 header words, 6 offset words
    # and 2 words for each of the 10 causal tasks), rounded to 256 bytes
    words = 8 + ((1 * 4 + 2) & ~1) + 2 * 10
    assert dash.dash_attn_bwd_workspace_size(1, 2, 2, 256, 64, 1, dash.AUTO) == \
        dash.dash_attn_bwd_workspace_size(1, 2, 2, 256, 64, 1, dash.NAIVE) + ((4 * words + 255) & ~255)
    assert dash.dash_attn_bwd_workspace_size(1, 2, 2, 256, 64, 1, 7) == 0
    assert dash.dash_attn_bwd_workspace_size(1, 2, 2, 256, 64, 1, dash.TABLE) == \
        dash.dash_attn_bwd_workspace_size(1, 2, 2, 256, 64, 1, dash.AUTO)
    assert L.dash_attn_bwd_auto_schedule(1, 3, 2, 256, 64, 1) == -dash.DASH_ERR_SHAPE
    assert L.dash_attn_bwd_auto_schedule(1, 2, 2, 256, 64, 2) == -dash.DASH_ERR_SCHEDULE_MASK
    assert L.dash_attn_bwd_auto_schedule(0, 2, 2, 256, 64, 1) == dash.NAIVE  # empty
    # argument errors come before the device is needed to resolve AUTO
    assert _bwd(sched=dash.AUTO, q=None) == dash.DASH_ERR_NULL
    assert _bwd(sched=dash.AUTO, ws=None) == dash.DASH_ERR_WORKSPACE
    assert _bwd(sched=dash.AUTO, S=0, q=None, ws=None) == dash.DASH_OK


def test_sim_report_closed_forms(capsys):
    """bench.py --sim-report on the large workloads; two cases have closed
    forms.  dit_full at P = 256, r = 0, with 256-key tiles (N = 16): 48 groups
    x 16 chains of 16 unit tasks on 256 workers are 3 rounds of 16, so every
    schedule's critical path is 48.
    llama8b_causal, symmetric shift, P = 256, r = 0, with 256-key tiles (N =
    16): 32 groups x 8 pairs of 17 tasks for each of 4 query heads (68 per
    item) in one round: 68, with efficiency 1 and no Lemma 1 violation."""
    import json
    sys.path.insert(0, str(ROOT))
    import bench
    bench.sim_report()
    rows = [json.loads(l) for l in capsys.readouterr().out.splitlines() if l.startswith("{")]
    assert len(rows) == 84 + 24  # closed forms, then one searched table per case
    pick = {(r["workload"], r["P"], r["r_over_c"], r["schedule"]): r for r in rows}
    # the searched table is never longer than the best closed form of its case
    for (w, P, r, sname), row in pick.items():
        if sname != "table":
            continue
        assert not row["deadlock"]
        best = min(v["critical_path"] for (w2, P2, r2, s2), v in pick.items()
                   if (w2, P2, r2) == (w, P, r) and s2 != "table" and not v["deadlock"]
                   and v["head_parts"] == 1)
        assert row["critical_path"] <= best + 1e-9
    q = pick[("qwen7b_causal", 256, 0.1, "table")]
    assert q["family"][0] == dash.FAMILY_PACKED and q["per_head"]
    assert q["critical_path"] < pick[("qwen7b_causal", 256, 0.1, "symmetric_shift")]["critical_path"]
    for s in ("naive", "descending_q", "shift"):
        assert pick[("dit_full", 256, 0.0, s)]["critical_path"] == 48.0
    assert dash.dash_attn_tile_size(4096, 64) == 256
    sym = pick[("llama8b_causal", 256, 0.0, "symmetric_shift")]
    assert dash.dash_attn_tile_size(4096, 128) == 256
    assert sym["critical_path"] == 68.0 and sym["lemma1_violations"] == 0
    assert abs(sym["efficiency"] - 1.0) < 1e-12
    assert not any(r["deadlock"] for r in rows)


def test_library_schedule_equals_hand_written_g2_table():
    # the closed forms of the library against the hand-written G = 2, N = 4
    # table (step outer, head inner), independently of the oracle
    import json
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "schedules_n4_g2.json")))
    N, G = gold["N"], gold["G"]
    names = {"naive": 0, "descending": 1, "shift": 2, "symmetric": 3, "atomic": 4}
    for key, rows in gold["items"].items():
        name, mname = key.split("_")
        s, m = names[name], {"full": 0, "causal": 1}[mname]
        assert dash.dash_schedule_num_items(m, s, N) == len(rows), key
        for n, row in enumerate(rows):
            want = [tuple(int(v) for v in t.split(",")) for t in row.split()]
            assert dash.dash_schedule_item_len(m, s, N, G, n) == len(want), (key, n)
            got = [dash.dash_schedule_task(m, s, N, G, n, st) for st in range(len(want))]
            assert got == want, (key, n)


def test_binding_rejects_mismatched_tensors():
    # every tensor's shape is checked against (B, S, Hq, D), (B, S, Hkv, D)
    # and (B, Hq, S) before the C ABI gets raw pointers; CPU tensors with the
    # right shapes are refused as not on a GPU
    import torch
    B, S, Hq, Hkv, D = 1, 8, 4, 2, 64
    bf = torch.bfloat16

    def mk(*shape, dtype=bf):
        return torch.zeros(shape, dtype=dtype)

    q, o, do, dq = (mk(B, S, Hq, D) for _ in range(4))
    k, v, dk, dv = (mk(B, S, Hkv, D) for _ in range(4))
    lse = mk(B, Hq, S, dtype=torch.float32)
    ws = torch.zeros(1 << 20, dtype=torch.uint8)
    bad = {"v": mk(B, S - 1, Hkv, D), "o": mk(B, S, Hq, D // 2), "dout": mk(B, S, Hkv, D),
           "dq": mk(B, S, Hq + 1, D), "dk": mk(B, S, Hq, D), "dv": mk(B, 2 * S, Hkv, D),
           "lse": mk(B, S, Hq, dtype=torch.float32)}
    args = dict(q=q, k=k, v=v, o=o, dout=do, lse=lse, dq=dq, dk=dk, dv=dv)
    for name, t in bad.items():
        a = dict(args)
        a[name] = t
        with pytest.raises(ValueError, match="shape"):
            dash.dash_attn_bwd(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"],
                               a["dk"], a["dv"], 0, dash.SHIFT, ws)
    with pytest.raises(ValueError, match="shape"):
        dash.dash_attn_fwd(q, k, bad["v"], o, lse, 0)
    with pytest.raises(ValueError, match="shape"):
        dash.dash_attn_fwd(q, k, v, o, bad["lse"], 0)
    with pytest.raises(ValueError, match="shape"):
        dash.dash_attn_bwd_run(q, k, v, do, dq, bad["dk"], dv, 0, dash.SHIFT, ws)
    with pytest.raises(ValueError, match="shape"):
        dash.dash_attn_bwd_prepare(o, bad["dout"], lse, (B, S, Hq, D), Hkv, 0, dash.SHIFT, ws)
    with pytest.raises(ValueError, match="GPU"):
        dash.dash_attn_bwd(q, k, v, o, do, lse, dq, dk, dv, 0, dash.SHIFT, ws)
    with pytest.raises(ValueError, match="GPU"):
        dash.dash_attn_fwd(q, k, v, o, lse, 0)


def test_not_prepared_status():
    assert dash.DASH_ERR_NOT_PREPARED == 8
    assert "not prepared" in dash.dash_status_string(8)


def test_head_parts_rule():
    # with 256-key tiles, the smallest divisor of G giving at least 256 items
    hp = dash.dash_attn_bwd_head_parts
    # the 7B-Qwen-shaped causal layer: 4 groups x 32 symmetric pairs = 128
    # items, so its 7 heads go to 7 parts; its chains (64 per group) suffice
    assert hp(1, 28, 4, 16384, 128, 1, dash.SYMMETRIC_SHIFT) == 7
    assert hp(1, 28, 4, 16384, 128, 1, dash.SHIFT) == 1
    assert hp(1, 28, 4, 16384, 128, 1, dash.AUTO) == 7
    # the 8B-Llama-shaped layer: 32 groups x 8 pairs = 256 items, no split
    assert hp(4, 32, 8, 4096, 128, 1, dash.SYMMETRIC_SHIFT) == 1
    # small shapes take every divisor up to G
    assert hp(1, 4, 2, 1024, 128, 1, dash.NAIVE) == 2
    assert hp(1, 6, 1, 1024, 128, 0, dash.SHIFT) == 6
    # 256-key tiles at head dim 64 split the same way
    assert hp(1, 8, 2, 4096, 64, 1, dash.NAIVE) == 4
    # 64- and 128-key tiles and single-head groups are never split
    assert hp(1, 8, 2, 512, 128, 1, dash.NAIVE) == 1
    assert hp(1, 8, 2, 512, 64, 1, dash.NAIVE) == 1
    assert hp(1, 8, 8, 4096, 128, 1, dash.NAIVE) == 1
    assert hp(1, 3, 2, 4096, 128, 1, dash.NAIVE) == 0  # invalid


@pytest.mark.parametrize("s,m", COMBOS)
@pytest.mark.parametrize("N,G,parts", [(4, 2, 2), (5, 6, 3), (8, 7, 7)])
def test_library_split_items_equal_oracle(s, m, N, G, parts):
    # the kernels take item `local` of a group as part local // base of base
    # item local % base, evaluated by the closed forms with G / parts heads
    if s == sch.SYMMETRIC_SHIFT and N % 2:
        return
    its = sch.items(s, m, N, G, parts)
    rk = sch.ranks(s, m, N, G)
    Gp = G // parts
    base = dash.dash_schedule_num_items(m, s, N)
    assert len(its) == base * parts
    for n, it in enumerate(its):
        k, b = divmod(n, base)
        assert dash.dash_schedule_item_len(m, s, N, Gp, b) == len(it)
        for step, (g, i, j) in enumerate(it):
            gl, il, jl, rl = dash.dash_schedule_task(m, s, N, Gp, b, step)
            assert (k * Gp + gl, il, jl, rl) == (g, i, j, rk[(g, i, j)]), (n, step)


def test_bench_searched_table_row(monkeypatch):
    """bench.py's table row on a 256-workgroup grid (the MI355X's, set here
    since no device is present): the search returns exactly a closed form
    that splits no heads for four workloads, which the line names instead of
    timing it twice, and the packed per-head table for the 16k causal layer
    with seven heads per KV head."""
    sys.path.insert(0, str(ROOT))
    import bench
    monkeypatch.setattr(dash, "dash_attn_bwd_grid_size", lambda S, D, mask: 256)
    want = {"long_full": "shift", "llama8b_causal": "symmetric_shift", "dit_full": "shift",
            "qwen7b_causal": None}
    for name, same in want.items():
        t = bench.searched_table(dash, bench.CONFIGS[name])
        assert t["same_as"] == same, (name, t["family"])
        if name == "qwen7b_causal":
            assert t["per_head"] and t["family"][0] == dash.FAMILY_PACKED
            assert t["items"] == 64
        else:
            assert not t["per_head"]


def test_sim_workers_beyond_the_items():
    # more workers than items: the same result as one worker per item, for
    # closed forms and tables, and no state kept for the idle workers
    for m, s, N, G, groups in ((sch.CAUSAL, dash.SYMMETRIC_SHIFT, 8, 2, 3), (sch.FULL, dash.SHIFT, 6, 1, 2)):
        items = groups * dash.dash_schedule_num_items(m, s, N)
        for disp in (0, 1):
            a = dash.dash_sim_run(m, s, N, G, groups, items, disp, 1.0, 0.5, 0.125)
            b = dash.dash_sim_run(m, s, N, G, groups, 1 << 30, disp, 1.0, 0.5, 0.125)
            assert a == b
    offs, tasks = dash.dash_schedule_table_closed_form(sch.CAUSAL, dash.SHIFT, 8, 2)
    a = dash.dash_sim_table(sch.CAUSAL, 8, 2, 3, 24, 1, offs, tasks, 1.0, 0.5, 0.125)
    b = dash.dash_sim_table(sch.CAUSAL, 8, 2, 3, 1 << 30, 1, offs, tasks, 1.0, 0.5, 0.125)
    assert a == b

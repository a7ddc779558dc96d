"""The task trace of the debug build against the schedule closed forms.

libdash_attn_trace.so is the library compiled with DASH_TASK_TRACE: thread 0
of each persistent workgroup records every task it runs -- item, step, query
head, key/value tile, query tile, rank, workgroup and start/end wall clock --
in a region of the workspace.  For every schedule on shapes that use each
kernel (128-key tiles, 256-key tiles, 256-key tiles with split query heads),
the test checks that the device ran exactly the task lists the schedule
defines (the oracle's items, in dispatch order, and the library's closed forms
for the ranks), that each item ran whole on one workgroup in step order, and
that each dQ tile's contributions started in an order consistent with its
ranks at the hand-off points the trace can see (a contribution's task cannot
end before its predecessor's task started).  The trace build's gradients are
also checked bit for bit against the product build (the trace writes touch
nothing else).
"""

import ctypes
import sys

import numpy as np
import pytest
import torch

import scheduling_persistent_attn_amd as dash
from oracle import schedule as sch

sys.path.insert(0, __file__.rsplit("/", 1)[0])
import gpu_util as gu  # noqa: E402

pytestmark = pytest.mark.gpu

CASES = [
    # B, S, Hq, Hkv, D, causal
    (1, 512, 4, 2, 64, True),      # 64-key tiles (D = 64, S <= 512): the 128-key-tile kernel
    (2, 1024, 4, 4, 64, False),    # 128-key tiles
    (1, 2048, 4, 2, 128, True),    # 256-key tiles, heads split into parts
    (1, 2048, 16, 16, 128, False), # 256-key tiles, one head per group
]


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _run(L, x, o, lse, causal, sched, ws):
    B, S, Hq, D = x["q"].shape
    Hkv = x["k"].shape[2]
    dq, dk, dv = (torch.empty_like(x[k]) for k in ("q", "k", "v"))
    st = L.dash_attn_bwd(_ptr(x["q"]), _ptr(x["k"]), _ptr(x["v"]), _ptr(o), _ptr(x["do"]), _ptr(lse),
                         _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv, S, D, int(causal), int(sched),
                         _ptr(ws), ws.numel(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, st
    assert L.dash_attn_bwd_check(_ptr(ws), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    return dq, dk, dv


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dS%dH%d-%dD%d%s" % (
    c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "f"))
def test_trace_equals_schedule(case):
    B, S, Hq, Hkv, D, causal = case
    mask = int(causal)
    T = dash.dash_attn_tile_size(S, D)
    N = (S + T - 1) // T
    G = Hq // Hkv
    L = dash.trace_lib()
    x = gu.gpu_inputs(B, S, Hq, Hkv, D, seed=3900)
    o, lse = gu.run_forward(x, causal)
    scheds = [dash.NAIVE, dash.DESCENDING_Q, dash.SHIFT, dash.ATOMIC]
    if causal and N % 2 == 0:
        scheds.append(dash.SYMMETRIC_SHIFT)
    for sched in scheds:
        print("trace", case, "schedule", sched, flush=True)
        n = L.dash_attn_bwd_workspace_size(B, Hq, Hkv, S, D, mask, sched)
        ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
        got = _run(L, x, o, lse, causal, sched, ws)
        ref = gu.run_backward(x, o, lse, causal, sched)
        if sched != dash.ATOMIC:
            for a, b in zip(got, ref):
                assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        parts = dash.dash_attn_bwd_head_parts(B, Hq, Hkv, S, D, mask, sched)
        Gp = G // parts
        its = sch.items(sched, mask, N, G, parts)
        rk = sch.ranks(sched, mask, N, G)
        tlen = Gp * (N + 1 if (sched == dash.SYMMETRIC_SHIFT or (sched == dash.ATOMIC and causal and N % 2 == 0))
                     else N)
        n_items = B * Hkv * len(its)
        # the trace is the workspace's last region: record item * tlen + step,
        # 8 int64 each, then padding to a multiple of 256 bytes
        nrec = n_items * tlen
        region = (nrec * 64 + 255) // 256 * 256
        start = (ws.numel() - region) // 8
        rec = ws.view(torch.int64)[start:start + nrec * 8].cpu().numpy().reshape(nrec, 8)
        recs = {}
        for r in rec:
            if r[3] == 0:
                continue  # a step past the end of a shorter item
            item, step = int(r[0]) & 0xffffffff, int(r[0]) >> 32
            pk = int(r[1])
            recs[(item, step)] = ((pk & 0xffff, (pk >> 16) & 0xffff, (pk >> 32) & 0xffff, (pk >> 48) & 0xffff),
                                  int(r[2]), int(r[3]), int(r[4]))
        want = 0
        for grp in range(B * Hkv):
            for n_it, it in enumerate(its):
                item = grp * len(its) + n_it
                wgs = set()
                last_end = 0
                for step, (g, i, j) in enumerate(it):
                    assert (item, step) in recs, (sched, item, step)
                    (tg, ti, tj, tr), wg, t0, t1 = recs[(item, step)]
                    assert (tg, ti, tj) == (g, i, j), (sched, item, step, (tg, ti, tj), (g, i, j))
                    if sched != dash.ATOMIC:
                        assert tr == rk[(g, i, j)], (sched, item, step)
                    assert t1 >= t0 >= last_end  # steps run in order, one after another
                    last_end = t1
                    wgs.add(wg)
                    want += 1
                assert len(wgs) == 1, (sched, item)  # a whole item on one workgroup
        assert len(recs) == want
        if sched != dash.ATOMIC:
            # a contribution of rank r + 1 to a dQ tile cannot finish its task
            # before the rank r contribution's task has started
            by_tile = {}
            for (item, step), ((g, i, j, r), wg, t0, t1) in recs.items():
                grp = item // len(its)
                by_tile.setdefault((grp, g, j), {})[r] = (t0, t1)
            for tile, d in by_tile.items():
                for r in range(1, len(d)):
                    assert d[r][1] >= d[r - 1][0], (sched, tile, r)
        del ws

"""Python binding of libdash_attn.so (deterministic attention backward, gfx950).

Argument marshalling only: every step of the computation runs in the HIP
library.  The names follow the C ABI in include/dash_attn.h.  PyTorch provides
device memory and streams.  If the library is missing the binding raises; it
has no fallback.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdash_attn.so")
# the debug build: the same library with a per-task trace in the workspace
TRACE_LIB_PATH = os.path.join(HERE, "libdash_attn_trace.so")

MASK_FULL, MASK_CAUSAL = 0, 1
NAIVE, DESCENDING_Q, SHIFT, SYMMETRIC_SHIFT, ATOMIC, AUTO, TABLE = 0, 1, 2, 3, 4, 5, 6
SCHEDULES = {"naive": NAIVE, "descending_q": DESCENDING_Q, "shift": SHIFT,
             "symmetric_shift": SYMMETRIC_SHIFT, "atomic": ATOMIC}
DETERMINISTIC = (NAIVE, DESCENDING_Q, SHIFT, SYMMETRIC_SHIFT)

DASH_OK = 0
DASH_ERR_NULL = 1
DASH_ERR_SHAPE = 2
DASH_ERR_UNSUPPORTED = 3
DASH_ERR_SCHEDULE_MASK = 4
DASH_ERR_WORKSPACE = 5
DASH_ERR_HIP = 6
DASH_ERR_TIMEOUT = 7
DASH_ERR_NOT_PREPARED = 8
DASH_ERR_TABLE = 9

# family kinds of dash_schedule_search
FAMILY_SYMMETRIC, FAMILY_SHIFT, FAMILY_DESCENDING, FAMILY_ASCENDING, FAMILY_PACKED = 0, 1, 2, 3, 4

SYMBOLS = (
    "dash_attn_tile_size", "dash_attn_bwd_workspace_size", "dash_attn_fwd",
    "dash_attn_bwd", "dash_attn_bwd_prepare", "dash_attn_bwd_run", "dash_attn_bwd_check", "dash_status_string",
    "dash_attn_bwd_grid_size", "dash_schedule_num_items",
    "dash_schedule_item_len", "dash_schedule_task", "dash_sim_run", "dash_sim_select",
    "dash_attn_bwd_auto_schedule", "dash_attn_bwd_auto_schedule_on", "dash_attn_set_watchdog", "dash_attn_bwd_wait_stats",
    "dash_attn_bwd_noalloc", "dash_attn_bwd_head_parts",
    "dash_schedule_table_tasks", "dash_schedule_table_closed_form", "dash_schedule_table_family",
    "dash_schedule_table_check",
    "dash_schedule_table_pack", "dash_sim_table", "dash_schedule_search", "dash_attn_bwd_table",
    "dash_attn_bwd_table_run",
)

# bytes of the static device workspace behind dash_attn_bwd_noalloc
NOALLOC_WORKSPACE_BYTES = 64 << 20


class DashError(RuntimeError):
    def __init__(self, status, where=""):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, dash_status_string(status), status))


class SimResult(ctypes.Structure):
    _fields_ = [("makespan", ctypes.c_double), ("base_makespan", ctypes.c_double),
                ("total_work", ctypes.c_double), ("efficiency", ctypes.c_double),
                ("max_deficit", ctypes.c_double), ("order_edges", ctypes.c_longlong),
                ("violations", ctypes.c_longlong), ("deadlock", ctypes.c_int)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


_lib = None
_trace_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


def trace_lib():
    """The debug build (per-task trace in the workspace); raises if it has not
    been built.  Same entry points as lib()."""
    global _trace_lib
    if _trace_lib is None:
        _trace_lib = _load(TRACE_LIB_PATH)
    return _trace_lib


def _load(path):
    if not os.path.exists(path):
        raise RuntimeError("%s is not built (run `python -m scheduling_persistent_attn_amd.build`)"
                           % os.path.basename(path))
    L = ctypes.CDLL(path)
    i, p, sz, d = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_double
    L.dash_attn_tile_size.argtypes = [i, i]
    L.dash_attn_tile_size.restype = i
    L.dash_attn_bwd_workspace_size.argtypes = [i] * 7
    L.dash_attn_bwd_workspace_size.restype = sz
    L.dash_attn_fwd.argtypes = [p, p, p, p, p] + [i] * 6 + [p]
    L.dash_attn_fwd.restype = i
    L.dash_attn_bwd.argtypes = [p] * 9 + [i] * 7 + [p, sz, p]
    L.dash_attn_bwd.restype = i
    L.dash_attn_bwd_prepare.argtypes = [p] * 3 + [i] * 7 + [p, sz, p]
    L.dash_attn_bwd_prepare.restype = i
    L.dash_attn_bwd_run.argtypes = [p] * 7 + [i] * 7 + [p, sz, p]
    L.dash_attn_bwd_run.restype = i
    L.dash_attn_bwd_head_parts.argtypes = [i] * 7
    L.dash_attn_bwd_head_parts.restype = i
    L.dash_attn_bwd_noalloc.argtypes = [p] * 9 + [i] * 7 + [p]
    L.dash_attn_bwd_noalloc.restype = i
    L.dash_attn_bwd_check.argtypes = [p, p]
    L.dash_attn_bwd_check.restype = i
    L.dash_attn_set_watchdog.argtypes = [d]
    L.dash_attn_set_watchdog.restype = i
    L.dash_attn_bwd_wait_stats.argtypes = [p, sz, p, ctypes.POINTER(ctypes.c_longlong),
                                           ctypes.POINTER(ctypes.c_longlong),
                                           ctypes.POINTER(ctypes.c_double)]
    L.dash_attn_bwd_wait_stats.restype = i
    L.dash_status_string.argtypes = [i]
    L.dash_status_string.restype = ctypes.c_char_p
    L.dash_attn_bwd_grid_size.argtypes = [i, i, i]
    L.dash_attn_bwd_grid_size.restype = i
    L.dash_schedule_num_items.argtypes = [i, i, i]
    L.dash_schedule_num_items.restype = i
    L.dash_schedule_item_len.argtypes = [i] * 5
    L.dash_schedule_item_len.restype = i
    L.dash_schedule_task.argtypes = [i] * 6 + [ctypes.POINTER(i)] * 4
    L.dash_schedule_task.restype = i
    L.dash_sim_run.argtypes = [i] * 7 + [d, d, d, ctypes.POINTER(SimResult)]
    L.dash_sim_run.restype = i
    L.dash_sim_select.argtypes = [i] * 6 + [d, d, d, ctypes.POINTER(ctypes.c_int),
                                            ctypes.POINTER(SimResult)]
    L.dash_sim_select.restype = i
    L.dash_attn_bwd_auto_schedule.argtypes = [i] * 6
    L.dash_attn_bwd_auto_schedule.restype = i
    L.dash_attn_bwd_auto_schedule_on.argtypes = [i] * 7
    L.dash_attn_bwd_auto_schedule_on.restype = i
    ip = ctypes.POINTER(ctypes.c_int)
    L.dash_schedule_table_tasks.argtypes = [i, i, i]
    L.dash_schedule_table_tasks.restype = ctypes.c_longlong
    L.dash_schedule_table_closed_form.argtypes = [i] * 4 + [ip, ip, ip]
    L.dash_schedule_table_closed_form.restype = i
    L.dash_schedule_table_family.argtypes = [i] * 6 + [ip, ip, ip]
    L.dash_schedule_table_family.restype = i
    L.dash_schedule_table_check.argtypes = [i] * 6 + [ip, ip]
    L.dash_schedule_table_check.restype = i
    L.dash_schedule_table_pack.argtypes = [i] * 5 + [ip, ip, p, sz, ip]
    L.dash_schedule_table_pack.restype = sz
    L.dash_sim_table.argtypes = [i] * 6 + [d, d, d, i, ip, ip, ctypes.POINTER(SimResult)]
    L.dash_sim_table.restype = i
    L.dash_schedule_search.argtypes = [i] * 6 + [d, d, d, ip, ip, ip, ip, ctypes.POINTER(SimResult)]
    L.dash_schedule_search.restype = i
    L.dash_attn_bwd_table.argtypes = [p] * 9 + [i] * 6 + [p, sz, i, i, p, sz, p]
    L.dash_attn_bwd_table.restype = i
    L.dash_attn_bwd_table_run.argtypes = [p] * 7 + [i] * 6 + [p, sz, i, i, p, sz, p]
    L.dash_attn_bwd_table_run.restype = i
    return L


# --- plain wrappers (same names as the C ABI) -------------------------------

def dash_status_string(status):
    return lib().dash_status_string(int(status)).decode()


def dash_attn_tile_size(S, D):
    return lib().dash_attn_tile_size(S, D)


def dash_attn_bwd_workspace_size(B, Hq, Hkv, S, D, mask, schedule):
    return lib().dash_attn_bwd_workspace_size(B, Hq, Hkv, S, D, mask, schedule)


def dash_attn_bwd_head_parts(B, Hq, Hkv, S, D, mask, schedule):
    return lib().dash_attn_bwd_head_parts(B, Hq, Hkv, S, D, int(mask), int(schedule))


def dash_attn_bwd_grid_size(S, D, mask):
    return lib().dash_attn_bwd_grid_size(S, D, mask)


def dash_schedule_num_items(mask, schedule, N):
    return lib().dash_schedule_num_items(mask, schedule, N)


def dash_schedule_item_len(mask, schedule, N, G, item):
    return lib().dash_schedule_item_len(mask, schedule, N, G, item)


def dash_schedule_task(mask, schedule, N, G, item, step):
    g, i, j, r = (ctypes.c_int() for _ in range(4))
    st = lib().dash_schedule_task(mask, schedule, N, G, item, step,
                                  ctypes.byref(g), ctypes.byref(i), ctypes.byref(j),
                                  ctypes.byref(r))
    if st != 0:
        raise ValueError("task out of range")
    return g.value, i.value, j.value, r.value


def dash_sim_select(mask, N, G=1, groups=1, P=256, dispatch=1, c_full=1.0, c_diag=None, r=0.0):
    """(schedule, report) of the deterministic schedule with the shortest
    simulated critical path."""
    if c_diag is None:
        c_diag = c_full
    sched = ctypes.c_int(-1)
    out = SimResult()
    st = lib().dash_sim_select(mask, N, G, groups, P, dispatch, float(c_full), float(c_diag),
                               float(r), ctypes.byref(sched), ctypes.byref(out))
    if st != DASH_OK:
        raise DashError(st, "dash_sim_select")
    return sched.value, out.as_dict()


def dash_attn_bwd_auto_schedule(B, Hq, Hkv, S, D, mask):
    """The schedule AUTO runs for this shape on the current device."""
    r = lib().dash_attn_bwd_auto_schedule(B, Hq, Hkv, S, D, mask)
    if r < 0:
        raise DashError(-r, "dash_attn_bwd_auto_schedule")
    return r


def dash_attn_bwd_auto_schedule_on(B, Hq, Hkv, S, D, mask, grid):
    """The schedule AUTO picks for a device whose persistent grid is `grid`
    workgroups, computed on the host alone."""
    r = lib().dash_attn_bwd_auto_schedule_on(B, Hq, Hkv, S, D, mask, grid)
    if r < 0:
        raise DashError(-r, "dash_attn_bwd_auto_schedule_on")
    return r


def dash_sim_run(mask, schedule, N, G=1, groups=1, P=256, dispatch=1,
                 c_full=1.0, c_diag=None, r=0.0):
    if c_diag is None:
        c_diag = c_full
    out = SimResult()
    st = lib().dash_sim_run(mask, schedule, N, G, groups, P, dispatch,
                            float(c_full), float(c_diag), float(r), ctypes.byref(out))
    if st != DASH_OK:
        raise DashError(st, "dash_sim_run")
    return out.as_dict()


# --- task tables ---------------------------------------------------------------
# A table is (item_offsets, tasks): item_offsets a sequence of items + 1 ints,
# tasks an [n, 4] array of (g, i, j, rank) rows, as in include/dash_attn.h.

def _int_array(x, shape_tail=()):
    import numpy as np
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
    if shape_tail and (a.ndim != 1 + len(shape_tail) or a.shape[1:] != shape_tail):
        raise ValueError("expected an array of shape [n, %s]" % ", ".join(map(str, shape_tail)))
    return a


def _iptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int))


def _table_out(n_tasks, max_items):
    import numpy as np
    return np.zeros(max_items + 1, dtype=np.int32), np.zeros((n_tasks, 4), dtype=np.int32)


def dash_schedule_table_tasks(mask, N, G):
    return lib().dash_schedule_table_tasks(int(mask), int(N), int(G))


def dash_schedule_table_closed_form(mask, schedule, N, G):
    """A closed-form schedule as a table: (item_offsets, tasks)."""
    n = dash_schedule_table_tasks(mask, N, G)
    if n < 0:
        raise ValueError("invalid mask, N or G")
    offs, tasks = _table_out(n, N)
    items = ctypes.c_int()
    st = lib().dash_schedule_table_closed_form(int(mask), int(schedule), int(N), int(G),
                                               ctypes.byref(items), _iptr(offs), _iptr(tasks))
    if st != DASH_OK:
        raise DashError(st, "dash_schedule_table_closed_form")
    return offs[:items.value + 1], tasks


def dash_schedule_table_family(mask, N, G, kind, order, block):
    """One member of the searched family as a table: (item_offsets, tasks)."""
    if order == 1 and kind == FAMILY_PACKED:
        raise ValueError("the packed kind has order 0 only")
    n = dash_schedule_table_tasks(mask, N, G)
    if n < 0:
        raise ValueError("invalid mask, N or G")
    offs, tasks = _table_out(n, G * N)
    items = ctypes.c_int()
    st = lib().dash_schedule_table_family(int(mask), int(N), int(G), int(kind), int(order), int(block),
                                          ctypes.byref(items), _iptr(offs), _iptr(tasks))
    if st != DASH_OK:
        raise DashError(st, "dash_schedule_table_family")
    return offs[:items.value + 1], tasks


def dash_schedule_table_check(S, D, mask, G, P, item_offsets, tasks):
    """Status of the table's checks (DASH_OK or an error code)."""
    offs = _int_array(item_offsets)
    tk = _int_array(tasks, (4,))
    return lib().dash_schedule_table_check(int(S), int(D), int(mask), int(G), int(P),
                                           len(offs) - 1, _iptr(offs), _iptr(tk))


def dash_schedule_table_pack(S, D, mask, G, item_offsets, tasks):
    """The table's device form as bytes (raises DashError if invalid)."""
    offs = _int_array(item_offsets)
    tk = _int_array(tasks, (4,))
    st = ctypes.c_int()
    n = lib().dash_schedule_table_pack(int(S), int(D), int(mask), int(G), len(offs) - 1,
                                       _iptr(offs), _iptr(tk), None, 0, ctypes.byref(st))
    if st.value != DASH_OK:
        raise DashError(st.value, "dash_schedule_table_pack")
    buf = ctypes.create_string_buffer(n)
    lib().dash_schedule_table_pack(int(S), int(D), int(mask), int(G), len(offs) - 1,
                                   _iptr(offs), _iptr(tk), buf, n, ctypes.byref(st))
    if st.value != DASH_OK:
        raise DashError(st.value, "dash_schedule_table_pack")
    return buf.raw


def dash_sim_table(mask, N, G, groups, P, dispatch, item_offsets, tasks, c_full=1.0,
                   c_diag=None, r=0.0):
    if c_diag is None:
        c_diag = c_full
    offs = _int_array(item_offsets)
    tk = _int_array(tasks, (4,))
    out = SimResult()
    st = lib().dash_sim_table(int(mask), int(N), int(G), int(groups), int(P), int(dispatch),
                              float(c_full), float(c_diag), float(r), len(offs) - 1,
                              _iptr(offs), _iptr(tk), ctypes.byref(out))
    if st != DASH_OK:
        raise DashError(st, "dash_sim_table")
    return out.as_dict()


def dash_schedule_search(S, D, mask, G=1, groups=1, P=256, c_full=1.0, c_diag=None, r=0.0):
    """The searched schedule: dict with item_offsets, tasks, family (kind,
    order, block) and the simulator's report."""
    if c_diag is None:
        c_diag = c_full
    T = dash_attn_tile_size(S, D)
    if T == 0 or S < 1:
        raise ValueError("unsupported S or D")
    N = (S + T - 1) // T
    n = dash_schedule_table_tasks(mask, N, G)
    if n < 0:
        raise ValueError("invalid mask or G")
    offs, tasks = _table_out(n, G * N)
    items = ctypes.c_int()
    fam = (ctypes.c_int * 3)()
    out = SimResult()
    st = lib().dash_schedule_search(int(S), int(D), int(mask), int(G), int(groups), int(P),
                                    float(c_full), float(c_diag), float(r), ctypes.byref(items),
                                    _iptr(offs), _iptr(tasks), fam, ctypes.byref(out))
    if st != DASH_OK:
        raise DashError(st, "dash_schedule_search")
    return {"item_offsets": offs[:items.value + 1], "tasks": tasks,
            "family": tuple(fam), "report": out.as_dict()}


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else None


def _dims(q, k):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be 4-d [B, S, H, D] tensors")
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    return B, S, Hq, Hkv, D


def _check_tensors(named, dtype):
    for name, t in named:
        if t is None:
            continue
        if t.dtype != dtype:
            raise TypeError("%s must be %s" % (name, dtype))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)


def _check_layout(dims, q_like=(), kv_like=(), row_like=()):
    """Shapes and device of every tensor the C ABI will read or write through
    a raw pointer: q_like are [B, S, Hq, D], kv_like [B, S, Hkv, D] and
    row_like [B, Hq, S]; all on one GPU.  A mismatch would make a kernel read
    or write past an allocation, so it raises ValueError before any call."""
    B, S, Hq, Hkv, D = dims
    want = {"q": (B, S, Hq, D), "kv": (B, S, Hkv, D), "row": (B, Hq, S)}
    named = ([(n, t, "q") for n, t in q_like] + [(n, t, "kv") for n, t in kv_like]
             + [(n, t, "row") for n, t in row_like])
    device = None
    for name, t, kind in named:
        if t is None:
            continue
        if tuple(t.shape) != want[kind]:
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), want[kind]))
    for name, t, _ in named:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError("%s must be a GPU tensor (is on %s)" % (name, t.device))
        if device is None:
            device = t.device
        elif t.device != device:
            raise ValueError("%s is on %s, the other tensors on %s" % (name, t.device, device))
    return device


def _check_workspace(workspace, device):
    if workspace is None:
        return
    if workspace.dtype.itemsize != 1 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous byte tensor")
    if device is not None and workspace.device != device:
        raise ValueError("workspace is on %s, the tensors on %s" % (workspace.device, device))


def dash_attn_fwd(q, k, v, o, lse, mask, stream=None):
    """Forward into preallocated o [B,S,Hq,D] bf16 and lse [B,Hq,S] fp32."""
    import torch
    _check_tensors([("q", q), ("k", k), ("v", v), ("o", o)], torch.bfloat16)
    _check_tensors([("lse", lse)], torch.float32)
    dims = _dims(q, k)
    _check_layout(dims, [("q", q), ("o", o)], [("k", k), ("v", v)], [("lse", lse)])
    B, S, Hq, Hkv, D = dims
    st = lib().dash_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                             B, Hq, Hkv, S, D, int(mask), _stream(stream))
    if st != DASH_OK:
        raise DashError(st, "dash_attn_fwd")


def dash_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, mask, schedule, workspace,
                  stream=None):
    """Backward into preallocated dq, dk, dv; workspace is a uint8 device tensor."""
    import torch
    _check_tensors([("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout),
                    ("dq", dq), ("dk", dk), ("dv", dv)], torch.bfloat16)
    _check_tensors([("lse", lse)], torch.float32)
    dims = _dims(q, k)
    dev = _check_layout(dims, [("q", q), ("o", o), ("dout", dout), ("dq", dq)],
                        [("k", k), ("v", v), ("dk", dk), ("dv", dv)], [("lse", lse)])
    _check_workspace(workspace, dev)
    B, S, Hq, Hkv, D = dims
    st = lib().dash_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                             _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv, S, D, int(mask),
                             int(schedule), _ptr(workspace),
                             workspace.numel() if workspace is not None else 0,
                             _stream(stream))
    if st != DASH_OK:
        raise DashError(st, "dash_attn_bwd")


def dash_attn_bwd_prepare(o, dout, lse, q_shape, kv_heads, mask, schedule, workspace,
                          stream=None):
    """First phase of dash_attn_bwd (the per-row values, counter reset).
    q_shape is (B, S, Hq, D); kv_heads is Hkv."""
    import torch
    _check_tensors([("o", o), ("dout", dout)], torch.bfloat16)
    _check_tensors([("lse", lse)], torch.float32)
    B, S, Hq, D = q_shape
    Hkv = int(kv_heads)
    dev = _check_layout((B, S, Hq, Hkv, D), [("o", o), ("dout", dout)], [], [("lse", lse)])
    _check_workspace(workspace, dev)
    st = lib().dash_attn_bwd_prepare(_ptr(o), _ptr(dout), _ptr(lse), B, Hq, Hkv, S,
                                     D, int(mask), int(schedule), _ptr(workspace),
                                     workspace.numel() if workspace is not None else 0,
                                     _stream(stream))
    if st != DASH_OK:
        raise DashError(st, "dash_attn_bwd_prepare")


def dash_attn_bwd_run(q, k, v, dout, dq, dk, dv, mask, schedule, workspace, stream=None):
    """Second phase of dash_attn_bwd (the persistent backward kernel)."""
    import torch
    _check_tensors([("q", q), ("k", k), ("v", v), ("dout", dout), ("dq", dq), ("dk", dk),
                    ("dv", dv)], torch.bfloat16)
    dims = _dims(q, k)
    dev = _check_layout(dims, [("q", q), ("dout", dout), ("dq", dq)],
                        [("k", k), ("v", v), ("dk", dk), ("dv", dv)])
    _check_workspace(workspace, dev)
    B, S, Hq, Hkv, D = dims
    st = lib().dash_attn_bwd_run(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk),
                                 _ptr(dv), B, Hq, Hkv, S, D, int(mask), int(schedule),
                                 _ptr(workspace),
                                 workspace.numel() if workspace is not None else 0,
                                 _stream(stream))
    if st != DASH_OK:
        raise DashError(st, "dash_attn_bwd_run")


def dash_attn_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, mask, schedule, stream=None):
    """dash_attn_bwd on the library's static device workspace (no workspace
    argument; the library allocates nothing).  Problems whose workspace
    exceeds NOALLOC_WORKSPACE_BYTES raise DashError (DASH_ERR_WORKSPACE)."""
    import torch
    _check_tensors([("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout),
                    ("dq", dq), ("dk", dk), ("dv", dv)], torch.bfloat16)
    _check_tensors([("lse", lse)], torch.float32)
    dims = _dims(q, k)
    _check_layout(dims, [("q", q), ("o", o), ("dout", dout), ("dq", dq)],
                  [("k", k), ("v", v), ("dk", dk), ("dv", dv)], [("lse", lse)])
    B, S, Hq, Hkv, D = dims
    st = lib().dash_attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                     _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv, S, D, int(mask),
                                     int(schedule), _stream(stream))
    if st != DASH_OK:
        raise DashError(st, "dash_attn_bwd_noalloc")


def dash_attn_bwd_table(q, k, v, o, dout, lse, dq, dk, dv, mask, table, items, grid, workspace,
                        stream=None):
    """dash_attn_bwd under a task table; `table` is a uint8 device tensor
    holding what dash_schedule_table_pack returned, `items` its item count,
    `grid` the cap on persistent workgroups (0 = the device's grid)."""
    import torch
    _check_tensors([("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout),
                    ("dq", dq), ("dk", dk), ("dv", dv)], torch.bfloat16)
    _check_tensors([("lse", lse)], torch.float32)
    _check_tensors([("table", table)], torch.uint8)
    dims = _dims(q, k)
    dev = _check_layout(dims, [("q", q), ("o", o), ("dout", dout), ("dq", dq)],
                        [("k", k), ("v", v), ("dk", dk), ("dv", dv)], [("lse", lse)])
    _check_workspace(workspace, dev)
    if table is not None and table.device != dev:
        raise ValueError("table must be on the tensors' device")
    B, S, Hq, Hkv, D = dims
    st = lib().dash_attn_bwd_table(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                   _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv, S, D, int(mask),
                                   _ptr(table), table.numel() if table is not None else 0,
                                   int(items), int(grid), _ptr(workspace),
                                   workspace.numel() if workspace is not None else 0,
                                   _stream(stream))
    if st != DASH_OK:
        raise DashError(st, "dash_attn_bwd_table")


def dash_attn_bwd_table_run(q, k, v, dout, dq, dk, dv, mask, table, items, grid, workspace,
                            stream=None):
    """Run phase of dash_attn_bwd_table, after dash_attn_bwd_prepare with
    the TABLE schedule on the same workspace."""
    import torch
    _check_tensors([("q", q), ("k", k), ("v", v), ("dout", dout), ("dq", dq), ("dk", dk),
                    ("dv", dv)], torch.bfloat16)
    _check_tensors([("table", table)], torch.uint8)
    dims = _dims(q, k)
    dev = _check_layout(dims, [("q", q), ("dout", dout), ("dq", dq)],
                        [("k", k), ("v", v), ("dk", dk), ("dv", dv)])
    _check_workspace(workspace, dev)
    if table is not None and table.device != dev:
        raise ValueError("table must be on the tensors' device")
    B, S, Hq, Hkv, D = dims
    st = lib().dash_attn_bwd_table_run(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk),
                                       _ptr(dv), B, Hq, Hkv, S, D, int(mask), _ptr(table),
                                       table.numel() if table is not None else 0, int(items),
                                       int(grid), _ptr(workspace),
                                       workspace.numel() if workspace is not None else 0,
                                       _stream(stream))
    if st != DASH_OK:
        raise DashError(st, "dash_attn_bwd_table_run")


def dash_attn_bwd_check(workspace, stream=None):
    st = lib().dash_attn_bwd_check(_ptr(workspace), _stream(stream))
    if st != DASH_OK:
        raise DashError(st, "dash_attn_bwd_check")


def dash_attn_bwd_wait_stats(workspace, stream=None):
    """Turn waits of the last backward on this workspace: a dict with the
    number of waits, their re-polls and the seconds they took (summed over
    waves)."""
    n, p, s = ctypes.c_longlong(), ctypes.c_longlong(), ctypes.c_double()
    st = lib().dash_attn_bwd_wait_stats(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                        _stream(stream), ctypes.byref(n), ctypes.byref(p),
                                        ctypes.byref(s))
    if st != DASH_OK:
        raise DashError(st, "dash_attn_bwd_wait_stats")
    return {"waits": n.value, "polls": p.value, "wait_seconds": s.value}


def dash_attn_set_watchdog(seconds):
    st = lib().dash_attn_set_watchdog(float(seconds))
    if st != DASH_OK:
        raise DashError(st, "dash_attn_set_watchdog")


# --- conveniences that allocate outputs with torch --------------------------

def new_workspace(q, k, mask, schedule):
    import torch
    B, S, Hq, Hkv, D = _dims(q, k)
    n = dash_attn_bwd_workspace_size(B, Hq, Hkv, S, D, int(mask), int(schedule))
    if n == 0:
        raise ValueError("invalid arguments for the backward workspace")
    # torch's caching allocator returns 256-byte aligned blocks
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def forward(q, k, v, causal):
    import torch
    B, S, Hq, Hkv, D = _dims(q, k)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    dash_attn_fwd(q, k, v, o, lse, MASK_CAUSAL if causal else MASK_FULL)
    return o, lse


def upload_table(q, k, causal, item_offsets, tasks):
    """Packs a table for q/k's shape and copies it to q's device: (uint8
    tensor, items)."""
    import torch
    B, S, Hq, Hkv, D = _dims(q, k)
    raw = dash_schedule_table_pack(S, D, MASK_CAUSAL if causal else MASK_FULL, Hq // Hkv,
                                   item_offsets, tasks)
    host = torch.frombuffer(bytearray(raw), dtype=torch.uint8)
    return host.to(q.device), len(item_offsets) - 1


def backward_table(q, k, v, o, dout, lse, causal, table, items, grid=0, workspace=None,
                   stream=None, check=True):
    """Allocates dq, dk, dv and runs dash_attn_bwd_table (see backward)."""
    import torch
    mask = MASK_CAUSAL if causal else MASK_FULL
    if workspace is None:
        workspace = new_workspace(q, k, mask, TABLE)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dash_attn_bwd_table(q, k, v, o, dout, lse, dq, dk, dv, mask, table, items, grid,
                        workspace, stream)
    if check and q.numel() > 0:
        dash_attn_bwd_check(workspace, stream)
    return dq, dk, dv


def backward(q, k, v, o, dout, lse, causal, schedule=SHIFT, workspace=None, stream=None,
             check=True):
    """Allocates dq, dk, dv and runs dash_attn_bwd.  With check (the default)
    it then waits for the stream and raises DashError if the device watchdog
    fired, in which case the outputs would be undefined; with check=False the
    call stays asynchronous and the caller must call dash_attn_bwd_check on
    the workspace before trusting the result."""
    import torch
    mask = MASK_CAUSAL if causal else MASK_FULL
    if workspace is None:
        workspace = new_workspace(q, k, mask, schedule)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dash_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, mask, schedule, workspace, stream)
    if check and q.numel() > 0:
        # (an empty problem launches nothing and leaves the workspace as it was)
        dash_attn_bwd_check(workspace, stream)
    return dq, dk, dv

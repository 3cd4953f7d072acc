"""Timing of the oracle on the host cores (test infrastructure; only the
``cpu_baseline`` leg of bench.py uses it).

The oracle runs in worker processes started with the ``spawn`` method, each
pinned to one host core with one BLAS thread. The processes are started before
the benchmark touches the GPU and hold only host arrays (NumPy and this
package; nothing here imports torch).

A sample of queries is measured in four phases:
  1. ``load``: each worker receives its share of the queries' host inputs;
  2. ``discover`` (untimed): the oracle runs once with a main-KV cache that
     records which rows attention reads and returns zero rows (the selected
     indices do not depend on the rows' values, so the set is exact);
  3. ``stage`` (untimed): the oracle packs exactly those rows (RoPE, then FP4)
     from the bf16 source rows the caller sends;
  4. timed runs over the staged rows: per query the write path of its step (the
     sequence's new main-KV row: RoPE + FP4, stored at its slot) and the whole
     layer group (scans, pool, Top-K, Reuse, attention in every layer). The
     one-core figure runs the workers one after another, each alone on its core;
     the all-core figure starts them together and takes the wall time from the
     first start to the last end.
"""

import multiprocessing as mp
import os
import time

import numpy as np


class RecordingRows:
    """Cache stand-in for the discovery pass: records the rows asked for and
    returns zero rows (attention values are discarded in that pass)."""

    def __init__(self, n_rows):
        self.n = int(n_rows)
        self.seen = set()

    def __len__(self):
        return self.n

    def __getitem__(self, sel):
        sel = np.asarray(sel, dtype=np.int64).reshape(-1)
        self.seen.update(int(j) for j in sel)
        return np.zeros((sel.shape[0], 288), dtype=np.uint8)


class StagedRows:
    """Packed main-KV rows staged by position; a position that was not staged
    raises (the timed pass never computes rows it was not given)."""

    def __init__(self, n_rows, rows):
        self.n = int(n_rows)
        self.rows = dict(rows)

    def __len__(self):
        return self.n

    def __getitem__(self, sel):
        sel = np.asarray(sel, dtype=np.int64).reshape(-1)
        if sel.shape[0] == 0:
            return np.zeros((0, 288), dtype=np.uint8)
        return np.stack([self.rows[int(j)] for j in sel])


def _run_query(task, rows_cache):
    from . import group as OG
    sched = OG.layer_schedule(task["kind"])
    return OG.run_group(sched, task["q_idx"], task["w"], task["q"], task["swa"], task["k"],
                        rows_cache, task["n_vis"], task["t"], task["swa_pos0"],
                        k_scales=task["k_scales"])


def _write_new_row(task, rows):
    """The step's write path for this query's sequence: RoPE at the new slot's
    position, then FP4 packing, stored at the slot."""
    from . import formats as OF
    from . import rope as OR
    if task.get("new_row") is None:
        return
    slot = int(task["new_slot"])
    y = OR.apply_rope(task["new_row"][None, :], [slot * int(task["m"])])
    rows[slot] = OF.quantize_rows(y)[0]


def _w_load(state, tasks):
    state["tasks"] = list(tasks)
    state["staged"] = [None] * len(state["tasks"])
    return len(state["tasks"])


def _w_discover(state):
    out = []
    for task in state["tasks"]:
        rec = RecordingRows(task["n_cap"])
        _run_query(task, rec)
        seen = rec.seen
        if task.get("new_row") is not None:
            seen.discard(int(task["new_slot"]))       # written by the timed write path
        out.append(sorted(seen))
    return out


def _w_stage(state, i, positions, rows_f32):
    """Pack the bf16 source rows (given as float32) of task i's positions."""
    from . import formats as OF
    from . import rope as OR
    task = state["tasks"][i]
    positions = np.asarray(positions, dtype=np.int64)
    if positions.shape[0]:
        packed = OF.quantize_rows(OR.apply_rope(np.asarray(rows_f32, dtype=np.float32),
                                                positions * int(task["m"])))
    else:
        packed = np.zeros((0, 288), dtype=np.uint8)
    state["staged"][i] = {int(p): r for p, r in zip(positions, packed)}
    return int(positions.shape[0])


def _w_run(state, budget_s=None):
    """Time the worker's queries over their staged rows (until budget_s seconds
    have been spent, if given). Returns (monotonic start, monotonic end,
    per-query seconds)."""
    times = []
    start = time.monotonic()
    for task, staged in zip(state["tasks"], state["staged"]):
        t0 = time.perf_counter()
        rows = dict(staged)
        _write_new_row(task, rows)
        _run_query(task, StagedRows(task["n_cap"], rows))
        times.append(time.perf_counter() - t0)
        if budget_s is not None and sum(times) >= budget_s:
            break
    return start, time.monotonic(), times


_FUNCS = {"load": _w_load, "discover": _w_discover, "stage": _w_stage, "run": _w_run}


def _worker(conn, core):
    try:
        os.sched_setaffinity(0, {core})
    except (AttributeError, OSError):
        pass
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except ImportError:           # pragma: no cover
        pass
    state = {}
    while True:
        msg = conn.recv()
        if msg is None:
            break
        name, args = msg
        try:
            conn.send(("ok", _FUNCS[name](state, *args)))
        except Exception as e:     # reported to the caller, which raises
            conn.send(("err", repr(e)))
    conn.close()


def host_cpu():
    """(CPU model name, cores this process may run on, os.cpu_count())."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:        # pragma: no cover
        usable = os.cpu_count() or 1
    return model, usable, os.cpu_count()


class Workers:
    """Spawned oracle workers, one per core (at most `max_workers`)."""

    def __init__(self, max_workers=16):
        try:
            cores = sorted(os.sched_getaffinity(0))
        except AttributeError:    # pragma: no cover
            cores = list(range(os.cpu_count() or 1))
        cores = cores[:max(1, int(max_workers))]
        ctx = mp.get_context("spawn")
        self.conns, self.procs, self.cores = [], [], cores
        for c in cores:
            a, b = ctx.Pipe()
            p = ctx.Process(target=_worker, args=(b, c), daemon=True)
            p.start()
            self.conns.append(a)
            self.procs.append(p)

    def __len__(self):
        return len(self.conns)

    def _send(self, i, name, *args):
        self.conns[i].send((name, args))

    def _recv(self, i):
        status, val = self.conns[i].recv()
        if status != "ok":
            raise RuntimeError("oracle worker %d: %s" % (i, val))
        return val

    def call(self, i, name, *args):
        self._send(i, name, *args)
        return self._recv(i)

    def call_all(self, name, args_per_worker):
        for i, a in enumerate(args_per_worker):
            self._send(i, name, *a)
        return [self._recv(i) for i in range(len(args_per_worker))]

    def close(self):
        for c in self.conns:
            try:
                c.send(None)
                c.close()
            except (OSError, BrokenPipeError):
                pass
        for p in self.procs:
            p.join(timeout=10)
            if p.is_alive():
                p.terminate()
        self.conns, self.procs = [], []


def measure(workers, tasks, source_rows, budget_1core_s=10.0):
    """Time the oracle on `tasks` (dicts of host inputs, see _run_query) with
    the spawned `workers`.

    source_rows(task_index, positions) -> float32 [len(positions), 512]: the
    bf16 main-KV source rows of that task's sequence at those positions.
    Returns a dict with the one-core and all-core throughputs."""
    n = min(len(workers), len(tasks))
    share = [tasks[w::n] for w in range(n)]        # task qi is share[qi % n][qi // n]
    workers.call_all("load", [(s,) for s in share])
    found = workers.call_all("discover", [()] * n)
    for j in range(len(share[0])):
        busy = [w for w in range(n) if j < len(share[w])]
        for w in busy:
            pos = found[w][j]
            rows = source_rows(j * n + w, pos) if pos else np.zeros((0, 512), np.float32)
            workers._send(w, "stage", j, pos, rows)
        for w in busy:
            workers._recv(w)
    # one core: each worker alone in turn, until the budget is spent
    one, spent = 0, 0.0
    for w in range(n):
        _, _, times = workers.call(w, "run", budget_1core_s - spent)
        one += len(times)
        spent += sum(times)
        if spent >= budget_1core_s:
            break
    # all cores: every worker at once over its whole share
    res = workers.call_all("run", [(None,)] * n)
    wall = max(r[1] for r in res) - min(r[0] for r in res)
    n_all = sum(len(r[2]) for r in res)
    return {"value_1core": one / spent, "queries_1core": one, "seconds_1core": spent,
            "value_all_cores": n_all / wall, "queries_all_cores": n_all,
            "seconds_all_cores": wall, "cores_all": n}

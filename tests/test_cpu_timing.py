"""The oracle timing harness behind bench.py's cpu_baseline (CPU only): the rows
found by the discovery pass are exactly the rows attention reads, the staged
run gives the oracle's own outputs over a fully packed cache, and the spawned
workers run the whole protocol."""

import numpy as np
import torch

from oracle import cpu_timing as CT
from oracle import formats as OF
from oracle import group as OG
from oracle import rope as OR


def _task(rng, n_cap=3000, kind="decoder", m=1, new_row=True):
    L = len(OG.layer_schedule(kind))
    idx_layers = [li for li, (mode, _) in enumerate(OG.layer_schedule(kind)) if mode != "U"]

    def e4m3(shape):
        x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32))
        return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()

    t = n_cap * m - 1
    return {
        "kind": kind, "n_cap": n_cap, "m": m, "t": t, "n_vis": n_cap, "swa_pos0": t - 127,
        "k": e4m3((n_cap, 128)), "k_scales": None,
        "q_idx": {li: e4m3((32, 128)) for li in idx_layers},
        "w": {li: (rng.uniform(0, 1, 32) / 32).astype(np.float32) for li in idx_layers},
        "q": {li: (rng.standard_normal((64, 512)) / np.sqrt(512)).astype(np.float32)
              for li in range(L)},
        "swa": {li: e4m3((128, 512)) for li in range(L)},
        "new_row": rng.standard_normal(512).astype(np.float32) if new_row else None,
        "new_slot": n_cap - 1}


def _source(rng, n_cap):
    return rng.standard_normal((n_cap, 512)).astype(np.float32)


def test_staged_rows_reproduce_the_oracle_on_a_full_cache():
    rng = np.random.default_rng(11)
    task = _task(rng)
    src = _source(rng, task["n_cap"])
    src[task["new_slot"]] = task["new_row"]
    full = OF.quantize_rows(OR.apply_rope(src, np.arange(task["n_cap"]) * task["m"]))
    ref = CT._run_query(task, full)
    state = {}
    CT._w_load(state, [task])
    (pos,) = CT._w_discover(state)
    assert task["new_slot"] not in pos
    assert len(pos) >= 512
    CT._w_stage(state, 0, pos, src[np.asarray(pos)])
    rows = dict(state["staged"][0])
    CT._write_new_row(task, rows)
    got = CT._run_query(task, CT.StagedRows(task["n_cap"], rows))
    for li in ref[0]:
        assert np.array_equal(ref[0][li], got[0][li])
        assert np.array_equal(ref[1][li], got[1][li])
    # every staged row is read by some layer's attention
    used = set()
    for li in got[0]:
        used.update(int(j) for j in got[0][li] if j >= 0)
    assert set(pos) <= used


def test_spawned_workers_run_the_whole_protocol():
    rng = np.random.default_rng(12)
    tasks = [_task(rng, n_cap=2000, kind="encoder", m=2), _task(rng, n_cap=2000, kind="full")]
    srcs = [_source(rng, 2000) for _ in tasks]
    workers = CT.Workers(max_workers=2)
    try:
        r = CT.measure(workers, tasks, lambda qi, pos: srcs[qi][np.asarray(pos)],
                       budget_1core_s=0.5)
    finally:
        workers.close()
    assert r["queries_1core"] >= 1 and r["value_1core"] > 0
    assert r["queries_all_cores"] == 2 and r["value_all_cores"] > 0
    assert r["cores_all"] == min(2, len(workers.cores))
    model, usable, total = CT.host_cpu()
    assert isinstance(model, str) and usable >= 1 and total >= 1

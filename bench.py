"""Benchmark of the CSA2 per-layer hot path on one MI355X.

A step is one pass of the whole path over one batch of decode queries: the
write path (one new main-KV row per sequence, RoPE + FP4, into the newest
slot), then the layer group -- for the 1M-context decoder group
[Full, Reindex, Reuse, Reindex, Reuse, Reindex, Reuse]: the Full-mode scan of
all 1,048,576 positions with block maxima, the 2,048-block pool, Top-512,
Reindex scans inside the pool, Reuse, and sparse attention in every layer.
Inputs are seeded synthetic tensors already resident in HBM.

Prints ONE JSON line (rank 0) with the queries/s, the roofline of the dominant
kernel (the Full-mode scan) and the oracle's throughput on the host cores for a
bounded sample. With graph replay (the default) each step is one HIP graph and
the scan's duration comes from HIP events around a graph of `--steps`
back-to-back scan launches on the same stream; with --eager the events bracket
the scan inside every timed step.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload c2|c4|c1|c3]
                       [--index-k fp8|fp4]

The default workload is the 1M-context decoder group. `--workload c3` times the
4,096-query prefill chunk instead (no write path; its scan is an FP8 MFMA
contraction, so its roofline is reported against the FP8 MFMA peak).
`--index-k fp4` runs a decode workload with FP4 indexer keys (E2M1 codes plus
one E8M0 scale per 32 channels, 68 bytes per key instead of 128) drawn from the
same N(0,1) keys; the default line uses the workloads' FP8 keys.
"""

import argparse
import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

HBM_PEAK_GBS = 8000.0
FP8_MFMA_PEAK_TFLOPS = 5000.0      # dense FP8 MFMA, MI355X
SCAN_KERNEL = "k_index_score_decode"
TRAFFIC_FILE = os.path.join(HERE, "profiles", "traffic_index_score_full_c2.json")
SCAN_SOURCE = os.path.join(HERE, "compressed_kv_cache_02_amd", "csrc", "index_score.hip")


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="c2", choices=["c1", "c2", "c3", "c4"])
    p.add_argument("--index-k", default="fp8", choices=["fp8", "fp4"],
                   help="indexer-key format: FP8 E4M3 (the workloads' format) or FP4 "
                        "E2M1 with one E8M0 scale per 32 channels (decode workloads)")
    p.add_argument("--write-path", default="main", choices=["main", "full"],
                   help="per-step write path of the decode workloads: 'main' packs one "
                        "already-compressed main-KV row per sequence (the workloads' "
                        "definition); 'full' also compresses each sequence's newest m "
                        "tokens on the device, appends the compressed indexer key and "
                        "appends the new token's window row in every layer")
    p.add_argument("--spec-tokens", type=int, default=1,
                   help="query tokens per sequence of a decode workload (the last T "
                        "positions, e.g. speculative decode); 1 = the workload as defined")
    p.add_argument("--fused-topk", default="auto", choices=["auto", "on", "off"],
                   help="groups without a pool (c1, c3, c4) take the Full layer's Top-K from "
                        "the fused scan + Top-K entry point (no score rows written): 'auto' "
                        "where it is faster (prefill chunks, decode over >= 262,144 positions)")
    p.add_argument("--rotate", type=int, default=None,
                   help="copies of the indexer keys and the main cache that consecutive timed "
                        "steps cycle through, so that a working set the 256 MB MALL could hold "
                        "is read from HBM (default: 3 for decode workloads whose keys fit in "
                        "1 GiB, else 1)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--graph", dest="graph", action="store_true", default=True,
                   help="replay each step segment as a HIP graph (default)")
    p.add_argument("--eager", dest="graph", action="store_false",
                   help="launch every kernel from Python instead of graph replay")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 1 GiB device copy (for counter calibration)")
    return p.parse_args()


def key_bytes(index_k):
    """Bytes of one indexer key: 128 E4M3 codes, or 64 bytes of E2M1 codes plus
    four E8M0 scales."""
    return 68 if index_k == "fp4" else 128


def scan_algorithmic_bytes(B, T, n_keys, index_k="fp8"):
    """Bytes the Full-mode scan must move per launch: one indexer key per
    position visible to some query of its sequence (n_keys, summed over the
    sequences; the query tokens of a sequence share the key reads) plus each
    query's 32x128 E4M3 query and 32 float weights."""
    return key_bytes(index_k) * n_keys + (32 * 128 + 32 * 4) * B * T


def step_algorithmic_bytes(w, n_keys, index_k="fp8"):
    """Whole-step bytes per the path's definition: scans, attention, write path."""
    q = w.B * w.T
    kb = key_bytes(index_k)
    full = kb * n_keys + (4096 + 128 + 2048) * q
    reindex = (16384 * kb + 4224 + 8192 + 2048) * q
    attn = 411648 * q
    n_x = {"decoder": 3}.get(w.kind, 0)
    return full + n_x * reindex + w.n_layers * attn + 1568 * w.B


def source_sha(path):
    """Hash of a kernel source's code: `//` comments and blank lines are left
    out, so a comment edit does not void counters taken on the same code."""
    import re
    with open(path, encoding="utf-8") as f:
        lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in f.read().splitlines()]
    return hashlib.sha256("\n".join(ln for ln in lines if ln.strip()).encode()).hexdigest()[:16]


def scan_kernel_name(kf, B, T, n_cap):
    """The decode-shaped Full scan's instantiation: <mode 0, key format,
    queries per wave, tiles per wave>. Single-token scans whose grid at 8
    tiles per wave (1,024 positions per work-group) has fewer than 16,384
    work-groups run 4 tiles per wave; query groups share each tile 2 at a time."""
    if T == 1:
        tiles = 4 if B * ((n_cap + 1023) // 1024) < 16384 else 8
        return "%s<0, %d, 1, %d>" % (SCAN_KERNEL, kf, tiles)
    return "%s<0, %d, 2, 8>" % (SCAN_KERNEL, kf)


def read_traffic(n_launch_bytes):
    """HBM traffic per scan launch from the committed rocprofv3 counter summary
    (one entry per key format), or None if no entry was taken on this version of
    the kernel source with this many algorithmic bytes per launch."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    sha = source_sha(SCAN_SOURCE)
    for e in t.get("entries", []):
        if e.get("source_sha") == sha and e.get("algorithmic_bytes_per_launch") == n_launch_bytes:
            return e.get("traffic_bytes_per_launch")
    return None


def cpu_baseline(workers, w, inp, seed, new_rows, budget_s=10.0, index_k="fp8",
                 oracle_rows=None):
    """The oracle on the host cores, on whole queries through the whole group
    (write-path row included): a sample of the workload's queries (every query
    of a decode workload up to two per worker; 64 evenly spaced queries of a
    prefill chunk, the first and last included), each through the whole layer
    group. The packed main-KV rows the oracle reads are staged before any
    timing (found by an untimed oracle pass, packed by the oracle from the bf16
    source rows); the timed region holds only oracle arithmetic on host arrays:
    the step's new row (RoPE + FP4) and the group. One-core throughput: the
    workers one after another, each alone on its core, until `budget_s` seconds
    are spent; all-core throughput: every worker at once over its share."""
    import numpy as np
    import torch
    from oracle import cpu_timing as CT
    from oracle.compress import n_visible
    from oracle import mxfp4 as OM
    import synth

    n_cap, m = w.n_cap, w.m
    n_q = w.B * w.T
    if w.T >= 64:
        picks = sorted(set(np.linspace(0, n_q - 1, 64).round().astype(int).tolist()))
    else:
        picks = list(range(min(n_q, 2 * len(workers))))
    n_layers = w.n_layers
    keys_of = {}

    def keys(b):
        if b not in keys_of:
            keys_of.clear()
            if index_k == "fp4":
                kn, ks = OM.quantize_index_keys(inp["k_bf16"][b].float().cpu().numpy())
            else:
                kn, ks = inp["k_idx"][b].cpu().numpy().copy(), None
            if oracle_rows is not None:
                # the full write path's appended key, as the oracle computes it
                if index_k == "fp4":
                    kn[n_cap - 1], ks[n_cap - 1] = oracle_rows["k"][0][b], oracle_rows["k"][1][b]
                else:
                    kn[n_cap - 1] = oracle_rows["k"][b]
            keys_of[b] = (kn, ks)
        return keys_of[b]

    tasks, seq_of = [], []
    for qi in picks:
        b, t = divmod(qi, w.T)
        kn, ks = keys(b)
        swa = {li: inp["swa"][li][b].cpu().numpy() for li in range(n_layers)}
        if oracle_rows is not None:
            for li in range(n_layers):
                swa[li] = swa[li].copy()
                swa[li][-1] = oracle_rows["win"][li][b]
        tq = int(w.q_positions[t])
        tasks.append({
            "kind": w.kind, "n_cap": n_cap, "m": m, "t": tq, "n_vis": int(n_visible(tq, m)),
            "swa_pos0": int(w.swa_pos0), "k": kn, "k_scales": ks,
            "q_idx": {li: inp["q_idx"][li][b, t].cpu().numpy() for li in inp["q_idx"]},
            "w": {li: inp["w"][li][b, t].cpu().numpy() for li in inp["w"]},
            "q": {li: inp["q"][li][b, t].float().cpu().numpy() for li in range(n_layers)},
            "swa": swa,
            "new_row": (new_rows[b].float().cpu().numpy() if new_rows is not None else None),
            "new_slot": n_cap - 1})
        seq_of.append(b)
    keys_of.clear()
    src = {}

    def source_rows(qi, pos):
        b = seq_of[qi]
        if b not in src:
            src.clear()
            src[b] = synth.pooled_main_rows(n_cap, m, "cuda", seed, w.name, "main", b,
                                            outliers=w.outliers)
        sel = torch.as_tensor(np.asarray(pos, dtype=np.int64), device=src[b].device)
        return src[b][sel].float().cpu().numpy()

    r = CT.measure(workers, tasks, source_rows, budget_1core_s=budget_s)
    src.clear()
    model, usable, total = CT.host_cpu()
    sched_len = n_layers
    return {"value": round(r["value_all_cores"], 4), "unit": "queries/s",
            "cores": r["cores_all"], "kind": "oracle",
            "value_1core": round(r["value_1core"], 4),
            "value_all_cores": round(r["value_all_cores"], 4),
            "cpu_model": model, "nproc": usable, "cpu_count": total,
            "sample": "%d of %d queries, each through all %d layers%s, packed rows staged "
                      "before timing; one core: %d queries in %.1f s (workers alone in turn); "
                      "all cores: %d queries on %d single-threaded processes in %.1f s" % (
                          len(picks), n_q, sched_len,
                          " incl. the write-path row" if new_rows is not None else "",
                          r["queries_1core"], r["seconds_1core"], r["queries_all_cores"],
                          r["cores_all"], r["seconds_all_cores"])}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    workers = None
    if not args.no_cpu_baseline:
        # the oracle's worker processes start before anything touches the GPU
        from oracle import cpu_timing as CT
        workers = CT.Workers(max_workers=16)
    import numpy as np
    import torch
    import compressed_kv_cache_02_amd as C
    from compressed_kv_cache_02_amd.group import LayerGroup, visible_entries
    from synth.configs import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    if args.fused_topk == "on" and not args.graph:
        print("--fused-topk on times the scan in its own graph: use it without --eager",
              file=sys.stderr)
        sys.exit(2)
    if args.spec_tokens > 1:
        import dataclasses
        if w.T != 1 or args.spec_tokens >= 64:
            print("--spec-tokens applies to the decode workloads, below 64", file=sys.stderr)
            sys.exit(2)
        w = dataclasses.replace(w, name=w.name, T=args.spec_tokens,
                                first_q=w.first_q - (args.spec_tokens - 1))
    dev = "cuda"
    torch.cuda.set_device(0)
    seed = 0
    log("generating inputs for %s" % w.name)
    inp = make_inputs(w, dev, seed=seed, index_k=args.index_k)
    B, T, n_cap, m = w.B, w.T, w.n_cap, w.m
    if args.index_k == "fp4":
        codes = torch.empty((B, n_cap, 64), dtype=torch.uint8, device=dev)
        scales = torch.empty((B, n_cap, 4), dtype=torch.uint8, device=dev)
        C.csa2_quantize_index_k(inp["k_bf16"].reshape(B * n_cap, 128), None, codes, scales)
        keys = (codes, scales)
    else:
        keys = inp["k_idx"]
    # cache build: every sequence's rows through the write-path kernel
    cache = torch.empty((B, n_cap, 288), dtype=torch.uint8, device=dev)
    cs_all = torch.from_numpy(C.csa2_rope_table(np.arange(n_cap, dtype=np.int64) * m)).to(dev)
    for b in range(B):
        C.csa2_quantize_kv(inp["main_rows_per_seq"][b], cs_all, None, cache[b])
    del cs_all
    inp["main_rows_per_seq"] = None
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    # per-step write path of a decode step: one new row per sequence into the
    # newest slot (the prefill chunk has none)
    prefill = T >= 64
    if prefill:
        new_rows, write = None, None
    else:
        if "write_bf16" in inp:
            new_rows = inp["write_bf16"]
        else:
            import synth
            new_rows = synth.token_rows_bf16(B, dev, seed, w.name, "write")
        slot = torch.arange(B, dtype=torch.int64, device=dev) * n_cap + (n_cap - 1)
        cs_new = torch.from_numpy(C.csa2_rope_table(np.full(B, (n_cap - 1) * m,
                                                            dtype=np.int64))).to(dev)
        write = (new_rows, cs_new, slot)
    full_write = None
    if args.write_path == "full" and not prefill:
        import synth
        from oracle import compress as OCm            # the oracle's rows for cpu_baseline only
        from oracle import formats as OFm
        from oracle import mxfp4 as OMm
        # the newest group of m tokens of every sequence (main latent and indexer key),
        # the new token's window row per layer; the compressed entry replaces new_rows
        tok_main = synth.token_rows_bf16(B * m, dev, seed, w.name, "write_tok", outliers=w.outliers)
        tok_k = synth.normal_rows(B * m, 128, dev, seed, w.name, "write_k",
                                  outliers=w.outliers).to(torch.bfloat16)
        win = [synth.normal_rows(B, 512, dev, seed, w.name, "write_win", li,
                                 outliers=w.outliers).to(torch.bfloat16) for li in range(w.n_layers)]
        entry = torch.empty((B, 512), dtype=torch.bfloat16, device=dev)
        kentry = torch.empty((B, 128), dtype=torch.bfloat16, device=dev)
        wslot = torch.arange(B, dtype=torch.int64, device=dev) * w.S + (w.S - 1)
        full_write = (tok_main, tok_k, win, entry, kentry, wslot)
        write = (entry, cs_new, slot)

        def _bits(t):
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        # oracle-side rows for the cpu_baseline: compressed entry, appended key, window rows
        new_rows = torch.from_numpy(OCm.bf16_bits_to_f32(OCm.compress_mean(_bits(tok_main), m))).to(
            torch.bfloat16).to(dev)
        k_new = OCm.bf16_bits_to_f32(OCm.compress_mean(_bits(tok_k), m))
        oracle_rows = {"k": (OMm.quantize_index_keys(k_new) if args.index_k == "fp4"
                             else OFm.e4m3_encode(k_new)),
                       "win": [OFm.e4m3_encode(x.float().cpu().numpy()) for x in win]}
    else:
        oracle_rows = None

    n_vis = visible_entries(inp["q_pos"], m).to(torch.int32)
    n_vis_total = int(n_vis.sum().item())
    # keys visible to some query of each sequence: what a scan that shares the
    # key reads among a sequence's query tokens must move (decode shapes)
    n_keys = int(n_vis.max(dim=1).values.sum().item())
    fused = {"auto": "auto", "on": True, "off": False}[args.fused_topk]
    if not args.graph:
        fused = False          # eager timing brackets the scan inside the step
    g = LayerGroup(w.kind, B, T, n_cap, device=dev, fused_topk=fused)
    stream = torch.cuda.current_stream()

    # copies of the keys and the main cache that consecutive steps cycle through
    key_total = B * n_cap * key_bytes(args.index_k)
    rot = args.rotate if args.rotate is not None else (3 if not prefill and key_total < (1 << 30)
                                                        else 1)
    rot = max(1, rot)
    sets = [(keys, cache)]
    for _ in range(rot - 1):
        kc = tuple(t.clone() for t in keys) if isinstance(keys, tuple) else keys.clone()
        sets.append((kc, cache.clone()))
    cur = [0]

    def seg_write():
        keys, cache = sets[cur[0]]
        if full_write is not None:
            tok_main, tok_k, win, entry, kentry, wslot = full_write
            C.csa2_compress_tokens(tok_main, m, entry)
            C.csa2_compress_tokens(tok_k, m, kentry)
            if args.index_k == "fp4":
                C.csa2_quantize_index_k(kentry, slot, keys[0], keys[1])
            else:
                C.csa2_quantize_e4m3(kentry, slot, keys)
            for li in range(w.n_layers):
                C.csa2_quantize_e4m3(win[li], wslot, inp["swa"][li])
        if write is not None:
            g.write(cache, write)

    def seg_scan():
        g.scan(sets[cur[0]][0], n_vis, inp["q_idx"], inp["w"])

    def seg_scan_timed():
        # the Full scan alone, for its roofline (with --fused-topk the step runs
        # it inside csa2_index_topk, writing block maxima only, as here)
        g.scan_only(sets[cur[0]][0], n_vis, inp["q_idx"], inp["w"])

    def seg_rest():
        keys, cache = sets[cur[0]]
        g.rest(keys, cache, n_vis, inp["q_pos"], inp["swa_pos0"], inp["q_idx"], inp["w"], inp["q"],
               inp["swa"])

    log("cache built; warmup %d steps" % args.warmup)
    for _ in range(max(1, args.warmup)):
        seg_write()
        seg_scan()
        seg_rest()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step():
        seg_write()
        seg_scan()
        seg_rest()

    if args.graph:
        # The whole step is one HIP graph (every call inside only launches
        # kernels); the scan's own duration is taken from a second graph that
        # launches the scan R times back to back, bracketed by HIP events on the
        # stream it runs on (events between graphs would add launch gaps to
        # the step).
        R = args.steps
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        step_graphs = []
        for ci in range(rot):
            cur[0] = ci
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                step()
            step_graphs.append(gr)
        scan_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(scan_graph):
            for r in range(R):
                cur[0] = r % rot
                seg_scan_timed()
        cur[0] = 0
        torch.cuda.synchronize()
        for i in range(max(1, args.warmup)):
            step_graphs[i % rot].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step_graphs[i % rot].replay()
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        scan_graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        scan_ms = e0.elapsed_time(e1) / R
        step()                       # leave the buffers of a plain step behind
        torch.cuda.synchronize()
    else:
        # eager: events bracket the scan inside every timed step
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            cur[0] = i % rot
            seg_write()
            ev[i][0].record(stream)
            seg_scan()
            ev[i][1].record(stream)
            seg_rest()
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        scan_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        b2 = torch.empty_like(a)
        b2.copy_(a)
        torch.cuda.synchronize()
        del a, b2

    ms = el * 1e3 / args.steps
    qps = B * T * args.steps / el
    scan_bytes = scan_algorithmic_bytes(B, T, n_keys, args.index_k)
    kf = 1 if args.index_k == "fp4" else 0
    mfma_scan = T >= (C.PREFILL_MIN_T_FP4 if kf else C.PREFILL_MIN_T_FP8)
    if mfma_scan:
        # a dense FP8 contraction: 32 heads x 128 channels x 2 FLOP per visible pair
        scan_flop = 8192 * n_vis_total
        achieved = scan_flop / (scan_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP8_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / FP8_MFMA_PEAK_TFLOPS, 4),
                "traffic": None,
                # the group always keeps block maxima (scores only without a pool or
                # a fused Top-K); 16-query tiles up to 16 tokens
                "kernel": "k_index_score_prefill<true, %d, %d, %s>" % (
                    kf, 2 if T <= 16 else 4, "false" if g.scores is None else "true"),
                "kernel_ms": round(scan_ms, 4), "algorithmic_flop_per_launch": scan_flop}
    else:
        achieved = scan_bytes / (scan_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": read_traffic(scan_bytes),
                "kernel": scan_kernel_name(kf, B, T, n_cap),
                "kernel_ms": round(scan_ms, 4), "algorithmic_bytes_per_launch": scan_bytes}
    step_roof = None
    if not prefill:
        step_bytes = step_algorithmic_bytes(w, n_keys, args.index_k)
        step_roof = {"algorithmic_bytes": step_bytes,
                     "achieved_GBps": round(step_bytes / (ms * 1e-3) / 1e9, 1),
                     "frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    res = {
        "metric": ("CSA2 prefill queries/s, 4,096-query chunk after 262,144 tokens; % MFMA roofline"
                   if prefill else
                   "CSA2 decode queries/s at 1M ctx (Top-512 + SWA-128); % HBM/MFMA roofline"),
        "value": round(qps, 2),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3/fp4-e2m1 storage; fp32 scores; bf16/fp16 MFMA attention",
        "data": "synthetic (seeded N(0,1) per the workload recipe)",
        "config": {"workload": "%s: %s" % (w.name, {
            "c2": "decoder layer group [F,X,U,X,U,X,U] at 1,048,576 positions (m=1), batch 8 decode, + write path",
            "c4": "encoder group [F,U x5] at 1,048,576 tokens (m=2, 524,288 entries), batch 64 decode, write path, outliers",
            "c1": "Full-mode decode, batch 32, 131,072 tokens (m=2, 65,536 entries)",
            "c3": "Full-mode prefill of 4,096 queries after 262,144 tokens (m=2, 131,072-133,120 visible entries)"}[w.name]),
            "batch": B, "queries_per_seq": T, "n_cap": n_cap, "layers": len(g.sched),
            "topk": 512, "window": 128,
            "spec_tokens": T if not prefill else None,
            "write_path": {"main": "one compressed main-KV row per sequence (RoPE + FP4)",
                           "full": "m tokens compressed on device, main row RoPE + FP4, indexer "
                                   "key appended, window row appended in every layer"}[args.write_path],
            "fused_topk": bool(g.fused),
            "cache_copies": rot,
            "index_k": {"fp8": "FP8 E4M3 indexer keys (128 B)",
                        "fp4": "FP4 E2M1 indexer keys + E8M0 per 32 channels (68 B)"}[args.index_k],
            "timing": ("one HIP graph per step; scan timed over back-to-back launches"
                       if args.graph else "eager")},
        "roofline": roof,
        "step_roofline": step_roof,
    }
    log("timed %d steps: %.3f ms/step; running the oracle sample" % (args.steps, ms))
    if not args.no_cpu_baseline:
        try:
            res["cpu_baseline"] = cpu_baseline(workers, w, inp, seed, new_rows,
                                               index_k=args.index_k, oracle_rows=oracle_rows)
        finally:
            workers.close()
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

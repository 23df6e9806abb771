"""Benchmark of one DSA decode step on one MI355X.

A step is the whole hot path for one batch: lightning-indexer logits over the
paged fp8 K cache, per-row top-2048, and sparse MLA over the selected latent
rows (split-KV partials + merge when the split heuristic picks more than one).
Inputs are seeded synthetic tensors resident in HBM before timing starts; the
timed steps rotate through several copies of the caches so that the 256 MB
Infinity Cache cannot serve one step's reads from the previous step.  The
timed region replays a HIP graph holding ten steps back to back, rotating
through the copies (as a decoder replays its layers' steps inside one graph,
so a graph launch is paid once per many steps); the one-graph-per-step rate is
reported beside it.

Prints one JSON line: metric, value = steps/s of the headline workload (by
default c5, MTP decode over 64 sequences at 128 MLA heads: the largest decode
workload one GPU takes), the roofline of its dominant kernel, the other decode
workloads of the same run under "also" (by default c2), and the float64 oracle
timed on the host, stage by stage, as cpu_baseline.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
BF16_PEAK_TFLOPS = 2500.0
CHAIN_STEPS = 10               # steps per timed graph (at least one per cache copy)
WARM_S = 0.3                   # untimed warm-up (whole steps) before the timed region, seconds


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c5", choices=["c1", "c2", "c3", "c4", "c5", "x1m"],
                    help="headline workload (default c5: the largest single-GPU decode workload)")
    ap.add_argument("--also", default="c2",
                    help="comma-separated workloads measured after the headline in the same run and reported "
                         "under 'also' (empty: none)")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--copies", type=int, default=0, help="cache copies to rotate through (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--kv", default="bf16", choices=["bf16", "fp8"],
                    help="latent cache of the step's sparse MLA (fp8: e4m3 latent in 4 scaled groups + bf16 rope)")
    return ap.parse_args()


def algorithmic_bytes(wl):
    """Bytes each stage must move at minimum (inputs read once, outputs written once)."""
    seq_lens = wl.seq_lens.numpy().astype(np.int64)
    qs = wl.query_start.numpy().astype(np.int64)
    q_lens = qs[1:] - qs[:-1]
    _, ext = _row_extents(seq_lens, qs)
    k, H = wl.topk, wl.num_heads
    idx_in = int((132 * seq_lens + q_lens * 64 * (128 + 4) + 4 * ((seq_lens + 63) // 64)).sum())
    logit_bytes = int(4 * ext.sum())
    sel = np.minimum(ext, k)
    mla = int((1152 * sel + 4 * k + H * (1152 + 1024 + 4)).sum())
    mla8 = int((656 * sel + 4 * k + H * (1152 + 1024 + 4)).sum())
    return {"indexer": idx_in + logit_bytes, "topk": logit_bytes + 4 * k * len(ext), "sparse_mla": mla,
            "sparse_mla_fp8": mla8,
            "indexer_flops": int(16384 * ext.sum()),
            "mla_flops": int(2 * H * (576 + 512) * sel.sum())}


def _row_extents(seq_lens, qs):
    R = int(qs[-1])
    seq = np.zeros(R, np.int64)
    ext = np.zeros(R, np.int64)
    for b in range(len(seq_lens)):
        q = int(qs[b + 1] - qs[b])
        for i in range(q):
            seq[qs[b] + i] = b
            ext[qs[b] + i] = max(0, int(seq_lens[b]) - q + i + 1)
    return seq, ext


STAGE_SOURCES = {"indexer": ("indexer_paged.hip",), "indexer_prefill": ("indexer_prefill.hip",),
                 "topk": ("topk.hip",), "sparse_mla": ("sparse_mla.hip", "mla_common.h"),
                 "sparse_mla_fp8": ("sparse_mla_fp8.hip", "mla_common.h")}


def stage_source_sha(stage):
    """sha256 prefix of the kernel sources of one stage (its files + common.h)."""
    import hashlib
    m = hashlib.sha256()
    for f in STAGE_SOURCES[stage] + ("common.h",):
        with open(os.path.join(ROOT, "sparse_attention_fp8_amd", "csrc", f), "rb") as fh:
            m.update(fh.read())
    return m.hexdigest()[:16]


def measured_traffic(config, stage):
    """HBM bytes per launch of `stage` from the committed rocprofv3 PMC summary of
    this workload, or None when there is none or the stage's sources changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"dsa_step_{config}_traffic.md")
    if not os.path.exists(path):
        return None
    want = stage_source_sha(stage)
    with open(path) as fh:
        for line in fh:
            parts = line.split()
            if len(parts) == 4 and parts[0] == "traffic:" and parts[1] == stage and parts[2] == want:
                return int(parts[3])
    return None


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, budget_s):
    """Time the float64 oracle on a bounded, seeded sample of the step's rows,
    stage by stage (indexer logits, top-k, sparse MLA), scaled to whole steps."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        blas_threads = 1
    R = wl.num_rows
    rng = np.random.default_rng(0)
    order = rng.permutation(R)
    q8, w, cache = wl.q_fp8.numpy(), wl.weights.numpy(), wl.idx_cache.numpy()
    bt, sl, qs = wl.block_table.numpy(), wl.seq_lens.numpy(), wl.query_start.numpy()
    qm, kv = wl.q_mla.view(torch.int16).numpy(), wl.kv_cache.view(torch.int16).numpy()
    stride = wl.max_seq_len
    # Rows in a seeded order until the budget runs out; a step that finishes
    # early is repeated until at least half the budget is spent, so the
    # figure averages over several seconds of work.
    stage_s = {"indexer": 0.0, "topk": 0.0, "sparse_mla": 0.0}
    done, passes, t0 = 0, 0, time.perf_counter()
    out_of_time = False
    while not out_of_time:
        for r in order:
            t1 = time.perf_counter()
            lg, _, _ = oracle.indexer_logits(q8, w, cache, bt, sl, qs, stride, rows=[int(r)])
            t2 = time.perf_counter()
            idx = oracle.topk(lg, sl, qs, wl.topk, rows=[int(r)])
            t3 = time.perf_counter()
            oracle.sparse_mla(qm, kv, bt, sl, qs, idx, wl.softmax_scale, rows=[int(r)])
            t4 = time.perf_counter()
            stage_s["indexer"] += t2 - t1
            stage_s["topk"] += t3 - t2
            stage_s["sparse_mla"] += t4 - t3
            done += 1
            if t4 - t0 > budget_s:
                out_of_time = True
                break
        else:
            passes += 1
            out_of_time = time.perf_counter() - t0 > budget_s / 2
    dt = time.perf_counter() - t0
    steps = done / R
    if passes >= 1:
        sample = (f"{passes} whole step(s) plus {done - passes * R} rows, {done} rows in all "
                  f"(indexer+top-k+sparse MLA per row, float64 numpy), {dt:.1f} s")
    else:
        sample = (f"{done} of {R} rows of one step (indexer+top-k+sparse MLA per row, float64 numpy), "
                  f"{dt:.1f} s, scaled by {R}/{done}")
    return {"value": steps / dt, "unit": "steps/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": sample,
            "stage_s_per_step": {k: v / steps for k, v in stage_s.items()},
            "threads_note": "cores = the BLAS pool's threads (the matrix products); the rest of the oracle "
                            "runs on one thread",
            "host_cpus": os.cpu_count(), "cpu_model": _cpu_model()}


def pre_path(dsa, wl, batch_dev, base, dev, steps):
    """Times the steps just before the path on this workload's new tokens: the
    indexer-q quantiser over its R rows, and the indexer-K and latent cache
    writers for the R tokens this step appends (the last q_len positions of
    each sequence).  Inputs rotate through enough copies that one round moves
    more than 1 GB, so the Infinity Cache cannot serve re-reads."""
    R = wl.num_rows
    if R == 0:
        return {}
    seq_lens = wl.seq_lens.numpy().astype(np.int64)
    qs = wl.query_start.numpy().astype(np.int64)
    bt = wl.block_table.numpy().astype(np.int64)
    slots = np.empty(R, dtype=np.int64)
    for b in range(len(seq_lens)):
        ql = int(qs[b + 1] - qs[b])
        pos = seq_lens[b] - ql + np.arange(ql)
        slots[qs[b]:qs[b + 1]] = bt[b, pos // 64] * 64 + pos % 64
    per = {"indexer_q_quant_fp8": R * 64 * (256 + 128 + 4 + 4),
           "indexer_k_quant_and_cache": R * (256 + 128 + 4 + 8),
           "latent_cache_write": R * (1152 + 1152 + 8)}
    copies = int(min(16, max(2, math.ceil(1.0e9 / max(per["indexer_q_quant_fp8"], 1)))))
    g = torch.Generator().manual_seed(1234)
    ins = []
    for _ in range(copies):
        ins.append({"q": torch.randn(R, 64, 128, generator=g).to(torch.bfloat16).to(dev),
                    "w": (torch.randn(R, 64, generator=g) / 8).to(dev),
                    "k": torch.randn(R, 128, generator=g).to(torch.bfloat16).to(dev),
                    "lat": torch.randn(R, 512, generator=g).to(torch.bfloat16).to(dev),
                    "rope": torch.randn(R, 64, generator=g).to(torch.bfloat16).to(dev)})
    slot_t = torch.from_numpy(slots).to(dev)
    q8 = torch.empty(R, 64, 128, dtype=torch.uint8, device=dev)
    w2 = torch.empty(R, 64, dtype=torch.float32, device=dev)
    ops = {
        "indexer_q_quant_fp8": lambda x: dsa.indexer_q_quant_fp8(x["q"], x["w"], q8, w2),
        "indexer_k_quant_and_cache": lambda x: dsa.indexer_k_quant_and_cache(x["k"], slot_t, base["idx_cache"]),
        "latent_cache_write": lambda x: dsa.latent_cache_write(x["lat"], x["rope"], slot_t, base["kv_cache"]),
    }
    stream = torch.cuda.current_stream()
    res = {}
    for name, fn in ops.items():
        for x in ins:
            fn(x)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for x in ins:
                fn(x)
        graph.replay()
        rounds = max(2, steps // copies)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(rounds):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (rounds * copies)
        gbs = per[name] / (us * 1e-6) / 1e9
        res[name] = {"us": us, "bytes": per[name], "GBps": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                     "items": R}
    return res


def measure(dsa, synth, name, args, kv="bf16", splits=0, seed=None, details=True):
    """Times one workload's step (and each stage) from HIP graph replays.
    Returns the figures of one JSON line (without the CPU baseline)."""
    dev = torch.device("cuda:0")
    wl = synth.make_config(name, seed)
    R, H, k = wl.num_rows, wl.num_heads, wl.topk
    prefill = wl.max_q_len > 2
    nbytes = algorithmic_bytes(wl)
    touched = nbytes["indexer"] + nbytes["sparse_mla"]
    copies = args.copies or int(min(8, max(2, math.ceil(1.0e9 / max(touched, 1)))))

    batch = dsa.Batch.from_host(wl.seq_lens, wl.query_start, wl.block_table, wl.num_pages, device=dev)
    sets = []
    base = {"q_fp8": wl.q_fp8.to(dev), "weights": wl.weights.to(dev), "idx_cache": wl.idx_cache.to(dev),
            "q_mla": wl.q_mla.to(dev), "kv_cache": wl.kv_cache.to(dev)}
    # the fp8 latent cache of the same rows, written by the library's own writer
    num_slots = wl.num_pages * 64
    kv8 = torch.zeros(wl.num_pages, dsa.binding.KV8_PAGE_BYTES, dtype=torch.uint8, device=dev)
    rows = base["kv_cache"][:, :64 * 576].reshape(num_slots, 576)
    dsa.latent_cache_write_fp8(rows[:, :512], rows[:, 512:], torch.arange(num_slots, dtype=torch.int64, device=dev),
                               kv8)
    base["kv8"] = kv8
    sets.append(base)
    for _ in range(copies - 1):
        sets.append({n: t.clone() for n, t in base.items()})
    stride = (wl.max_seq_len + 3) // 4 * 4
    logits = torch.empty(R, stride, dtype=torch.float32, device=dev)
    indices = torch.empty(R, k, dtype=torch.int32, device=dev)
    out = torch.empty(R, H, 512, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(R, H, dtype=torch.float32, device=dev)
    ws_topk = torch.empty(max(dsa.topk_workspace_bytes(batch, k), 1), dtype=torch.uint8, device=dev)
    ws_mla = torch.empty(max(dsa.sparse_mla_workspace_bytes(batch, H, k, splits), 1), dtype=torch.uint8,
                         device=dev)
    nsplits = splits or dsa.sparse_mla_pick_splits(batch, H, k)
    indexer = dsa.indexer_logits_prefill if prefill else dsa.indexer_logits_paged

    def run_stage(stage, i):
        t = sets[i % copies]
        if stage == "indexer":
            indexer(batch, t["q_fp8"], t["weights"], t["idx_cache"], logits, clean_logits=False)
        elif stage == "topk":
            dsa.topk(batch, logits, indices, k=k, workspace=ws_topk)
        elif stage == "sparse_mla_fp8":
            dsa.sparse_mla_decode_fp8(batch, t["q_mla"], t["kv8"], indices, wl.softmax_scale, out, lse,
                                      num_splits=splits, workspace=ws_mla)
        else:
            dsa.sparse_mla_decode(batch, t["q_mla"], t["kv_cache"], indices, wl.softmax_scale, out, lse,
                                  num_splits=splits, workspace=ws_mla)

    mla_stage = "sparse_mla_fp8" if kv == "fp8" else "sparse_mla"
    stages = ("indexer", "topk", mla_stage)
    other_mla = "sparse_mla" if kv == "fp8" else "sparse_mla_fp8"
    timed_stages = stages + ((other_mla,) if details else ())

    def step(i):
        for stage in stages:
            run_stage(stage, i)

    # eager warm-up (also loads every code object before capture)
    for i in range(max(args.warmup, 1)):
        step(i)
    torch.cuda.synchronize()

    # One HIP graph per cache copy holds one whole step, and a chain graph holds
    # `chain_len` steps back to back, rotating through the copies (a decoder
    # replays its layers' DSA steps inside one graph the same way, so a graph
    # launch is paid once per many steps).  The timed region runs exactly
    # `steps` steps: steps // chain_len chain replays, then single-step graphs.
    chain_len = max(copies, min(args.steps, CHAIN_STEPS))
    step_graphs = []
    for c in range(copies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(c)
        step_graphs.append(g)
    chain = torch.cuda.CUDAGraph()
    with torch.cuda.graph(chain):
        for c in range(chain_len):
            step(c % copies)
    # Per-stage graphs: `reps` launches of one entry point, rotating copies, so
    # the stage's average launch duration is measured on its own stream.
    reps = 2 * copies
    stage_graphs = {}
    for stage in timed_stages:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                run_stage(stage, i)
        stage_graphs[stage] = g
    torch.cuda.synchronize()
    for i in range(args.warmup):
        step_graphs[i % copies].replay()
    # Untimed warm-up until the clocks have settled: whole steps (chain
    # replays) for at least WARM_S seconds of GPU time.  A c5 step measured
    # after 5 warm-up steps only reads ~15 % slower than in steady state.
    t_warm = time.perf_counter()
    warm_replays = 0
    while True:
        chain.replay()
        warm_replays += 1
        if warm_replays % 8 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t_warm >= WARM_S:
                break
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps // chain_len):
        chain.replay()
    for i in range(args.steps % chain_len):
        step_graphs[i % copies].replay()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps

    # the same number of steps with one graph launch per step
    start.record(stream)
    for i in range(args.steps):
        step_graphs[i % copies].replay()
    stop.record(stream)
    torch.cuda.synchronize()
    ms_graph_each = start.elapsed_time(stop) / args.steps

    # Each stage: `stage_rounds` replays of its graph (`reps` launches each),
    # each replay bracketed by events; the median replay gives the average
    # launch duration (one replay disturbed by a clock or power transient moves
    # the median little, where it would move the mean by its full size).
    stage_ms = {}
    stage_rounds = max(5, args.steps // reps)
    for stage in timed_stages:
        stage_graphs[stage].replay()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(stage_rounds + 1)]
        evs[0].record(stream)
        for i in range(stage_rounds):
            stage_graphs[stage].replay()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(stage_rounds))
        stage_ms[stage] = per[stage_rounds // 2] / reps

    alt_ms = stage_ms.pop(other_mla) if details else None
    total_bytes = nbytes["indexer"] + nbytes["topk"] + nbytes[mla_stage]
    if prefill:
        dom = "indexer"
        achieved = nbytes["indexer_flops"] / (stage_ms[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / FP8_PEAK_TFLOPS, "traffic": measured_traffic(name, "indexer_prefill"),
                "kernel": "indexer_prefill", "per_launch": f"{nbytes['indexer_flops']} flop"}
    else:
        dom = max(stage_ms, key=stage_ms.get)
        achieved = nbytes[dom] / (stage_ms[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(name, dom), "kernel": dom,
                "per_launch": f"{nbytes[dom]} B"}
    res = {
        "ms": ms, "ms_graph_each": ms_graph_each, "stage_ms": stage_ms, "roofline": roof,
        "step_bytes": total_bytes, "step_hbm_frac": total_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "stage_hbm_frac": {st: nbytes[st] / (stage_ms[st] * 1e-3) / 1e9 / HBM_PEAK_GBS for st in stages},
        "mla_mfma_frac": nbytes["mla_flops"] / (stage_ms[mla_stage] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "config": {"workload": synth.CONFIGS[name], "name": name, "rows": R, "mla_heads": H,
                   "topk": k, "splits": nsplits, "cache_copies": copies,
                   "seed": seed if seed is not None else synth.DEFAULT_SEEDS[name]},
        "timing": f"HIP graph replays after {args.warmup} warm-up steps and {warm_replays * chain_len} more "
                  f"untimed steps ({WARM_S} s, clocks settled): a graph of {chain_len} steps (rotating {copies} "
                  f"cache copies) replayed {args.steps // chain_len} times plus {args.steps % chain_len} single-step "
                  f"graphs; stage times: median of {stage_rounds} replays of a graph of {reps} launches of one "
                  f"entry point",
        "rows": R,
    }
    if details:
        res["other_kv_stage"] = {"stage": other_mla, "us": alt_ms * 1e3, "bytes": nbytes[other_mla],
                                 "GBps": nbytes[other_mla] / (alt_ms * 1e-3) / 1e9,
                                 "hbm_frac": nbytes[other_mla] / (alt_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                 "note": "the same indices through the other latent-cache format"}
        res["pre_path"] = pre_path(dsa, wl, batch, base, dev, args.steps)
        if not prefill:
            res["page_read"] = page_read_ceiling(wl, [t["idx_cache"] for t in sets], dev, reps)
        res["wl"] = wl
    del sets, base
    torch.cuda.synchronize()
    return res


def page_read_ceiling(wl, caches, dev, reps):
    """Rate at which this GPU reads the indexer's pages with the indexer's copy
    scheme and no arithmetic: the probe library reads every page the paged
    indexer reads (same page list, order and launch shape), rotating over the
    same cache copies.  Returns None when the probe library is not built."""
    import ctypes
    path = os.path.join(ROOT, "sparse_attention_fp8_amd", "libdsa_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.dsa_probe_page_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.dsa_probe_page_read.restype = ctypes.c_int
    bt, sl, qs = wl.block_table.numpy(), wl.seq_lens.numpy(), wl.query_start.numpy()
    ids = []
    for b in range(len(sl)):
        if qs[b + 1] > qs[b]:
            n = (min(int(sl[b]), wl.max_seq_len) + 63) // 64
            ids.extend(int(x) for x in bt[b, :n])
    ids_dev = torch.tensor(ids, dtype=torch.int32, device=dev)
    assert len(ids) == 0 or (0 <= int(ids_dev.min()) and int(ids_dev.max()) < wl.num_pages)
    max_pages = len(sl) * ((wl.max_seq_len + 63) // 64)
    grid = max(1, min(torch.cuda.get_device_properties(0).multi_processor_count, (max_pages + 7) // 8))
    out = torch.empty(grid * 512, dtype=torch.int32, device=dev)
    page_bytes = 64 * 132
    stride = caches[0].stride(0) * caches[0].element_size()
    stream = torch.cuda.current_stream()

    def launch(i):
        # the stream current at the call: under capture that is the capturing stream
        rc = lib.dsa_probe_page_read(ctypes.c_void_p(caches[i % len(caches)].data_ptr()), stride,
                                     ctypes.c_void_p(ids_dev.data_ptr()), len(ids), ctypes.c_void_p(out.data_ptr()),
                                     grid, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert rc == 0, f"page-read probe launch failed ({rc})"

    launch(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            launch(i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rounds = 4
    e0.record(stream)
    for _ in range(rounds):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (rounds * reps)
    nbytes = len(ids) * page_bytes
    return {"us": ms * 1e3, "GBps": nbytes / (ms * 1e-3) / 1e9, "pages": len(ids), "bytes": nbytes,
            "grid": grid, "note": "the paged indexer's pages read with its copy scheme and launch shape, "
                                  "no arithmetic (probe/page_read.hip)"}


def copy_rate_gbs():
    """Device-to-device copy rate of this run (1 GiB), for reference."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    cbuf = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cdst = torch.empty_like(cbuf)
    cdst.copy_(cbuf)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        cdst.copy_(cbuf)
    e1.record(stream)
    torch.cuda.synchronize()
    return 5 * 2 * cbuf.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only; run with --gpus 1"}))
        sys.exit(2)
    import sparse_attention_fp8_amd as dsa
    from sparse_attention_fp8_amd import synth

    dsa.load()
    head = measure(dsa, synth, args.config, args, kv=args.kv, splits=args.splits, seed=args.seed)
    copy_gbs = copy_rate_gbs()
    ms = head["ms"]
    line = {
        "metric": "DSA decode steps/s (indexer+topk+sparse MLA) and % of HBM roofline at 1 GPU",
        "kv_cache": args.kv,
        "value": 1000.0 / ms,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 indexer / bf16 MLA, fp32 accumulate" if args.kv == "bf16"
                 else "fp8 indexer / fp8-cache MLA (bf16 operands), fp32 accumulate",
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
        "stages_ms": head["stage_ms"],
        "stage_hbm_frac": head["stage_hbm_frac"],
        "mla_mfma_frac": head["mla_mfma_frac"],
        "step_bytes": head["step_bytes"],
        "step_hbm_frac": head["step_hbm_frac"],
        "copy_GBps": copy_gbs,
        "timing": head["timing"],
        "ms_per_step_one_graph_each": head["ms_graph_each"],
        "rows_per_s": head["rows"] * 1000.0 / ms,
        "other_kv_stage": head["other_kv_stage"],
        "pre_path": head["pre_path"],
    }
    if head.get("page_read"):
        pr = head["page_read"]
        pr["indexer_stage_over_page_read"] = head["stage_ms"]["indexer"] * 1e3 / pr["us"]
        line["page_read"] = pr
    wl = head.pop("wl")
    del head
    # the other decode workloads, measured in the same run (same timing method)
    extra = {}
    for name in [x for x in args.also.split(",") if x and x != args.config]:
        r = measure(dsa, synth, name, args, kv=args.kv, details=False)
        extra[name] = {"workload": r["config"]["workload"], "ms_per_step": r["ms"], "steps_per_s": 1000.0 / r["ms"],
                       "stages_ms": r["stage_ms"], "step_bytes": r["step_bytes"],
                       "step_hbm_frac": r["step_hbm_frac"], "stage_hbm_frac": r["stage_hbm_frac"],
                       "roofline": r["roofline"], "splits": r["config"]["splits"],
                       "ms_per_step_one_graph_each": r["ms_graph_each"]}
    if extra:
        line["also"] = extra
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget_s)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the SparDA hot path on one MI355X; prints one JSON line.

The headline (the metric's workload): one decode layer-step of the batched
128K-context workload (B=16, T=131072, 32 query / 8 KV heads, d=128, 64-token
blocks, top-64): Forecast block scoring of the next layer's compressed keys,
top-k and GQA block-sparse attention of this layer, inputs resident in HBM,
one ``sparda_decode_layer`` launch per layer. The same run measures the other
four workloads (tiny fp32 decode, 32K single-sequence decode, the two-layer
offloaded decode with lookahead prefetch, the 4096-query chunked prefill) as
extra keys, each with its own roofline, the parity of every workload against
the fp64 oracle, and the oracle itself on the host cores (one core, and all
of them).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --workload decode|offload|prefill|pipeline   # one workload only

Timing: W untimed steps, then exactly K steps captured in one HIP graph
(replayed three times untimed after capture: a new graph's first replays run
slower), replayed 5 times, each replay between two HIP events on the launch stream
with a device synchronisation on both sides (three untimed steps run between
the synchronisation and the start event, so the timed steps do not begin on
an idle GPU); ms_per_step is the median replay / K (the spread is reported).
Input sets rotate (3 independent sets) so no step finds its data in the
256 MB last-level cache.
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode steps/s/layer at 128K ctx (select+sparse attn); % of HBM peak GB/s"
HBM_PEAK_GBPS = 8000.0
HOST_LINK_PEAK_GBPS = 63.0   # PCIe 5.0 x16, one direction
MFMA_BF16_PEAK_TFLOPS = 2500.0
N_SETS = 3
REPEATS = 5
MAX_POOL = 16  # host threads a GPU machine grants one GPU


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ timing ----
def _stats(per_call_ms) -> dict:
    xs = sorted(per_call_ms)
    return {"median": statistics.median(xs), "min": xs[0], "max": xs[-1], "n": len(xs)}


def time_graph_stats(fn, n: int, repeats: int = REPEATS, prime: int = 3) -> dict:
    """fn(0) .. fn(n-1) captured once in a HIP graph (no host launch cost
    inside), replayed `repeats` times, each replay between HIP events on the
    replay stream with a device synchronisation on both sides. Before each
    replay's start event, `prime` untimed fn calls run eagerly, so that the
    GPU is busy (clocks up) when the timed region begins rather than idle
    after the synchronisation. Returns the median / min / max ms per fn call
    over the replays."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(n):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    stream = torch.cuda.current_stream()
    for _ in range(3):  # the first replays of a new graph run slower: untimed
        g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(repeats):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        for i in range(prime):
            fn(i)
        start.record(stream)
        g.replay()
        end.record(stream)
        torch.cuda.synchronize()
        out.append(start.elapsed_time(end) / n)
    del g
    return _stats(out)


def time_graph(fn, n: int, repeats: int = REPEATS) -> float:
    """Median ms per fn call (see time_graph_stats)."""
    return time_graph_stats(fn, n, repeats)["median"]


def time_loop_stats(fn, n: int, stream, repeats: int = REPEATS) -> dict:
    """fn(0) .. fn(n-1) launched eagerly, `repeats` times, each run between HIP
    events on `stream` (after one untimed call that keeps the GPU busy up to
    the start event); median / min / max ms per call."""
    import torch
    out = []
    for _ in range(repeats):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        fn(0)
        start.record(stream)
        for i in range(n):
            fn(i)
        end.record(stream)
        torch.cuda.synchronize()
        out.append(start.elapsed_time(end) / n)
    return _stats(out)


def time_loop(fn, n: int, stream, repeats: int = REPEATS) -> float:
    return time_loop_stats(fn, n, stream, repeats)["median"]


def _us(st: dict) -> dict:
    return {k: (round(v * 1e3, 2) if k != "n" else v) for k, v in st.items()}


# ------------------------------------------------- the oracle on the host ----
def _f64(u16):
    """bf16 bit patterns (uint16) -> exact fp64 values."""
    import numpy as np
    return (np.asarray(u16, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def oracle_step_rows(rows, meta, reps: int) -> float:
    """The oracle, as it stands, on (sequence, KV head) rows of a decode step:
    Forecast scoring of every visible window, top-k of the blocks, the union
    of their tokens up to the query, and attention of the group's query
    heads over them. rows: per row (F, Kc, Q, K_sel, V_sel) as bf16 bit
    patterns, K_sel / V_sel being the keys and values of the oracle's own
    selection (gathered beforehand). Inputs are widened to fp64 outside the
    timed region; one thread. Returns the seconds of the `reps` timed passes."""
    import oracle
    from threadpoolctl import threadpool_limits
    T, q_start, scale, k = meta["T"], meta["q_start"], meta["scale"], meta["k"]
    data = [tuple(_f64(a) for a in r) for r in rows]
    timed = 0.0
    with threadpool_limits(limits=1):
        for _ in range(reps):
            t0 = time.perf_counter()
            for F, Kc, Q, KJ, VJ in data:
                sc = oracle.select_forecast_tile(F[None, :], Kc, [q_start], T, scale)
                idx = oracle.topk_row(sc, k)
                oracle.selected_keys(idx, q_start)
                for g in range(Q.shape[0]):
                    oracle.attend(Q[g], KJ, VJ, scale)
            timed += time.perf_counter() - t0
    return timed


def start_oracle_pool():
    """Worker processes for the all-cores oracle, started before anything
    touches the GPU (spawned interpreters that import numpy and the oracle
    only). As many as the host cores this process may use, up to MAX_POOL."""
    import multiprocessing as mp
    n = min(MAX_POOL, len(os.sched_getaffinity(0)))
    return mp.get_context("spawn").Pool(n), n


def cpu_baseline(w, s, pool, n_workers: int, reps: int = 20) -> dict:
    """The oracle timed on the benchmark's own step (all B x Hkv rows of input
    set 0): on one thread in this process, and split over the pool's worker
    processes (one thread each). The selection the oracle attends over is its
    own; the keys and values of those blocks are gathered from the GPU copy
    before timing."""
    import numpy as np
    import torch
    import oracle
    rows = []
    meta = {"T": w.T, "q_start": w.q_start, "scale": w.scale, "k": w.k}

    def u16(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    for b in range(w.B):
        for h in range(w.Hkv):
            F, Kc, Q = u16(s["F"][b, h, 0]), u16(s["Kc"][b, h]), u16(s["Q"][b, h * w.G:(h + 1) * w.G, 0])
            sc = oracle.select_forecast_tile(_f64(F)[None, :], _f64(Kc), [w.q_start], w.T, w.scale)
            J = oracle.selected_keys(oracle.topk_row(sc, w.k), w.q_start)
            Jt = torch.from_numpy(J).to(s["K"].device)
            rows.append((F, Kc, Q, u16(s["K"][b, h].index_select(0, Jt)), u16(s["V"][b, h].index_select(0, Jt))))
    one = oracle_step_rows(rows, meta, reps) / reps
    out = {"value": None, "unit": "steps/s/layer", "cores": 1, "kind": "oracle",
           "sample": f"the full step, all {len(rows)} (sequence, KV head) rows of one input set: Forecast scoring of "
                     f"{w.W} windows, top-{w.k} of {w.nB} blocks, attention of {w.G} heads over {w.k * w.block} keys; "
                     f"fp64 numpy, {reps} passes timed per configuration; fp64 widening of the inputs untimed",
           "single_core": {"value": round(1.0 / one, 4), "cores": 1, "s_per_step": round(one, 4),
                           "seconds_timed": round(one * reps, 2)},
           "nproc": len(os.sched_getaffinity(0)), "hardware_concurrency": os.cpu_count()}
    if pool is not None:
        chunks = [rows[i::n_workers] for i in range(n_workers)]
        t0 = time.perf_counter()
        secs = pool.starmap(oracle_step_rows, [(c, meta, reps) for c in chunks if c])
        wall = time.perf_counter() - t0
        per_step = max(secs) / reps  # a step ends when the slowest worker's rows are done
        out.update(value=round(1.0 / per_step, 4), cores=n_workers)
        out["all_cores"] = {"value": round(1.0 / per_step, 4), "cores": n_workers, "s_per_step": round(per_step, 4),
                            "cpu_seconds_timed": round(sum(secs), 2), "wall_seconds_with_transfer": round(wall, 2)}
    else:
        out["value"] = out["single_core"]["value"]
    return out


# ------------------------------------------------------------ parity ----
def _check(fn, *a, **kw):
    """Run a parity check; a failure is reported in the JSON line, not raised."""
    try:
        return fn(*a, **kw)
    except AssertionError as e:
        return f"FAIL: {e}"


def parity_decode(w, kbs, s, rows=None, mh_scores=None, positions=None) -> dict:
    """The GPU's own results of one decode input set against the oracle:
    block scores (the oracle scores the GPU's compressed keys), the selection
    by the band rule, and attention run by the oracle over the GPU's
    selection, for the given (sequence, KV head) rows (all by default)."""
    import numpy as np
    import torch
    import oracle
    from tests import parity
    rows = rows if rows is not None else [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    positions = positions or [w.q_start] * w.B
    worst = worst_mh = err = 0.0
    banded = 0
    status = "ok"
    for b, h in rows:
        p = positions[b]
        Kc = parity.to_f64(s["Kc"][b, h])
        ref = oracle.select_forecast_tile(parity.to_f64(s["F"][b, h]), Kc, [p], w.T, w.scale)[None, :]
        got = parity.to_f64(s["scores"][b, h])
        idx = s["idx"][b, h].cpu().numpy()
        r1 = _check(parity.check_scores, got, ref)
        r2 = _check(parity.check_topk_band, idx, ref, w.k)
        J = oracle.selected_keys(idx[0], p)
        Q = parity.to_f64(s["Q"][b, h * w.G:(h + 1) * w.G, 0])
        o_ref = np.zeros((w.G, w.d))
        if J.size:
            Jt = torch.from_numpy(J).to(s["K"].device)
            KJ, VJ = parity.to_f64(s["K"][b, h].index_select(0, Jt)), parity.to_f64(s["V"][b, h].index_select(0, Jt))
            for g in range(w.G):
                o_ref[g] = oracle.attend(Q[g], KJ, VJ, w.scale)
        tol = parity.ATTN_ATOL_BF16 if w.dtype == "bf16" else 1e-4
        r3 = _check(parity.check_attention, parity.to_f64(s["out"][b, h * w.G:(h + 1) * w.G, 0]), o_ref, tol)
        for r in (r1, r2, r3):
            if isinstance(r, str):
                status = r
        worst = max(worst, r1) if not isinstance(r1, str) else worst
        banded += r2 if not isinstance(r2, str) else 0
        err = max(err, r3) if not isinstance(r3, str) else err
        if mh_scores is not None:
            ref_mh = oracle.select_multihead_tile(parity.to_f64(s["Q"][b, h * w.G:(h + 1) * w.G]), Kc, [p], w.T,
                                                  w.scale)[None, :]
            r4 = _check(parity.check_scores, parity.to_f64(mh_scores[b, h]), ref_mh)
            if isinstance(r4, str):
                status = r4
            else:
                worst_mh = max(worst_mh, r4)
    out = {"status": status, "rows_checked": len(rows), "score_worst_rel": float(f"{worst:.3g}"),
           "banded_rows": int(banded), "attn_max_abs": float(f"{err:.3g}")}
    if mh_scores is not None:
        out["multihead_score_worst_rel"] = float(f"{worst_mh:.3g}")
    return out


# ------------------------------------------------------ algorithmic bytes ----
def algorithmic_bytes(w) -> dict:
    """Bytes each kernel must move for one layer-step (storage dtype)."""
    e = 2 if w.dtype == "bf16" else 4
    rows = w.B * w.Hkv
    kc = rows * w.W * w.d * e
    f = rows * w.d * e
    q = w.B * w.Hq * w.d * e
    o = q
    scores = rows * w.nB * 4
    idx = rows * w.k * 4
    kv = 2 * rows * w.k * 64 * w.d * e
    return {
        "select_forecast": kc + f + scores,
        "select_multihead": kc + q + scores,
        "topk": scores + idx,
        "attention": kv + q + idx + o,
        "topk_attention": scores + idx + kv + q + o,
        "topk_attention_partial": scores + idx + kv + q,
        "select_forecast_merge": kc + f + scores + o,
        # one launch: the next layer's selection and this layer's top-k + attention
        "decode_layer": (kc + f + scores) + (scores + idx + kv + q + o),
        "step": kc + f + scores + (scores + idx) + (kv + q + idx + o),
    }


def pmc_traffic(kernel_files, summary: str):
    """HBM bytes per launch from a committed rocprofv3 PMC summary, or None when
    a kernel source changed since the counters were taken (sha256 of the
    sources' bytes, concatenated in the order given)."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", summary)) as f:
            rec = json.load(f)
        h = hashlib.sha256()
        for kernel_file in ([kernel_files] if isinstance(kernel_files, str) else kernel_files):
            with open(os.path.join(ROOT, kernel_file), "rb") as f:
                h.update(f.read())
        digest = h.hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != digest:
        return None
    return rec.get("traffic_bytes_per_launch")


def calibration_copy(dev) -> None:
    """A plain 1 GiB device copy, ten times: the known-size reference for the
    profiler's FETCH_SIZE / WRITE_SIZE counters in the same run."""
    import torch
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


PREFILL_ATTN_SOURCES = ["kv_block_selection_amd/csrc/attn_prefill.hip", "kv_block_selection_amd/csrc/lds_dma.h",
                        "kv_block_selection_amd/csrc/common.h"]

LAYER_SOURCES = ["kv_block_selection_amd/csrc/attn_decode.hip", "kv_block_selection_amd/csrc/topk_row.h",
                 "kv_block_selection_amd/csrc/select_row.h", "kv_block_selection_amd/csrc/reduce16.h",
                 "kv_block_selection_amd/csrc/common.h"]


def make_sets(kbs, w, dev, n_sets: int):
    import synth.gpu as sg
    import torch
    from synth import workloads as wl
    sets = []
    for i in range(n_sets):
        wi = wl.scaled(w, seed=w.seed + 1000 * i)
        s = {n: sg.tensor(wi.recipe(n), wi.shape(n), dev) for n in ("Q", "F", "K", "V")}
        s["Kc"] = kbs.compress_keys(s["K"])
        s["scores"] = torch.empty((w.B, w.Hkv, 1, w.nB), dtype=torch.float32, device=dev)
        s["idx"] = torch.empty((w.B, w.Hkv, 1, w.k), dtype=torch.int32, device=dev)
        s["out"] = torch.empty_like(s["Q"])
        sets.append(s)
    return sets


# --------------------------------------------- small decode configs (c1, c2) ----
def bench_small_decode(kbs, w, dev, steps: int, warmup: int) -> dict:
    """One decode layer-step of a one-sequence workload (the tiny fp32 one and
    the 32K bf16 one): Forecast selection, top-k and attention per step. bf16
    runs one sparda_decode_layer call per layer (its few rows keep block ranges,
    merged by a second launch); fp32 runs the selection and the fused top-k +
    attention (the layer call is bf16 only). Three input sets rotate. Both
    selectors' cost (scoring + top-k) is timed too, and parity of the step's
    own results against the oracle (every row)."""
    import torch
    sets = make_sets(kbs, w, dev, N_SETS)
    ws_mh = torch.empty(max(1, kbs.workspace_bytes(kbs.OP_SELECT_MULTIHEAD, w.B, w.Hq, w.Hkv, 1, w.T)),
                        dtype=torch.uint8, device=dev)
    ws_l = torch.empty(max(1, kbs.workspace_bytes(kbs.OP_DECODE_LAYER, w.B, w.Hq, w.Hkv, 1, w.T, w.k)),
                       dtype=torch.uint8, device=dev)
    ws_a = torch.empty(max(1, kbs.workspace_bytes(kbs.OP_BLOCK_SPARSE_ATTN, w.B, w.Hq, w.Hkv, 1, w.T, w.k)),
                       dtype=torch.uint8, device=dev)
    mh = [torch.empty_like(s["scores"]) for s in sets]
    idx_mh = [torch.empty_like(s["idx"]) for s in sets]
    bf16 = w.dtype == "bf16"
    for s in sets:
        kbs.select_forecast(s["F"], s["Kc"], w.T, w.q_start, out=s["scores"])

    def step(i):
        s, nxt = sets[i % N_SETS], sets[(i + 1) % N_SETS]
        if bf16:
            kbs.decode_layer(s["scores"], s["Q"], s["K"], s["V"], w.k, w.T, w.q_start, ws_l, idx=s["idx"],
                             out=s["out"], select_next=(nxt["F"], nxt["Kc"], nxt["scores"], w.T, w.q_start))
        else:
            kbs.select_forecast(s["F"], s["Kc"], w.T, w.q_start, out=s["scores"])
            kbs.topk_block_sparse_attn(s["scores"], s["Q"], s["K"], s["V"], w.k, w.T, w.q_start, idx=s["idx"],
                                       out=s["out"], ws=ws_a)

    def sel_f(i):
        s = sets[i % N_SETS]
        kbs.select_forecast(s["F"], s["Kc"], w.T, w.q_start, out=s["scores"])
        kbs.topk_blocks(s["scores"], w.k, out=s["idx"])

    def sel_m(i):
        s = sets[i % N_SETS]
        kbs.select_multihead(s["Q"], s["Kc"], w.T, w.q_start, out=mh[i % N_SETS], ws=ws_mh)
        kbs.topk_blocks(mh[i % N_SETS], w.k, out=idx_mh[i % N_SETS])

    for i in range(max(warmup, N_SETS)):
        step(i)
    torch.cuda.synchronize()
    n = max(N_SETS, steps)
    st = time_graph_stats(step, n)
    sf = time_graph_stats(sel_f, 3 * N_SETS * 10)
    sm = time_graph_stats(sel_m, 3 * N_SETS * 10)
    # each set's scores, selection and output as the step leaves them (every
    # set's scores were computed from its own Forecast and compressed keys)
    for i in range(N_SETS + 1):
        step(i)
    kbs.select_multihead(sets[0]["Q"], sets[0]["Kc"], w.T, w.q_start, out=mh[0], ws=ws_mh)
    torch.cuda.synchronize()
    nbytes = algorithmic_bytes(w)["step"]
    gbps = nbytes / (st["median"] * 1e-3) / 1e9
    par = parity_decode(w, kbs, sets[0], mh_scores=mh[0])
    del sets
    return {"workload": w.description, "steps_per_s_per_layer": round(1e3 / st["median"], 1),
            "us_per_step": _us(st), "steps": n,
            "step": "sparda_decode_layer (+ its merge launch)" if bf16 else
                    "sparda_select_forecast + sparda_topk_block_sparse_attn (fp32)",
            "selection_us": {"forecast": round(sf["median"] * 1e3, 2), "multihead": round(sm["median"] * 1e3, 2)},
            "forecast_vs_multihead_select_speedup": round(sm["median"] / sf["median"], 3),
            "roofline": {"bound": "hbm", "kernel": "step", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                         "algorithmic_bytes": nbytes,
                         "note": "launch-latency bound at this size: the bytes take a few microseconds at peak"},
            "parity": par}


# -------------------------------------------------- the headline (c3) ----
def bench_decode(args, pool=None, n_workers: int = 0) -> dict:
    import torch
    import kv_block_selection_amd as kbs
    from synth import workloads as wl

    kbs.load()
    w = wl.C3_DECODE_128K
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] generating {N_SETS} input sets of {w.name}")
    sets = make_sets(kbs, w, dev, N_SETS)
    for s in sets:
        # the newest token of every sequence again, for the cache-append timings
        s["Knew1"] = s["K"][:, :, w.T - 1:].contiguous()
        s["Vnew1"] = s["V"][:, :, w.T - 1:].contiguous()
        s["Knew2"] = s["K"][:, :, w.T - 2:w.T - 1].contiguous()
        s["Vnew2"] = s["V"][:, :, w.T - 2:w.T - 1].contiguous()
    pos_last = torch.full((w.B,), w.q_start, dtype=torch.int32, device=dev)
    len_win = torch.full((w.B,), w.T - 1, dtype=torch.int32, device=dev)  # token T-1 completes window W-1
    len_nowin = torch.full((w.B,), w.T - 2, dtype=torch.int32, device=dev)  # token T-2 completes none
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ws_attn = torch.zeros(max(1, kbs.workspace_bytes(kbs.OP_BLOCK_SPARSE_ATTN, w.B, w.Hq, w.Hkv, 1, w.T, w.k)),
                          dtype=torch.uint8, device=dev)
    ws_mh = torch.empty(max(1, kbs.workspace_bytes(kbs.OP_SELECT_MULTIHEAD, w.B, w.Hq, w.Hkv, 1, w.T)),
                        dtype=torch.uint8, device=dev)
    ws_layer = torch.zeros(max(1, kbs.workspace_bytes(kbs.OP_DECODE_LAYER, w.B, w.Hq, w.Hkv, 1, w.T, w.k)),
                           dtype=torch.uint8, device=dev)
    mh_scores = [torch.empty_like(s["scores"]) for s in sets]

    def sel(i):
        s = sets[i % N_SETS]
        kbs.select_forecast(s["F"], s["Kc"], w.T, w.q_start, out=s["scores"])

    def sel_mh(i):
        s = sets[i % N_SETS]
        kbs.select_multihead(s["Q"], s["Kc"], w.T, w.q_start, out=mh_scores[i % N_SETS], ws=ws_mh)

    def topk(i):
        s = sets[i % N_SETS]
        kbs.topk_blocks(s["scores"], w.k, out=s["idx"])

    def attn(i):
        s = sets[i % N_SETS]
        kbs.block_sparse_attn(s["Q"], s["K"], s["V"], s["idx"], w.T, w.q_start, out=s["out"], ws=ws_attn)

    def topk_attn(i):  # top-k and attention in one launch, then the merge launch
        s = sets[i % N_SETS]
        kbs.topk_block_sparse_attn(s["scores"], s["Q"], s["K"], s["V"], w.k, w.T, w.q_start, idx=s["idx"],
                                   out=s["out"], ws=ws_attn)

    def topk_attn_partial(i):  # the same without the merge (left in ws_attn)
        s = sets[i % N_SETS]
        kbs.topk_block_sparse_attn(s["scores"], s["Q"], s["K"], s["V"], w.k, w.T, w.q_start, idx=s["idx"],
                                   out=s["out"], ws=ws_attn, merge=False)

    def sel_merge(i):  # selection + the merge of the previous layer's attention
        s, prev = sets[i % N_SETS], sets[(i - 1) % N_SETS]
        kbs.select_forecast(s["F"], s["Kc"], w.T, w.q_start, out=s["scores"],
                            merge_from=(ws_attn, prev["out"], w.T, w.k))

    def step_one_launch(i):
        # layer i in one launch: its top-k + attention (finished output) and
        # layer i+1's Forecast selection, both from layer i's projections
        s, nxt = sets[i % N_SETS], sets[(i + 1) % N_SETS]
        kbs.decode_layer(s["scores"], s["Q"], s["K"], s["V"], w.k, w.T, w.q_start, ws_layer, idx=s["idx"],
                         out=s["out"], select_next=(nxt["F"], nxt["Kc"], nxt["scores"], w.T, w.q_start))

    def step_two_launches(i):
        # layer i as two launches: top-k + attention leaving its block ranges
        # in ws_attn, then the next layer's selection merging them
        s, nxt = sets[i % N_SETS], sets[(i + 1) % N_SETS]
        kbs.topk_block_sparse_attn(s["scores"], s["Q"], s["K"], s["V"], w.k, w.T, w.q_start, idx=s["idx"],
                                   out=s["out"], ws=ws_attn, merge=False)
        kbs.select_forecast(nxt["F"], nxt["Kc"], w.T, w.q_start, out=nxt["scores"],
                            merge_from=(ws_attn, s["out"], w.T, w.k))

    def step_layer(i):  # one layer at a time: selection, then top-k + attention + merge
        sel(i)
        topk_attn(i)

    def step_separate(i):  # the same with top-k as a launch of its own
        sel(i)
        topk(i)
        attn(i)

    # Decode-time state maintenance: append the step's token to K, V and
    # compress the window it completes (every 16th step) or none. The tokens
    # written are the ones already there, so the inputs stay as they are.
    def append_win(i):
        s = sets[i % N_SETS]
        kbs.append_kv(s["Knew1"], s["Vnew1"], s["K"], s["V"], len_win, k_cmp=s["Kc"])

    def append_nowin(i):
        s = sets[i % N_SETS]
        kbs.append_kv(s["Knew2"], s["Vnew2"], s["K"], s["V"], len_nowin, k_cmp=s["Kc"])

    def step_q_pos(i):  # the one-launch step with per-sequence positions (all at T - 1)
        s, nxt = sets[i % N_SETS], sets[(i + 1) % N_SETS]
        kbs.decode_layer(s["scores"], s["Q"], s["K"], s["V"], w.k, w.T, 0, ws_layer, idx=s["idx"], out=s["out"],
                         q_pos=pos_last, select_next=(nxt["F"], nxt["Kc"], nxt["scores"], w.T, 0, pos_last))

    log("[bench] warmup (eager)")
    for i in range(N_SETS):
        sel(i)
    for i in range(max(args.warmup, 2 * N_SETS)):
        step_one_launch(i)
    torch.cuda.synchronize()
    eager = time_loop_stats(step_one_launch, args.steps, stream)
    log(f"[bench] eager step {eager['median'] * 1e3:.1f} us; timing {args.steps} steps x {REPEATS} graph replays")
    main_st = time_graph_stats(step_one_launch, args.steps)
    ms_step = main_st["median"]
    n_var = 3 * N_SETS * max(1, 60 // (3 * N_SETS))  # 54 calls per graph for the comparisons
    variants = {"two_launches_per_layer": time_graph_stats(step_two_launches, n_var),
                "one_layer_at_a_time": time_graph_stats(step_layer, n_var),
                "topk_separate": time_graph_stats(step_separate, n_var)}
    log(f"[bench] graph step {ms_step * 1e3:.1f} us (median of {REPEATS} x {args.steps}; two launches per layer "
        f"{variants['two_launches_per_layer']['median'] * 1e3:.1f} us, one layer at a time "
        f"{variants['one_layer_at_a_time']['median'] * 1e3:.1f} us, top-k on its own "
        f"{variants['topk_separate']['median'] * 1e3:.1f} us); per-kernel graphs")
    for i in range(N_SETS):
        sel(i)
    kn = {"select_forecast": sel, "topk": topk, "attention": attn, "select_multihead": sel_mh,
          "topk_attention": topk_attn, "topk_attention_partial": topk_attn_partial,
          "select_forecast_merge": sel_merge}
    kst = {k: time_graph_stats(fn, n_var) for k, fn in kn.items()}
    kst["decode_layer"] = main_st
    ms = {k: v["median"] for k, v in kst.items()}
    ms_extra = {"append_kv_with_window": time_graph(append_win, n_var), "append_kv": time_graph(append_nowin, n_var),
                "step_with_q_pos": time_graph(step_q_pos, n_var)}
    # leave every set's Forecast scores, selection and output as the step makes them
    for i in range(N_SETS):
        sel(i)
    for i in range(N_SETS + 1):
        step_one_launch(i)
    sel_mh(0)
    torch.cuda.synchronize()
    projection = bench_projection(kbs, w, dev, REPEATS)
    token_level = bench_token_level(kbs, w, sets, dev, n_var)
    decoupled = (decoupled_layers(kbs, w, sets, ws_attn, dev, algorithmic_bytes(w)["step"], n_layers=3 * args.steps)
                 if args.decoupled_layers else None)
    log("[bench] parity of the step's results (all rows of one input set) against the oracle")
    par = parity_decode(w, kbs, sets[0], mh_scores=mh_scores[0])

    nbytes = algorithmic_bytes(w)
    gbps = {k: nbytes[k] / (ms[k] * 1e-3) / 1e9 for k in ms}
    dominant = "decode_layer"  # the step is one launch per layer: that launch is the roofline kernel
    step_gbps = nbytes["step"] / (ms_step * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(1e3 / ms_step, 2),
        "unit": "steps/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.description, "B": w.B, "T": w.T, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d,
                   "block": w.block, "top_k": w.k, "selector": "forecast", "input_sets_rotated": N_SETS,
                   "schedule": "consecutive layers (the input sets in turn), one launch per layer: layer l's top-k + "
                               "attention (finished output) and layer l+1's Forecast selection, both from layer l's "
                               "projections"},
        "timing": {"repeats": REPEATS, "steps_per_repeat": args.steps, "ms_per_step_min": round(main_st["min"], 5),
                   "ms_per_step_max": round(main_st["max"], 5), "ms_per_step_eager": round(eager["median"], 5)},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(gbps[dominant], 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps[dominant] / HBM_PEAK_GBPS, 4),
                     "traffic": pmc_traffic(LAYER_SOURCES, "decode_layer_c3_traffic.json"),
                     "algorithmic_bytes_per_launch": nbytes[dominant]},
        "step_hbm_GBps": round(step_gbps, 1),
        "step_hbm_frac": round(step_gbps / HBM_PEAK_GBPS, 4),
        "ms_per_step_variants": {k: round(v["median"], 5) for k, v in variants.items()},
        "kernel_us": {k: round(v * 1e3, 2) for k, v in ms.items()},
        "kernel_us_spread": {k: [round(v["min"] * 1e3, 2), round(v["max"] * 1e3, 2)] for k, v in kst.items()},
        "kernel_GBps": {k: round(v, 1) for k, v in gbps.items()},
        "selection_us": {"forecast": round((ms["select_forecast"] + ms["topk"]) * 1e3, 2),
                         "multihead": round((ms["select_multihead"] + ms["topk"]) * 1e3, 2)},
        "forecast_vs_multihead_select_speedup": round(ms["select_multihead"] / ms["select_forecast"], 3),
        "multihead_bytes_bound_ratio": round((nbytes["select_multihead"] + 2 * w.B * w.Hkv * w.G * w.W * 4) /
                                             nbytes["select_forecast"], 3),
        "state_maintenance_us": {k: round(v * 1e3, 2) for k, v in ms_extra.items()},
        "upstream_projection": projection,
        "token_level": token_level,
        "parity": par,
    }
    if decoupled is not None:
        result["decoupled_layers"] = decoupled
    if args.calibration_copy:
        calibration_copy(dev)
        result["calibration_copy_bytes"] = 1 << 30
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: the oracle on the step's rows, 1 thread and {n_workers} worker processes")
        result["cpu_baseline"] = cpu_baseline(w, sets[0], pool, n_workers)
    del sets
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return result


def decoupled_layers(kbs, w, sets, ws_attn, dev, step_bytes: int, n_layers: int) -> dict:
    """Consecutive layers in the order the method runs them: layer j's Forecast
    selects layer j+1's blocks, so at the start of layer j the selection and
    top-k for layer j+1 go on a second stream while layer j attends with the
    blocks selected during layer j-1. Layer j+1 begins when layer j's
    attention has finished. The input sets stand in for the layers (set j % 3).
    Each layer does the whole step (Forecast scoring, top-k, attention) on its
    own data; timed with HIP events on the attention stream, after warm-up,
    and beside the same layers run one after another on one stream."""
    import torch
    main = torch.cuda.current_stream(dev)
    side = torch.cuda.Stream(device=dev)
    ev_sel = [torch.cuda.Event() for _ in range(N_SETS)]
    ev_begin = torch.cuda.Event()

    def select(j, stream):
        s = sets[j % N_SETS]
        kbs.select_forecast(s["F"], s["Kc"], w.T, w.q_start, out=s["scores"], stream=stream)
        kbs.topk_blocks(s["scores"], w.k, out=s["idx"], stream=stream)

    def attend(j):
        s = sets[j % N_SETS]
        kbs.block_sparse_attn(s["Q"], s["K"], s["V"], s["idx"], w.T, w.q_start, out=s["out"], ws=ws_attn,
                              stream=main)

    def layers(j0, n, overlap):
        for j in range(j0, j0 + n):
            if overlap:
                side.wait_event(ev_begin)  # layer j has begun: its Forecast exists
                select(j + 1, side)
                ev_sel[(j + 1) % N_SETS].record(side)
                main.wait_event(ev_sel[j % N_SETS])
            else:
                select(j + 1, main)
            attend(j)
            ev_begin.record(main)

    out = {}
    for name, overlap in (("sequential", False), ("overlapped", True)):
        select(0, main)
        ev_sel[0].record(main)
        ev_begin.record(main)
        layers(0, 6, overlap)  # warm-up
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(main)
        layers(6, n_layers, overlap)
        end.record(main)
        torch.cuda.synchronize()
        us = start.elapsed_time(end) * 1e3 / n_layers
        out[name] = {"us_per_layer": round(us, 2), "steps_per_s_per_layer": round(1e6 / us, 1),
                     "hbm_frac": round(step_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    out["layers_timed"] = n_layers
    return out


def bench_token_level(kbs, w, sets, dev, per_graph: int) -> dict:
    """The token-level Forecast variant at the same shape: the Forecast vector
    scores all T key tokens of every row, the top k_tok = 64 * k tokens are
    kept (the block path's token budget) and attended. Algorithmic bytes: all
    of K plus the scores for the scoring, the scores and the kept indices for
    the top-k, the kept K and V rows plus Q, O and the indices for the
    attention (its staging copy is the implementation's own traffic)."""
    import torch
    k_tok = 64 * w.k
    rows = w.B * w.Hkv
    bufs = []
    for s in sets:
        bufs.append({"tok_scores": torch.empty((w.B, w.Hkv, 1, w.T), dtype=torch.float32, device=dev),
                     "tok_idx": torch.empty((w.B, w.Hkv, 1, k_tok), dtype=torch.int32, device=dev),
                     "out": torch.empty_like(s["Q"])})
    need = kbs.workspace_bytes(kbs.OP_TOKEN_ATTN, w.B, w.Hq, w.Hkv, 1, w.T, k_tok)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def score(i):
        s, b = sets[i % N_SETS], bufs[i % N_SETS]
        kbs.select_tokens(s["F"], s["K"], w.q_start, scale=w.scale, out=b["tok_scores"])

    def topk(i):
        b = bufs[i % N_SETS]
        kbs.topk_blocks(b["tok_scores"], k_tok, out=b["tok_idx"])

    def attn(i):
        s, b = sets[i % N_SETS], bufs[i % N_SETS]
        kbs.token_sparse_attn(s["Q"], s["K"], s["V"], b["tok_idx"], w.q_start, scale=w.scale, out=b["out"], ws=ws)

    for i in range(N_SETS):
        score(i)
        topk(i)
        attn(i)
    torch.cuda.synchronize()
    ms = {"select_tokens": time_graph(score, per_graph), "topk_tokens": time_graph(topk, per_graph),
          "token_attention": time_graph(attn, per_graph)}
    row_bytes = w.d * 2
    nbytes = {"select_tokens": rows * w.T * row_bytes + rows * row_bytes + rows * w.T * 4,
              "topk_tokens": rows * w.T * 4 + rows * k_tok * 4,
              "token_attention": 2 * rows * k_tok * row_bytes + 2 * w.B * w.Hq * row_bytes + rows * k_tok * 4}
    step = sum(ms.values())
    log(f"[bench] token-level variant: {step * 1e3:.1f} us per layer-step")
    return {"k_tok": k_tok,
            "kernel_us": {k: round(v * 1e3, 2) for k, v in ms.items()},
            "kernel_GBps": {k: round(nbytes[k] / (ms[k] * 1e-3) / 1e9, 1) for k in ms},
            "ms_per_step": round(step, 5),
            "what": "token scores over all of K, top-k of 131072 scores per row, attention over the kept tokens"}


def bench_projection(kbs, w, dev, replays: int, D: int = 4096, n_layers: int = 8) -> dict:
    """The Q/K/V/Forecast projection GEMM upstream of selection (not part of
    the step): one decode token per sequence, hidden size D, one Forecast set.
    Weights of n_layers layers rotate (470 MB at B = 16), so each launch
    streams its weights from HBM as a real decode pass over the layers would;
    algorithmic bytes = weights + hidden states + outputs."""
    import torch
    import synth.gpu as sg
    from synth import workloads as wl
    out = {}
    for B in (w.B, 64):
        wB = wl.scaled(w, B=B)
        N = wl.qkvf_rows(wB, 1)
        xs = [sg.tensor(wl.hidden_recipe(wB, layer=l), (B, D), dev) for l in range(n_layers)]
        ws = [sg.tensor(wl.qkvf_weight_recipe(wB, D, layer=l), (N, D), dev) for l in range(n_layers)]
        outs = (torch.empty((B, w.Hq, 1, w.d), dtype=torch.bfloat16, device=dev),
                torch.empty((B, w.Hkv, 1, w.d), dtype=torch.bfloat16, device=dev),
                torch.empty((B, w.Hkv, 1, w.d), dtype=torch.bfloat16, device=dev),
                torch.empty((1, B, w.Hkv, 1, w.d), dtype=torch.bfloat16, device=dev))

        def proj(i):
            kbs.project_qkvf(xs[i % n_layers], ws[i % n_layers], w.Hq, w.Hkv, 1, out=outs)

        ms = time_graph(proj, n_layers, max(1, replays))
        nbytes = N * D * 2 + B * D * 2 + B * N * 2
        gbps = nbytes / (ms * 1e-3) / 1e9
        out[f"B{B}"] = {"us": round(ms * 1e3, 2), "bytes": nbytes, "GBps": round(gbps, 1),
                        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
                        "TFLOPs": round(2.0 * B * N * D / (ms * 1e-3) / 1e12, 1)}
        del xs, ws
    out["shape"] = f"x [B, {D}] times W [{wl.qkvf_rows(w, 1)}, {D}] (32 Q + 8 K + 8 V + 8 Forecast heads of 128)"
    return out




# ------------------------------------------------------ offload (c4) ----
def bench_offload_cfg(args) -> dict:
    """Two-layer decode step at B=64, T=128K with layer 1's KV (32 GiB) in pinned
    host memory: both selections, layer 0's attention from HBM overlapped with
    the gather of layer 1's selected blocks over the host link on a side stream,
    then layer 1's attention from staging. Also times each part alone, a plain
    1 GiB pinned host-to-device copy (the link's practical rate), a sweep of the
    gather's workgroups and the staging buffer kept as a block cache; parity of
    both layers' results on sampled rows."""
    import numpy as np
    import torch
    import kv_block_selection_amd as kbs
    from kv_block_selection_amd.lookahead import LookaheadStep
    from synth import workloads as wl
    from synth.offload import offload_layers

    kbs.load()
    w = wl.C4_OFFLOAD
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] generating {w.name} (32 GiB KV in HBM, 32 GiB pinned host)")
    l0, l1 = offload_layers(w, kbs.compress_keys, dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    st = LookaheadStep(w.B, w.Hq, w.Hkv, w.T, w.k, torch.bfloat16, dev)
    T, q = w.T, w.q_start
    link_bytes = 2 * w.B * w.Hkv * w.k * w.block * w.d * 2

    def step(i):
        st.step(l0, l1, stream)

    def select(i):
        st.select(l0, l1, stream)

    def attn0(i):
        kbs.block_sparse_attn(l0["Q"], l0["K"], l0["V"], st.idx0, T, q, out=st.out0, ws=st.ws, stream=stream)

    def attn1(i):
        kbs.block_sparse_attn(l1["Q"], st.stage_k, st.stage_v, st.idx1, T, q, kv_mode=kbs.KV_STAGING,
                              out=st.out1, ws=st.ws, stream=stream)

    def gather(nwg):
        return lambda i: kbs.prefetch_blocks(l1["host_K"], l1["host_V"], st.idx1.view(w.B, w.Hkv, w.k),
                                             st.stage_k, st.stage_v, num_workgroups=nwg, stream=stream)

    for i in range(max(2, args.warmup)):
        step(i)
    torch.cuda.synchronize()
    n = 4
    step_st = time_loop_stats(step, n, stream)
    ms_step = step_st["median"]
    log(f"[bench] offload step {ms_step:.3f} ms; parts alone")
    parts = {"select_both_layers": time_loop(select, n, stream), "attn_layer0_hbm": time_loop(attn0, n, stream),
             "gather_layer1": time_loop(gather(0), n, stream), "attn_layer1_staging": time_loop(attn1, n, stream)}
    host = l1["host_K"].view(-1).view(torch.uint8)[: 1 << 30]
    dst = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    ms_copy = time_loop(lambda i: dst.copy_(host, non_blocking=True), 2, stream)
    del dst
    sweep = {}
    for nwg in (16, 32, 64, 128, 256):
        g = time_loop(gather(nwg), 1, stream, repeats=3)
        sweep[nwg] = {"gather_ms": round(g, 4), "gather_GBps": round(link_bytes / (g * 1e-3) / 1e9, 2)}
    cached = bench_cached_gather(kbs, w, l1, st, stream, dev)
    # results of one step, for parity (sampled rows of both layers)
    step(0)
    torch.cuda.synchronize()
    par = parity_offload(w, kbs, l0, l1, st)
    cpu_loop = bench_cpu_in_loop_gather(w, l1, st, stream)
    serial = sum(parts.values())
    # the gather waits only for layer 1's selection; layer 0's selection and
    # attention can hide behind it
    hideable = min(parts["select_both_layers"] / 2 + parts["attn_layer0_hbm"], parts["gather_layer1"])
    link_gbps = link_bytes / (parts["gather_layer1"] * 1e-3) / 1e9
    h2d = (1 << 30) / (ms_copy * 1e-3) / 1e9
    out = {"workload": w.description, "steps_per_s_per_layer": round(2e3 / ms_step, 3),
           "ms_per_step": {k: (round(v, 4) if k != "n" else v) for k, v in step_st.items()},
           "roofline": {"bound": "host_link", "kernel": "prefetch", "achieved": round(link_gbps, 2),
                        "peak": HOST_LINK_PEAK_GBPS, "unit": "GB/s", "frac": round(link_gbps / HOST_LINK_PEAK_GBPS, 4),
                        "traffic": None, "frac_of_measured_h2d": round(link_gbps / h2d, 4)},
           "link_bytes_per_step": link_bytes,
           "h2d_memcpy_1GiB_GBps": round(h2d, 2),
           "parts_ms": {k: round(v, 4) for k, v in parts.items()},
           "serial_ms": round(serial, 4),
           "overlap_hidden_frac": round((serial - ms_step) / hideable, 3) if hideable > 0 else None,
           "overlap_note": "hideable = layer 0 selection (half of both selections) + layer 0 attention",
           "workgroup_sweep": sweep,
           "cached_gather": cached,
           "cpu_in_the_loop_gather": cpu_loop,
           "parity": par}
    del l0, l1, st, host
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def bench_cpu_in_loop_gather(w, l1, st, stream, n_rows: int = 64) -> dict:
    """The gather with the CPU in the loop, for contrast with the device-side
    gather: the host copies layer 1's selected indices back (a sync on the
    step's path) and issues one hipMemcpyAsync per selected K and V block from
    pinned host memory into the staging slots. Timed over n_rows (sequence, KV
    head) rows and scaled to the step's B * Hkv rows (the cost is per copy);
    the staged bytes of those rows are checked against the device gather's."""
    import ctypes
    import os
    import time
    import torch
    hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
    hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    hip.hipMemcpyAsync.restype = ctypes.c_int
    h2d = 1  # hipMemcpyHostToDevice
    blk = w.block * w.d * 2
    rows = [(r // w.Hkv, r % w.Hkv) for r in range(0, w.B * w.Hkv, (w.B * w.Hkv) // n_rows)][:n_rows]
    hk, hv = l1["host_K"], l1["host_V"]
    ref_k = torch.stack([st.stage_k[b, h].clone() for b, h in rows])
    ref_v = torch.stack([st.stage_v[b, h].clone() for b, h in rows])
    for b, h in rows:
        st.stage_k[b, h].zero_()
        st.stage_v[b, h].zero_()
    torch.cuda.synchronize()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    times = []
    for rep in range(3):
        t0 = time.perf_counter()
        idx = st.idx1.view(w.B, w.Hkv, w.k).cpu()  # device -> host, waits for the selection
        for b, h in rows:
            for j in range(w.k):
                bi = int(idx[b, h, j])
                if bi < 0:
                    continue
                for src, dst in ((hk, st.stage_k), (hv, st.stage_v)):
                    rc = hip.hipMemcpyAsync(dst[b, h, j].data_ptr(), src[b, h, bi * w.block].data_ptr(), blk, h2d,
                                            sptr)
                    if rc != 0:
                        raise RuntimeError(f"hipMemcpyAsync failed ({rc})")
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
    same = all(torch.equal(st.stage_k[b, h], ref_k[i]) and torch.equal(st.stage_v[b, h], ref_v[i])
               for i, (b, h) in enumerate(rows))
    t = sorted(times)[1]
    copies = 2 * w.k * len(rows)
    scale = (w.B * w.Hkv) / len(rows)
    return {"rows_timed": len(rows), "copies_timed": copies, "ms_rows_timed": round(t * 1e3, 3),
            "ms_per_step_scaled": round(t * 1e3 * scale, 2), "us_per_copy": round(t * 1e6 / copies, 2),
            "GBps": round(copies * blk / t / 1e9, 2), "staged_bytes_match_device_gather": bool(same),
            "how": "D2H of the indices, then one hipMemcpyAsync per selected 16 KiB K or V block from pinned "
                   "host memory, issued from a Python loop through ctypes (median of 3)"}


def parity_offload(w, kbs, l0, l1, st, n_rows: int = 32) -> dict:
    """Both layers of the offloaded step on sampled (sequence, KV head) rows:
    scores (layer 0 by its own Forecast, layer 1 by layer 0's Forecast of the
    next layer), selection by the band rule, attention of layer 1 from the
    host copy of its KV over the GPU's selection."""
    import numpy as np
    import torch
    import oracle
    from tests import parity
    rng = np.random.default_rng(0)
    flat = rng.choice(w.B * w.Hkv, n_rows, replace=False)
    worst = err = 0.0
    banded = 0
    status = "ok"
    for layer in (0, 1):
        F = l0["F_self"] if layer == 0 else l0["F_next"]
        Kc = l0["Kc"] if layer == 0 else l1["Kc"]
        scores = st.scores0 if layer == 0 else st.scores1
        idx = st.idx0 if layer == 0 else st.idx1
        out = st.out0 if layer == 0 else st.out1
        Q = l0["Q"] if layer == 0 else l1["Q"]
        for r in flat:
            b, h = divmod(int(r), w.Hkv)
            ref = oracle.select_forecast_tile(parity.to_f64(F[b, h]), parity.to_f64(Kc[b, h]), [w.q_start], w.T,
                                              w.scale)[None, :]
            r1 = _check(parity.check_scores, parity.to_f64(scores[b, h]), ref)
            gi = idx[b, h].cpu().numpy()
            r2 = _check(parity.check_topk_band, gi, ref, w.k)
            J = oracle.selected_keys(gi[0], w.q_start)
            if layer == 0:
                Jt = torch.from_numpy(J).to(Q.device)
                KJ, VJ = l0["K"][b, h].index_select(0, Jt), l0["V"][b, h].index_select(0, Jt)
            else:
                Jt = torch.from_numpy(J)
                KJ, VJ = l1["host_K"][b, h].index_select(0, Jt), l1["host_V"][b, h].index_select(0, Jt)
            KJ, VJ = parity.to_f64(KJ), parity.to_f64(VJ)
            Qr = parity.to_f64(Q[b, h * w.G:(h + 1) * w.G, 0])
            o_ref = np.stack([oracle.attend(Qr[g], KJ, VJ, w.scale) for g in range(w.G)]) if J.size else 0 * Qr
            r3 = _check(parity.check_attention, parity.to_f64(out[b, h * w.G:(h + 1) * w.G, 0]), o_ref,
                        parity.ATTN_ATOL_BF16)
            for x in (r1, r2, r3):
                if isinstance(x, str):
                    status = x
            worst = max(worst, r1) if not isinstance(r1, str) else worst
            banded += r2 if not isinstance(r2, str) else 0
            err = max(err, r3) if not isinstance(r3, str) else err
    return {"status": status, "rows_checked": 2 * n_rows, "score_worst_rel": float(f"{worst:.3g}"),
            "banded_rows": int(banded), "attn_max_abs": float(f"{err:.3g}")}


# ------------------------------------------------------- prefill (c5) ----
def bench_prefill_cfg(args) -> dict:
    """A 4096-query chunk at the end of a 128K context (B=1, 32/8 heads): Forecast
    scoring of every 64-query tile, top-64 per tile, block-sparse attention,
    each on the matrix cores except top-k; inputs resident in HBM. The
    multi-head selector is timed beside the Forecast."""
    import torch
    import kv_block_selection_amd as kbs
    import synth.gpu as sg
    from synth import workloads as wl

    kbs.load()
    w = wl.C5_PREFILL
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] generating {w.name}")
    s = {n: sg.tensor(w.recipe(n), w.shape(n), dev) for n in ("Q", "F", "K", "V")}
    s["Kc"] = kbs.compress_keys(s["K"])
    scores = torch.empty((w.B, w.Hkv, w.n_tiles, w.nB), dtype=torch.float32, device=dev)
    mh = torch.empty_like(scores)
    idx = torch.empty((w.B, w.Hkv, w.n_tiles, w.k), dtype=torch.int32, device=dev)
    out = torch.empty_like(s["Q"])

    def sel(i):
        kbs.select_forecast(s["F"], s["Kc"], w.T, w.q_start, out=scores)

    def topk(i):
        kbs.topk_blocks(scores, w.k, out=idx)

    def attn(i):
        kbs.block_sparse_attn(s["Q"], s["K"], s["V"], idx, w.T, w.q_start, out=out)

    def sel_mh(i):
        kbs.select_multihead(s["Q"], s["Kc"], w.T, w.q_start, out=mh)

    def step(i):
        sel(i)
        topk(i)
        attn(i)

    for i in range(max(3, args.warmup)):
        step(i)
    torch.cuda.synchronize()
    n = 20
    step_st = time_graph_stats(step, n)
    kst = {"select_forecast": time_graph_stats(sel, n), "topk": time_graph_stats(topk, n),
           "attention": time_graph_stats(attn, n), "select_multihead": time_graph_stats(sel_mh, 5)}
    ms = {k: v["median"] for k, v in kst.items()}
    step(0)
    sel_mh(0)
    torch.cuda.synchronize()
    fl = prefill_flops(w, idx.cpu().numpy())
    tf = {k: fl[k] / (ms[k] * 1e-3) / 1e12 for k in fl}
    roof = {k: {"bound": "mfma", "kernel": k, "achieved": round(tf[k], 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tf[k] / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None}
            for k in fl}
    # HBM bytes of the attention launch from the committed PMC record (null
    # when its source changed since the counters were taken)
    roof["attention"]["traffic"] = pmc_traffic(PREFILL_ATTN_SOURCES, "prefill_attn_c5_traffic.json")
    if args.calibration_copy:
        calibration_copy(dev)
    par = parity_prefill(w, s, scores, mh, idx, out)
    del s
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {"workload": w.description, "chunks_per_s": round(1e3 / step_st["median"], 3),
            "us_per_chunk": _us(step_st),
            "roofline": roof["attention"], "roofline_per_kernel": roof,
            "kernel_us": {k: round(v * 1e3, 2) for k, v in ms.items()},
            "kernel_us_spread": {k: [round(v["min"] * 1e3, 2), round(v["max"] * 1e3, 2)] for k, v in kst.items()},
            "algorithmic_gflop": {k: round(v / 1e9, 3) for k, v in fl.items()},
            "mfma_utilisation": {k: round(v / MFMA_BF16_PEAK_TFLOPS, 4) for k, v in tf.items()},
            "selection_us": {"forecast": round((ms["select_forecast"] + ms["topk"]) * 1e3, 2),
                             "multihead": round((ms["select_multihead"] + ms["topk"]) * 1e3, 2)},
            "forecast_vs_multihead_select_speedup": round(ms["select_multihead"] / ms["select_forecast"], 3),
            "multihead_exp_per_chunk": 2 * w.G * fl["select_forecast"] // (2 * w.d),
            "parity": par}


def parity_prefill(w, s, scores, mh, idx, out, n_pairs: int = 12) -> dict:
    """Sampled (KV head, query tile) pairs of the chunk, all 64 queries of
    each: Forecast and multi-head tile scores (the oracle scores the GPU's
    compressed keys), the selection by the band rule, and attention of every
    query head of the group over the GPU's selection."""
    import numpy as np
    import oracle
    from tests import parity
    rng = np.random.default_rng(1)
    pairs = [(0, 0), (w.Hkv - 1, w.n_tiles - 1)] + [(int(h), int(t)) for h, t in
                                                    zip(rng.integers(0, w.Hkv, n_pairs - 2),
                                                        rng.integers(0, w.n_tiles, n_pairs - 2))]
    worst = worst_mh = err = 0.0
    banded = 0
    status = "ok"
    for h, t in pairs:
        i0, i1 = t * w.tile, min(w.Tq, (t + 1) * w.tile)
        pos = [w.q_start + i for i in range(i0, i1)]
        Kc = parity.to_f64(s["Kc"][0, h])
        ref = oracle.select_forecast_tile(parity.to_f64(s["F"][0, h, i0:i1]), Kc, pos, w.T, w.scale)[None, :]
        Qg = parity.to_f64(s["Q"][0, h * w.G:(h + 1) * w.G, i0:i1])
        ref_mh = oracle.select_multihead_tile(Qg, Kc, pos, w.T, w.scale)[None, :]
        r1 = _check(parity.check_scores, parity.to_f64(scores[0, h, t])[None, :], ref)
        r4 = _check(parity.check_scores, parity.to_f64(mh[0, h, t])[None, :], ref_mh)
        gi = idx[0, h, t].cpu().numpy()
        r2 = _check(parity.check_topk_band, gi[None, :], ref, w.k)
        K64, V64 = parity.to_f64(s["K"][0, h, : pos[-1] + 1]), parity.to_f64(s["V"][0, h, : pos[-1] + 1])
        o_ref = np.zeros((w.G, i1 - i0, w.d))
        for qi, p in enumerate(pos):
            J = oracle.selected_keys(gi, p)
            if J.size:
                for g in range(w.G):
                    o_ref[g, qi] = oracle.attend(Qg[g, qi], K64[J], V64[J], w.scale)
        r3 = _check(parity.check_attention, parity.to_f64(out[0, h * w.G:(h + 1) * w.G, i0:i1]), o_ref,
                    parity.ATTN_ATOL_BF16)
        for x in (r1, r2, r3, r4):
            if isinstance(x, str):
                status = x
        worst = max(worst, r1) if not isinstance(r1, str) else worst
        worst_mh = max(worst_mh, r4) if not isinstance(r4, str) else worst_mh
        banded += r2 if not isinstance(r2, str) else 0
        err = max(err, r3) if not isinstance(r3, str) else err
    return {"status": status, "tiles_checked": len(pairs), "queries_per_tile": w.tile,
            "score_worst_rel": float(f"{worst:.3g}"), "multihead_score_worst_rel": float(f"{worst_mh:.3g}"),
            "banded_tiles": int(banded), "attn_max_abs": float(f"{err:.3g}")}


def bench_cached_gather(kbs, w, l1, st, stream, dev, steps: int = 8) -> dict:
    """The gather of layer 1 with the staging buffer kept as a block cache
    (k slots per row, the same 1 GiB per tensor): sequences of selections in
    which a fixed share of each row's blocks stays from one step to the next
    (synthetic: the pages give no figure for it), the first step cold and
    untimed. Reports ms per gather and the link bytes it moved."""
    import numpy as np
    import torch

    rows = w.B * w.Hkv
    block_bytes = 2 * w.block * w.d * 2  # K and V, bf16
    out = {}
    tags = torch.empty((w.B, w.Hkv, w.k), dtype=torch.int32, device=dev)
    slot_of = torch.empty((w.B, w.Hkv, w.k), dtype=torch.int32, device=dev)
    for keep in (0.0, 0.5, 0.9):
        rng = np.random.default_rng(int(keep * 100) + 7)
        cur = np.stack([rng.choice(w.nB, w.k, replace=False) for _ in range(rows)])
        seq = [cur.copy()]
        n_new = w.k - int(round(keep * w.k))
        for _ in range(steps - 1):
            nxt = cur.copy()
            for r in range(rows):
                drop = rng.choice(w.k, n_new, replace=False)
                pool = np.setdiff1d(np.arange(w.nB), cur[r])
                nxt[r, drop] = rng.choice(pool, n_new, replace=False)
            seq.append(nxt)
            cur = nxt
        idx = [torch.from_numpy(np.sort(x, axis=1).astype(np.int32)).view(w.B, w.Hkv, w.k).to(dev) for x in seq]
        tags.fill_(-1)
        kbs.prefetch_blocks_cached(l1["host_K"], l1["host_V"], idx[0], tags, slot_of, st.stage_k, st.stage_v,
                                   stream=stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for x in idx[1:]:
            kbs.prefetch_blocks_cached(l1["host_K"], l1["host_V"], x, tags, slot_of, st.stage_k, st.stage_v,
                                       stream=stream)
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1) / (steps - 1)
        moved = rows * n_new * block_bytes
        out[f"keep_{int(keep * 100)}pct"] = {"ms_per_gather": round(ms, 4), "link_bytes": moved,
                                            "link_GBps": round(moved / (ms * 1e-3) / 1e9, 2)}
        log(f"[bench] cached gather, {int(keep * 100)}% of blocks kept: {ms:.3f} ms, {moved} B")
    return out


def bench_pipeline(args, L: int = 4, B: int = 16) -> int:
    """An L-layer offloaded decode step (layer 0 in HBM, layers 1 .. L-1 with
    K/V in pinned host memory, B=16, T=128K, top-64): each layer's blocks are
    gathered into one of two staging buffers while the previous layer attends
    from the other. Also times each layer's gather and the device work alone."""
    import torch
    import kv_block_selection_amd as kbs
    from kv_block_selection_amd.pipeline import LayerPipeline
    from synth import workloads as wl
    from synth.offload import offload_stack, set_lookahead

    kbs.load()
    w = wl.scaled(wl.C4_OFFLOAD, B=B)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] generating a {L}-layer stack at B={B} ({L - 1} x {B * 8 * 2 * w.T * 256 >> 30} GiB pinned host)")
    layers = offload_stack(w, L, kbs.compress_keys, dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    pipe = LayerPipeline(L, w.B, w.Hq, w.Hkv, w.T, w.k, torch.bfloat16, dev)
    T, q = w.T, w.q_start
    link_bytes = (L - 1) * 2 * w.B * w.Hkv * w.k * w.block * w.d * 2
    for i in range(args.warmup):
        pipe.step(layers, stream)
    torch.cuda.synchronize()
    n = max(3, min(args.steps, 10))
    ms_step = time_loop(lambda i: pipe.step(layers, stream), n, stream)
    sk, sv = pipe.stage[0]

    def gather_only(i):
        for l in range(1, L):
            kbs.prefetch_blocks(layers[l]["host_K"], layers[l]["host_V"], pipe.idx[l].view(w.B, w.Hkv, w.k), sk, sv,
                                stream=stream)

    def device_only(i):
        kbs.select_forecast(layers[0]["F_self"], layers[0]["Kc"], T, q, out=pipe.scores[0], stream=stream)
        kbs.topk_blocks(pipe.scores[0], w.k, out=pipe.idx[0], stream=stream)
        kbs.block_sparse_attn(layers[0]["Q"], layers[0]["K"], layers[0]["V"], pipe.idx[0], T, q, out=pipe.out[0],
                              ws=pipe.ws, stream=stream)
        for l in range(1, L):
            kbs.select_forecast(layers[l - 1]["F_next"], layers[l]["Kc"], T, q, out=pipe.scores[l], stream=stream)
            kbs.topk_blocks(pipe.scores[l], w.k, out=pipe.idx[l], stream=stream)
            kbs.block_sparse_attn(layers[l]["Q"], sk, sv, pipe.idx[l], T, q, kv_mode=kbs.KV_STAGING,
                                  out=pipe.out[l], ws=pipe.ws, stream=stream)

    ms_gather = time_loop(gather_only, max(3, n // 4), stream)
    ms_device = time_loop(device_only, max(3, n // 4), stream)
    sweep = {}
    for nwg in (16, 32, 64, 128, 256):
        def g(i, nwg=nwg):
            for l in range(1, L):
                kbs.prefetch_blocks(layers[l]["host_K"], layers[l]["host_V"], pipe.idx[l].view(w.B, w.Hkv, w.k), sk,
                                    sv, num_workgroups=nwg, stream=stream)
        t = time_loop(g, max(3, n // 4), stream)
        sweep[nwg] = {"gather_ms": round(t, 4), "gather_GBps": round(link_bytes / (t * 1e-3) / 1e9, 2)}
        log(f"[bench] gather of {L - 1} layers with {nwg} workgroups: {t:.3f} ms")
    # lookahead of more than one layer: layer l's Forecast picks layer l + D's
    # blocks, D + 1 staging buffers (inputs: the same stack plus those vectors)
    depth_sweep = {1: {"ms_per_step": round(ms_step, 4), "staging_buffers": len(pipe.stage)}}
    del pipe
    for D in (2, 3):
        set_lookahead(w, layers, D, dev)
        pd = LayerPipeline(L, w.B, w.Hq, w.Hkv, w.T, w.k, torch.bfloat16, dev, depth=D)
        for i in range(max(2, args.warmup // 4)):
            pd.step(layers, stream)
        torch.cuda.synchronize()
        t = time_loop(lambda i: pd.step(layers, stream), max(3, n // 2), stream)
        depth_sweep[D] = {"ms_per_step": round(t, 4), "staging_buffers": len(pd.stage)}
        log(f"[bench] lookahead depth {D}: {t:.3f} ms per step")
        del pd
    link_gbps = link_bytes / (ms_gather * 1e-3) / 1e9
    result = {
        "metric": f"offloaded decode steps/s/layer at 128K ctx, B={B}, {L}-layer stack with lookahead prefetch",
        "value": round(L * 1e3 / ms_step, 3), "unit": "steps/s/layer",
        "n_gpus": 1, "steps": n, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{L}-layer offloaded decode stack, bf16: B={B}, T={w.T}, {w.Hq}/{w.Hkv} heads, "
                               f"d={w.d}, top-{w.k}; layer 0 KV in HBM, layers 1-{L - 1} KV in pinned host memory",
                   "layers": L, "B": B, "T": w.T, "top_k": w.k, "staging_buffers": 2},
        "roofline": {"bound": "host_link", "kernel": "prefetch", "achieved": round(link_gbps, 2),
                     "peak": HOST_LINK_PEAK_GBPS, "unit": "GB/s", "frac": round(link_gbps / HOST_LINK_PEAK_GBPS, 4),
                     "traffic": None},
        "link_bytes_per_step": link_bytes,
        "gather_all_layers_ms": round(ms_gather, 4),
        "device_work_all_layers_ms": round(ms_device, 4),
        "serial_ms": round(ms_gather + ms_device, 4),
        "workgroup_sweep": sweep,
        "lookahead_depth_sweep": depth_sweep,
    }
    print(json.dumps(result), flush=True)
    return 0


def prefill_flops(w, idx) -> dict:
    """Algorithmic flops of the chunk: Forecast scoring of every visible
    (query, window) pair, and attention over every selected key at or before
    each query (QK and PV, 2 x 128 flops each)."""
    import numpy as np
    pos = w.q_start + np.arange(w.Tq)
    vis = np.where(pos >= w.kernel - 1, np.minimum(w.W, (pos - w.kernel + 1) // w.stride + 1), 0)
    sel = 2 * w.d * int(vis.sum()) * w.B * w.Hkv
    keys = 0
    for t in range(w.n_tiles):
        p = pos[t * w.tile:(t + 1) * w.tile]
        blk = idx[:, :, t, :]                                   # [B, Hkv, k]
        valid = blk >= 0
        start = 64 * np.where(valid, blk, 0)
        cnt = np.clip(p[None, None, None, :] - start[..., None] + 1, 0, 64) * valid[..., None]
        keys += int(cnt.sum())
    # the multi-head selector scores every (query, head, visible window) twice:
    # once for the softmax normalisers, once for the normalised group sums
    return {"select_forecast": sel, "select_multihead": 2 * w.G * sel, "attention": 4 * w.d * keys * w.G}




# ------------------------------------------------------------------ main ----
def _line(metric: str, value, unit: str, ms_per_step, steps: int, args, workload: str, extra: dict) -> dict:
    out = {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": steps, "warmup": args.warmup,
           "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic", "config": {"workload": workload}}
    out.update(extra)
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", choices=("all", "decode", "offload", "prefill", "pipeline"), default="all",
                    help="all (default): the batch-16 128K decode step as the headline, the other four workloads "
                         "as extra keys; decode: the headline only; offload: the batch-64 two-layer step with "
                         "lookahead prefetch from pinned host memory; prefill: a 4096-query chunk at 128K; "
                         "pipeline: a four-layer offloaded stack")
    ap.add_argument("--config", type=int, choices=(1, 2, 3, 4, 5), default=None,
                    help="one benchmark configuration alone: 1 tiny fp32 decode, 2 single-sequence 32K decode, "
                         "3 batch-16 128K decode (the headline; as --workload decode), 4 offloaded batch-64 decode "
                         "(as --workload offload), 5 chunked prefill (as --workload prefill)")
    ap.add_argument("--decoupled-layers", action="store_true",
                    help="decode: also time consecutive layers with the next layer's selection on a second stream "
                         "beside this layer's attention, against the same layers on one stream")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (torch copy_) ten times, as the known-size reference "
                         "for scaling the profiler's FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): this path is built and timed on a single "
              f"MI355X; sharding across GPUs is not implemented.", file=sys.stderr)
        return 2
    if args.steps < 1:
        print("--steps must be at least 1", file=sys.stderr)
        return 2
    if args.config in (3, 4, 5):
        args.workload = {3: "decode", 4: "offload", 5: "prefill"}[args.config]
    elif args.config in (1, 2):
        import torch
        import kv_block_selection_amd as kbs
        from synth import workloads as wl
        kbs.load()
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        w = wl.C1_TINY if args.config == 1 else wl.C2_DECODE_32K
        r = bench_small_decode(kbs, w, dev, args.steps, args.warmup)
        print(json.dumps(_line("decode steps/s/layer (select+sparse attn)", r["steps_per_s_per_layer"],
                               "steps/s/layer", round(r["us_per_step"]["median"] / 1e3, 5), r["steps"], args,
                               r["workload"], r)), flush=True)
        return 0
    # the all-cores oracle's worker processes start before anything touches the GPU
    pool, n_workers = (None, 0)
    if args.workload in ("all", "decode") and not args.no_cpu_baseline:
        pool, n_workers = start_oracle_pool()
    try:
        if args.workload == "pipeline":
            return bench_pipeline(args)
        if args.workload == "offload":
            r = bench_offload_cfg(args)
            print(json.dumps(_line("offloaded decode steps/s/layer at 128K ctx, B=64, two layers with lookahead "
                                   "prefetch", r["steps_per_s_per_layer"], "steps/s/layer",
                                   r["ms_per_step"]["median"], 4, args, r["workload"], r)), flush=True)
            return 0
        if args.workload == "prefill":
            r = bench_prefill_cfg(args)
            print(json.dumps(_line("chunked-prefill chunks/s at 128K ctx (4096 queries, select+sparse attn)",
                                   r["chunks_per_s"], "chunks/s", round(r["us_per_chunk"]["median"] / 1e3, 5), 20,
                                   args, r["workload"], r)), flush=True)
            return 0
        import torch
        from synth import workloads as wl
        configs = {}
        if args.workload == "all":
            import kv_block_selection_amd as kbs
            kbs.load()
            dev = torch.device("cuda:0")
            torch.cuda.set_device(dev)
            for w in (wl.C1_TINY, wl.C2_DECODE_32K):
                log(f"[bench] {w.name}")
                configs[w.name] = bench_small_decode(kbs, w, dev, args.steps, args.warmup)
        result = bench_decode(args, pool, n_workers)
        if args.workload == "all":
            log("[bench] c5: chunked prefill")
            configs[wl.C5_PREFILL.name] = bench_prefill_cfg(args)
            log("[bench] c4: offloaded decode with lookahead prefetch")
            configs[wl.C4_OFFLOAD.name] = bench_offload_cfg(args)
            result["other_configs"] = configs
        print(json.dumps(result), flush=True)
        return 0
    finally:
        if pool is not None:
            pool.terminate()
            pool.join()


if __name__ == "__main__":
    sys.exit(main())

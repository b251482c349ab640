"""Benchmark of the SparDA decode hot path on one MI355X.

One step = Forecast block scoring of every compressed key window, top-k block
choice and GQA block-sparse attention over the chosen blocks, for one layer of
the batched 128K-context decode workload (B=16, T=131072, 32 query / 8 KV
heads, d=128, 64-token blocks, top-64), inputs resident in HBM. Prints one
JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --workload offload   # two-layer step, layer-1 KV in pinned host memory
    python bench.py --workload prefill   # 4096-query chunk at 128K on the matrix cores
    python bench.py --workload pipeline  # four-layer step, layers 1-3 KV in pinned host memory

Timing: W untimed steps, then K steps between two HIP events on the stream the
kernels run on, with a device synchronisation on both sides. Input sets rotate
(3 independent sets) so no step finds its data in the 256 MB last-level cache.
Per-kernel averages come from their own event-bracketed loops.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode steps/s/layer at 128K ctx (select+sparse attn); % of HBM peak GB/s"
HBM_PEAK_GBPS = 8000.0
N_SETS = 3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(w) -> dict:
    """Bytes each kernel must move for one layer-step (bf16 = 2 B)."""
    e = 2
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
        # one launch: the next layer's selection, this layer's top-k + attention, the merge of the layer before
        "decode_layer": (kc + f + scores) + (scores + idx + kv + q) + o,
        "step": kc + f + scores + (scores + idx) + (kv + q + idx + o),
    }


def time_loop(fn, iters: int, stream) -> float:
    """Average ms of fn(i) over iters eager launches, HIP events on `stream`."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(iters):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / iters


def time_graph(fn, per_graph: int, replays: int) -> float:
    """Average ms per fn(i) call: fn(0..per_graph-1) captured once in a HIP graph
    (no host launch cost inside), replayed `replays` times between HIP events on
    the replay stream."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(per_graph):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per_graph):
            fn(i)
    stream = torch.cuda.current_stream()
    g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(replays):
        g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / (replays * per_graph)


def cpu_baseline(w, sets, min_seconds: float = 10.0, max_reps: int = 30) -> dict:
    """The fp64 oracle, as it stands, on the benchmark's own step: Forecast
    scoring + top-k + attention for every (sequence, KV head) row of the first
    input set, single-threaded. The whole step is repeated until about
    min_seconds of CPU time have accumulated; inputs are converted to fp64
    outside the timed region (the blocks an attention row reads are gathered
    after the oracle's own selection)."""
    import oracle
    from tests import parity
    from threadpoolctl import threadpool_limits
    s = sets[0]
    cache = []
    timed = 0.0
    with threadpool_limits(limits=1):
        for b in range(w.B):
            for h in range(w.Hkv):
                F = parity.to_f64(s["F"][b, h])
                Kc = parity.to_f64(s["Kc"][b, h])
                Q = parity.to_f64(s["Q"][b, h * w.G:(h + 1) * w.G])
                t0 = time.perf_counter()
                sc = oracle.select_forecast_tile(F, Kc, [w.q_start], w.T, w.scale)
                idx = oracle.topk_row(sc, w.k)
                J = oracle.selected_keys(idx, w.q_start)
                timed += time.perf_counter() - t0
                import torch
                Jt = torch.from_numpy(J).to(s["K"].device)
                KJ = parity.to_f64(s["K"][b, h].index_select(0, Jt))
                VJ = parity.to_f64(s["V"][b, h].index_select(0, Jt))
                t0 = time.perf_counter()
                for g in range(w.G):
                    oracle.attend(Q[g, 0], KJ, VJ, w.scale)
                timed += time.perf_counter() - t0
                cache.append((F, Kc, Q, KJ, VJ))
        reps = 1
        while timed < min_seconds and reps < max_reps:
            t0 = time.perf_counter()
            for F, Kc, Q, KJ, VJ in cache:
                sc = oracle.select_forecast_tile(F, Kc, [w.q_start], w.T, w.scale)
                idx = oracle.topk_row(sc, w.k)
                oracle.selected_keys(idx, w.q_start)
                for g in range(w.G):
                    oracle.attend(Q[g, 0], KJ, VJ, w.scale)
            timed += time.perf_counter() - t0
            reps += 1
    per_step = timed / reps
    return {"value": round(1.0 / per_step, 4), "unit": "steps/s/layer", "cores": 1, "kind": "oracle",
            "sample": f"the full step ({w.B * w.Hkv} (sequence, KV head) rows: Forecast scoring of {w.W} windows, "
                      f"top-{w.k} of {w.nB} blocks, attention of {w.G} heads over {w.k * w.block} keys), fp64 numpy "
                      f"on 1 thread, repeated {reps}x ({timed:.1f} s timed); fp64 conversion of inputs untimed"}


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


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", choices=("decode", "offload", "prefill", "pipeline"), default="decode",
                    help="decode: the batch-16 128K decode step (the headline line); offload: the batch-64 two-layer "
                         "step with lookahead prefetch from pinned host memory; prefill: a 4096-query chunk at 128K")
    ap.add_argument("--kernel-iters", type=int, default=100)
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

    if args.workload == "offload":
        return bench_offload(args)
    if args.workload == "pipeline":
        return bench_pipeline(args)
    if args.workload == "prefill":
        return bench_prefill(args)
    return bench_decode(args)


def bench_decode(args) -> int:
    import torch
    import kv_block_selection_amd as kbs
    import synth.gpu as sg
    from synth import workloads as wl

    kbs.load()
    w = wl.C3_DECODE_128K
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] generating {N_SETS} input sets of {w.name}")
    sets = []
    for i in range(N_SETS):
        wi = wl.scaled(w, seed=w.seed + 1000 * i)
        s = {n: sg.tensor(wi.recipe(n), wi.shape(n), dev) for n in ("Q", "F", "K", "V")}
        s["Kc"] = kbs.compress_keys(s["K"])
        s["scores"] = torch.empty((w.B, w.Hkv, 1, w.nB), dtype=torch.float32, device=dev)
        s["idx"] = torch.empty((w.B, w.Hkv, 1, w.k), dtype=torch.int32, device=dev)
        s["out"] = torch.empty_like(s["Q"])
        # the newest token of every sequence again, for the cache-append timings
        s["Knew1"] = s["K"][:, :, w.T - 1:].contiguous()
        s["Vnew1"] = s["V"][:, :, w.T - 1:].contiguous()
        s["Knew2"] = s["K"][:, :, w.T - 2:w.T - 1].contiguous()
        s["Vnew2"] = s["V"][:, :, w.T - 2:w.T - 1].contiguous()
        sets.append(s)
    pos_last = torch.full((w.B,), w.q_start, dtype=torch.int32, device=dev)
    len_win = torch.full((w.B,), w.T - 1, dtype=torch.int32, device=dev)  # token T-1 completes window W-1
    len_nowin = torch.full((w.B,), w.T - 2, dtype=torch.int32, device=dev)  # token T-2 completes none
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ws_attn = torch.zeros(max(1, kbs.workspace_bytes(kbs.OP_BLOCK_SPARSE_ATTN, w.B, w.Hq, w.Hkv, 1, w.T, w.k)),
                          dtype=torch.uint8, device=dev)
    ws_mh = torch.empty(max(1, kbs.workspace_bytes(kbs.OP_SELECT_MULTIHEAD, w.B, w.Hq, w.Hkv, 1, w.T)),
                        dtype=torch.uint8, device=dev)

    def sel(i):
        s = sets[i % N_SETS]
        kbs.select_forecast(s["F"], s["Kc"], w.T, w.q_start, out=s["scores"])

    def sel_mh(i):
        s = sets[i % N_SETS]
        kbs.select_multihead(s["Q"], s["Kc"], w.T, w.q_start, out=s["scores"], ws=ws_mh)

    def topk(i):
        s = sets[i % N_SETS]
        kbs.topk_blocks(s["scores"], w.k, out=s["idx"])

    def attn(i):
        s = sets[i % N_SETS]
        kbs.block_sparse_attn(s["Q"], s["K"], s["V"], s["idx"], w.T, w.q_start, out=s["out"], ws=ws_attn)

    def topk_attn(i):  # top-k and attention in one launch
        s = sets[i % N_SETS]
        kbs.topk_block_sparse_attn(s["scores"], s["Q"], s["K"], s["V"], w.k, w.T, w.q_start, idx=s["idx"],
                                   out=s["out"], ws=ws_attn)

    def step(i):
        sel(i)
        topk_attn(i)

    def step_separate(i):  # the same step with top-k as a launch of its own
        sel(i)
        topk(i)
        attn(i)

    def topk_attn_partial(i):  # the same without the merge (left in ws_attn)
        s = sets[i % N_SETS]
        kbs.topk_block_sparse_attn(s["scores"], s["Q"], s["K"], s["V"], w.k, w.T, w.q_start, idx=s["idx"],
                                   out=s["out"], ws=ws_attn, merge=False)

    def sel_merge(i):  # selection + the merge of the previous layer's attention
        s, prev = sets[i % N_SETS], sets[(i - 1) % N_SETS]
        kbs.select_forecast(s["F"], s["Kc"], w.T, w.q_start, out=s["scores"],
                            merge_from=(ws_attn, prev["out"], w.T, w.k))

    ws_layer = torch.zeros(max(1, kbs.workspace_bytes(kbs.OP_DECODE_LAYER, w.B, w.Hq, w.Hkv, 1, w.T, w.k)),
                           dtype=torch.uint8, device=dev)

    def step_one_launch(i):
        # layer i in one launch: its top-k + attention (finished output) and
        # layer i+1's Forecast selection, both from layer i's projections
        s, nxt = sets[i % N_SETS], sets[(i + 1) % N_SETS]
        kbs.decode_layer(s["scores"], s["Q"], s["K"], s["V"], w.k, w.T, w.q_start, ws_layer, idx=s["idx"],
                         out=s["out"], select_next=(nxt["F"], nxt["Kc"], nxt["scores"], w.T, w.q_start))

    def step_pipelined(i):
        # layer i in the method's layer order: its selection (from the layer
        # before's Forecast) shares a launch with the merge of the layer
        # before's attention, which leaves its block-range results in ws_attn
        s, prev = sets[i % N_SETS], sets[(i - 1) % N_SETS]
        kbs.select_forecast(s["F"], s["Kc"], w.T, w.q_start, out=s["scores"],
                            merge_from=(ws_attn, prev["out"], w.T, w.k))
        kbs.topk_block_sparse_attn(s["scores"], s["Q"], s["K"], s["V"], w.k, w.T, w.q_start, idx=s["idx"],
                                   out=s["out"], ws=ws_attn, merge=False)

    # Decode-time state maintenance: append the step's token to K, V and
    # compress the window it completes (every 16th step) or none. The tokens
    # written are the ones already there, so the inputs stay as they are.
    def append_win(i):
        s = sets[i % N_SETS]
        kbs.append_kv(s["Knew1"], s["Vnew1"], s["K"], s["V"], len_win, k_cmp=s["Kc"])

    def append_nowin(i):
        s = sets[i % N_SETS]
        kbs.append_kv(s["Knew2"], s["Vnew2"], s["K"], s["V"], len_nowin, k_cmp=s["Kc"])

    def step_q_pos(i):  # the same step with per-sequence positions (all at T - 1)
        s = sets[i % N_SETS]
        kbs.select_forecast(s["F"], s["Kc"], w.T, 0, out=s["scores"], q_pos=pos_last)
        kbs.topk_block_sparse_attn(s["scores"], s["Q"], s["K"], s["V"], w.k, w.T, 0, idx=s["idx"], out=s["out"],
                                   ws=ws_attn, q_pos=pos_last)

    log("[bench] warmup (eager)")
    for i in range(args.warmup):
        step(i)
    for i in range(args.warmup):
        step_pipelined(i)
    torch.cuda.synchronize()
    for i in range(6):
        step_one_launch(i)
    torch.cuda.synchronize()
    ms_step_eager = time_loop(step_one_launch, 6 * max(1, args.steps // 6), stream)
    log(f"[bench] eager step {ms_step_eager * 1e3:.1f} us; timing {args.steps} steps through a HIP graph")
    per_graph = 3 * N_SETS
    replays = max(1, args.steps // per_graph)
    # six layers per graph: the three input sets and the two workspaces both cycle
    ms_step = time_graph(step_one_launch, 6, max(1, args.steps // 6))
    steps_timed = 6 * max(1, args.steps // 6)
    ms_step_two_launches = time_graph(step_pipelined, per_graph, replays)
    ms_step_layer = time_graph(step, per_graph, replays)
    ms_step_separate = time_graph(step_separate, per_graph, replays)
    log(f"[bench] graph step {ms_step * 1e3:.1f} us (two launches per layer {ms_step_two_launches * 1e3:.1f} us, one "
        f"layer at a time {ms_step_layer * 1e3:.1f} us, with top-k launched on its own {ms_step_separate * 1e3:.1f} "
        f"us); per-kernel graphs")
    kr = max(1, args.kernel_iters // per_graph)
    ms = {"select_forecast": time_graph(sel, per_graph, kr), "topk": time_graph(topk, per_graph, kr),
          "attention": time_graph(attn, per_graph, kr), "select_multihead": time_graph(sel_mh, per_graph, kr),
          "topk_attention": time_graph(topk_attn, per_graph, kr),
          "topk_attention_partial": time_graph(topk_attn_partial, per_graph, kr),
          "select_forecast_merge": time_graph(sel_merge, per_graph, kr),
          "decode_layer": ms_step}
    ms_extra = {"append_kv_with_window": time_graph(append_win, per_graph, kr),
                "append_kv": time_graph(append_nowin, per_graph, kr),
                "step_with_q_pos": time_graph(step_q_pos, per_graph, kr)}
    for i in range(N_SETS):  # leave each set's Forecast scores / idx in place
        step(i)
    torch.cuda.synchronize()
    projection = bench_projection(kbs, w, dev, kr)
    token_level = bench_token_level(kbs, w, sets, dev, per_graph, kr)
    decoupled = (decoupled_layers(kbs, w, sets, ws_attn, dev, algorithmic_bytes(w)["step"], n_layers=3 * args.steps)
                 if args.decoupled_layers else None)

    nbytes = algorithmic_bytes(w)
    gbps = {k: nbytes[k] / (ms[k] * 1e-3) / 1e9 for k in ms}
    # the timed step is one launch per layer: that launch is the roofline kernel
    dominant = "decode_layer"
    step_gbps = nbytes["step"] / (ms_step * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(1e3 / ms_step, 2),
        "unit": "steps/s/layer",
        "n_gpus": 1,
        "steps": steps_timed,
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
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(gbps[dominant], 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps[dominant] / HBM_PEAK_GBPS, 4),
                     "traffic": pmc_traffic(["kv_block_selection_amd/csrc/attn_decode.hip",
                                             "kv_block_selection_amd/csrc/topk_row.h",
                                             "kv_block_selection_amd/csrc/select_row.h",
                                             "kv_block_selection_amd/csrc/merge_row.h",
                                             "kv_block_selection_amd/csrc/reduce16.h"],
                                            "decode_layer_c3_traffic.json")},
        "step_hbm_GBps": round(step_gbps, 1),
        "step_hbm_frac": round(step_gbps / HBM_PEAK_GBPS, 4),
        "ms_per_step_eager": round(ms_step_eager, 5),
        "ms_per_step_two_launches_per_layer": round(ms_step_two_launches, 5),
        "ms_per_step_one_layer_at_a_time": round(ms_step_layer, 5),
        "ms_per_step_topk_separate": round(ms_step_separate, 5),
        "kernel_us": {k: round(v * 1e3, 2) for k, v in ms.items()},
        "kernel_GBps": {k: round(v, 1) for k, v in gbps.items()},
        "selection_us": {"forecast": round((ms["select_forecast"] + ms["topk"]) * 1e3, 2),
                         "multihead": round((ms["select_multihead"] + ms["topk"]) * 1e3, 2)},
        "forecast_vs_multihead_select_speedup": round(ms["select_multihead"] / ms["select_forecast"], 3),
        "state_maintenance_us": {k: round(v * 1e3, 2) for k, v in ms_extra.items()},
        "upstream_projection": projection,
        "token_level": token_level,
    }
    if decoupled is not None:
        result["decoupled_layers"] = decoupled
    if args.calibration_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["calibration_copy_bytes"] = 1 << 30
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle sample)")
        result["cpu_baseline"] = cpu_baseline(w, sets)
    print(json.dumps(result), flush=True)
    return 0


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


def bench_token_level(kbs, w, sets, dev, per_graph: int, kr: int) -> dict:
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
    ms = {"select_tokens": time_graph(score, per_graph, kr), "topk_tokens": time_graph(topk, per_graph, kr),
          "token_attention": time_graph(attn, per_graph, kr)}
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


HOST_LINK_PEAK_GBPS = 63.0   # PCIe 5.0 x16, one direction
MFMA_BF16_PEAK_TFLOPS = 2500.0


def bench_offload(args) -> int:
    """Two-layer decode step at B=64, T=128K with layer 1's KV (32 GiB) in pinned
    host memory: both selections, layer 0's attention from HBM overlapped with
    the gather of layer 1's selected blocks over the host link on a side stream,
    then layer 1's attention from staging. Also times each part alone, a plain
    1 GiB pinned host-to-device copy, and a sweep of the gather's workgroups."""
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

    log("[bench] warmup")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    n = max(5, args.steps)
    ms_step = time_loop(step, n, stream)
    log(f"[bench] step {ms_step:.3f} ms; parts alone")
    parts = {"select_both_layers": time_loop(select, n, stream), "attn_layer0_hbm": time_loop(attn0, n, stream),
             "gather_layer1": time_loop(gather(0), n, stream), "attn_layer1_staging": time_loop(attn1, n, stream)}
    host = l1["host_K"].view(-1).view(torch.uint8)[: 1 << 30]
    dst = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    ms_copy = time_loop(lambda i: dst.copy_(host, non_blocking=True), max(5, n // 4), stream)
    del dst
    sweep = {}
    for nwg in (8, 16, 32, 64, 128, 256):
        st.num_workgroups = nwg
        g = time_loop(gather(nwg), max(5, n // 4), stream)
        s_ms = time_loop(step, max(5, n // 4), stream)
        sweep[nwg] = {"gather_ms": round(g, 4), "gather_GBps": round(link_bytes / (g * 1e-3) / 1e9, 2),
                      "step_ms": round(s_ms, 4)}
        log(f"[bench] gather with {nwg} workgroups: {g:.3f} ms, step {s_ms:.3f} ms")
    st.num_workgroups = 0
    cached = bench_cached_gather(kbs, w, l1, st, stream, dev)
    # the gather waits only for layer 1's selection; layer 0's selection and
    # attention can hide behind it
    serial = sum(parts.values())
    hideable = min(parts["select_both_layers"] / 2 + parts["attn_layer0_hbm"], parts["gather_layer1"])
    link_gbps = link_bytes / (parts["gather_layer1"] * 1e-3) / 1e9
    result = {
        "metric": "offloaded decode steps/s/layer at 128K ctx, B=64, two layers with lookahead prefetch",
        "value": round(2e3 / ms_step, 3),
        "unit": "steps/s/layer",
        "n_gpus": 1, "steps": n, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.description, "B": w.B, "T": w.T, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d,
                   "block": w.block, "top_k": w.k, "layers": 2, "gather_workgroups": "library default"},
        "roofline": {"bound": "host_link", "kernel": "prefetch", "achieved": round(link_gbps, 2),
                     "peak": HOST_LINK_PEAK_GBPS, "unit": "GB/s", "frac": round(link_gbps / HOST_LINK_PEAK_GBPS, 4),
                     "traffic": None},
        "link_bytes_per_step": link_bytes,
        "h2d_memcpy_1GiB_GBps": round((1 << 30) / (ms_copy * 1e-3) / 1e9, 2),
        "parts_ms": {k: round(v, 4) for k, v in parts.items()},
        "serial_ms": round(serial, 4),
        "overlap_hidden_frac": round((serial - ms_step) / hideable, 3) if hideable > 0 else None,
        "overlap_note": "hideable = layer 0 selection (half of both selections) + layer 0 attention",
        "workgroup_sweep": sweep,
        "cached_gather": cached,
    }
    print(json.dumps(result), flush=True)
    return 0


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
    n = max(5, args.steps)
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


def bench_prefill(args) -> int:
    """A 4096-query chunk at the end of a 128K context (B=1, 32/8 heads): Forecast
    scoring of every 64-query tile, top-64 per tile, block-sparse attention,
    each on the matrix cores except top-k; inputs resident in HBM."""
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
    Kc = kbs.compress_keys(s["K"])
    scores = torch.empty((w.B, w.Hkv, w.n_tiles, w.nB), dtype=torch.float32, device=dev)
    idx = torch.empty((w.B, w.Hkv, w.n_tiles, w.k), dtype=torch.int32, device=dev)
    out = torch.empty_like(s["Q"])
    stream = torch.cuda.current_stream(dev)

    def sel(i):
        kbs.select_forecast(s["F"], Kc, w.T, w.q_start, out=scores)

    def topk(i):
        kbs.topk_blocks(scores, w.k, out=idx)

    def attn(i):
        kbs.block_sparse_attn(s["Q"], s["K"], s["V"], idx, w.T, w.q_start, out=out)

    def sel_mh(i):
        kbs.select_multihead(s["Q"], Kc, w.T, w.q_start, out=scores)

    def step(i):
        sel(i)
        topk(i)
        attn(i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    n = max(5, args.steps)
    ms_step = time_loop(step, n, stream)
    ms = {"select_forecast": time_loop(sel, n, stream), "topk": time_loop(topk, n, stream),
          "attention": time_loop(attn, n, stream), "select_multihead": time_loop(sel_mh, n, stream)}
    step(0)
    torch.cuda.synchronize()
    fl = prefill_flops(w, idx.cpu().numpy())
    tf = {k: fl[k] / (ms[k] * 1e-3) / 1e12 for k in fl}
    result = {
        "metric": "chunked-prefill chunks/s at 128K ctx (4096 queries, select+sparse attn)",
        "value": round(1e3 / ms_step, 3),
        "unit": "chunks/s",
        "n_gpus": 1, "steps": n, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.description, "B": w.B, "T": w.T, "Tq": w.Tq, "q_start": w.q_start, "Hq": w.Hq,
                   "Hkv": w.Hkv, "d": w.d, "block": w.block, "tile": w.tile, "top_k": w.k},
        "roofline": {"bound": "mfma", "kernel": "attention", "achieved": round(tf["attention"], 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf["attention"] / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None},
        "kernel_us": {k: round(v * 1e3, 2) for k, v in ms.items()},
        "algorithmic_gflop": {k: round(v / 1e9, 3) for k, v in fl.items()},
        "kernel_TFLOPs": {k: round(v, 1) for k, v in tf.items()},
        "mfma_utilisation": {k: round(v / MFMA_BF16_PEAK_TFLOPS, 4) for k, v in tf.items()},
        "selection_us": {"forecast": round((ms["select_forecast"] + ms["topk"]) * 1e3, 2),
                         "multihead": round((ms["select_multihead"] + ms["topk"]) * 1e3, 2)},
        "forecast_vs_multihead_select_speedup": round(ms["select_multihead"] / ms["select_forecast"], 3),
        "multihead_exp_per_chunk": 2 * w.G * prefill_flops(w, idx.cpu().numpy())["select_forecast"] // (2 * w.d),
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

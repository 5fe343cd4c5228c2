"""MoE-layer forward benchmark on one MI355X.

One step = one pass of the whole layer (route -> permute -> expert FFN ->
combine, plus the shared expert where the workload has one) over one batch,
inputs already resident in HBM.  Weight sets of several layers are rotated so
that the touched expert bytes of consecutive steps do not sit in the 256 MB
last-level cache (a model walks its layers the same way), and every step gets
a fresh batch of logits and activations.

Prints ONE JSON line: tokens/s of the whole job, the dominant kernel's
roofline fraction (HIP events around the expert-FFN call on its stream inside
the timed region), and the CPU oracle timed on a bounded sample as baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
LLC_BYTES = 256 << 20           # Infinity Cache

DEFAULTS = {  # workload -> (steps, warmup, batches)
    "tiny_bf16": (200, 20, 16),
    "decode_mxfp4": (400, 40, 64),
    "prefill_nvfp4": (50, 5, 8),
    "fp8_lru_pool": (24, 2, 12),
    "large_prefill_mxfp4": (10, 2, 2),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="decode_mxfp4")
    ap.add_argument("--rot", type=int, default=0, help="weight sets rotated (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--variant", default="auto")
    ap.add_argument("--eager", action="store_true", help="launch eagerly instead of graph replay")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 64 MiB device copy (for HBM counter calibration)")
    ap.add_argument("--calibrate-read", action="store_true",
                    help="only time plain streaming reads of several sizes (the practical HBM "
                         "read ceiling next to the published peak)")
    ap.add_argument("--resident", action="store_true",
                    help="cache workloads: keep every expert in HBM instead of the slot pool")
    ap.add_argument("--layers", type=int, default=1,
                    help="decode-sized workloads: one step = this many MoE layers chained "
                         "(each layer's y is the next one's x; one graph per run)")
    ap.add_argument("--slots", type=int, default=None,
                    help="cache workloads: pool slots (default: the workload's)")
    ap.add_argument("--slot-sweep", type=str, default=None,
                    help="cache workloads: comma-separated pool sizes; replays the run's routing "
                         "through the same LRU policy at each size (misses per layer-step)")
    ap.add_argument("--fill-groups", type=int, default=8,
                    help="cache workloads: copy groups the FFN runs behind (0 = fill all misses, "
                         "then run the FFN)")
    ap.add_argument("--tokens", type=int, default=None,
                    help="override the workload's batch size T (e.g. a decode batch-size sweep)")
    return ap.parse_args()


# kernel sources the timed launches of each workload are compiled from
KERNEL_SOURCES = {
    "decode": ("decode.hip", "ffn_common.h", "moe_internal.h", "route_common.h"),
    "layer": ("ffn.hip", "ffn_common.h", "moe_internal.h", "route.hip", "route_common.h",
              "permute.hip", "combine.hip"),
}


def source_hash(workload: str) -> str:
    """sha256 over the workload's kernel sources: counter readings are valid only for these
    bytes (decode_mxfp4 runs the decode-layer kernels, the other workloads the separate
    route / permute / expert FFN / combine kernels)."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES["decode" if workload == "decode_mxfp4" else "layer"]:
        with open(os.path.join(ROOT, "moe_expert_ffn_router_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per step from committed rocprofv3 FETCH_SIZE / WRITE_SIZE readings, scaled by
    the copy-kernel calibration; None when the readings were taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("TRAFFIC "):
            rec = json.loads(line[len("TRAFFIC "):])
            if rec.get("source_hash") != source_hash(workload):
                return None
            return int(sum(k["fetch_kib"] * 1024 * rec["fetch_scale"] +
                           k["write_kib"] * 1024 * rec["write_scale"]
                           for k in rec["kernels"].values()))
    return None


def calibrate_copy():
    """A plain device copy of known size: the reference for the counters' scale."""
    import torch
    n = 64 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": n, "launches": 5}), flush=True)


def calibrate_read():
    """moe_hbm_read_probe over sizes from a decode launch's bytes to 1 GiB, 24 launches
    in one graph replay; each launch reads a region the previous launches did not (the
    buffer spans 8x the largest size, well past the memory-side cache)."""
    import torch
    import moe_expert_ffn_router_amd as moe
    big = 1 << 30
    buf = torch.ones(8 * big, dtype=torch.uint8, device="cuda")
    sink = torch.empty(8192 * 256, dtype=torch.int32, device="cuda")
    rows = []
    for nbytes in (16 << 20, 34_000_000, 68_000_000, 96_404_480, 256 << 20, big):
        n = nbytes // 16 * 16
        regions = buf.numel() // n
        for grid in (512, 1024, 2048, 4096):
            for r in range(3):
                moe.moe_hbm_read_probe(buf[(r % regions) * n:], n, grid, sink)
            reps = 24
            g = torch.cuda.CUDAGraph()  # launches back to back, no host gaps
            with torch.cuda.graph(g):
                for r in range(reps):
                    moe.moe_hbm_read_probe(buf[((3 + r) % regions) * n:], n, grid, sink)
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            rows.append({"bytes": n, "grid": grid, "us": round(us, 2),
                         "tb_s": round(n / (us * 1e-6) / 1e12, 3)})
    best = {}
    for r in rows:
        if r["bytes"] not in best or r["us"] < best[r["bytes"]]["us"]:
            best[r["bytes"]] = r
    print(json.dumps({"calibration_read": rows, "best_per_size": list(best.values())}),
          flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer has no "
              "multi-GPU path (experts and tokens are not sharded).", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.calibrate_read:
        calibrate_read()
        return
    import torch

    import moe_expert_ffn_router_amd as moe
    import synth

    wl = synth.WORKLOADS[args.workload]
    if args.tokens is not None:
        wl = wl.scaled(T=args.tokens)
    if wl.pool_slots and not args.resident:
        return bench_cached(args, wl)
    steps_d, warm_d, nb = DEFAULTS[wl.name]
    steps = args.steps if args.steps is not None else steps_d
    warmup = args.warmup if args.warmup is not None else warm_d
    dev = torch.device("cuda")
    torch.cuda.set_device(0)

    lay = synth.record_layout(wl.fmt, wl.H, wl.I)
    stride, payload = lay["stride"], lay["payload"]

    # ---- inputs, resident in HBM -------------------------------------------
    t0 = time.time()
    base_set = synth.make_expert_records(wl.fmt, wl.E, wl.H, wl.I, wl.seed, device=dev)
    logits = [torch.from_numpy(synth.make_logits(wl, b)).to(dev) for b in range(nb)]
    xs = [torch.from_numpy(synth.make_x(wl, b).view(np.int16)).to(dev).view(torch.bfloat16)
          for b in range(nb)]
    shared = None
    if wl.shared_I:
        shared = synth.make_shared_record(wl.seed, wl.H, wl.shared_I, device=dev)

    layer = moe.MoELayer(wl.fmt, wl.E, wl.H, wl.I, wl.k, wl.T, stride, shared_I=wl.shared_I,
                         shared_stride=shared.shape[1] if shared is not None else 0)
    Ws = moe.experts("bf16", 1, wl.H, wl.shared_I, shared, shared.shape[1]) if shared is not None else None

    # touched experts per batch (from the device routing) -> algorithmic bytes
    touched = []
    for b in range(nb):
        layer.route_permute(logits[b])
        touched.append(int((layer.counts[:wl.E] > 0).sum().item()))
    touched_bytes = float(np.mean(touched)) * payload

    rot = args.rot or max(1, int(np.ceil(4 * LLC_BYTES / max(touched_bytes, 1))))
    rot = min(rot, max(1, int(0.5 * torch.cuda.mem_get_info()[0] // (wl.E * stride))))
    sets = [base_set] + [base_set.clone() for _ in range(rot - 1)]
    Wsets = [layer.weights(s) for s in sets]
    setup_s = time.time() - t0

    stream = torch.cuda.current_stream()
    use_graph = not args.eager

    # decode-sized batches: the two-launch whole-layer path (route+permute+gate/up,
    # down+combine); otherwise the separate calls
    whole = layer.decode_ws is not None and Ws is None and args.variant == "auto"

    L = args.layers
    if L > 1 and not whole:
        print("bench.py: --layers needs a decode-sized workload (whole-layer decode path) "
              "or a cache workload", file=sys.stderr)
        sys.exit(2)
    stack = [layer] + [moe.MoELayer(wl.fmt, wl.E, wl.H, wl.I, wl.k, wl.T, stride)
                       for _ in range(L - 1)]

    def step(i):
        b = i % nb
        if whole:
            x = xs[b]
            for li, lay_l in enumerate(stack):  # layer li of step i: its own weight set
                x = lay_l.forward_decode(logits[(b + li) % nb], x, Wsets[(i * L + li) % rot])
            return
        layer.route_permute(logits[b])
        layer.expert_ffn(Wsets[i % rot], xs[b], wl.T, variant=args.variant)
        if Ws is not None:
            layer.shared_ffn(Ws, xs[b], wl.T, variant=args.variant)
        layer.combine(wl.T, Ws is not None)

    # per-batch routing state, so the FFN launches can be replayed on their own
    perm = []
    for b in range(nb):
        layer.route_permute(logits[b])
        perm.append((layer.counts.clone(), layer.offsets.clone(), layer.sorted_idx.clone()))

    def ffn_only(i):
        b = i % nb
        c, o, sidx = perm[b]
        moe.moe_expert_ffn(Wsets[i % rot], None, xs[b], wl.T, wl.k, c, o, sidx, layer.y_perm,
                           layer.ffn_ws, args.variant)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    def timed(fn, first):
        """Run fn(first .. first+steps-1) once as a captured graph (or eagerly) and return ms."""
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if use_graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(steps):
                    fn(first + i)
            g.replay()  # untimed warm replay (graph upload)
            torch.cuda.synchronize()
            start.record()
            g.replay()
            end.record()
        else:
            start.record()
            for i in range(steps):
                fn(first + i)
            end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end)

    total_ms = timed(step, warmup)
    # dominant kernel time: the whole-layer launches when the layer is two kernels,
    # else the expert-FFN launches replayed on their own
    ffn_ms = total_ms / steps if whole else timed(ffn_only, warmup) / steps
    ms_per_step = total_ms / steps
    # MoE-layer tokens: each of the L chained layers of a step processes T tokens
    tokens_per_s = wl.T * L * steps / (total_ms / 1e3)

    # ---- roofline of the dominant kernel (expert FFN) -------------------------
    A = wl.T * wl.k
    step_batches = [(warmup + i + li) % nb for i in range(steps) for li in range(L)]
    t_mean = float(np.mean([touched[b] for b in step_batches]))
    # per step: L layers (one unless --layers)
    ffn_bytes = L * (t_mean * payload + wl.T * wl.H * 2 + 2 * A * wl.I * 2 + A * wl.H * 2)
    ffn_flops = L * 2.0 * A * 3 * wl.H * wl.I
    # binding roofline: the larger of the HBM floor and the MFMA floor
    # (bf16 rate: the rate of the instructions the prefill kernels issue)
    t_hbm = ffn_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = ffn_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    if t_hbm >= t_mfma:
        achieved = ffn_bytes / (ffn_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        achieved = ffn_flops / (ffn_ms / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": None}
    if whole:
        # the two launches also read logits, write routing outputs and y
        ffn_bytes += L * (wl.T * wl.E * 4 + wl.T * wl.H * 2)
        achieved = ffn_bytes / (ffn_ms / 1e3) / 1e9
        roof.update({"achieved": round(achieved, 1), "frac": round(achieved / HBM_PEAK_GBS, 4)})
    if use_graph and args.tokens is None and L == 1:
        # HBM bytes per step of the timed kernels, from the committed counter
        # readings of this workload's configuration (None without them)
        roof["traffic"] = measured_traffic(wl.name)
    roof.update({"kernel": ("moe_forward_decode, token-major (2 launches: the expert FFN with "
                            "routing, then the combine)" if whole and wl.T <= 16 else
                            "moe_forward_decode (4 launches)" if whole
                            else "moe_expert_ffn (gate/up + down launches)"),
                 "ffn_ms": round(ffn_ms, 5),
                 "timing": ("HIP events around one replay of a graph of the %d steps"
                            % steps + (" (%d layers each)" % L if L > 1 else ""))
                           if use_graph else "HIP events, eager",
                 "algorithmic_bytes_per_launch": int(ffn_bytes),
                 "algorithmic_flops_per_launch": int(ffn_flops),
                 "touched_experts_mean": round(t_mean, 2)})

    # ---- CPU baseline: the oracle on a bounded sample ---------------------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, base_set, shared, args.cpu_seconds)

    out = {
        "metric": "MoE-layer tokens/s at 1 GPU; % HBM roofline (decode), % MFMA peak (prefill)",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "E": wl.E, "I": wl.I, "k": wl.k,
                   "weights": wl.fmt, "shared_I": wl.shared_I, "global_batch": wl.T,
                   "weight_sets_rotated": rot, "batches_rotated": nb,
                   "layers_per_step": L, "us_per_layer": round(ms_per_step * 1e3 / L, 2),
                   "boundary": ("route->permute->expert_ffn->combine on one stream, "
                                + ("as two whole-layer launches, " if whole else "")
                                + ("one captured HIP graph of the K steps" if use_graph
                                   else "eager launches")),
                   "parallelism": "none (1 GPU)", "setup_s": round(setup_s, 1)},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_cached(args, wl):
    """The slot-pool workload: experts live in a pinned host bank, a pool of wl.pool_slots HBM
    slots holds the ones in use, the LRU lookup runs on the host after each routing, misses are
    copied on a side stream and the FFN reads the pool through the slot table.  One step =
    route+permute, counts to the host, lookup, fills, expert FFN, combine (eager: the host
    decision sits in the middle of every step).  Batches rotate over the domain-biased routing
    distributions, so the pool churns."""
    import torch

    import moe_expert_ffn_router_amd as moe
    import synth

    steps_d, warm_d, _ = DEFAULTS[wl.name]
    nb = wl.batches
    steps = args.steps if args.steps is not None else steps_d
    warmup = args.warmup if args.warmup is not None else warm_d
    dev = torch.device("cuda")
    lay = synth.record_layout(wl.fmt, wl.H, wl.I)
    stride, payload = lay["stride"], lay["payload"]
    E = wl.E
    S = args.slots or wl.pool_slots
    L = args.layers  # a stack of L layers sharing the one pool, keys (layer, expert)

    t0 = time.time()
    bank = torch.empty((L * E, stride), dtype=torch.uint8, pin_memory=True)
    for li in range(L):
        for e0 in range(0, E, 16):
            ids = list(range(e0, min(E, e0 + 16)))
            bank[li * E + e0:li * E + e0 + len(ids)].copy_(
                synth.make_expert_records(wl.fmt, E, wl.H, wl.I, wl.seed, layer=li, device=dev,
                                          experts=ids))
    pool = torch.empty((S, stride), dtype=torch.uint8, device=dev)
    table = torch.full((L * E,), -1, dtype=torch.int32, device=dev)
    cache = moe.ExpertCache(L, E, S, stride, pool, bank, table)
    layer = moe.MoELayer(wl.fmt, E, wl.H, wl.I, wl.k, wl.T, stride)
    pool_W = moe.experts(wl.fmt, E, wl.H, wl.I, pool, stride)
    logits = [[torch.from_numpy(synth.make_logits(wl, b, layer=li)).to(dev) for b in range(nb)]
              for li in range(L)]
    xs = [torch.from_numpy(synth.make_x(wl, b).view(np.int16)).to(dev).view(torch.bfloat16)
          for b in range(nb)]
    side = torch.cuda.Stream()
    setup_s = time.time() - t0

    def step(i):
        """One step: every layer of the stack on batch i (each layer's own router logits)."""
        infos = []
        for li in range(L):
            lg, x = logits[li][i % nb], xs[i % nb]
            if args.fill_groups > 0:
                infos.append(layer.forward_streamed(lg, x, li, cache, pool_W, table, side=side,
                                                    groups=args.fill_groups)[1])
            else:
                infos.append(layer.forward_cached(lg, x, li, cache, pool_W, table,
                                                  side=side)[1])
        return infos

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    st0 = cache.stats()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    touched, misses, waves = [], [], []
    start.record()
    for i in range(steps):
        for info in step(warmup + i):
            touched.append(info["hits"] + info["misses"])
            misses.append(info["misses"])
            waves.append(info.get("waves", 1))
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    st1 = cache.stats()
    filled = st1["bytes_filled"] - st0["bytes_filled"]

    # miss rate against pool size: the run's own routing (device route + permute, counts
    # to host) replayed through the same policy on host-only handles, waves as above
    sweep = None
    if args.slot_sweep:
        from moe_expert_ffn_router_amd.layer import plan_waves
        counts = {}
        for li in range(L):
            for b in range(nb):
                layer.route_permute(logits[li][b])
                counts[li, b] = layer.counts[:E].cpu().numpy().copy()
        sweep = []
        for S_s in [int(v) for v in args.slot_sweep.split(",")]:
            h = moe.ExpertCache(L, E, S_s, stride)
            m_t = n_t = w_t = 0
            for i in range(warmup + steps):
                for li in range(L):
                    c = counts[li, i % nb]
                    for wave in plan_waves(c, S_s, h.expert_cache_row(li).numpy()):
                        cw = np.zeros(E, dtype=np.int32)
                        cw[wave] = c[wave]
                        _, _, nm, nh, _ = h.expert_cache_lookup(li, torch.from_numpy(cw))
                        if i >= warmup:
                            m_t, n_t, w_t = m_t + nm, n_t + nm + nh, w_t + 1
            h.close()
            sweep.append({"slots": S_s, "misses_per_layer_step": round(m_t / (steps * L), 2),
                          "hit_rate": round(1 - m_t / max(1, n_t), 4),
                          "waves_per_layer_step": round(w_t / (steps * L), 2),
                          "fill_gb_per_layer_step": round(m_t * payload / (steps * L) / 1e9, 3)})

    # elastic resize of the live pool (in place): halve it, keeping the most recently
    # used residents, then grow back; wall time of each host-synchronous call
    t_r = time.time()
    cache.moe_cache_resize(max(1, S // 2), side=side)
    shrink_ms = (time.time() - t_r) * 1e3
    t_r = time.time()
    cache.moe_cache_resize(S, side=side)
    grow_ms = (time.time() - t_r) * 1e3

    # pinned host -> HBM copy rate of this machine (the fill path's ceiling)
    n_copy = min(64, S)
    h2d = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    h2d[0].record(side)
    with torch.cuda.stream(side):
        pool[:n_copy].copy_(bank[:n_copy], non_blocking=True)
    h2d[1].record(side)
    torch.cuda.synchronize()
    h2d_gbs = n_copy * stride / (h2d[0].elapsed_time(h2d[1]) / 1e3) / 1e9
    # (the cache is not used after this point: the pool is rewritten below)

    # hit path: the expert FFN on the pool with every expert of the last batch resident,
    # replayed in a graph (slot table: touched expert -> its slot)
    b = (warmup + steps - 1) % nb
    layer.route_permute(logits[0][b])
    ids_needed = torch.nonzero(layer.counts[:E] > 0).flatten().to(torch.int32)
    ident = torch.full((E,), 0, dtype=torch.int32, device=dev)
    ident[ids_needed.long()] = torch.arange(len(ids_needed), dtype=torch.int32, device=dev)
    for j, e in enumerate(ids_needed.tolist()):
        pool[j].copy_(bank[e], non_blocking=True)
    torch.cuda.synchronize()
    reps = 10
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            layer.expert_ffn(pool_W, xs[b], wl.T, ident)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    ffn_ms = e0.elapsed_time(e1) / reps
    A = wl.T * wl.k
    n_t = len(ids_needed)
    ffn_bytes = n_t * payload + wl.T * wl.H * 2 + 2 * A * wl.I * 2 + A * wl.H * 2
    achieved = ffn_bytes / (ffn_ms / 1e3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": "moe_expert_ffn on the slot pool (gate/up + down launches), hit path",
            "ffn_ms": round(ffn_ms, 5),
            "timing": f"HIP events around one replay of a graph of {reps} FFN launches",
            "algorithmic_bytes_per_launch": int(ffn_bytes),
            "algorithmic_flops_per_launch": int(2.0 * A * 3 * wl.H * wl.I),
            "touched_experts": n_t}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, bank[:E], None, args.cpu_seconds)

    out = {
        "metric": "MoE-layer tokens/s at 1 GPU; % HBM roofline (decode), % MFMA peak (prefill)",
        "value": round(wl.T * L * steps / (total_ms / 1e3), 1),  # MoE-layer tokens
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(total_ms / steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "E": E, "I": wl.I, "k": wl.k,
                   "weights": wl.fmt, "global_batch": wl.T, "pool_slots": S,
                   "layers_per_step": L, "ms_per_layer": round(total_ms / steps / L, 4),
                   "domains": wl.domains, "batches_rotated": nb,
                   "boundary": ("route+permute -> counts to host -> expert_cache_lookup -> "
                                "expert_cache_fill_groups (%d copy groups on a side stream, "
                                "pinned bank) -> expert_ffn on the pool via the slot table for "
                                "the hits at once and for each group as it lands -> combine; "
                                "eager" % args.fill_groups) if args.fill_groups > 0 else
                               ("route+permute -> counts to host -> expert_cache_lookup -> "
                                "expert_cache_fill (side stream, pinned bank) -> expert_ffn on "
                                "the pool via the slot table -> combine; eager"),
                   "fill_groups": args.fill_groups,
                   "parallelism": "none (1 GPU)", "setup_s": round(setup_s, 1)},
        "cache": {"touched_mean": round(float(np.mean(touched)), 1),
                  "misses_mean": round(float(np.mean(misses)), 1),
                  "waves_mean": round(float(np.mean(waves)), 2),
                  "per": "layer-step",
                  "hit_rate": round(1 - sum(misses) / max(1, sum(touched)), 4),
                  "bytes_filled": int(filled),
                  "fill_gb_per_step": round(filled / steps / 1e9, 3),
                  "pinned_h2d_gbs": round(h2d_gbs, 1),
                  "resize_ms": {"to_%d" % max(1, S // 2): round(shrink_ms, 2),
                                "to_%d" % S: round(grow_ms, 2)},
                  "slot_sweep": sweep},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    cache.close()


def cpu_baseline(wl, base_set, shared, budget_s):
    """Time the CPU oracle (float64 numpy) on whole batches of the same workload."""
    import torch
    from oracle import layer as OL
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    recs = {}

    def rec(e):
        if e not in recs:
            recs[e] = base_set[e].cpu().numpy()
        return recs[e]

    sh = None
    if shared is not None:
        s_host = shared[0].cpu().numpy()
        sh = OL.ExpertSet("bf16", wl.H, wl.shared_I, lambda e: s_host)
    T_sample = wl.T
    # large batches: a token subset of the batch (per-token outputs are independent)
    if wl.T * wl.k * 3 * wl.H * wl.I * 2 > 2e11:
        T_sample = max(1, int(2e11 / (wl.k * 3 * wl.H * wl.I * 2)))
    done_tokens, t0, b = 0, time.time(), 0
    while True:
        ex = OL.ExpertSet(wl.fmt, wl.H, wl.I, rec)
        lg = synth_logits(wl, b)[:T_sample]
        xb = synth_x(wl, b)[:T_sample]
        OL.forward(lg, xb, wl.k, ex, shared=sh)
        done_tokens += T_sample
        b += 1
        recs.clear()
        if time.time() - t0 >= budget_s:
            break
    el = time.time() - t0
    del torch
    return {"value": round(done_tokens / el, 3), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{b} batch(es) of {T_sample} of {wl.T} tokens, {wl.name} weights "
                      f"(float64 numpy, weights decoded per call), {el:.1f} s"}


def synth_logits(wl, b):
    import synth
    return synth.make_logits(wl, b)


def synth_x(wl, b):
    import synth
    return synth.make_x(wl, b)


if __name__ == "__main__":
    main()

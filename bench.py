"""MoE-layer forward benchmark on one MI355X.

One step = one pass of the whole layer (route -> permute -> expert FFN ->
combine, plus the shared expert where the workload has one) over one batch,
inputs already resident in HBM.  Weight sets of several layers are rotated so
that the touched expert bytes of consecutive steps do not sit in the 256 MB
last-level cache (a model walks its layers the same way), and every step gets
a fresh batch of logits and activations.

Default run: the decode layer (decode_mxfp4, T=8, H=2048, E=256, I=512, top-8,
MXFP4 experts) is the headline (`value`, `roofline`, `cpu_baseline`), timed for
exactly --steps steps after --warmup untimed ones; then every other synthetic
layer is timed with its own step count and reported in `per_workload`
(tokens/s, ms per step, the roofline of its dominant launches, the arithmetic
its kernels issue, and the CPU oracle on a bounded sample).  `--workload NAME`
times one layer alone.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
MFMA_FP8_PEAK_TFLOPS = 5000.0   # dense fp8 (and fp8 x fp4) MFMA
MFMA_FP4_PEAK_TFLOPS = 10100.0  # dense fp4 x fp4 MFMA
LLC_BYTES = 256 << 20           # Infinity Cache
METRIC = "MoE-layer tokens/s at 1 GPU; % HBM roofline (decode), % MFMA peak (prefill)"

HEADLINE = "decode_mxfp4"
ORDER = ("decode_mxfp4", "tiny_bf16", "prefill_nvfp4", "large_prefill_mxfp4", "fp8_lru_pool")

DEFAULTS = {  # workload -> (steps, warmup, batches)
    "tiny_bf16": (200, 20, 16),
    "decode_mxfp4": (400, 40, 64),
    "prefill_nvfp4": (50, 5, 8),
    "fp8_lru_pool": (24, 2, 12),
    "large_prefill_mxfp4": (10, 2, 2),
}

# the arithmetic each workload's kernels issue (operand types of the MFMAs, accumulator)
DTYPE = {
    "tiny_bf16": "bf16*bf16->f32",
    "decode_mxfp4": "e4m3(hi+lo)*e2m1->f32",
    "prefill_nvfp4": "bf16*bf16->f32",
    "fp8_lru_pool": "e4m3(hi+lo)*e4m3->f32",
    "large_prefill_mxfp4": "e4m3(hi+lo)*e2m1->f32 (+shared bf16*bf16->f32)",
}
DTYPE_NOTE = {
    "tiny_bf16": "bf16 weights and activations on the bf16 MFMA, fp32 accumulation",
    "decode_mxfp4": ("block-scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4): packed E2M1 "
                     "weights with their E8M0 scales as stored; each bf16 activation split "
                     "into E4M3 hi + lo with one E8M0 scale per 32, two MFMAs per product; "
                     "fp32 accumulation"),
    "prefill_nvfp4": ("E2M1 codes times their E4M3 block scales decoded to bf16 in registers "
                      "(exact), bf16 MFMA 32x32x16, fp32 accumulation, per-tensor fp32 scale "
                      "on the accumulators"),
    "fp8_lru_pool": ("block-scaled MFMA with E4M3 weights as stored (unit MFMA scale), bf16 "
                     "activations split into E4M3 hi + lo, fp32 128x128 block scales applied "
                     "to fp32 partial sums"),
    "large_prefill_mxfp4": ("routed experts as decode_mxfp4 (block-scaled MFMA, hi + lo "
                            "activations); shared expert bf16 MFMA"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="all",
                    help="'all' (default: the decode headline plus every other workload) or "
                         "one workload name")
    ap.add_argument("--rot", type=int, default=0, help="weight sets rotated (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=5.0,
                    help="CPU oracle budget per workload (at least one batch is run)")
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
    "layer": ("ffn.hip", "ffn_common.h", "lds_copy.h", "moe_internal.h", "route.hip",
              "route_common.h", "permute.hip", "combine.hip"),
}


def source_hash(workload: str) -> str:
    """sha256 over the workload's kernel sources: counter readings are valid only for these
    bytes (decode_mxfp4 runs the decode-layer kernels, the other workloads the separate
    route / permute / expert FFN / combine kernels)."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES["decode" if workload == "decode_mxfp4" else "layer"]:
        with open(os.path.join(ROOT, "moe_expert_ffn_router_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """(HBM bytes per step, source) from committed rocprofv3 FETCH_SIZE / WRITE_SIZE readings,
    scaled by the copy-kernel calibration; (None, reason) when there are none or they were
    taken on other kernel sources."""
    rel = os.path.join("profiles", f"traffic_{workload}.txt")
    path = os.path.join(ROOT, rel)
    if not os.path.exists(path):
        return None, "no counter reading for this workload"
    for line in open(path):
        if line.startswith("TRAFFIC "):
            rec = json.loads(line[len("TRAFFIC "):])
            if rec.get("source_hash") != source_hash(workload):
                return None, f"{rel}: taken on other kernel sources (stale)"
            return (int(sum(k["fetch_kib"] * 1024 * rec["fetch_scale"] +
                            k["write_kib"] * 1024 * rec["write_scale"]
                            for k in rec["kernels"].values())),
                    f"{rel}: rocprofv3 FETCH_SIZE + WRITE_SIZE passes on these kernel sources, "
                    "committed reading (not counted in this run)")
    return None, f"{rel}: no TRAFFIC line"


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
    """Plain streaming reads (the measurement library's moe_measure_hbm_read) of sizes from a
    decode launch's bytes to 1 GiB, 24 launches in one graph replay; each launch reads a
    region the previous launches did not (the buffer spans 8x the largest size, well past
    the memory-side cache)."""
    import torch

    from moe_expert_ffn_router_amd import measure
    big = 1 << 30
    buf = torch.ones(8 * big, dtype=torch.uint8, device="cuda")
    sink = torch.empty(8192 * 256, dtype=torch.int32, device="cuda")
    rows = []
    for nbytes in (16 << 20, 34_000_000, 68_000_000, 96_404_480, 256 << 20, big):
        n = nbytes // 16 * 16
        regions = buf.numel() // n
        for grid in (512, 1024, 2048, 4096):
            for r in range(3):
                measure.moe_measure_hbm_read(buf[(r % regions) * n:], n, grid, sink)
            reps = 24
            g = torch.cuda.CUDAGraph()  # launches back to back, no host gaps
            with torch.cuda.graph(g):
                for r in range(reps):
                    measure.moe_measure_hbm_read(buf[((3 + r) % regions) * n:], n, grid, sink)
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


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def roofline_mfma(flops: float, ms: float, issued: str) -> dict:
    """MFMA roofline: algorithmic flops over the launches' time against the peak of the
    instruction the kernels issue for an exact product (see `issued`)."""
    achieved = flops / (ms / 1e3) / 1e12
    r = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
         "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4)}
    if issued == "hilo":
        r["peak_note"] = ("two fp8-rate block-scaled MFMAs (hi, lo) per product: executed "
                          "flops = 2 x algorithmic against the 5.0 PFLOP/s fp8 peak, the same "
                          "fraction as algorithmic flops against 2.5 PFLOP/s")
    else:
        r["peak_note"] = "bf16 MFMA, 2.5 PFLOP/s dense"
    r["frac_of_fp8_peak_algorithmic"] = round(achieved / MFMA_FP8_PEAK_TFLOPS, 4)
    r["frac_of_fp4_peak_algorithmic"] = round(achieved / MFMA_FP4_PEAK_TFLOPS, 4)
    return r


def roofline_hbm(nbytes: float, ms: float) -> dict:
    achieved = nbytes / (ms / 1e3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4)}


def graph_time(torch, fn, first: int, steps: int, use_graph: bool) -> float:
    """Run fn(first .. first+steps-1) once as a captured graph (or eagerly); return ms."""
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


# ---------------------------------------------------------------------------
# all experts resident in HBM
# ---------------------------------------------------------------------------
def bench_resident(args, wl, steps, warmup, want_cpu: bool):
    import torch

    import moe_expert_ffn_router_amd as moe
    import synth

    _, _, nb = DEFAULTS[wl.name]
    dev = torch.device("cuda")
    torch.cuda.set_device(0)
    lay = synth.record_layout(wl.fmt, wl.H, wl.I)
    stride, payload = lay["stride"], lay["payload"]

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
    Ws = (moe.experts("bf16", 1, wl.H, wl.shared_I, shared, shared.shape[1])
          if shared is not None else None)

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

    use_graph = not args.eager
    # decode-sized batches: the whole-layer path (moe_forward_decode); otherwise the
    # separate calls
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
    if not whole:
        for b in range(nb):
            layer.route_permute(logits[b])
            perm.append((layer.counts.clone(), layer.offsets.clone(), layer.sorted_idx.clone()))

    def ffn_only(i):
        b = i % nb
        c, o, sidx = perm[b]
        moe.moe_expert_ffn(Wsets[i % rot], None, xs[b], wl.T, wl.k, c, o, sidx, layer.y_perm,
                           layer.ffn_ws, args.variant)

    def shared_only(i):
        layer.shared_ffn(Ws, xs[i % nb], wl.T)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    total_ms = graph_time(torch, step, warmup, steps, use_graph)
    # dominant work: the whole-layer launches for decode batches, else the expert-FFN
    # launches replayed on their own
    ffn_ms = total_ms / steps if whole else graph_time(torch, ffn_only, warmup, steps,
                                                       use_graph) / steps
    shared_ms = (graph_time(torch, shared_only, warmup, steps, use_graph) / steps
                 if Ws is not None else None)
    ms_per_step = total_ms / steps
    tokens_per_s = wl.T * L * steps / (total_ms / 1e3)

    # ---- roofline of the dominant launches ----------------------------------
    A = wl.T * wl.k
    step_batches = [(warmup + i + li) % nb for i in range(steps) for li in range(L)]
    t_mean = float(np.mean([touched[b] for b in step_batches]))
    ffn_flops = L * 2.0 * A * 3 * wl.H * wl.I
    if whole:
        # one call per layer: logits in, touched experts' weights once, x in, routing
        # outputs and y out (h never leaves the chip on the one-stream path; the fp32
        # partials it writes and re-reads are implementation traffic, in `traffic`)
        ffn_bytes = L * (t_mean * payload + wl.T * wl.E * 4 + wl.T * wl.H * 2
                         + wl.T * wl.H * 2 + A * 4 * 4 + (2 * wl.E + 1) * 4)
    else:
        # touched weights once, x in, h written and read, y_perm written
        ffn_bytes = L * (t_mean * payload + wl.T * wl.H * 2 + 2 * A * wl.I * 2 + A * wl.H * 2)
    t_hbm = ffn_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = ffn_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    issued = "hilo" if wl.fmt in ("mxfp4", "fp8_b128") else "bf16"
    if wl.name == "tiny_bf16":
        roof = roofline_hbm(ffn_bytes, ffn_ms)
        roof["bound"] = "latency"
        roof["note"] = ("1.7 MB and 25 MFLOP per step: the launches' fixed latency binds, "
                        "neither HBM nor MFMA (frac shown against 8 TB/s for reference)")
    elif t_hbm >= t_mfma:
        roof = roofline_hbm(ffn_bytes, ffn_ms)
    else:
        roof = roofline_mfma(ffn_flops, ffn_ms, issued)
    traffic, tsrc = (None, "graph replay of the default configuration only")
    if use_graph and args.tokens is None and L == 1:
        traffic, tsrc = measured_traffic(wl.name)
    roof["traffic"] = traffic
    roof.update({"traffic_source": tsrc,
                 "kernel": ("moe_forward_decode, one weight stream (2 launches: the expert FFN "
                            "with routing, then the combine)" if whole and wl.T <= 16 else
                            "moe_forward_decode (4 launches)" if whole
                            else "moe_expert_ffn (gate/up + down launches)"),
                 "ffn_ms": round(ffn_ms, 5),
                 "timing": ("HIP events on the launch stream around one replay of a graph of "
                            "the %d steps" % steps + (" (%d layers each)" % L if L > 1 else "")
                            + ("" if whole else "; FFN launches replayed in a graph of their "
                               "own"))
                           if use_graph else "HIP events, eager",
                 "algorithmic_bytes_per_launch": int(ffn_bytes),
                 "algorithmic_flops_per_launch": int(ffn_flops),
                 "touched_experts_mean": round(t_mean, 2)})
    res = {
        "workload": wl.name, "value": round(tokens_per_s, 1), "unit": "tokens/s",
        "ms_per_step": round(ms_per_step, 5), "steps": steps, "warmup": warmup,
        "dtype": DTYPE.get(wl.name, "bf16*bf16->f32"), "dtype_note": DTYPE_NOTE.get(wl.name, ""),
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "E": wl.E, "I": wl.I, "k": wl.k,
                   "weights": wl.fmt, "shared_I": wl.shared_I, "global_batch": wl.T,
                   "weight_sets_rotated": rot, "batches_rotated": nb,
                   "layers_per_step": L, "us_per_layer": round(ms_per_step * 1e3 / L, 2),
                   "boundary": ("route->permute->expert_ffn->combine on one stream, "
                                + ("as whole-layer decode launches, " if whole else "")
                                + ("one captured HIP graph of the K steps" if use_graph
                                   else "eager launches")),
                   "parallelism": "none (1 GPU)", "setup_s": round(setup_s, 1)},
        "roofline": roof,
    }
    if shared_ms is not None:
        sflops = 2.0 * wl.T * 3 * wl.H * wl.shared_I
        res["shared_expert"] = {"ms": round(shared_ms, 5), "flops": int(sflops),
                                "roofline": roofline_mfma(sflops, shared_ms, "bf16"),
                                "kernel": "moe_shared_ffn"}
        routed_flops = ffn_flops
        res["layer_roofline"] = roofline_mfma(routed_flops + sflops, ms_per_step, issued)
        res["layer_roofline"]["note"] = "whole step (route .. combine) against the MFMA peak"
    if want_cpu:
        res["cpu_baseline"] = cpu_baseline(wl, lambda e: base_set[e].cpu().numpy(), shared,
                                           args.cpu_seconds)
        if wl.name in ("tiny_bf16", "decode_mxfp4"):
            res["cpu_baseline_1thread"] = cpu_baseline(
                wl, lambda e: base_set[e].cpu().numpy(), shared, args.cpu_seconds, threads=1)
    del sets, Wsets, base_set, layer, stack, perm, logits, xs, shared
    gc.collect()
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# experts in a pinned host bank, an HBM slot pool in front of it
# ---------------------------------------------------------------------------
def bench_cached(args, wl, steps, warmup, want_cpu: bool):
    """The slot-pool workload: experts live in a pinned host bank, a pool of wl.pool_slots HBM
    slots holds the ones in use, the LRU lookup runs on the host after each routing, misses are
    copied on a side stream and the FFN reads the pool through the slot table.  One step =
    route+permute, counts to the host, lookup, fills, expert FFN, combine (eager: the host
    decision sits in the middle of every step).  Batches rotate over the domain-biased routing
    distributions, so the pool churns.  Three boundaries: end to end (the step), the fill path
    alone (route+permute, lookup, fills; no FFN) against the measured pinned copy rate, and
    the hit path (the expert FFN with every expert of a batch resident)."""
    import torch

    import moe_expert_ffn_router_amd as moe
    import synth

    nb = wl.batches
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

    # fill path alone: the same kind of steps without the FFN and the combine (the next
    # batches of the rotation, so the pool keeps churning)
    st0 = cache.stats()
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cs = torch.cuda.current_stream()
    f0.record()
    for i in range(steps):
        for li in range(L):
            layer.route_permute(logits[li][(warmup + steps + i) % nb])
            counts_host = layer.counts[:E].to("cpu")
            me, ms, _, _, _ = cache.expert_cache_lookup(li, counts_host)
            cache.expert_cache_fill(li, me, ms, side=side, compute=cs)
    f1.record()
    torch.cuda.synchronize()
    fill_ms = f0.elapsed_time(f1)
    fill_bytes = cache.stats()["bytes_filled"] - st0["bytes_filled"]

    # miss rate against pool size: the run's own routing (device route + permute, counts
    # to host) replayed through the same policy on host-only handles, waves as above
    sweep = None
    if args.slot_sweep:
        counts = {}
        for li in range(L):
            for b in range(nb):
                layer.route_permute(logits[li][b])
                counts[li, b] = layer.counts[:E].cpu().clone()
        sweep = []
        for S_s in [int(v) for v in args.slot_sweep.split(",")]:
            h = moe.ExpertCache(L, E, S_s, stride)
            m_t = n_t = w_t = 0
            for i in range(warmup + steps):
                for li in range(L):
                    r = h.expert_cache_plan(li, counts[li, i % nb])
                    if i >= warmup:
                        m_t, n_t = m_t + r["misses"], n_t + r["misses"] + r["hits"]
                        w_t += r["n_waves"]
            h.close()
            sweep.append({"slots": S_s, "misses_per_layer_step": round(m_t / (steps * L), 2),
                          "hit_rate": round(1 - m_t / max(1, n_t), 4),
                          "waves_per_layer_step": round(w_t / (steps * L), 2),
                          "fill_gb_per_layer_step": round(m_t * payload / (steps * L) / 1e9, 3)})

    # waves: a pool smaller than one step's experts (two staging sets of S/2 slots:
    # each wave's copies overlap the FFN of the wave before), same bank and batches,
    # timed against the fill floor of its own copies
    wave_case = None
    if L == 1 and args.slots is None:
        S_w = 48
        pool_w = torch.empty((S_w, stride), dtype=torch.uint8, device=dev)
        table_w = torch.full((E,), -1, dtype=torch.int32, device=dev)
        cache_w = moe.ExpertCache(1, E, S_w, stride, pool_w, bank, table_w)
        pool_Ww = moe.experts(wl.fmt, E, wl.H, wl.I, pool_w, stride)
        n_w = 6
        layer.forward_streamed(logits[0][0], xs[0], 0, cache_w, pool_Ww, table_w, side=side,
                               groups=args.fill_groups or 1)
        torch.cuda.synchronize()
        s0 = cache_w.stats()
        w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        wv = []
        w0.record()
        for i in range(n_w):
            _, info = layer.forward_streamed(logits[0][(1 + i) % nb], xs[(1 + i) % nb], 0,
                                             cache_w, pool_Ww, table_w, side=side,
                                             groups=args.fill_groups or 1)
            wv.append(info["waves"])
        w1.record()
        torch.cuda.synchronize()
        wms = w0.elapsed_time(w1) / n_w
        wbytes = (cache_w.stats()["bytes_filled"] - s0["bytes_filled"]) / n_w
        wave_case = {"pool_slots": S_w, "steps": n_w, "ms_per_step": round(wms, 3),
                     "waves_per_step": round(float(np.mean(wv)), 2),
                     "fill_gb_per_step": round(wbytes / 1e9, 3),
                     "fill_floor_ms_per_step": round(wbytes / (h2d_gbs_probe(torch, pool_w, bank, side)
                                                               * 1e9) * 1e3, 3)}
        wave_case["frac_of_fill_floor"] = round(wave_case["fill_floor_ms_per_step"] / wms, 4)
        cache_w.close()
        del cache_w, pool_w, table_w

    # hybrid steps (part of each step's misses on the CPU, from the bank): calibrate the
    # host-memory and PCIe rates with the real kernels, split at the calibrated fetch
    # fraction (q*), and time steps on a fresh pool of the same size
    hybrid = None
    if L == 1 and args.slots is None:
        threads = max(1, len(os.sched_getaffinity(0)))
        cpu_pool = moe.CpuPool(threads)
        pool_h = torch.empty((S, stride), dtype=torch.uint8, device=dev)
        bank_W = moe.experts(wl.fmt, E, wl.H, wl.I, bank.data_ptr(), stride)
        prof = moe.moe_bench_bw(cpu_pool, bank_W, pool_h, 16, 2.0, stream=side)
        table_h = torch.full((E,), -1, dtype=torch.int32, device=dev)
        cache_h = moe.ExpertCache(1, E, S, stride, pool_h, bank, table_h)
        pool_Wh = moe.experts(wl.fmt, E, wl.H, wl.I, pool_h, stride)
        q = float(prof["fetch_fraction"])
        n_h = 4
        for i in range(2):   # fill the pool, as the offload run did in its warm-up
            layer.forward_hybrid(logits[0][i % nb], xs[i % nb], 0, cache_h, pool_Wh, table_h,
                                 cpu_pool, q, side=side, groups=args.fill_groups or 1)
        torch.cuda.synchronize()
        h0, h1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n_cpu, n_fetch = [], []
        t_h = time.time()
        h0.record()
        for i in range(n_h):
            _, info = layer.forward_hybrid(logits[0][(2 + i) % nb], xs[(2 + i) % nb], 0, cache_h,
                                           pool_Wh, table_h, cpu_pool, q, side=side,
                                           groups=args.fill_groups or 1)
            n_cpu.append(len(info["cpu"]))
            n_fetch.append(info["fetched"])
        h1.record()
        torch.cuda.synchronize()
        hybrid = {"calibration": {"h2d_gbs": round(prof["h2d_bytes_per_s"] / 1e9, 2),
                                  "cpu_gbs": round(prof["cpu_bytes_per_s"] / 1e9, 2),
                                  "cpu_threads": threads, "threshold": prof["threshold"],
                                  "hybrid_recommended": bool(prof["hybrid_recommended"]),
                                  "fetch_fraction_q": round(q, 4)},
                  "steps": n_h, "ms_per_step": round(h0.elapsed_time(h1) / n_h, 3),
                  "wall_ms_per_step": round((time.time() - t_h) * 1e3 / n_h, 3),
                  "cpu_experts_per_step": round(float(np.mean(n_cpu)), 1),
                  "fetched_per_step": round(float(np.mean(n_fetch)), 1),
                  "tokens_per_s": round(wl.T * n_h / (h0.elapsed_time(h1) / 1e3), 1),
                  "offload_ms_per_step": round(total_ms / steps, 3),
                  "note": ("auto would " + ("choose hybrid" if prof["hybrid_recommended"]
                                            else "stay on offload") +
                           " (CPU rate vs threshold x PCIe rate); timed at the calibrated split")}
        cache_h.close()
        cpu_pool.close()
        del cache_h, pool_h, table_h

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
    roof = roofline_hbm(ffn_bytes, ffn_ms)
    traffic, tsrc = measured_traffic(wl.name)
    roof.update({"traffic": traffic, "traffic_source": tsrc,
                 "kernel": "moe_expert_ffn on the slot pool (gate/up + down launches), hit path",
                 "ffn_ms": round(ffn_ms, 5),
                 "timing": f"HIP events around one replay of a graph of {reps} FFN launches",
                 "algorithmic_bytes_per_launch": int(ffn_bytes),
                 "algorithmic_flops_per_launch": int(2.0 * A * 3 * wl.H * wl.I),
                 "touched_experts": n_t})

    res = {
        "workload": wl.name,
        "value": round(wl.T * L * steps / (total_ms / 1e3), 1),  # MoE-layer tokens
        "unit": "tokens/s", "steps": steps, "warmup": warmup,
        "ms_per_step": round(total_ms / steps, 4),
        "dtype": DTYPE[wl.name], "dtype_note": DTYPE_NOTE[wl.name],
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
        "end_to_end": {"ms_per_step": round(total_ms / steps, 4),
                       "tokens_per_s": round(wl.T * L * steps / (total_ms / 1e3), 1),
                       "fill_floor_ms_per_step": round(filled / steps / (h2d_gbs * 1e9) * 1e3, 3),
                       "frac_of_fill_floor": round(filled / steps / (h2d_gbs * 1e9) * 1e3
                                                   / (total_ms / steps), 4)},
        "fill_path": {"ms_per_step": round(fill_ms / steps, 4),
                      "gb_per_step": round(fill_bytes / steps / 1e9, 3),
                      "achieved_gbs": round(fill_bytes / (fill_ms / 1e3) / 1e9, 2),
                      "pinned_h2d_gbs": round(h2d_gbs, 2),
                      "frac_of_h2d": round(fill_bytes / (fill_ms / 1e3) / 1e9 / h2d_gbs, 4),
                      "boundary": "route+permute -> counts to host -> lookup -> "
                                  "expert_cache_fill, no FFN; eager"},
        "hit_path": {"ffn_ms": round(ffn_ms, 5), "frac_of_hbm": roof["frac"]},
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
        "waves": wave_case,
        "hybrid": hybrid,
        "roofline": roof,
    }
    if want_cpu:
        res["cpu_baseline"] = cpu_baseline(wl, lambda e: bank[e].numpy(), None, args.cpu_seconds)
    cache.close()
    del cache, pool, bank, table, layer, logits, xs, g
    gc.collect()
    torch.cuda.empty_cache()
    return res


def h2d_gbs_probe(torch, pool, bank, side) -> float:
    """Pinned host -> HBM copy rate of whole expert records on `side` (GB/s)."""
    n = min(16, pool.shape[0])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(side)
    with torch.cuda.stream(side):
        pool[:n].copy_(bank[:n], non_blocking=True)
    e1.record(side)
    torch.cuda.synchronize()
    return n * pool.shape[1] / (e0.elapsed_time(e1) / 1e3) / 1e9


# ---------------------------------------------------------------------------
# CPU oracle baseline
# ---------------------------------------------------------------------------
def cpu_baseline(wl, rec_of, shared, budget_s, threads=None):
    """Time the CPU oracle (float64 numpy, as it stands) on token batches of the same
    workload until budget_s has passed (at least one batch)."""
    import contextlib

    from oracle import layer as OL
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_info = threadpool_limits = None
    ctx = (threadpool_limits(limits=threads) if (threads and threadpool_limits)
           else contextlib.nullcontext())
    with ctx:
        if threadpool_info is not None:
            used = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        else:
            used = len(os.sched_getaffinity(0))
        recs = {}

        def rec(e):
            if e not in recs:
                recs[e] = rec_of(e)
            return recs[e]

        sh = None
        if shared is not None:
            s_host = shared[0].cpu().numpy()
            sh = OL.ExpertSet("bf16", wl.H, wl.shared_I, lambda e: s_host)
        # large batches: a token subset of the batch (per-token outputs are independent)
        T_sample = wl.T
        if wl.T * wl.k * 3 * wl.H * wl.I * 2 > 2e10:
            T_sample = max(1, int(2e10 / (wl.k * 3 * wl.H * wl.I * 2)))
        done_tokens, t0, b = 0, time.time(), 0
        import synth
        while True:
            ex = OL.ExpertSet(wl.fmt, wl.H, wl.I, rec)
            lg = synth.make_logits(wl, b)[:T_sample]
            xb = synth.make_x(wl, b)[:T_sample]
            OL.forward(lg, xb, wl.k, ex, shared=sh)
            done_tokens += T_sample
            b += 1
            recs.clear()
            if time.time() - t0 >= budget_s:
                break
        el = time.time() - t0
    return {"value": round(done_tokens / el, 3), "unit": "tokens/s", "cores": int(used),
            "kind": "oracle",
            "sample": f"{b} batch(es) of the first {T_sample} of {wl.T} tokens, {wl.name} "
                      f"(float64 numpy, weights decoded per batch), {el:.1f} s"}


def cpu_info() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def run_one(args, name, steps, warmup, want_cpu):
    import synth
    wl = synth.WORKLOADS[name]
    if args.tokens is not None:
        wl = wl.scaled(T=args.tokens)
    if wl.pool_slots and not args.resident:
        return bench_cached(args, wl, steps, warmup, want_cpu)
    return bench_resident(args, wl, steps, warmup, want_cpu)


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
    want_cpu = not args.no_cpu_baseline
    head = HEADLINE if args.workload == "all" else args.workload
    d_steps, d_warm, _ = DEFAULTS[head]
    steps = args.steps if args.steps is not None else d_steps
    warmup = args.warmup if args.warmup is not None else d_warm
    t_all = time.time()
    log(f"{head}: {steps} steps after {warmup} warm-up steps")
    hr = run_one(args, head, steps, warmup, want_cpu)
    per = {}
    if args.workload == "all":
        per[head] = {k: v for k, v in hr.items() if k not in ("config",)}
        for name in ORDER:
            if name == head:
                continue
            s, w, _ = DEFAULTS[name]
            log(f"{name}: {s} steps after {w} warm-up steps")
            r = run_one(args, name, s, w, want_cpu)
            per[name] = r
    out = {
        "metric": METRIC,
        "value": hr["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": hr["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": hr["dtype"],
        "data": "synthetic",
        "config": hr["config"],
        "roofline": hr["roofline"],
        "cpu_baseline": hr.get("cpu_baseline"),
    }
    for key, val in hr.items():
        if key not in out and key not in ("workload", "unit", "steps", "warmup", "dtype_note"):
            out[key] = val
    if per:
        out["per_workload"] = per
    out["host"] = {"cpu": cpu_info(), "affinity_cores": len(os.sched_getaffinity(0))}
    out["wall_s"] = round(time.time() - t_all, 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

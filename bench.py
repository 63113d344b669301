#!/usr/bin/env python3
"""Benchmark of the quantized MoE FFN block on one MI355X.

Metric: MoE-layer tokens/s at decode batch 1 (one Gemma-4-26B-A4B-like layer:
d_model 2816, 128 experts of d_ff 704 with 4-bit affine group-64 weights, shared
expert d_ff 2112, 8-bit router, top-8), with the fraction of the HBM roofline
on active-expert bytes. The 128-row prefill chunk (Zipf-skewed routing) is
measured in the same run and reported under "prefill" with its roofline and
MFMA utilisation, and the 30-layer stacks (decode 1 row, prefill chunks of 256
rows, residual add between layers) under "stack".

Inputs are synthetic and seeded (see synth/): every step uses a different layer
of a pool of independently drawn layers and a fresh activation row, so the
weights a step touches are not resident in the 256 MB Infinity Cache from the
previous step. All inputs are in HBM before the timed region. Steps are
captured in HIP graphs (one graph = one pass over the rotation) and replayed.

One JSON line on stdout; progress on stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # B/s, MI355X HBM3E
MFMA_F16_PEAK = 2.5e15     # flop/s, dense fp16/bf16 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_bytes(shape):
    """Algorithmic HBM bytes of one decode token-layer: router + top_k experts +
    shared expert weights, x in (bf16) and y out (fp32)."""
    import quantized_mixture_experts_bit_amd as q
    s = q.as_shape(shape)
    return (q.moe_router_blob_bytes(s) + shape.top_k * q.moe_expert_blob_bytes(s) + q.moe_shared_blob_bytes(s)
            + 2 * shape.d_model + 4 * shape.d_model)


def prefill_roofline(shape, counts, rows):
    """Ideal time of one prefill chunk: per GEMM group max(bytes / HBM, flops / MFMA)."""
    import quantized_mixture_experts_bit_amd as q
    s = q.as_shape(shape)
    d, f, fs = shape.d_model, shape.d_ff, shape.d_ff_shared
    t = 0.0
    flops = 0.0
    nbytes = 0.0
    for c in counts:
        if c > 0:
            fl = 2.0 * c * 3 * f * d
            by = q.moe_expert_blob_bytes(s)
            t += max(by / HBM_PEAK, fl / MFMA_F16_PEAK)
            flops += fl
            nbytes += by
    fl = 2.0 * rows * 3 * fs * d
    by = q.moe_shared_blob_bytes(s)
    t += max(by / HBM_PEAK, fl / MFMA_F16_PEAK)
    flops += fl
    nbytes += by
    rb = q.moe_router_blob_bytes(s) + rows * d * 2 + rows * d * 4
    t += rb / HBM_PEAK
    nbytes += rb
    return t, flops, nbytes


CSRC = os.path.join(ROOT, "quantized_mixture_experts_bit_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_decode_fused_gemma4_decode_traffic.txt")


# the files k_decode_fused is built and launched from (its counters stay valid while these do)
DECODE_KERNEL_SOURCES = ("common.h", "decode_fused.h", "moe_lib.hip")


def csrc_digest(names=None):
    """sha256 over the HIP sources (names and bytes, sorted), or over `names` only:
    identifies the kernel build."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        p = os.path.join(CSRC, name)
        if names is not None and name not in names:
            continue
        if os.path.isfile(p) and name.endswith((".h", ".hip", ".cpp")):
            h.update(name.encode())
            with open(p, "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per k_decode_fused launch from the committed counter summary (FETCH_SIZE and
    WRITE_SIZE passes, each divided by the factor the same counter shows on a plain copy of
    known size), or None when the summary is missing or the kernel's sources changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None, None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                a, b = line.split(":", 1)
                kv[a.strip()] = b.strip()
    if kv.get("decode_sources_sha256") != csrc_digest(DECODE_KERNEL_SOURCES):
        return None, "counters were taken on other kernel sources"
    fetch = float(kv["fetch_bytes_per_launch"]) / float(kv["copy_factor_fetch"])
    write = float(kv["write_bytes_per_launch"]) / float(kv["copy_factor_write"])
    return fetch + write, {"fetch_bytes": fetch, "write_bytes": write, "source": os.path.relpath(TRAFFIC_FILE, ROOT)}


def calibrate_copy(mbytes):
    """A plain device copy of known size (for the counter calibration): src -> dst, 5 times."""
    import torch
    n = int(mbytes * 1e6) // 16 * 16
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    src.fill_(7)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 5}), flush=True)


def time_replays(graph, replays, warmup):
    """Replays `graph` `warmup` times untimed, then `replays` times with a HIP event before
    each replay and one after the last, all on the current stream (where replay() launches).
    Returns the per-replay times in ms."""
    import torch
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(replays + 1)]
    ev[0].record()
    for i in range(replays):
        graph.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(replays)]


def spread(per_replay_ms, units):
    """Median, p10 and p90 of the per-unit time (us) over replays of `units` units each."""
    import numpy as np
    v = np.asarray(per_replay_ms, dtype=np.float64) * 1e3 / units
    return {"median_us": float(np.median(v)), "p10_us": float(np.percentile(v, 10)),
            "p90_us": float(np.percentile(v, 90)), "replays": int(v.size), "units_per_replay": int(units)}


def measured_ceilings(dev):
    """Achievable rates on this GPU, run as black boxes: a streaming read (torch sum over
    4 GiB of fp32, far past the 256 MB Infinity Cache) and a large bf16 GEMM (torch matmul,
    hipBLASLt), each the best of 10 timed runs."""
    import torch
    res = {}
    n = 1 << 30
    a = torch.ones(n, dtype=torch.float32, device=dev)
    out = torch.empty((), dtype=torch.float32, device=dev)
    ts = []
    for _ in range(12):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.sum(a, dim=0, out=out)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    res["stream_read_GBps"] = 4.0 * n / (min(ts[2:]) * 1e-3) / 1e9
    res["stream_read"] = "torch.sum over 4 GiB of fp32 (read once), best of 10"
    del a
    m = 8192
    x = torch.randn(m, m, dtype=torch.bfloat16, device=dev)
    y = torch.randn(m, m, dtype=torch.bfloat16, device=dev)
    ts = []
    for _ in range(12):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.matmul(x, y)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    res["bf16_gemm_TFLOPs"] = 2.0 * m ** 3 / (min(ts[2:]) * 1e-3) / 1e12
    res["bf16_gemm"] = "torch.matmul bf16 8192x8192x8192, best of 10"
    del x, y
    torch.cuda.empty_cache()
    return res


def flagged_rows(logits, k, gap=1e-4):
    """Rows whose k-th and (k+1)-th largest logits (the GPU's own fp64 logits) are closer
    than `gap`: the rows where the picks are a near-tie."""
    import numpy as np
    srt = -np.sort(-np.asarray(logits), axis=1)
    return int(((srt[:, k - 1] - srt[:, k]) < gap).sum())


TIMELINE_SLOTS = {  # slot -> meaning, per item kind of the whole-block decode kernel
    "router": {0: "start", 1: "weights and x in", 2: "logits published"},
    "shared gate/up": {0: "start", 1: "router published", 3: "dot products done", 4: "h stored"},
    "routed gate/up": {0: "start", 1: "key words held", 2: "picks ranked", 3: "dot products done", 4: "h stored"},
    "routed down": {0: "start", 1: "key words held", 2: "picks ranked", 3: "first h in", 4: "all h in",
                    5: "dot products done", 7: "outputs stored"},
    "shared down": {0: "start", 4: "all h in", 5: "dot products done", 7: "outputs stored"},
    "combine": {0: "start", 1: "key words held", 2: "picks ranked", 4: "all shared h in", 5: "dot products done",
                6: "all expert outputs in", 7: "y stored"},
}


def decode_timeline(q, shape, run_step, n_steps, dev):
    """Per-phase times of the whole-block decode kernel from the timeline build's
    per-workgroup stamps (100 MHz counter): for each item kind and phase, the median
    and the slowest workgroup, in us from the earliest start of the step; medians of
    those over n_steps steps."""
    import ctypes as C
    import numpy as np
    import torch
    E, k, d, f, fs = shape.n_experts, shape.top_k, shape.d_model, shape.d_ff, shape.d_ff_shared
    n = {"router": E // 2, "shared gate/up": fs // 16, "routed gate/up": k * (f // 16), "routed down": k * (d // 64),
         "shared down": d // 64, "combine": d // 64}
    grid = sum(n.values()) + 1
    buf = torch.zeros(grid * 8, dtype=torch.int64, device=dev)
    fn = q.lib().moe_debug_set_timeline
    fn.restype, fn.argtypes = C.c_int, [C.c_void_p]
    assert fn(buf.data_ptr()) == 0
    per = {kind: {slot: [] for slot in slots} for kind, slots in TIMELINE_SLOTS.items()}
    for i in range(n_steps):
        buf.zero_()
        run_step(i)
        torch.cuda.synchronize()
        t = buf.cpu().numpy().reshape(grid, 8).astype(np.float64)
        t0 = t[:grid - 1, 0].min()
        b = 0
        for kind, cnt in n.items():
            for slot in TIMELINE_SLOTS[kind]:
                v = (t[b:b + cnt, slot] - t0) / 100.0  # 100 MHz ticks -> us
                per[kind][slot].append((float(np.median(v)), float(v.max())))
            b += cnt
    assert fn(None) == 0
    out = {}
    for kind, slots in TIMELINE_SLOTS.items():
        out[kind] = {"items": n[kind]}
        for slot, name in slots.items():
            a = np.asarray(per[kind][slot])
            out[kind][name] = {"median_us": float(np.median(a[:, 0])), "slowest_us": float(np.median(a[:, 1]))}
    return out


def stack_timeline(q, shape, run_stack, n_layers, n_steps, dev):
    """Per-phase times of the one-launch stacked decode from the timeline build: for
    layers 1.. (whose items start while the previous layer finishes), each phase in us
    from the previous layer's last y store, as the median workgroup / slowest workgroup,
    medians over the layers and the n_steps steps; layer 0 from the first start."""
    import ctypes as C
    import numpy as np
    import torch
    E, k, d, f, fs = shape.n_experts, shape.top_k, shape.d_model, shape.d_ff, shape.d_ff_shared
    n = {"router": E // 2, "shared gate/up": fs // 16, "routed gate/up": k * (f // 16), "routed down": k * (d // 64),
         "shared down": d // 64, "combine": d // 64}
    grid = sum(n.values()) + 1
    buf = torch.zeros(n_layers * grid * 8, dtype=torch.int64, device=dev)
    fn = q.lib().moe_debug_set_timeline
    fn.restype, fn.argtypes = C.c_int, [C.c_void_p]
    assert fn(buf.data_ptr()) == 0
    slots = dict(TIMELINE_SLOTS)
    per = {kind: {slot: [] for slot in sl} for kind, sl in slots.items()}
    first = {kind: {slot: [] for slot in sl} for kind, sl in slots.items()}
    ends = []
    for _ in range(n_steps):
        buf.zero_()
        run_stack()
        torch.cuda.synchronize()
        t = buf.cpu().numpy().reshape(n_layers, grid, 8).astype(np.float64) / 100.0  # 100 MHz ticks -> us
        t0 = t[0, :grid - 1, 0].min()
        b0 = grid - 1 - n["combine"]
        y_end = t[:, b0:grid - 1, 7].max(axis=1)  # each layer's last y store
        ends.append(np.diff(y_end))
        b = 0
        for kind, cnt in n.items():
            for slot in slots[kind]:
                v = t[:, b:b + cnt, slot]
                first[kind][slot].append((float(np.median(v[0] - t0)), float((v[0] - t0).max())))
                rel = v[1:] - y_end[:-1, None]
                per[kind][slot].append((float(np.median(np.median(rel, axis=1))), float(np.median(rel.max(axis=1)))))
            b += cnt
    assert fn(None) == 0
    out = {"layers": n_layers, "us_per_layer_median": float(np.median(np.concatenate(ends)))}
    for kind, sl in slots.items():
        out[kind] = {"items": n[kind]}
        for slot, name in sl.items():
            a = np.asarray(per[kind][slot])
            a0 = np.asarray(first[kind][slot])
            out[kind][name] = {"median_us": float(np.median(a[:, 0])), "slowest_us": float(np.median(a[:, 1])),
                               "layer0_median_us": float(np.median(a0[:, 0])),
                               "layer0_slowest_us": float(np.median(a0[:, 1]))}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=600, help="timed decode steps (prefill: steps/10 chunks)")
    ap.add_argument("--warmup", type=int, default=2, help="untimed graph replays before timing")
    ap.add_argument("--layers", type=int, default=30, help="distinct seeded layers in the pool (rotation and stacks)")
    ap.add_argument("--prefill-rows", type=int, default=128)
    ap.add_argument("--stack-rows", type=int, default=256, help="rows per chunk of the 30-layer prefill stack")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the single-layer decode leg (profiling of the others)")
    ap.add_argument("--cache-slots", type=int, default=0,
                    help="also decode through HBM expert slots per layer in front of a pinned host tier (0: off)")
    ap.add_argument("--cache-layers", type=int, default=8, help="layers of the tiered-store decode leg")
    ap.add_argument("--cache-tokens", type=int, default=40, help="timed tokens of the tiered-store decode leg")
    ap.add_argument("--sweep-chunks", default="", metavar="R1,R2,...",
                    help="also time prefill chunks of these row counts (reported under prefill_chunk_sweep)")
    ap.add_argument("--no-stack", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the streaming-read and bf16 GEMM ceilings")
    ap.add_argument("--timeline", type=int, default=0, metavar="STEPS",
                    help="also record the per-phase timelines of the decode kernel and of the one-launch stack "
                         "over STEPS eager steps each (needs the timeline build: "
                         "QMOE_LIB=.../libqmoe_timeline.so, from build.py --timeline)")
    ap.add_argument("--cpu-rows", type=int, default=1536, help="rows in the oracle's timed CPU sample")
    ap.add_argument("--calibrate-copy", type=float, default=0.0, metavar="MB",
                    help="only run a plain device copy of MB megabytes 5 times (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (every box has one GPU); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy > 0:
        return calibrate_copy(args.calibrate_copy)

    import numpy as np
    import torch

    import synth
    import quantized_mixture_experts_bit_amd as q
    from quantized_mixture_experts_bit_amd.weights import ExpertPool

    dev = torch.device("cuda:0")
    shape = synth.GEMMA4
    E, k, d = shape.n_experts, shape.top_k, shape.d_model
    L = args.layers

    # ---------------------------------------------------------------- weights
    t0 = time.time()
    pool = ExpertPool(shape, L * E, dev)
    layers_c = []
    dls = []
    for i in range(L):
        lay = synth.make_layer(shape, seed=0, layer=i)
        dls.append(pool.add_layer(lay, i * E))
        if i == 0:
            layers_c.append(lay)  # layer 0 kept for the CPU baseline
        del lay
    log("pool: %d layers x %d experts, %.2f GB, built in %.1f s" % (L, E, pool.buf.numel() / 1e9,
                                                                      time.time() - t0))

    # ---------------------------------------------------------------- decode
    steps_per_graph = 4 * L
    n_x = steps_per_graph
    xs = torch.from_numpy(synth.make_x(shape, n_x, seed=1, dtype="bf16")).view(torch.bfloat16).to(dev)
    ws = torch.empty(q.moe_workspace_bytes(shape, max(1, args.prefill_rows, args.stack_rows)), dtype=torch.uint8,
                     device=dev)
    q.moe_workspace_init(ws)
    idx = torch.empty(n_x, k, dtype=torch.int32, device=dev)
    w = torch.empty(n_x, k, dtype=torch.float32, device=dev)
    eo = torch.empty(k, d, dtype=torch.float32, device=dev)
    y = torch.empty(n_x, d, dtype=torch.float32, device=dev)

    def decode_step(i):
        q.moe_layer_decode(shape, dls[i % L].c, xs[i:i + 1], None, idx[i], w[i], eo, y[i], None, ws)

    cap = torch.cuda.Stream()
    dbytes = decode_bytes(shape)
    dec_ms = dec_tok_s = dec_bw = dec_spread = dec_flagged = None
    dec_steps = 0
    if not args.no_decode:
        # eager pass (also warms up the code objects)
        for i in range(steps_per_graph):
            decode_step(i)
        torch.cuda.synchronize()
        assert q.moe_check_device_error() == 0

        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for i in range(steps_per_graph):
                decode_step(i)
        # at least 10 replays of the whole rotation, whatever --steps asks for
        replays = max(10, -(-args.steps // steps_per_graph))
        per_rep = time_replays(g, replays, args.warmup)
        dec_steps = replays * steps_per_graph
        dec_ms = sum(per_rep) / dec_steps
        dec_spread = spread(per_rep, steps_per_graph)
        # near-ties among the decode rows, from the GPU's own fp64 logits
        lg_dec = torch.empty(n_x, E, dtype=torch.float64, device=dev)
        for i in range(steps_per_graph):
            q.moe_router_topk(shape, dls[i % L].c, xs[i:i + 1], 1, None, idx[i], w[i], lg_dec[i], ws)
        dec_flagged = flagged_rows(lg_dec.cpu().numpy(), k)
        dec_tok_s = 1000.0 / dec_ms
        dec_bw = dbytes / (dec_ms * 1e-3)
        log("decode: %d steps, %.2f us/step (median %.2f, p10 %.2f, p90 %.2f over %d replays), %.0f tok/s, %.2f TB/s "
            "on active bytes (%.1f%% of 8 TB/s), %d flagged rows of %d"
            % (dec_steps, dec_ms * 1e3, dec_spread["median_us"], dec_spread["p10_us"], dec_spread["p90_us"], replays,
               dec_tok_s, dec_bw / 1e12, 100 * dec_bw / HBM_PEAK, dec_flagged, steps_per_graph))

    timeline = None
    if args.timeline > 0 and not args.no_decode:
        timeline = decode_timeline(q, shape, decode_step, args.timeline, dev)
        log("decode timeline (us from the first workgroup's start; median workgroup / slowest workgroup, "
            "medians over %d steps):" % args.timeline)
        for kind, rec in timeline.items():
            log("  %-15s (%3d items) " % (kind, rec["items"]) + "; ".join(
                "%s %.2f / %.2f" % (name, v["median_us"], v["slowest_us"]) for name, v in rec.items()
                if name != "items"))

    # ---------------------------------------------------------------- prefill
    def measure_prefill(R):
        """Chunks of R rows rotating over the L layers (one Zipf offset per layer), replayed
        from one HIP graph; returns the prefill record."""
        n_chunks = L
        zipf = [torch.from_numpy(synth.make_zipf_offset(shape, seed=0, layer=i)).to(dev) for i in range(L)]
        xp = [torch.from_numpy(synth.make_x(shape, R, seed=2, stream=i, dtype="bf16")).view(torch.bfloat16).to(dev)
              for i in range(n_chunks)]
        wsp = torch.empty(q.moe_workspace_bytes(shape, R), dtype=torch.uint8, device=dev)
        q.moe_workspace_init(wsp)
        pidx = torch.empty(n_chunks, R, k, dtype=torch.int32, device=dev)
        pw = torch.empty(n_chunks, R, k, dtype=torch.float32, device=dev)
        cnt = torch.empty(n_chunks, E, dtype=torch.int32, device=dev)
        off = torch.empty(n_chunks, E + 1, dtype=torch.int32, device=dev)
        perm = torch.empty(n_chunks, R * k, dtype=torch.int32, device=dev)
        inv = torch.empty(n_chunks, R * k, dtype=torch.int32, device=dev)
        peo = torch.empty(R * k, d, dtype=torch.float32, device=dev)
        py = torch.empty(n_chunks, R, d, dtype=torch.float32, device=dev)

        def prefill_step(i):
            q.moe_layer_prefill(shape, dls[i % L].c, xp[i], R, zipf[i % L], pidx[i], pw[i], cnt[i], off[i], perm[i],
                                inv[i], peo, py[i], None, wsp)

        for i in range(n_chunks):
            prefill_step(i)
        torch.cuda.synchronize()
        assert q.moe_check_device_error() == 0
        counts = cnt.cpu().numpy()
        gp = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gp, stream=cap):
            for i in range(n_chunks):
                prefill_step(i)
        p_replays = max(10, args.steps // 10 // n_chunks)
        p_per = time_replays(gp, p_replays, args.warmup)
        p_ms = sum(p_per) / (p_replays * n_chunks)
        lgp = torch.empty(R, E, dtype=torch.float64, device=dev)
        p_flagged = 0
        for i in range(n_chunks):
            q.moe_router_topk(shape, dls[i % L].c, xp[i], R, zipf[i % L], pidx[i], pw[i], lgp, wsp)
            p_flagged += flagged_rows(lgp.cpu().numpy(), k)
        ideal = [prefill_roofline(shape, counts[i], R) for i in range(n_chunks)]
        t_ideal = float(np.mean([t for t, _, _ in ideal]))
        flops = float(np.mean([fl for _, fl, _ in ideal]))
        nbytes = float(np.mean([by for _, _, by in ideal]))
        distinct = float(np.mean((counts > 0).sum(1)))
        rec = {
            "workload": "prefill chunk of %d rows, same layer shape, Zipf(1.1)-skewed router logits" % R,
            "metric": "MoE-layer tokens/s (prefill chunk %d)" % R,
            "value": R / (p_ms * 1e-3), "unit": "tokens/s", "ms_per_chunk": p_ms,
            "chunks": p_replays * n_chunks, "per_chunk": spread(p_per, n_chunks),
            "flagged_rows": p_flagged, "rows_checked_for_flags": n_chunks * R,
            "roofline": {"bound": "sum over GEMMs of max(bytes/HBM, flops/MFMA)", "ideal_ms": t_ideal * 1e3,
                         "frac": t_ideal / (p_ms * 1e-3)},
            "mfma_util": flops / (p_ms * 1e-3) / MFMA_F16_PEAK,
            "achieved_tflops": flops / (p_ms * 1e-3) / 1e12,
            "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
            "distinct_experts_mean": distinct,
            "rows_per_expert_max_mean": float(np.mean(counts.max(1))),
            # rows routed to an expert -> how many (chunk, expert) pairs had that many
            "rows_per_expert_hist": {str(b): int(v) for b, v in
                                     zip(*np.unique(counts[counts > 0], return_counts=True))},
        }
        log("prefill: %d rows, %.1f us/chunk, %.0f tok/s, roofline frac %.3f, MFMA util %.3f, %.1f distinct experts"
            % (R, p_ms * 1e3, rec["value"], rec["roofline"]["frac"], rec["mfma_util"], distinct))
        del gp
        return rec

    prefill = None
    if not args.no_prefill:
        prefill = measure_prefill(args.prefill_rows)
    sweep = None
    if args.sweep_chunks:
        sweep = [measure_prefill(int(r)) for r in args.sweep_chunks.split(",")]

    # ---------------------------------------------------------------- 30-layer stacks
    stack = None
    if not args.no_stack:
        NL = min(30, L)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # decode: one row through NL layers, x <- bf16(x + y) in place after each
        x0d = torch.from_numpy(synth.make_x(shape, 1, seed=41, dtype="bf16")).view(torch.bfloat16).to(dev)
        hd = x0d.clone()
        sid, sw = torch.empty(NL, k, dtype=torch.int32, device=dev), torch.empty(NL, k, device=dev)
        syd = torch.empty(1, d, device=dev)

        stack_layers = [dls[l].c for l in range(NL)]

        def stack_decode():  # the whole stack in one launch (moe_stack_decode)
            hd.copy_(x0d)
            q.moe_stack_decode(shape, stack_layers, hd, None, sid, sw, None, None, None, ws)

        def stack_decode_layer_calls():  # one whole-block launch per layer
            hd.copy_(x0d)
            for l in range(NL):
                q.moe_layer_decode(shape, dls[l].c, hd, None, sid[l], sw[l], eo, syd, hd, ws)

        sd_rep = max(20, args.steps // NL)  # at least 20 tokens
        stack_decode_layer_calls()
        torch.cuda.synchronize()
        gsl = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gsl, stream=cap):
            stack_decode_layer_calls()
        sl_ms = sum(time_replays(gsl, sd_rep, args.warmup)) / sd_rep
        del gsl
        stack_decode()
        torch.cuda.synchronize()
        assert q.moe_check_device_error() == 0
        gsd = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gsd, stream=cap):
            stack_decode()
        sd_per = time_replays(gsd, sd_rep, args.warmup)
        sd_ms = sum(sd_per) / sd_rep
        sd_timeline = None
        if args.timeline > 0:
            sd_timeline = stack_timeline(q, shape, stack_decode, NL, args.timeline, dev)
            log("stack decode timeline, layers 1..%d (us from the previous layer's last y; median workgroup / slowest "
                "workgroup, medians over layers and %d steps), %.2f us per layer:"
                % (NL - 1, args.timeline, sd_timeline["us_per_layer_median"]))
            for kind, rec in sd_timeline.items():
                if isinstance(rec, dict):
                    log("  %-15s (%3d items) " % (kind, rec["items"]) + "; ".join(
                        "%s %.2f / %.2f" % (name, v["median_us"], v["slowest_us"]) for name, v in rec.items()
                        if name != "items"))
        sd_bytes = NL * dbytes
        # prefill: chunks of RS rows through NL layers, Zipf-skewed routing per layer
        RS = args.stack_rows
        x0p = torch.from_numpy(synth.make_x(shape, RS, seed=42, dtype="bf16")).view(torch.bfloat16).to(dev)
        hp = x0p.clone()
        zl = [torch.from_numpy(synth.make_zipf_offset(shape, seed=0, layer=l)).to(dev) for l in range(NL)]
        s_idx = torch.empty(RS, k, dtype=torch.int32, device=dev)
        s_w = torch.empty(RS, k, device=dev)
        s_cnt = torch.empty(NL, E, dtype=torch.int32, device=dev)
        s_off = torch.empty(NL, E + 1, dtype=torch.int32, device=dev)
        s_perm = torch.empty(RS * k, dtype=torch.int32, device=dev)
        s_inv = torch.empty(RS * k, dtype=torch.int32, device=dev)
        s_eo = torch.empty(RS * k, d, device=dev)
        s_y = torch.empty(RS, d, device=dev)

        def stack_prefill():
            hp.copy_(x0p)
            for l in range(NL):
                q.moe_layer_prefill(shape, dls[l].c, hp, RS, zl[l], s_idx, s_w, s_cnt[l], s_off[l], s_perm, s_inv,
                                    s_eo, s_y, hp, ws)

        stack_prefill()
        torch.cuda.synchronize()
        assert q.moe_check_device_error() == 0
        s_counts = s_cnt.cpu().numpy()
        gsp = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gsp, stream=cap):
            stack_prefill()
        sp_rep = max(10, args.steps // 100)  # at least 10 chunks
        sp_per = time_replays(gsp, sp_rep, args.warmup)
        sp_ms = sum(sp_per) / sp_rep
        sp_ideal = [prefill_roofline(shape, s_counts[l], RS) for l in range(NL)]
        sp_t = sum(t for t, _, _ in sp_ideal)
        sp_fl = sum(fl for _, fl, _ in sp_ideal)
        sp_by = sum(by for _, _, by in sp_ideal)
        stack = {
            "decode": {
                "workload": "%d-layer stack of the same block (distinct seeded layers, %d experts each resident in "
                            "one pool behind per-layer slot tables), decode 1 row, in-place residual "
                            "x <- bf16(x + y) between layers; the whole stack in one launch (moe_stack_decode)"
                            % (NL, E),
                "metric": "tokens/s through the %d-layer stack (decode bs=1)" % NL,
                "value": 1000.0 / sd_ms, "unit": "tokens/s", "ms_per_token": sd_ms, "tokens": sd_rep,
                "per_token": spread(sd_per, 1),
                "ms_per_token_one_launch_per_layer": sl_ms,
                "timeline": sd_timeline,
                "roofline": {"bound": "hbm", "algorithmic_bytes_per_token": sd_bytes,
                             "achieved": sd_bytes / (sd_ms * 1e-3) / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                             "frac": sd_bytes / (sd_ms * 1e-3) / HBM_PEAK},
            },
            "prefill": {
                "workload": "%d-layer stack, prefill chunks of %d rows, Zipf(1.1)-skewed router logits per layer, "
                            "in-place residual; one HIP graph per chunk" % (NL, RS),
                "metric": "tokens/s through the %d-layer stack (prefill chunk %d)" % (NL, RS),
                "value": RS / (sp_ms * 1e-3), "unit": "tokens/s", "ms_per_chunk": sp_ms, "chunks": sp_rep,
                "per_chunk": spread(sp_per, 1),
                "roofline": {"bound": "sum over layers and GEMMs of max(bytes/HBM, flops/MFMA)",
                             "ideal_ms": sp_t * 1e3, "frac": sp_t / (sp_ms * 1e-3)},
                "mfma_util": sp_fl / (sp_ms * 1e-3) / MFMA_F16_PEAK,
                "algorithmic_bytes": sp_by, "algorithmic_flops": sp_fl,
                "distinct_experts_per_layer": [int(v) for v in (s_counts > 0).sum(1)],
            },
        }
        log("stack decode: %d layers in one launch, %.1f us/token, %.0f tok/s, %.1f%% of HBM peak on active bytes "
            "(one launch per layer: %.1f us/token)"
            % (NL, sd_ms * 1e3, 1000.0 / sd_ms, 100 * stack["decode"]["roofline"]["frac"], sl_ms * 1e3))
        log("stack prefill: %d layers x %d rows, %.2f ms/chunk, %.0f tok/s, roofline frac %.3f, MFMA util %.3f"
            % (NL, RS, sp_ms, stack["prefill"]["value"], stack["prefill"]["roofline"]["frac"],
               stack["prefill"]["mfma_util"]))

    # ---------------------------------------------------------------- tiered residency (HBM slots + pinned host tier)
    cache = None
    if args.cache_slots > 0:
        from quantized_mixture_experts_bit_amd.weights import HostExpertPool, TieredStore
        NLc = min(args.cache_layers, L)
        t0 = time.time()
        host = HostExpertPool(shape, NLc)
        for l in range(NLc):
            host.load_layer(l, synth.make_layer(shape, seed=0, layer=l))
        store = TieredStore(host, args.cache_slots, dev)
        cl = [store.layer(l, dls[l].router, dls[l].shared) for l in range(NLc)]
        # a second store over the same host tier: the overlapped flow runs the same tokens from
        # the same cache states as the serial one, so both see the same hits and misses
        store2 = TieredStore(host, args.cache_slots, dev)
        cl2 = [store2.layer(l, dls[l].router, dls[l].shared) for l in range(NLc)]
        # and two stores with the policy on the device (eager, and one HIP graph per token)
        store3 = TieredStore(host, args.cache_slots, dev, device_policy=True)
        cl3 = [store3.layer(l, dls[l].router, dls[l].shared) for l in range(NLc)]
        store4 = TieredStore(host, args.cache_slots, dev, device_policy=True)
        cl4 = [store4.layer(l, dls[l].router, dls[l].shared) for l in range(NLc)]
        log("tiered store: %d layers in pinned host memory (%.2f GB), %d HBM slots per layer, built in %.1f s"
            % (NLc, host.buf.numel() / 1e9, args.cache_slots, time.time() - t0))
        ws1 = torch.empty(q.moe_workspace_bytes(shape, 1), dtype=torch.uint8, device=dev)
        q.moe_workspace_init(ws1)
        cid, cw = torch.empty(k, dtype=torch.int32, device=dev), torch.empty(k, device=dev)
        ceo, cy = torch.empty(k, d, device=dev), torch.empty(1, d, device=dev)
        hc = torch.empty(1, d, dtype=torch.bfloat16, device=dev)
        zoff = [torch.from_numpy(synth.make_zipf_offset(shape, seed=0, layer=l)).to(dev) for l in range(NLc)]

        copy_stream = torch.cuda.Stream()

        def token(t, layers, offs, through_cache):
            # one token through the NLc layers with the residual in place. Through the cache
            # the picks go to the host (a synchronising copy); "overlap" copies the misses on
            # their own stream while the shared expert and the hits run (CachedLayer.decode)
            hc.copy_(torch.from_numpy(synth.make_x(shape, 1, seed=500 + t, dtype="bf16")).view(torch.bfloat16))
            if through_cache == "graph":
                token_graph[offs_key(offs)].replay()
                return
            for l in range(NLc):
                if through_cache:
                    layers[l].decode(hc, offs[l], cid, cw, ceo, cy, hc, ws1,
                                     copy_stream if through_cache == "overlap" else None)
                    continue
                q.moe_router_topk(shape, layers[l].c, hc, 1, offs[l], cid, cw, None, ws1)
                q.moe_expert_ffn_decode(shape, layers[l].c, hc, cid, ceo, ws1)
                q.moe_combine(shape, layers[l].c, hc, 1, ceo, None, cw, cy, hc, ws1)

        token_graph = {}

        def offs_key(offs):
            return "zipf" if offs[0] is not None else "uniform"

        def capture_token(layers, offs):
            # one token's layers through a device-policy store, captured once (the capture
            # runs nothing, so the store's history is untouched)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=torch.cuda.Stream()):
                for l in range(NLc):
                    layers[l].decode(hc, offs[l], cid, cw, ceo, cy, hc, ws1)
            token_graph[offs_key(offs)] = g

        def timed(layers, offs, through_cache, n_tok, first, st=store):
            for t in range(3):
                token(first + t, layers, offs, through_cache)
            torch.cuda.synchronize()
            h0, m0, b0 = st.stats()
            t0 = time.time()
            for t in range(n_tok):
                token(first + 3 + t, layers, offs, through_cache)
            torch.cuda.synchronize()
            dt = (time.time() - t0) / n_tok
            h1, m1, b1 = st.stats()
            hits, misses, nb = h1 - h0, m1 - m0, b1 - b0
            return dt, hits, misses, nb

        cache = {"workload": "decode, batch 1, %d-layer stack, residual in place; split calls with the picks "
                             "copied to the host after each router, the misses copied on their own stream while the "
                             "shared expert and the hits run (serially for comparison), and with the policy on the "
                             "device (no host round trip; eager, and one HIP graph per token); %d HBM "
                             "expert slots per layer (LFU) in front of all %d x %d blobs in pinned host memory"
                             % (NLc, args.cache_slots, NLc, E),
                 "slots_per_layer": args.cache_slots, "layers": NLc}
        n_tok = args.cache_tokens
        for name, offs in (("uniform_router", [None] * NLc), ("zipf_router", zoff)):
            first = 0 if name == "uniform_router" else 10000
            # the same tokens through the two stores: serial, then overlapped
            dt_s, hits_s, misses_s, nb_s = timed(cl, offs, "serial", n_tok, first)
            dt_c, hits, misses, nb = timed(cl2, offs, "overlap", n_tok, first, store2)
            dt_d, hits_d, misses_d, nb_d = timed(cl3, offs, "device", n_tok, first, store3)
            capture_token(cl4, offs)
            dt_g, hits_g, misses_g, nb_g = timed(cl4, offs, "graph", n_tok, first, store4)
            dt_r, _, _, _ = timed(dls, offs, False, n_tok, first)
            rec = {"ms_per_token": dt_c * 1e3, "tokens_per_s": 1.0 / dt_c, "hit_rate": hits / max(1, hits + misses),
                   "misses_per_token_layer": misses / (n_tok * NLc), "bytes_per_token": nb / n_tok,
                   "host_to_hbm_GBps": nb / n_tok / dt_c / 1e9,
                   "serial_ms_per_token": dt_s * 1e3, "serial_hit_rate": hits_s / max(1, hits_s + misses_s),
                   "serial_bytes_per_token": nb_s / n_tok, "overlap_gain": dt_s / dt_c,
                   "device_policy_ms_per_token": dt_d * 1e3,
                   "device_policy_hit_rate": hits_d / max(1, hits_d + misses_d),
                   "device_policy_graph_ms_per_token": dt_g * 1e3,
                   "device_policy_graph_hit_rate": hits_g / max(1, hits_g + misses_g),
                   "resident_ms_per_token": dt_r * 1e3, "slowdown_vs_resident": dt_c / dt_r, "tokens": n_tok}
            cache[name] = rec
            log("tiered decode (%s): %.2f ms/token (%.1f tok/s) with the misses copied beside the shared expert and "
                "the hits (serial: %.2f ms/token, %.2fx), hit rate %.3f (serial %.3f), %.2f misses per token-layer, "
                "%.1f MB/token from the host tier (%.1f GB/s), resident split path %.2f ms/token (%.2fx)"
                % (name, rec["ms_per_token"], rec["tokens_per_s"], rec["serial_ms_per_token"], rec["overlap_gain"],
                   rec["hit_rate"], rec["serial_hit_rate"], rec["misses_per_token_layer"],
                   rec["bytes_per_token"] / 1e6, rec["host_to_hbm_GBps"], rec["resident_ms_per_token"],
                   rec["slowdown_vs_resident"]))
            log("tiered decode (%s), policy on the device: %.2f ms/token eager, %.2f ms/token as one HIP graph per "
                "token (hit rates %.3f, %.3f)" % (name, rec["device_policy_ms_per_token"],
                                                  rec["device_policy_graph_ms_per_token"],
                                                  rec["device_policy_hit_rate"], rec["device_policy_graph_hit_rate"]))
        # prefill chunks of 128 rows through the same cache: the routed experts in passes of
        # at most `slots` experts (MOE_SLOT_SKIP for the others), against the same split
        # calls on the resident pool
        RPc = 128
        wsp = torch.empty(q.moe_workspace_bytes(shape, RPc), dtype=torch.uint8, device=dev)
        q.moe_workspace_init(wsp)
        po = dict(idx=torch.empty(RPc, k, dtype=torch.int32, device=dev), w=torch.empty(RPc, k, device=dev),
                  cnt=torch.empty(E, dtype=torch.int32, device=dev), off=torch.empty(E + 1, dtype=torch.int32, device=dev),
                  perm=torch.empty(RPc * k, dtype=torch.int32, device=dev),
                  inv=torch.empty(RPc * k, dtype=torch.int32, device=dev),
                  eo=torch.empty(RPc * k, d, device=dev), y=torch.empty(RPc, d, device=dev))
        xp_c = [torch.from_numpy(synth.make_x(shape, RPc, seed=700 + l, dtype="bf16")).view(torch.bfloat16).to(dev)
                for l in range(NLc)]

        def chunk_pass(l, through_cache):
            if through_cache:
                return cl[l].prefill(xp_c[l], RPc, zoff[l], po["idx"], po["w"], po["cnt"], po["off"], po["perm"],
                                     po["inv"], po["eo"], po["y"], None, wsp)
            q.moe_router_topk(shape, dls[l].c, xp_c[l], RPc, zoff[l], po["idx"], po["w"], None, wsp)
            q.moe_group_by_expert(shape, po["idx"], RPc, po["cnt"], po["off"], po["perm"], po["inv"], wsp)
            q.moe_expert_ffn_prefill_chunk(shape, dls[l].c, xp_c[l], RPc, po["off"], po["perm"], po["eo"], wsp)
            q.moe_combine(shape, dls[l].c, xp_c[l], RPc, po["eo"], po["inv"], po["w"], po["y"], None, wsp)
            return 0, 0

        def timed_prefill(through_cache, reps):
            for l in range(NLc):
                chunk_pass(l, through_cache)
            torch.cuda.synchronize()
            h0, m0, b0 = store.stats()
            n_pass = 0
            t0 = time.time()
            for _ in range(reps):
                for l in range(NLc):
                    n_pass += chunk_pass(l, through_cache)[0]
            torch.cuda.synchronize()
            dt = (time.time() - t0) / (reps * NLc)
            h1, m1, b1 = store.stats()
            return dt, n_pass / (reps * NLc), h1 - h0, m1 - m0, b1 - b0

        reps = max(1, n_tok // 10)
        dt_c, n_pass, hits, misses, nb = timed_prefill(True, reps)
        dt_r = timed_prefill(False, reps)[0]
        rec = {"workload": "prefill chunks of %d rows, Zipf(1.1)-skewed router, rotating over the %d layers" % (RPc, NLc),
               "ms_per_chunk": dt_c * 1e3, "tokens_per_s": RPc / dt_c, "passes_per_chunk": n_pass,
               "hit_rate": hits / max(1, hits + misses), "bytes_per_chunk": nb / (reps * NLc),
               "host_to_hbm_GBps": nb / (reps * NLc) / dt_c / 1e9, "resident_ms_per_chunk": dt_r * 1e3,
               "slowdown_vs_resident": dt_c / dt_r, "chunks": reps * NLc}
        cache["prefill_zipf_router"] = rec
        log("tiered prefill (%d rows, zipf): %.2f ms/chunk, %.2f passes/chunk, hit rate %.3f, %.1f MB/chunk from the "
            "host tier (%.1f GB/s), resident split path %.3f ms/chunk (%.1fx)"
            % (RPc, rec["ms_per_chunk"], rec["passes_per_chunk"], rec["hit_rate"], rec["bytes_per_chunk"] / 1e6,
               rec["host_to_hbm_GBps"], rec["resident_ms_per_chunk"], rec["slowdown_vs_resident"]))
        store.close()
        store2.close()
        store3.close()
        store4.close()

    # ---------------------------------------------------------------- CPU baseline (the oracle)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        # the host's share for one GPU: OMP_NUM_THREADS where set (16 on the GPU machines), at most
        # the logical CPUs the OS reports
        n_os = os.cpu_count() or 1
        cores = min(n_os, int(os.environ.get("OMP_NUM_THREADS", n_os)))
        ol = O.OracleLayer(layers_c[0])
        xc = synth.make_x(shape, args.cpu_rows, seed=3, dtype="bf16")
        O.set_threads(cores)
        t = time.time()
        O.moe_rows(ol, xc, want=("idx", "p", "y"))
        dt = time.time() - t
        used = O.threads()
        rows1 = max(8, args.cpu_rows // 16)
        O.set_threads(1)
        t = time.time()
        O.moe_rows(ol, xc[:rows1], want=("idx", "p", "y"))
        dt1 = time.time() - t
        O.set_threads(cores)
        cpu = {"value": args.cpu_rows / dt, "unit": "tokens/s", "cores": used, "kind": "oracle",
               "sample": "%d independent decode rows of the same layer shape (fp64 C oracle, OpenMP over rows), "
                         "%.1f s wall on %d threads; os.cpu_count() = %d" % (args.cpu_rows, dt, used, n_os),
               "os_cpu_count": n_os,
               "single_core": {"value": rows1 / dt1, "unit": "tokens/s", "cores": 1,
                               "sample": "the first %d of those rows on 1 thread, %.1f s wall" % (rows1, dt1)}}
        log("cpu oracle: %d rows in %.1f s on %d threads -> %.2f tok/s; %d rows on 1 thread -> %.2f tok/s "
            "(os.cpu_count() %d)" % (args.cpu_rows, dt, used, cpu["value"], rows1, rows1 / dt1, n_os))

    ceilings = None if args.no_ceilings else measured_ceilings(dev)
    if ceilings and dec_bw:
        log("ceilings: streaming read %.0f GB/s, bf16 GEMM %.0f TFLOP/s" % (ceilings["stream_read_GBps"],
                                                                         ceilings["bf16_gemm_TFLOPs"]))
        out_frac = dec_bw / (ceilings["stream_read_GBps"] * 1e9)
        ceilings["decode_frac_of_stream_read"] = out_frac
    traffic, traffic_detail = measured_traffic()
    out = {
        "metric": "MoE-layer tokens/s (decode bs=1)",
        "value": dec_tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": dec_steps,
        "warmup": args.warmup,
        "ms_per_step": dec_ms,
        "per_step": dec_spread,
        "flagged_rows": dec_flagged,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 activations, 4-bit/8-bit affine weights, fp32 accumulate (router fp64)",
        "data": "synthetic (seeded random weights and activations of the named shapes)",
        "config": {
            "workload": "decode, batch 1 token, one MoE layer: d_model 2816, 128 experts (gate/up 2816x704, "
                        "down 704x2816, 4-bit affine g64 bf16 scale+bias), shared expert d_ff 2112, 8-bit router "
                        "128x2816, top-8 softmax, GeGLU; rotating over %d seeded layers" % L,
            "global_batch": 1,
            "seq_len": 1,
            "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "k_decode_fused (moe_layer_decode: the whole block for one row in one launch)",
            "achieved": dec_bw / 1e9 if dec_bw else None,
            "peak": HBM_PEAK / 1e9,
            "unit": "GB/s",
            "frac": dec_bw / HBM_PEAK if dec_bw else None,
            "traffic": traffic,
            "traffic_detail": traffic_detail,
            "algorithmic_bytes_per_launch": dbytes,
        },
        "cpu_baseline": cpu,
        "measured_ceilings": ceilings,
        "prefill": prefill,
        "stack": stack,
    }
    if sweep is not None:
        out["prefill_chunk_sweep"] = sweep
    if timeline is not None:
        out["decode_timeline"] = timeline
    if cache is not None:
        out["tiered_residency"] = cache
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

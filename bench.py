"""Benchmark: CSM compression and log-N decode attention at 64K context on one MI355X.

Workload (synthetic, seeded): Llama-3.1-8B-shaped KV cache, 32 layers x 8 KV heads x d=128,
bf16, batch 1, 65536-token context, 4% of (layer, kv-head) slices flagged outlier, keys
AR(1) with rho ~ U[0.8, 0.99] per head, values N(0, 1), queries N(0, 1).

One step = one pass of the whole hot path:
  1. csm_compress: one CSM round (r = 0.5, c = 256, n1 = 16, n2 = 64) in place over the
     64K cache (its input is restored from a pristine copy and the 256 MB last-level cache is
     flushed before every step, outside the round's timed events);
  2. kv_append: one decode token appended to every slice of the serving cache, which was
     compressed beforehand (untimed) to the 20% budget by the annealed Algorithm 1 rounds;
  3. decode_attn_logn: GQA log-N attention for all 32 query heads of all 32 layers.
Inputs are resident in HBM before timing.  `value` is the CSM round's throughput in
slice-tokens/s (input tokens of the compressed slices per second of the csm_compress call,
timed with HIP events on the stream the library launches on); the decode figures are
reported beside it.  Roofline: algorithmic bytes (what the round must read and write: every
compressed slice reads its rows after the sinks once and writes its kept rows once; outlier
slices are not touched) / duration.
"""

import argparse
import json
import math
import os
import sys
import time
from statistics import median

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSM compress tokens/s + log-N decode-attn HBM GB/s (% of peak), 64K ctx"
PEAK_GBPS = 8000.0
ROW_BYTES = 128 * 2 * 2 + 4  # K + V (bf16, d = 128) + int32 degree
CSM_SOURCES = ["csm_kernel.hip", "csm_common.hpp", "device_common.hpp", "kernel_args.hpp"]
DEC_SOURCES = ["decode_kernel.hip", "device_common.hpp", "kernel_args.hpp"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-slices", type=int, default=246,
                    help="compressible slices the oracle baseline clusters (all 246 by default)")
    ap.add_argument("--offload-slices", type=int, default=32,
                    help="compressible slices the CPU-offloaded round is timed on")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter calibration)")
    ap.add_argument("--workloads", default="1,2,3,5,4:f16,4:d64,4:c512,4:g8",
                    help="other synthetic workloads to measure and report (comma list of ids, "
                         "id:dtype for another storage format, '' for none)")
    return ap.parse_args()


COUNTER_RECORD = os.path.join(ROOT, "profiles", "csm_decode_64k_hbm_counters.md")
CSRC = os.path.join(ROOT, "kv_cache_clustering_amd", "csrc")


def recorded_traffic(key, sources):
    """HBM bytes per launch from the recorded FETCH_SIZE / WRITE_SIZE passes (copy-calibrated),
    or None when the record is missing or the kernel sources changed since it was taken."""
    import hashlib
    try:
        text = open(COUNTER_RECORD).read()
        rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])[key]
    except (OSError, IndexError, KeyError, ValueError):
        return None
    h = hashlib.sha256()
    for f in sources:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return rec["traffic_bytes_per_launch"] if h.hexdigest()[:16] == rec["source_sha256_16"] else None


def csm_bytes(lens_in, lens_out, mask, n1):
    """Algorithmic HBM bytes of one round: every compressed slice reads its rows after the n1
    sinks once and writes its kept rows once; outlier slices are not read or written."""
    return sum(((s - n1) + (s2 - n1)) * ROW_BYTES
               for s, s2, m in zip(lens_in, lens_out, mask) if not m)


def csm_copy_bytes(lens_in, mask, n1):
    """Bytes the out-of-place round moves besides the algorithmic ones: the n1 sink rows of every
    compressed slice and every row of the outlier slices, each read once and written once."""
    return sum(2 * (s if m else n1) * ROW_BYTES for s, m in zip(lens_in, mask))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the hot path "
              "shards by slice with no exchange, and this benchmark measures one GPU's share.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import kvsynth
    # the oracle baseline forks its host workers first, before anything (the HIP library
    # included) touches the GPU, so that they start from a process with no GPU state
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(kvsynth.workload(4), args.cpu_slices)
    from kv_cache_clustering_amd import _lib as lib
    from kv_cache_clustering_amd.schedule import Algorithm1, round_output_length

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    w = kvsynth.workload(4)
    K, W = args.steps, args.warmup
    if K + W > w.steps:
        print(f"steps + warmup must be <= {w.steps} (appended-token capacity)", file=sys.stderr)
        sys.exit(1)

    t_setup = time.time()
    c = kvsynth.make_cache(w, dev)
    K0, V0, N0, L0, mask = c["K"], c["V"], c["N"], c["lens"], c["mask"]
    app_k, app_v = c["app_k"], c["app_v"]
    q_all = kvsynth.make_queries(w, dev, steps=K + W)
    S, cap, d = K0.shape
    maskh = mask.cpu().numpy()
    # the timed round works in place on a copy restored from the pristine cache every step
    Ki, Vi, Ni, Li = (torch.empty_like(t) for t in (K0, V0, N0, L0))
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    # serving cache: compressed to the budget by Algorithm 1's prefill rounds (untimed)
    Kd, Vd, Nd, Ld = K0.clone(), V0.clone(), N0.clone(), L0.clone()
    sched = Algorithm1(n=w.ctx, R=w.R, Gamma=w.steps, g=w.g, n1=w.n1, n2=w.n2, c=w.c)
    ws_c = lib.new_workspace(lib.csm_workspace_bytes(K0, w.n1, w.n2, w.c, max_len=w.ctx), dev)
    s_pre = w.ctx
    for r in sched.prefill_rounds():  # in place: the bound covers the compressed slices only
        lib.csm_compress(Kd, Vd, Nd, Ld, w.n1, w.n2, w.c, r, mask, max_len=s_pre, workspace=ws_c)
        s_pre = round_output_length(s_pre, w.n1, w.n2, w.c, r)
    assert lib.read_error(ws_c) == lib.OK
    ws_d = lib.new_workspace(lib.decode_workspace_bytes(Kd, w.H_q, w.H_kv), dev)
    O = torch.empty((w.groups, w.H_q, d), dtype=torch.float32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup
    stream = torch.cuda.current_stream(dev)
    # auxiliary: the decode-time round of Algorithm 1 (step 110 of this workload: the serving
    # cache, 13081 tokens after the prefill rounds, reaches B + g after 110 appended tokens and
    # one round at r = 0.1 runs), in place, input restored and cache flushed before each rep;
    # measured on a copy of the serving cache before the timed steps append to it
    trig = trigger_round(lib, w, sched, Kd, Vd, Nd, Ld, app_k, app_v, mask, maskh, flush, stream,
                         dev)
    # the hierarchical centroid index over the serving cache: build, and decode over the rows
    # it keeps with the workload's queries
    hier = index_decode(lib, w, Kd, Vd, Nd, Ld, q_all[0], stream, dev)
    # the CPU-offloaded variant: the same round on the host's cores over a host copy of a sample
    # of the slices, and the upload of its result
    offload = host_offload(lib, w, K0, V0, N0, L0, maskh, stream, dev, args.offload_slices)

    r0 = w.r_init
    s_out = round_output_length(w.ctx, w.n1, w.n2, w.c, r0)
    lens_in = [w.ctx] * S
    lens_out = [w.ctx if m else s_out for m in maskh]
    csm_alg = csm_bytes(lens_in, lens_out, maskh, w.n1)
    slice_tokens = int(sum(w.ctx for m in maskh if not m))

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]

    def restore(i):
        """The round's input back to the pristine cache, then the last-level cache flushed."""
        Ki.copy_(K0)
        Vi.copy_(V0)
        Ni.copy_(N0)
        Li.copy_(L0)
        flush.fill_(i & 0xFF)

    def step(i, evs=None):
        restore(i)
        if evs:
            evs[0].record(stream)
        lib.csm_compress(Ki, Vi, Ni, Li, w.n1, w.n2, w.c, r0, mask, max_len=w.ctx, workspace=ws_c)
        if evs:
            evs[1].record(stream)
        lib.kv_append(Kd, Vd, Nd, Ld, app_k[i], app_v[i], err)
        if evs:
            evs[2].record(stream)
        lib.decode_attn_logn(q_all[i], Kd, Vd, Nd, Ld, w.H_q, w.H_kv, out=O, workspace=ws_d)
        if evs:
            evs[3].record(stream)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(W + i, ev[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    assert lib.read_error(ws_c) == lib.OK and lib.read_error(ws_d) == lib.OK
    assert lib.read_error(err) == lib.OK
    ms_per_step = (t1 - t0) * 1e3 / K
    csm_ms = [e[0].elapsed_time(e[1]) for e in ev]
    app_ms = [e[1].elapsed_time(e[2]) for e in ev]
    dec_ms = [e[2].elapsed_time(e[3]) for e in ev]
    csm_avg, dec_avg, app_avg = (sum(x) / K for x in (csm_ms, dec_ms, app_ms))
    csm_med, dec_med = median(csm_ms), median(dec_ms)

    # decode bytes: every slice's rows once, plus q in and O out
    lens_d = Ld.cpu().numpy()
    dec_lens_mid = lens_d - (K // 2)  # lengths grow by one per step; use the mid-run length
    dec_alg = int(dec_lens_mid.sum()) * ROW_BYTES + w.groups * w.H_q * d * (2 + 4)
    assert np.all(Li.cpu().numpy() == np.array(lens_out))

    csm_gbps = csm_alg / (csm_avg * 1e-3) / 1e9
    dec_gbps = dec_alg / (dec_avg * 1e-3) / 1e9
    value = slice_tokens / (csm_avg * 1e-3)

    # decode as a model runs it: one call per layer (that layer's slices, its query heads)
    hk = w.H_kv
    layer_views = []
    for layer in range(w.layers):
        sl = slice(layer * hk, (layer + 1) * hk)
        layer_views.append((Kd[sl], Vd[sl], Nd[sl], Ld[sl], O[layer:layer + 1]))
    # host-known bound on every length: the outlier slices are never compressed and have grown
    # by one token per step
    dec_bound = w.ctx + W + K
    ws_l = lib.new_workspace(lib.decode_workspace_bytes(layer_views[0][0], w.H_q, w.H_kv,
                                                        max_len=dec_bound), dev)
    q_last = q_all[W + K - 1]

    def layer_calls():
        for layer, (Kl, Vl, Nl, Ll, Ol) in enumerate(layer_views):
            lib.decode_attn_logn(q_last[layer:layer + 1], Kl, Vl, Nl, Ll, w.H_q, w.H_kv, out=Ol,
                                 max_len=dec_bound, workspace=ws_l)

    for _ in range(3):
        layer_calls()
    torch.cuda.synchronize()
    layer_ms = []
    for _ in range(10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        layer_calls()
        e1.record(stream)
        torch.cuda.synchronize()
        layer_ms.append(e0.elapsed_time(e1))
    assert lib.read_error(ws_l) == lib.OK
    O_eager = O.clone()
    # the same 32 calls replayed from one HIP graph: the GPU's own time per layer, without the
    # host's per-call cost (argument checks, marshalling and two launches per call)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        layer_calls()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    layer_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(layer_graph):
        layer_calls()
    for _ in range(3):
        layer_graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(O, O_eager)
    layer_graph_ms = []
    for _ in range(10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        layer_graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        layer_graph_ms.append(e0.elapsed_time(e1))
    del layer_graph
    dec_alg_now = int(Ld.cpu().numpy().sum()) * ROW_BYTES + w.groups * w.H_q * d * (2 + 4)
    step_flows = per_layer_steps(lib, w, Kd, Vd, Nd, Ld, q_last, app_k[-1], app_v[-1], stream, dev)

    # auxiliary: the out-of-place round (csm_compress_into, pristine cache -> a second cache).
    # Its algorithmic bytes are the in-place round's; it also copies the sinks of every slice and
    # the whole outlier slices, reported apart.
    Kw, Vw, Nw, Lw = (torch.empty_like(t) for t in (K0, V0, N0, L0))
    oop_ms = []
    for rep in range(5):
        flush.fill_(rep & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        lib.csm_compress_into(K0, V0, N0, L0, Kw, Vw, Nw, Lw, w.n1, w.n2, w.c, r0, mask,
                              max_len=w.ctx, workspace=ws_c)
        e1.record(stream)
        torch.cuda.synchronize()
        oop_ms.append(e0.elapsed_time(e1))
    assert lib.read_error(ws_c) == lib.OK
    assert torch.equal(Lw, Li)
    oop_avg = sum(oop_ms) / len(oop_ms)
    oop_copy = csm_copy_bytes(lens_in, maskh, w.n1)
    del Kw, Vw, Nw, Lw

    # decode as the serving loop runs it (append + attention, step after step): wall time per
    # step, and HIP events around every attention call (its steady-state time, not preceded by
    # a 64K round as in the timed step)
    loop_steps = min(50, w.steps - K - W - 1)
    base = W + K
    lev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(loop_steps)]
    t0 = time.perf_counter()
    for i in range(loop_steps):
        lib.kv_append(Kd, Vd, Nd, Ld, app_k[base + i], app_v[base + i], err)
        lev[i][0].record(stream)
        lib.decode_attn_logn(q_all[i % (K + W)], Kd, Vd, Nd, Ld, w.H_q, w.H_kv, out=O,
                             max_len=cap, workspace=ws_d)
        lev[i][1].record(stream)
    torch.cuda.synchronize()
    eager_us = (time.perf_counter() - t0) * 1e6 / loop_steps
    steady_ms = [a.elapsed_time(b) for a, b in lev[1:]]
    steady_avg = sum(steady_ms) / len(steady_ms)
    steady_alg = int(Ld.cpu().numpy().sum() - loop_steps // 2 * S) * ROW_BYTES + w.groups * w.H_q * d * (2 + 4)
    q_in, k_in, v_in = q_all[0].clone(), app_k[0].clone(), app_v[0].clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lib.kv_append(Kd, Vd, Nd, Ld, k_in, v_in, err)
        lib.decode_attn_logn(q_in, Kd, Vd, Nd, Ld, w.H_q, w.H_kv, out=O, max_len=cap,
                             workspace=ws_d)
    graph.replay()  # one appended token
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    gsteps = min(loop_steps, w.steps - K - W - loop_steps - 2)
    for _ in range(gsteps):
        graph.replay()
    torch.cuda.synchronize()
    graph_us = (time.perf_counter() - t0) * 1e6 / max(1, gsteps)
    assert lib.read_error(err) == lib.OK and lib.read_error(ws_d) == lib.OK

    # the same steps with Algorithm 1's trigger decided on the device: 25 steps (append,
    # attention, triggered round) per graph; rounds fire whenever a slice reaches B + g
    tsteps = min(100, w.steps - K - W - loop_steps - gsteps - 2) // 25 * 25
    trig_us, trig_rounds = None, None
    if tsteps > 0:
        thr_v = math.ceil(sched.budget + sched.g)
        thr = torch.full((S,), thr_v, dtype=torch.int32, device=dev)
        ridx = torch.full((S,), len(sched.rounds), dtype=torch.int32, device=dev)
        s_now = int(Ld[int(np.argmin(maskh))].item())
        bound = min(cap, max(thr_v, s_now) + tsteps)
        ws_t = lib.new_workspace(lib.csm_workspace_bytes(Kd, w.n1, w.n2, w.c, max_len=bound), dev)
        tq = q_all[0].clone()
        tk = torch.stack([app_k[base + loop_steps + gsteps + 1 + i] for i in range(25)])
        tv = torch.stack([app_v[base + loop_steps + gsteps + 1 + i] for i in range(25)])
        torch.cuda.synchronize()
        tgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(tgraph):
            for i in range(25):
                lib.kv_append(Kd, Vd, Nd, Ld, tk[i], tv[i], err)
                lib.decode_attn_logn(tq, Kd, Vd, Nd, Ld, w.H_q, w.H_kv, out=O, max_len=cap,
                                     workspace=ws_d)
                lib.csm_compress_triggered(Kd, Vd, Nd, Ld, thr, ridx, w.n1, w.n2, w.c, w.r_init,
                                           0.05, 0.1, mask, max_len=bound, workspace=ws_t)
        torch.cuda.synchronize()
        per_replay = []
        for _ in range(tsteps // 25):
            t0 = time.perf_counter()
            tgraph.replay()
            torch.cuda.synchronize()
            per_replay.append((time.perf_counter() - t0) * 1e6 / 25)
        trig_us = {"mean": sum(per_replay) / len(per_replay), "per_replay": per_replay}
        assert lib.read_error(ws_t) == lib.OK and lib.read_error(err) == lib.OK
        trig_rounds = int(ridx[int(np.argmin(maskh))].item()) - len(sched.rounds)

    # achievable copy bandwidth on this machine (context for the roofline fraction)
    nbytes = 4 << 30
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        b.copy_(a)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * nbytes * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    if args.calibrate_copy:
        g = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        h = torch.empty_like(g)
        h.copy_(g)
        torch.cuda.synchronize()
        del g, h
    del a, b

    others = []
    wl = [x.strip() for x in args.workloads.split(",") if x.strip()]
    if wl:
        del K0, V0, N0, Ki, Vi, Ni, Kd, Vd, Nd, app_k, app_v, c, flush
        torch.cuda.empty_cache()
        for spec in wl:  # "<id>[:<dtype>][:d<head dim>][:c<chunk>][:g<q heads per kv head>]"
            cid, *mods = spec.split(":")
            num = {m[0]: int(m[1:]) for m in mods if m[:1] in ("d", "c", "g") and m[1:].isdigit()}
            dt = next((m for m in mods if not (m[:1] in ("d", "c", "g") and m[1:].isdigit())), None)
            others.append(measure_workload(int(cid), dt, num.get("d"), num.get("c"), num.get("g")))
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "slice-tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_per_step,
        "ms_per_step_includes": "per step: restore of the round's 8.6 GB input and a 512 MB "
                                "cache flush (untimed by the events), the round, append, decode",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": w.layers, "kv_heads": w.H_kv, "q_heads": w.H_q,
                   "d": d, "batch": w.batch, "ctx": w.ctx, "slices": S,
                   "outlier_slices": int(maskh.sum()), "c": w.c, "n1": w.n1, "n2": w.n2,
                   "r": r0, "round_out_len": s_out, "budget": sched.budget,
                   "decode_len": int(sched.s), "prefill_rounds": len(sched.rounds)},
        "csm": {"call": "csm_compress (in place; input restored and last-level cache flushed "
                        "before each step, outside the events)",
                "ms": csm_avg, "median_ms": csm_med, "min_ms": min(csm_ms),
                "alg_bytes": csm_alg, "GBps": csm_gbps, "frac": csm_gbps / PEAK_GBPS,
                "slice_tokens": slice_tokens,
                "model_tokens_per_s": w.ctx / (csm_avg * 1e-3),
                "whole_step_slice_tokens_per_s": slice_tokens / (ms_per_step * 1e-3),
                "out_of_place": {"call": "csm_compress_into", "ms": oop_avg,
                                 "median_ms": median(oop_ms), "min_ms": min(oop_ms),
                                 "alg_bytes": csm_alg,
                                 "GBps": csm_alg / (oop_avg * 1e-3) / 1e9,
                                 "frac": csm_alg / (oop_avg * 1e-3) / 1e9 / PEAK_GBPS,
                                 "copy_bytes": oop_copy,
                                 "GBps_with_copies": (csm_alg + oop_copy) / (oop_avg * 1e-3) / 1e9},
                "trigger_round": trig},
        "decode_attn": {"us": steady_avg * 1e3, "median_us": median(steady_ms) * 1e3,
                        "min_us": min(steady_ms) * 1e3, "alg_bytes": steady_alg,
                        "GBps": steady_alg / (steady_avg * 1e-3) / 1e9,
                        "timing": "events around each call of a run of append + attention "
                                  f"steps ({len(steady_ms)} timed)",
                        "in_step": {"us": dec_avg * 1e3, "median_us": dec_med * 1e3,
                                    "min_us": min(dec_ms) * 1e3, "alg_bytes": dec_alg,
                                    "GBps": dec_gbps, "frac": dec_gbps / PEAK_GBPS,
                                    "note": "the step's own call, right after the 64K round"},
                        "frac": steady_alg / (steady_avg * 1e-3) / 1e9 / PEAK_GBPS,
                        "layers": w.layers,
                        "per_layer_calls": {
                            "calls": w.layers, "median_us": median(layer_ms) * 1e3,
                            "min_us": min(layer_ms) * 1e3, "alg_bytes": dec_alg_now,
                            "GBps": dec_alg_now / (median(layer_ms) * 1e-3) / 1e9,
                            "hip_graph_median_us": median(layer_graph_ms) * 1e3,
                            "hip_graph_min_us": min(layer_graph_ms) * 1e3,
                            "hip_graph_GBps": dec_alg_now / (median(layer_graph_ms) * 1e-3) / 1e9},
                        "per_layer_steps_with_append": step_flows,
                        "traffic": recorded_traffic("dec_split_bf16_g4", DEC_SOURCES)},
        "append_us": app_avg * 1e3,
        "decode_loop_wall_us_per_step": {"eager": eager_us, "hip_graph": graph_us,
                                         "steps": loop_steps, "includes": "append + attention, 32 layers",
                                         "hip_graph_device_trigger": trig_us,
                                         "device_trigger_steps": tsteps,
                                         "device_trigger_rounds_fired": trig_rounds},
        "hbm_copy_GBps": copy_gbps,
        "roofline": {"bound": "hbm", "kernel": "csm_round_bf16_regs (csm_compress, in place)",
                     "achieved": csm_gbps, "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": csm_gbps / PEAK_GBPS,
                     "traffic": recorded_traffic("csm_round_bf16_regs", CSM_SOURCES)},
        "cpu_offload": offload,
        "hierarchical_index": hier,
        "cpu_baseline": cpu,
        "workloads": others,
        "setup_s": setup_s,
    }
    print(json.dumps(out), flush=True)


def per_layer_steps(lib, w, Kd, Vd, Nd, Ld, q, k_new, v_new, stream, dev, reps=10, warm=3):
    """A decode step as a model runs it, layer after layer, each layer appending its token and
    then attending: kv_append + decode_attn_logn per layer against kv_append_decode_attn_logn per
    layer, each flow captured in one HIP graph and replayed on its own copy of the serving cache
    (every replay appends one token to every slice).  After the same replays the two copies must
    hold the same cache and close outputs."""
    import torch

    hk = w.H_kv
    n_app = warm + reps + 1
    bound = int(Ld.max()) + n_app
    out = {}
    caches, outs = {}, {}
    for flow in ("two_calls", "fused"):
        K, V, N, L = (t.clone() for t in (Kd, Vd, Nd, Ld))
        O = torch.empty((w.groups, w.H_q, w.d), dtype=torch.float32, device=dev)
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        views = [(K[l * hk:(l + 1) * hk], V[l * hk:(l + 1) * hk], N[l * hk:(l + 1) * hk],
                  L[l * hk:(l + 1) * hk], O[l:l + 1], k_new[l * hk:(l + 1) * hk],
                  v_new[l * hk:(l + 1) * hk]) for l in range(w.layers)]
        ws = lib.new_workspace(lib.decode_workspace_bytes(views[0][0], w.H_q, hk, max_len=bound), dev)

        def step():
            for layer, (Kl, Vl, Nl, Ll, Ol, kl, vl) in enumerate(views):
                if flow == "two_calls":
                    lib.kv_append(Kl, Vl, Nl, Ll, kl, vl, err)
                    lib.decode_attn_logn(q[layer:layer + 1], Kl, Vl, Nl, Ll, w.H_q, hk, out=Ol,
                                         max_len=bound, workspace=ws)
                else:
                    lib.kv_append_decode_attn_logn(q[layer:layer + 1], Kl, Vl, Nl, Ll, w.H_q, hk,
                                                   kl, vl, out=Ol, max_len=bound, workspace=ws)
        step()  # one eager step, then the captured steps
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        ms = []
        for i in range(warm + reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            if i >= warm:
                ms.append(e0.elapsed_time(e1))
        del graph
        assert lib.read_error(ws) == lib.OK and lib.read_error(err) == lib.OK
        out[flow] = {"hip_graph_median_us": median(ms) * 1e3, "hip_graph_min_us": min(ms) * 1e3}
        caches[flow], outs[flow] = (K, V, N, L), O
    for a, b in zip(caches["two_calls"], caches["fused"]):
        assert torch.equal(a, b)
    out["max_abs_fused_vs_two_calls"] = float((outs["fused"] - outs["two_calls"]).abs().max())
    out["steps_replayed"] = n_app
    del caches, outs
    torch.cuda.empty_cache()
    return out


def index_decode(lib, w, Kd, Vd, Nd, Ld, q, stream, dev, B=64, tau=8.0):
    """The hierarchical centroid index over the serving cache (blocks of B rows): build time,
    then decode_attn_logn_pruned with the workload's queries (time, fraction of rows kept)
    beside the plain call, both timed with events over 10 calls."""
    import torch

    index = lib.new_index(Kd, B)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    lib.index_build(Kd, Nd, Ld, index, err, B)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    lib.index_build(Kd, Nd, Ld, index, err, B)
    e1.record(stream)
    torch.cuda.synchronize()
    build_ms = e0.elapsed_time(e1)
    O, kept, ws = lib.decode_attn_logn_pruned(q, Kd, Vd, Nd, Ld, w.H_q, w.H_kv, index, tau, w.n1,
                                              w.n2, B, kept=True)
    O_full = lib.decode_attn_logn(q, Kd, Vd, Nd, Ld, w.H_q, w.H_kv)
    times = {}
    for name in ("pruned", "plain"):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            if name == "pruned":
                lib.decode_attn_logn_pruned(q, Kd, Vd, Nd, Ld, w.H_q, w.H_kv, index, tau, w.n1,
                                            w.n2, B, out=O, workspace=ws)
            else:
                lib.decode_attn_logn(q, Kd, Vd, Nd, Ld, w.H_q, w.H_kv, out=O_full)
        e1.record(stream)
        torch.cuda.synchronize()
        times[name] = e0.elapsed_time(e1) / 10 * 1e3
    assert lib.read_error(err) == lib.OK and lib.read_error(ws) == lib.OK
    clustered = index_decode_clustered(lib, w, stream, dev, B, tau)
    lens = Ld.cpu().numpy()
    kh = kept.cpu().numpy()
    kept_rows = 0
    for z in range(len(lens)):
        for b in range(-(-int(lens[z]) // B)):
            kept_rows += min(B, int(lens[z]) - b * B) if kh[z, b] else 0
    out = {"block_rows": B, "tau": tau, "index_bytes": index.numel(), "build_ms": build_ms,
           "pruned_decode_us": times["pruned"], "plain_decode_us": times["plain"],
           "rows_kept_frac": kept_rows / float(lens.sum()),
           "max_abs_vs_plain": float((O - O_full).abs().max()),
           "queries": "the workload's (N(0, I)); on AR(1) keys the ball bounds drop little",
           "clustered_keys": clustered}
    del index, ws
    torch.cuda.empty_cache()
    return out


def index_decode_clustered(lib, w, stream, dev, B, tau, S=64, s=13081):
    """The same index path on keys the ball bounds can separate: S slices of s rows whose blocks
    of B rows are tight clusters (centre of norm sqrt(d) in a random direction, spread 0.05 per
    element), queries aligned with one key of their slice (norm 6 d^(1/4)), fp32 -> bf16; values
    N(0, 1), degrees 1.  Time of the pruned and the plain call (events over 10 calls each),
    fraction of rows kept, largest difference of the outputs."""
    import torch
    gen = torch.Generator(device=dev).manual_seed(404)
    d, cap = w.d, s + 64
    nb = -(-s // B)
    C = torch.randn((S, nb, d), generator=gen, device=dev)
    C = C * (d ** 0.5) / C.norm(dim=2, keepdim=True)
    K = torch.zeros((S, cap, d), dtype=torch.bfloat16, device=dev)
    K[:, :s] = (C.repeat_interleave(B, dim=1)[:, :s]
                + 0.05 * torch.randn((S, s, d), generator=gen, device=dev)).to(torch.bfloat16)
    V = torch.randn((S, cap, d), generator=gen, device=dev).to(torch.bfloat16)
    N = torch.ones((S, cap), dtype=torch.int32, device=dev)
    L = torch.full((S,), s, dtype=torch.int32, device=dev)
    H_kv, H_q = w.H_kv, w.H_q
    j = torch.randint(0, s, (S // H_kv, H_q), generator=gen, device=dev)
    zs = (torch.arange(S // H_kv, device=dev)[:, None] * H_kv
          + torch.arange(H_q, device=dev)[None, :] // (H_q // H_kv))
    kq = K[zs, j].float()
    q = (6.0 * d ** 0.25 * kq / kq.norm(dim=2, keepdim=True)).to(torch.bfloat16)
    index = lib.new_index(K, B)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    lib.index_build(K, N, L, index, err, B)
    O, kept, ws = lib.decode_attn_logn_pruned(q, K, V, N, L, H_q, H_kv, index, tau, w.n1, w.n2, B,
                                              kept=True)
    O_full = lib.decode_attn_logn(q, K, V, N, L, H_q, H_kv)
    times = {}
    for name in ("pruned", "plain"):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            if name == "pruned":
                lib.decode_attn_logn_pruned(q, K, V, N, L, H_q, H_kv, index, tau, w.n1, w.n2, B,
                                            out=O, workspace=ws)
            else:
                lib.decode_attn_logn(q, K, V, N, L, H_q, H_kv, out=O_full)
        e1.record(stream)
        torch.cuda.synchronize()
        times[name] = e0.elapsed_time(e1) / 10 * 1e3
    assert lib.read_error(err) == lib.OK and lib.read_error(ws) == lib.OK
    kept_rows = int(kept[:, :nb - 1].sum()) * B + int(kept[:, nb - 1].sum()) * (s - (nb - 1) * B)
    out = {"slices": S, "rows": s, "pruned_decode_us": times["pruned"],
           "plain_decode_us": times["plain"], "rows_kept_frac": kept_rows / float(S * s),
           "max_abs_vs_plain": float((O - O_full).abs().max())}
    del K, V, N, index, ws
    torch.cuda.empty_cache()
    return out


def host_offload(lib, w, K0, V0, N0, L0, maskh, stream, dev, nslices):
    """The CPU-offloaded round (csm_compress_host) on `nslices` compressible slices of the workload
    copied to pinned host memory, one host thread per core, then csm_upload_rows of its result
    (rows from n1 on, and the lengths) into a device cache of those slices, timed with events."""
    import torch

    comp = [int(z) for z in range(len(maskh)) if not maskh[z]]
    zs = comp[:: max(1, len(comp) // nslices)][:nslices]
    Kh, Vh, Nh, Lh = (torch.empty((len(zs),) + tuple(t.shape[1:]), dtype=t.dtype, pin_memory=True)
                      for t in (K0, V0, N0, L0))
    for h, t in ((Kh, K0), (Vh, V0), (Nh, N0), (Lh, L0)):
        h.copy_(t[zs])
    threads = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    lib.csm_compress_host(Kh, Vh, Nh, Lh, w.n1, w.n2, w.c, w.r_init, threads=threads)
    round_s = time.perf_counter() - t0
    Kd, Vd, Nd, Ld = (t[zs].clone() for t in (K0, V0, N0, L0))
    torch.cuda.synchronize()
    ms = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        lib.csm_upload_rows(Kh, Vh, Nh, Lh, Kd, Vd, Nd, Ld, row_begin=w.n1)
        e1.record(stream)
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    assert torch.equal(Ld.cpu(), Lh)
    up_bytes = int(sum(int(s) - w.n1 for s in Lh)) * ROW_BYTES + 4 * len(zs)
    rate = len(zs) * w.ctx / round_s
    del Kh, Vh, Nh, Lh, Kd, Vd, Nd, Ld
    torch.cuda.empty_cache()
    return {"call": "csm_compress_host + csm_upload_rows", "isa": lib.host_isa(),
            "threads": threads, "slices": len(zs), "round_s": round_s,
            "slice_tokens_per_s": rate,
            "round_s_all_compressible_slices": len(comp) * w.ctx / rate,
            "upload_ms": min(ms), "upload_bytes": up_bytes,
            "upload_GBps": up_bytes / (min(ms) * 1e-3) / 1e9}


def trigger_round(lib, w, sched, Kd, Vd, Nd, Ld, app_k, app_v, mask, maskh, flush, stream, dev):
    """Time the first decode-time round of Algorithm 1 on this workload by itself: a copy of the
    serving cache gets appended tokens until the compressed slices reach B + g, then the round
    runs in place at the schedule's r (input restored and cache flushed before each rep)."""
    import math

    import torch

    from kv_cache_clustering_amd.schedule import Algorithm1, round_output_length
    probe = Algorithm1(n=w.ctx, R=w.R, Gamma=w.steps, g=w.g, n1=w.n1, n2=w.n2, c=w.c)
    probe.prefill_rounds()
    steps = 0
    while not probe.over_budget():
        probe.append()
        steps += 1
    j = len(probe.rounds)
    r = probe.next_round(steps)
    s_in, s_out = probe.rounds[-1][2], probe.rounds[-1][3]
    Kt, Vt, Nt, Lt = Kd.clone(), Vd.clone(), Nd.clone(), Ld.clone()
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    for i in range(steps):
        lib.kv_append(Kt, Vt, Nt, Lt, app_k[i], app_v[i], err)
    Kr, Vr, Nr, Lr = Kt.clone(), Vt.clone(), Nt.clone(), Lt.clone()
    ws = lib.new_workspace(lib.csm_workspace_bytes(Kt, w.n1, w.n2, w.c, max_len=s_in), dev)
    ms = []
    for rep in range(5):
        Kr.copy_(Kt)
        Vr.copy_(Vt)
        Nr.copy_(Nt)
        Lr.copy_(Lt)
        flush.fill_(rep & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        lib.csm_compress(Kr, Vr, Nr, Lr, w.n1, w.n2, w.c, r, mask, max_len=s_in, workspace=ws)
        e1.record(stream)
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    assert lib.read_error(ws) == lib.OK and lib.read_error(err) == lib.OK
    comp = int((maskh == 0).sum())
    assert int(Lr[int(maskh.argmin())]) == s_out == round_output_length(s_in, w.n1, w.n2, w.c, r)
    alg = comp * ((s_in - w.n1) + (s_out - w.n1)) * ROW_BYTES
    avg = sum(ms) / len(ms)
    del Kt, Vt, Nt, Lt, Kr, Vr, Nr, Lr
    torch.cuda.empty_cache()
    return {"decode_step": steps, "round_index": j, "r": r, "s_in": s_in, "s_out": s_out,
            "threshold": math.ceil(sched.budget + sched.g), "ms": avg, "median_ms": median(ms),
            "min_ms": min(ms), "alg_bytes": alg, "GBps": alg / (avg * 1e-3) / 1e9,
            "frac": alg / (avg * 1e-3) / 1e9 / PEAK_GBPS,
            "slice_tokens_per_s": comp * s_in / (avg * 1e-3)}


ROUND0_WARMUP, ROUND0_REPS = 3, 10  # untimed and timed reps of a workload's round 0
DEC_WARMUP, DEC_STEPS = 3, 10        # untimed and timed decode steps of a workload


def measure_workload(cid, dtype=None, head_dim=None, chunk=None, group=None):
    """One synthetic workload: every prefill round in place (HIP events per round), then
    decode steps (append + attention) over the compressed cache.  Figures are algorithmic
    bytes / event time."""
    import numpy as np
    import torch

    import kvsynth
    from kv_cache_clustering_amd import _lib as lib
    from kv_cache_clustering_amd.schedule import Algorithm1, round_output_length

    w = kvsynth.workload(cid)
    if dtype is not None and dtype != w.dtype:
        w = kvsynth.workload(cid, dtype=dtype, name=f"{w.name}-as-{dtype}")
    if head_dim is not None and head_dim != w.d:
        w = kvsynth.workload(cid, dtype=w.dtype, d=head_dim, name=f"{w.name}-d{head_dim}")
    if chunk is not None and chunk != w.c:
        w = kvsynth.workload(cid, dtype=w.dtype, d=w.d, c=chunk, name=f"{w.name}-c{chunk}")
    if group is not None and group != w.G:
        w = kvsynth.workload(cid, dtype=w.dtype, d=w.d, c=w.c, H_q=group * w.H_kv,
                             name=f"{w.name}-g{group}")
    dev = torch.device("cuda:0")
    c = kvsynth.make_cache(w, dev, batch_slices=256)
    K, V, N, L, mask = c["K"], c["V"], c["N"], c["lens"], c["mask"]
    maskh = mask.cpu().numpy()
    S, cap, d = K.shape
    row = 2 * d * K.element_size() + 4
    ws = lib.new_workspace(lib.csm_workspace_bytes(K, w.n1, w.n2, w.c, max_len=w.ctx), dev)
    if w.R is None:
        rs = [w.r_init]
    else:
        sched = Algorithm1(n=w.ctx, R=w.R, Gamma=w.steps, g=w.g, n1=w.n1, n2=w.n2, c=w.c)
        rs = sched.prefill_rounds()
    stream = torch.cuda.current_stream(dev)
    n_comp = int((maskh == 0).sum())
    # round 0 by itself, as the headline round is timed: in place on a copy restored before every
    # rep, the last-level cache flushed, the first rep not counted (when two copies fit in HBM)
    round0_reps = None
    cache_bytes = sum(t.numel() * t.element_size() for t in (K, V, N, L))
    if 2 * cache_bytes < 160 * 2 ** 30:
        Kc, Vc, Nc, Lc = (t.clone() for t in (K, V, N, L))
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        reps = []
        for rep in range(ROUND0_WARMUP + ROUND0_REPS):
            for dst, src in ((Kc, K), (Vc, V), (Nc, N), (Lc, L)):
                dst.copy_(src)
            flush.fill_(rep)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            lib.csm_compress(Kc, Vc, Nc, Lc, w.n1, w.n2, w.c, rs[0], mask if maskh.any() else None,
                             max_len=w.ctx, workspace=ws)
            e1.record(stream)
            torch.cuda.synchronize()
            reps.append(e0.elapsed_time(e1))
        round0_reps = reps[ROUND0_WARMUP:]
        del Kc, Vc, Nc, Lc, flush
        torch.cuda.empty_cache()
    rounds = []
    s = w.ctx
    for r in rs:
        s2 = round_output_length(s, w.n1, w.n2, w.c, r)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        lib.csm_compress(K, V, N, L, w.n1, w.n2, w.c, r, mask if maskh.any() else None,
                         max_len=s, workspace=ws)  # in place: outlier slices need no cover
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        alg = n_comp * ((s - w.n1) + (s2 - w.n1)) * row
        rounds.append({"r": round(r, 4), "s_in": s, "s_out": s2, "ms": ms, "GBps": alg / ms / 1e6,
                       "slice_tokens_per_s": n_comp * s / (ms * 1e-3)})
        s = s2
    assert lib.read_error(ws) == lib.OK
    assert int(L[int(np.argmin(maskh))]) == s
    r0 = dict(rounds[0])
    if round0_reps:
        r0["first_call_ms"] = r0["ms"]  # the prefill sequence's own first round (cold)
        alg0 = n_comp * ((w.ctx - w.n1) + (r0["s_out"] - w.n1)) * row
        r0["ms"] = sum(round0_reps) / len(round0_reps)
        r0["median_ms"] = median(round0_reps)
        r0["min_ms"] = min(round0_reps)
        r0["GBps"] = alg0 / r0["ms"] / 1e6
        r0["slice_tokens_per_s"] = n_comp * w.ctx / (r0["ms"] * 1e-3)
        r0["timing"] = (f"mean of {len(round0_reps)} reps in place on a restored copy, last-level "
                        f"cache flushed before each, after {ROUND0_WARMUP} untimed reps")
    out = {"workload": w.name, "slices": S, "dtype": w.dtype, "d": w.d, "c": w.c, "G": w.G,
           "ctx": w.ctx,
           "round0": r0,
           "prefill": {"rounds": len(rounds), "len": s, "ms": sum(x["ms"] for x in rounds),
                       "GBps": sum(n_comp * ((x["s_in"] - w.n1) + (x["s_out"] - w.n1)) * row
                                   for x in rounds) / sum(x["ms"] for x in rounds) / 1e6}}
    ws_d = lib.new_workspace(lib.decode_workspace_bytes(K, w.H_q, w.H_kv), dev)
    q = kvsynth.make_queries(w, dev, steps=min(w.steps, DEC_WARMUP + DEC_STEPS))
    O = torch.empty((w.groups, w.H_q, d), dtype=torch.float32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    nsteps = q.shape[0]
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nsteps)]
    for i in range(nsteps):
        if w.append:
            lib.kv_append(K, V, N, L, c["app_k"][i], c["app_v"][i], err)
        evs[i][0].record(stream)
        lib.decode_attn_logn(q[i], K, V, N, L, w.H_q, w.H_kv, out=O, workspace=ws_d)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    assert lib.read_error(ws_d) == lib.OK and lib.read_error(err) == lib.OK
    warm = DEC_WARMUP if nsteps > DEC_WARMUP else 0
    times = [a.elapsed_time(b) for a, b in evs[warm:]]
    us = sum(times) / len(times) * 1e3
    dec_alg = int(L.sum()) * row + w.groups * w.H_q * d * (K.element_size() + 4)
    out["decode"] = {"us": us, "median_us": median(times) * 1e3, "min_us": min(times) * 1e3,
                     "GBps": dec_alg / (us * 1e-6) / 1e9,
                     "frac": dec_alg / (us * 1e-6) / 1e9 / PEAK_GBPS, "steps_timed": len(times)}
    out["round0"]["frac"] = out["round0"]["GBps"] / PEAK_GBPS
    del c, K, V, N, L, q, ws, ws_d
    torch.cuda.empty_cache()
    return out


def _oracle_worker(cid, zs, csm_zs, barrier, queue):
    """Runs _oracle_work and reports its stamps, or the error that stopped it (after which the
    barrier is broken, so that no other worker waits for this one)."""
    try:
        queue.put(("ok", _oracle_work(cid, zs, csm_zs, barrier)))
    except BaseException as e:  # reported to the parent, which raises
        barrier.abort()
        queue.put(("error", f"{type(e).__name__}: {e}"))


def _oracle_work(cid, zs, csm_zs, barrier):
    """One host worker of the oracle baseline: generates its slices of the workload on the host
    (the workload's per-slice seeds, AR(1) parameters and bf16 rounding; the host's random
    streams, so the same distribution but not the device's bits), then, between barriers shared
    with the other workers, times one CSM round on its compressible slices and one decode step
    (every query head of its slices at their serving lengths)."""
    # numpy only: torch's OpenMP pool is not safe to use in a forked child of a process that
    # has already run it (as a test process may have)
    import numpy as np
    from threadpoolctl import threadpool_limits

    import kvsynth
    from kvsynth import gen as kg
    from kv_cache_clustering_amd.schedule import Algorithm1
    from oracle import attention as oatt
    from oracle import bf16 as obf16
    from oracle import csm as ocsm

    w = kvsynth.workload(cid)
    mask = kg.outlier_mask(w)
    sched = Algorithm1(n=w.ctx, R=w.R, Gamma=w.steps, g=w.g, n1=w.n1, n2=w.n2, c=w.c)
    sched.prefill_rounds()
    serve_len = sched.s  # the compressed slices' length after the annealed prefill rounds
    data = []
    for z in zs:
        b, layer, head = kg._slice_coords(w, z)
        rho, sigma, mu = kg.slice_params(w, z)
        rng = np.random.default_rng(kg.seed_of(cid, b, layer, head, "K"))
        k = kg.ar1_numpy(rng, w.ctx, w.d, rho, sigma, mu)
        v = np.random.default_rng(kg.seed_of(cid, b, layer, head, "V")).standard_normal((w.ctx, w.d))
        # generated in fp64, stored as the device stores it: fp32, then bf16 (nearest even)
        k = obf16.round_to_bf16(k.astype(np.float32).astype(np.float64))
        v = obf16.round_to_bf16(v.astype(np.float32).astype(np.float64))
        data.append((z, k, v))
    q = np.random.default_rng(kg.seed_of(cid, 0, 0, 0, "q")).standard_normal((w.G, w.d))
    ones = np.ones(w.ctx, dtype=np.int64)
    with threadpool_limits(1):
        barrier.wait(timeout=900)
        t0 = time.perf_counter()
        for z, k, v in data:
            if z in csm_zs:
                ocsm.csm_round_slice(k, v, ones, w.ctx, w.n1, w.n2, w.c, w.r_init, "bf16")
        t1 = time.perf_counter()
        barrier.wait(timeout=900)
        t2 = time.perf_counter()
        for z, k, v in data:
            s = w.ctx if mask[z] else serve_len
            for h in range(w.G):
                oatt.logn_attention_one(q[h], k[:s], v[:s], ones[:s])
        t3 = time.perf_counter()
    return t0, t1, t2, t3


def cpu_baseline(w, nslices):
    """The fp64 oracle on the host cores, one worker process per core (at most 16): one CSM
    round over nslices of the workload's compressible slices (slice-tokens/s) and one decode
    step over every slice at the serving lengths (us/step).  Wall time from the first worker's
    start to the last one's end of each phase.  Must run before anything touches the GPU: the
    workers are forked."""
    import multiprocessing as mp

    import numpy as np

    from kvsynth import gen as kg

    cores = min(16, len(os.sched_getaffinity(0)))
    mask = kg.outlier_mask(w)
    comp = [z for z in range(w.slices) if not mask[z]]
    csm_zs = set(comp[:: max(1, len(comp) // max(1, nslices))][:nslices])
    ctx = mp.get_context("fork")
    barrier, queue = ctx.Barrier(cores), ctx.Queue()
    shares = [list(range(i, w.slices, cores)) for i in range(cores)]
    procs = [ctx.Process(target=_oracle_worker, args=(w.cid, zs, csm_zs, barrier, queue))
             for zs in shares]
    for p in procs:
        p.start()
    results = []
    try:
        for _ in procs:
            results.append(queue.get(timeout=900))
    finally:
        for p in procs:
            p.join(timeout=60)
            if p.is_alive():
                p.terminate()
    errors = [r[1] for r in results if r[0] != "ok"]
    if errors or len(results) != len(procs):
        raise RuntimeError(f"oracle baseline workers failed: {errors or 'no report'}")
    stamps = [r[1] for r in results]
    t_csm = max(s[1] for s in stamps) - min(s[0] for s in stamps)
    t_dec = max(s[3] for s in stamps) - min(s[2] for s in stamps)
    return {"value": len(csm_zs) * w.ctx / t_csm, "unit": "slice-tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"CSM round on {len(csm_zs)} of {len(comp)} compressible {w.ctx // 1024}K slices and a "
                      f"decode step over all {w.slices} slices at the serving lengths (fp64 "
                      f"numpy, {cores} worker processes (one per host core, at most 16), one "
                      f"thread each; slices drawn on the host from the workload's seeds and "
                      f"recipe, so the same distribution but not the device's bits; the decode "
                      f"leg attends with every degree 1)",
            "csm_s": t_csm, "decode_us_per_step": t_dec * 1e6,
            "host_cpus": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    main()

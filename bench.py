#!/usr/bin/env python
"""Decode-attention benchmark of the KV-cache refinement decode step on one GPU.

A step is one decode step of every layer of the workload: for each of the 32
layers, score all cached tokens from the resident base key codes, select the
top-T tokens per KV head, refine their K/V with the stored refinement bits,
and attend over all tokens (one sf_decode_step per layer, in layer order).
Inputs are seeded synthetic K/V/q of the named head geometry, resident in HBM
before timing starts.

Prints ONE JSON line: steps/s (whole job), the step's algorithmic HBM GB/s,
a roofline record of the dominant kernel (score or attention pass) timed live
with HIP events, the CPU oracle timed on a bounded sample on the host, and
secondary measurements (32K context; host-pinned refinement store with an
AR(1) query process: hit rate and bytes fetched per step).
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "decode-attention steps/s at 32K & 128K ctx; achieved HBM GB/s vs peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(w, lens):
    """Bytes one layer-step must move: base K/V codes + (lo, delta) read once,
    refinement rows of the selected K and V, query in and output out."""
    d, b, r, hkv = w.head_dim, w.base_bits, w.refine_bits, w.n_kv_heads
    tot = 0
    for n in lens:
        tot += 2 * n * hkv * (d * b // 8 + 8) + 2 * min(w.top_t, n) * hkv * d * r // 8 + 2 * w.n_q_heads * d * 4
    return tot


def kernel_bytes(w, lens):
    """The layer's algorithmic bytes, each credited to the one pass that moves
    it.  score: base K codes and (lo, delta) of every token, and the query.
    attend: base V codes and (lo, delta) of every token, the refinement rows
    of the selected K and V, and the output.  Implementation bytes (the
    per-head logits the score pass hands to the attention pass, partials, the
    re-read of the selected tokens' base K rows) are not credited; the two sum
    to algorithmic_bytes()."""
    d, b, r, hkv = w.head_dim, w.base_bits, w.refine_bits, w.n_kv_heads
    score = sum(n * hkv * (d * b // 8 + 8) + w.n_q_heads * d * 4 for n in lens)
    attend = sum(n * hkv * (d * b // 8 + 8) + 2 * min(w.top_t, n) * hkv * d * r // 8 + w.n_q_heads * d * 4
                 for n in lens)
    return {"score": score, "attend": attend}


class Model:
    """The workload's layers resident on the GPU."""

    def __init__(self, w, tier, layers=None):
        import torch
        from selective_kv_cache_amd import binding as B
        from selective_kv_cache_amd import workloads as W
        from selective_kv_cache_amd.kvcache import Decoder, LayerCache
        self.w = w
        self.lens = w.seq_lengths()
        self.off = W.seq_offsets(self.lens)
        self.L = w.layers if layers is None else layers
        g = B.geom(w.head_dim, w.n_q_heads, w.n_kv_heads, w.base_bits, w.refine_bits)
        ntot = int(self.off[-1])
        self.caches, self.qs = [], []
        for l in range(self.L):
            c = LayerCache(g, ntot, tier=tier, max_seqs=w.batch, cache_slots=w.cache_slots())
            k, v = W.layer_kv(w, l, device="cuda")
            c.append(k, v, 0)
            del k, v
            self.caches.append(c)
            self.qs.append(torch.as_tensor(W.query(w, l), device="cuda"))
        torch.cuda.synchronize()
        self.dec = Decoder(g, self.off, w.top_t)
        self.outs = [torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
                     for _ in range(self.L)]

    def step(self, qs=None, events=None, stats=False):
        acc = {"selected": 0, "hits": 0, "misses": 0, "h2d_bytes": 0}
        for l in range(self.L):
            ev = events[l] if events is not None else None
            res = self.dec.step(self.caches[l], (qs or self.qs)[l], out=self.outs[l], events=ev,
                                want_stats=stats)
            if stats:
                for k2 in acc:
                    acc[k2] += res[1][k2]
        return acc

    def close(self):
        for c in self.caches:
            c.close()


def time_steps(model, steps, warmup):
    import torch
    for _ in range(warmup):
        model.step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        model.step()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def capture_step(model):
    """The whole step (every layer's decode, device-tier store) captured as one
    HIP graph: the library launches only kernels on the caller's stream and
    allocates nothing per step, so a replay is the step without host launch
    overhead."""
    import torch
    model.step()                     # leaves the workspace histogram clear
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        model.step()
    torch.cuda.synchronize()
    return graph


def time_graph(graph, steps, warmup):
    """Exactly `steps` back-to-back graph replays, synchronized on both sides,
    with a HIP event between consecutive ones: (mean ms per step over the
    whole timed region, per-step ms)."""
    import torch
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        graph.replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return evs[0].elapsed_time(evs[-1]) / steps, per


def achievable_read_gbps():
    """Streaming read bandwidth of the box from a plain reduction over 4 GiB
    (torch's kernel; context for the peak, not a measurement of this path)."""
    import torch
    x = torch.ones(1 << 30, dtype=torch.float32, device="cuda")
    for _ in range(2):
        x.sum()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        x.sum()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    del x
    return x_bytes_per_ms(4 << 30, ms)


def source_hash():
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "selective_kv_cache_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch of each kernel from the committed counter summary
    (rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by a copy of known size), or {}
    when there is none or it was taken on other library sources."""
    path = os.path.join(ROOT, "profiles", f"decode_step_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return {}
    vals, sha = {}, None
    with open(path) as fh:
        for ln in fh:
            if ln.startswith("source_sha256_16:"):
                sha = ln.split(":", 1)[1].strip()
            elif ln.startswith("traffic_bytes "):
                k, v = ln[len("traffic_bytes "):].split(":")
                vals[k.strip()] = float(v)
    return vals if sha == source_hash() else {}


def x_bytes_per_ms(nbytes, ms):
    return nbytes / (ms * 1e-3) / 1e9


KERNELS = ("score", "scan", "resolve", "attend", "combine")


def time_kernels(model, steps):
    """Average duration of each kernel of the step, from a pair of HIP events
    around every launch: the start event is recorded just before the kernel's
    dispatch, the stop event completes with it (both created without the
    system-scope fence, so no cache write-back is added), and
    elapsed(start, stop) is the kernel's time as it ran inside the step."""
    import torch
    from selective_kv_cache_amd.binding import TimingEvent
    evs = [[tuple((TimingEvent(), TimingEvent()) for _ in KERNELS) for _ in range(model.L)]
           for _ in range(steps)]
    torch.cuda.synchronize()
    # hold the stream with a spin kernel while the host queues every timed
    # launch, so that the kernels run back to back instead of waiting on the
    # host (each launch costs the host more than some kernels take)
    torch.cuda._sleep(50_000_000)
    for s in range(steps):
        model.step(events=evs[s])
    torch.cuda.synchronize()
    dur = {k: [] for k in KERNELS}
    for row in evs:
        for quint in row:
            for k, (e0, e1) in zip(KERNELS, quint):
                dur[k].append(e0.elapsed_ms(e1))
                e0.close()
                e1.close()
    out = {}
    for k in KERNELS:
        out[k] = float(np.mean(dur[k]))
        out[k + "_median"] = float(np.median(dur[k]))
    return out


def cpu_baseline(w, min_s=10.0, max_s=30.0, n_layers=3):
    """The oracle timed on the host on a bounded sample: the decode of the
    first n_layers layers (all KV heads of every sequence), layer after layer
    and again until at least min_s of timed work (stopping at max_s), scaled
    to whole-model steps/s."""
    import torch
    import oracle.kv_oracle as O
    from selective_kv_cache_amd import workloads as W
    lens = w.seq_lengths()
    off = W.seq_offsets(lens)
    layers = []
    for l in range(min(n_layers, w.layers)):
        k, v = W.layer_kv(w, l, device="cuda")
        k, v = k.cpu().numpy(), v.cpu().numpy()
        layers.append((W.query(w, l), O.quantize_cache(k, v, w.base_bits, w.refine_bits)))   # setup, not timed
        del k, v
    heads = [(s, h) for s in range(w.batch) for h in range(w.n_kv_heads)]
    dt, done, full = 0.0, 0, 0
    while dt < min_s:
        for q, cache in layers:
            for sh in heads:
                t0 = time.perf_counter()
                O.decode_step(q, cache, off, w.top_t, heads=[sh])
                dt += time.perf_counter() - t0
                done += 1
                if dt > max_s:
                    break
            if dt > max_s:
                break
            full += 1
            if dt >= min_s:
                break
        if dt > max_s:
            break
    layer_s = dt * len(heads) / done
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    return {"value": 1.0 / (layer_s * w.layers), "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"layers 0-{len(layers) - 1} of {w.name}, in turn: {done} (sequence, KV head) units "
                      f"({full} whole layers) timed, {dt:.1f} s, scaled to {w.layers} layers; numpy fp64 "
                      f"oracle, quantization excluded"}


def host_tier_run(w, steps, warmup):
    """Host-pinned refinement store + device cache; queries follow an AR(1)
    process (rho = 0.9) so selections overlap across steps."""
    import torch
    from selective_kv_cache_amd import binding as B
    from selective_kv_cache_amd import workloads as W
    wq = W.Workload(**{**w.__dict__, "rho": 0.9})
    m = Model(w, B.SF_TIER_HOST_PINNED)
    try:
        n = warmup + steps
        per_layer = [W.queries(wq, l, n) for l in range(m.L)]
        qsteps = [[torch.as_tensor(per_layer[l][t], device="cuda") for l in range(m.L)] for t in range(n)]
        # timed without statistics (asking for them makes every call wait)
        for t in range(warmup):
            m.step(qsteps[t])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(warmup, n):
            m.step(qsteps[t])
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        # the same query sequence again from empty caches, with statistics
        for c in m.caches:
            c.clear_cache()
        tot = {"selected": 0, "hits": 0, "misses": 0, "h2d_bytes": 0}
        for t in range(n):
            st = m.step(qsteps[t], stats=True)
            if t >= warmup:
                for k2 in tot:
                    tot[k2] += st[k2]
        return {"workload": w.name, "store": "host_pinned", "query_process": "AR(1) rho=0.9",
                "steps": steps, "warmup": warmup, "ms_per_step": dt * 1e3, "steps_per_s": 1.0 / dt,
                "hit_rate": tot["hits"] / max(tot["selected"], 1),
                "h2d_bytes_per_step": tot["h2d_bytes"] / steps}
    finally:
        m.close()


def reuse_run(w, stats, skip=False, sample_every=0):
    """Multi-step reuse run: every layer's cache starts at w.ctx tokens with its
    refinement rows in pinned host memory; each of w.steps steps appends one
    token to every layer (quantized on the GPU, its refinement rows put in the
    store) and decodes with that step's AR(1) query over the grown context.
    Eager launches; with ``stats`` every decode call waits for its miss lists
    (hit rate and bytes), otherwise nothing waits on the host.  ``skip``:
    policy "skip" on a refinement-cache miss.  With ``sample_every`` > 0 the
    outputs of every layer at steps sample_every - 1, 2 sample_every - 1, ...
    are returned as well (copied after the timed region ends)."""
    import torch
    from selective_kv_cache_amd import binding as B
    from selective_kv_cache_amd import workloads as W
    from selective_kv_cache_amd.kvcache import Decoder, LayerCache
    g = B.geom(w.head_dim, w.n_q_heads, w.n_kv_heads, w.base_bits, w.refine_bits)
    n0, steps = w.ctx, w.steps
    caches, qs, app = [], [], []
    try:
        for l in range(w.layers):
            c = LayerCache(g, n0 + steps, tier=B.SF_TIER_HOST_PINNED, max_seqs=1, cache_slots=2 * w.top_t)
            caches.append(c)
            k, v = W.layer_kv(w, l, device="cuda")
            c.append(k, v, 0)
            del k, v
            qs.append(torch.as_tensor(W.queries(w, l, steps), device="cuda"))
            kv = [W.appended_kv(w, l, t) for t in range(steps)]
            app.append((torch.as_tensor(np.stack([x[0] for x in kv]), device="cuda"),
                        torch.as_tensor(np.stack([x[1] for x in kv]), device="cuda")))
        dec = Decoder(g, W.seq_offsets([n0 + 1]), w.top_t)
        outs = [torch.empty((1, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
                for _ in range(w.layers)]
        tot = {"selected": 0, "hits": 0, "misses": 0, "h2d_bytes": 0}
        kept = []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(steps):
            dec.set_offsets([0, n0 + t + 1])
            keep = sample_every > 0 and (t + 1) % sample_every == 0
            for l in range(w.layers):
                caches[l].append(app[l][0][t], app[l][1][t], n0 + t)
                out = torch.empty_like(outs[l]) if keep else outs[l]
                res = dec.step(caches[l], qs[l][t], out=out, want_stats=stats, skip_misses=skip)
                if keep:
                    kept.append(out)
                if stats:
                    for k2 in tot:
                        tot[k2] += res[1][k2]
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        return dt, tot, [x.cpu().numpy() for x in kept]
    finally:
        for c in caches:
            c.close()


def reuse_record(w):
    """The multi-step reuse run under the two policies on a miss: "wait"
    (every selected token refined) and "skip" (misses at base precision this
    step, fetched beside the attention for later steps), with the skip run's
    output difference from the wait run on every layer at every 16th step."""
    dt, _, o_wait = reuse_run(w, stats=False, sample_every=16)
    _, tot, _ = reuse_run(w, stats=True)
    dt_s, _, o_skip = reuse_run(w, stats=False, skip=True, sample_every=16)
    diff = np.concatenate([np.abs(a - b).ravel() for a, b in zip(o_skip, o_wait)])
    return {"workload": w.name, "store": "host_pinned", "query_process": f"AR(1) rho={w.rho}",
            "ctx": [w.ctx + 1, w.ctx + w.steps], "steps": w.steps, "layers": w.layers,
            "launch": "eager", "ms_per_step": dt * 1e3, "steps_per_s": 1.0 / dt,
            "hit_rate": tot["hits"] / max(tot["selected"], 1),
            "h2d_bytes_per_step": tot["h2d_bytes"] / w.steps,
            "per_step": "append one token to every layer (GPU quantization, refinement rows into the "
                        "pinned store), then decode every layer",
            "skip_on_miss": {"ms_per_step": dt_s * 1e3, "steps_per_s": 1.0 / dt_s,
                             "out_diff_vs_wait_max": float(diff.max()), "out_diff_vs_wait_mean": float(diff.mean()),
                             "compared": f"every layer's output at every 16th step ({len(o_skip)} outputs)"}}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama8b_128k")
    ap.add_argument("--tier", choices=["device", "host"], default="device")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only copy BYTES between two device buffers 3 times (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the decode step is measured on one GPU's share "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)

    import torch
    from selective_kv_cache_amd import binding as B
    from selective_kv_cache_amd import workloads as W
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        src = torch.ones(args.calibrate_copy // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.calibrate_copy} bytes 3 times")
        return
    w = W.WORKLOADS[args.workload]
    tier = B.SF_TIER_DEVICE if args.tier == "device" else B.SF_TIER_HOST_PINNED
    log(f"setup {w.name}: {w.layers} layers, ctx {w.seq_lengths()[:4]}, tier {args.tier}")
    model = Model(w, tier)
    log("timing steps (eager launches)")
    ms_eager = time_steps(model, args.steps, args.warmup)
    launch = "eager"
    ms, p50, p10, p90 = ms_eager, None, None, None
    if tier == B.SF_TIER_DEVICE:
        log(f"{ms_eager:.3f} ms/step eager; capturing the step as a HIP graph")
        graph = capture_step(model)
        ms, per = time_graph(graph, args.steps, args.warmup)
        p50, p10, p90 = (float(np.percentile(per, q)) for q in (50, 10, 90))
        launch = "hip_graph"
        del graph
    log(f"{ms:.3f} ms/step ({launch}); timing each kernel with HIP events")
    kt = time_kernels(model, max(2, args.steps // 4))
    model.close()
    del model
    step_bytes = algorithmic_bytes(w, w.seq_lengths()) * w.layers
    kb = kernel_bytes(w, w.seq_lengths())
    dom = max(kb, key=lambda k: kt[k])
    gbps = {k: kb[k] / (kt[k] * 1e-3) / 1e9 for k in kb}
    rec = {
        "metric": METRIC, "value": 1e3 / ms, "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "ctx": w.ctx or list(w.ctx_range),
                   "layers": w.layers, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "base_bits": w.base_bits, "refine_bits": w.refine_bits,
                   "top_t": w.top_t, "refinement_store": args.tier, "launch": launch},
        "ms_per_step_p50": p50, "ms_per_step_p10": p10, "ms_per_step_p90": p90, "eager_ms_per_step": ms_eager,
        "step_algorithmic_bytes": step_bytes,
        "step_hbm_gbps": step_bytes / (ms * 1e-3) / 1e9,
        "step_frac_of_peak": step_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "roofline": {"bound": "hbm", "achieved": gbps[dom], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": gbps[dom] / PEAK_HBM_GBPS,
                     "traffic": measured_traffic(w.name).get(dom + "_mfma"), "kernel": dom,
                     "bytes_per_launch": kb[dom], "avg_launch_ms": kt[dom],
                     "kernels": {k: {"bytes_per_launch": kb[k], "avg_launch_ms": kt[k],
                                     "median_launch_ms": kt[k + "_median"], "achieved_gbps": gbps[k]}
                                 for k in kb},
                     "other_kernels_avg_ms": {k: kt[k] for k in KERNELS if k not in kb},
                     "event_timing": "start/stop HIP event pair around each launch, in this run"},
    }
    if not args.no_secondary:
        sec = {}
        w2 = W.WORKLOADS["llama8b_32k"]
        log("secondary: llama8b_32k")
        m2 = Model(w2, B.SF_TIER_DEVICE)
        g2 = capture_step(m2)
        ms2 = time_graph(g2, args.steps, args.warmup)[0]
        del g2
        m2.close()
        del m2
        b2 = algorithmic_bytes(w2, w2.seq_lengths()) * w2.layers
        sec["llama8b_32k"] = {"steps_per_s": 1e3 / ms2, "ms_per_step": ms2, "launch": "hip_graph",
                              "step_hbm_gbps": b2 / (ms2 * 1e-3) / 1e9,
                              "step_frac_of_peak": b2 / (ms2 * 1e-3) / 1e9 / PEAK_HBM_GBPS}
        w4 = W.WORKLOADS["qwen8b_b16"]
        log("secondary: qwen8b_b16")
        m4 = Model(w4, B.SF_TIER_DEVICE)
        # one layer per step: a graph replay's own fixed cost is then a large
        # share, so the eager rate (the host queues ahead) is timed as well
        ms4e = time_steps(m4, 8 * args.steps, args.warmup)
        g4 = capture_step(m4)
        ms4g = time_graph(g4, 8 * args.steps, args.warmup)[0]
        del g4
        m4.close()
        del m4
        ms4, launch4 = (ms4g, "hip_graph") if ms4g <= ms4e else (ms4e, "eager")
        b4 = algorithmic_bytes(w4, w4.seq_lengths()) * w4.layers
        sec["qwen8b_b16"] = {"layer_steps_per_s": 1e3 / ms4, "ms_per_layer_step": ms4, "launch": launch4,
                             "ms_per_layer_step_graph": ms4g, "ms_per_layer_step_eager": ms4e,
                             "batch": w4.batch, "tokens": int(sum(w4.seq_lengths())),
                             "step_hbm_gbps": b4 / (ms4 * 1e-3) / 1e9,
                             "step_frac_of_peak": b4 / (ms4 * 1e-3) / 1e9 / PEAK_HBM_GBPS}
        if w.host_store:
            log("secondary: host-pinned store")
            sec["host_store"] = host_tier_run(w, max(4, args.steps // 2), 2)
        log("secondary: multi-step reuse run (llama8b_reuse)")
        sec["reuse"] = reuse_record(W.WORKLOADS["llama8b_reuse"])
        rec["secondary"] = sec
    rec["achievable_read_gbps"] = achievable_read_gbps()
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a bounded sample)")
        rec["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

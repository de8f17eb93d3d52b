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
    """Algorithmic bytes of one launch of each pass.  score: base K codes and
    scales of every token, plus the query.  attend: base K and V codes and
    scales, the refinement rows of the selected K and V, the query; the split
    partials it writes are not counted."""
    d, b, r, hkv = w.head_dim, w.base_bits, w.refine_bits, w.n_kv_heads
    score = sum(n * hkv * (d * b // 8 + 8) + w.n_q_heads * d * 4 for n in lens)
    attend = sum(2 * n * hkv * (d * b // 8 + 8) + 2 * min(w.top_t, n) * hkv * d * r // 8 + w.n_q_heads * d * 4
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


def time_kernels(model, steps):
    """Average duration of the score and attention kernels, from HIP events
    recorded around each of their launches on the decode stream."""
    import torch
    mk = lambda: torch.cuda.Event(enable_timing=True)
    evs = [[tuple(mk() for _ in range(4)) for _ in range(model.L)] for _ in range(steps)]
    for row in evs:
        for quad in row:
            for e in quad:
                e.record()          # materialise the events before handing them over
    torch.cuda.synchronize()
    for s in range(steps):
        model.step(events=evs[s])
    torch.cuda.synchronize()
    score = [q[0].elapsed_time(q[1]) for row in evs for q in row]
    attend = [q[2].elapsed_time(q[3]) for row in evs for q in row]
    return {"score": float(np.mean(score)), "attend": float(np.mean(attend)),
            "score_median": float(np.median(score)), "attend_median": float(np.median(attend))}


def cpu_baseline(w, layer_budget_s=30.0):
    """The oracle timed on the host on a bounded sample: one layer's decode
    (all KV heads of every sequence), scaled to whole-model steps/s."""
    import torch
    import oracle.kv_oracle as O
    from selective_kv_cache_amd import workloads as W
    lens = w.seq_lengths()
    off = W.seq_offsets(lens)
    k, v = W.layer_kv(w, 0, device="cuda")
    k, v = k.cpu().numpy(), v.cpu().numpy()
    q = W.query(w, 0)
    cache = O.quantize_cache(k, v, w.base_bits, w.refine_bits)     # setup, not timed
    del k, v
    heads = [(s, h) for s in range(w.batch) for h in range(w.n_kv_heads)]
    t0 = time.perf_counter()
    done = 0
    for sh in heads:
        O.decode_step(q, cache, off, w.top_t, heads=[sh])
        done += 1
        if time.perf_counter() - t0 > layer_budget_s:
            break
    dt = time.perf_counter() - t0
    layer_s = dt * len(heads) / done
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    return {"value": 1.0 / (layer_s * w.layers), "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"layer 0 of {w.name}: {done}/{len(heads)} (sequence, KV head) units timed "
                      f"({dt:.1f} s), scaled to {w.layers} layers; numpy fp64 oracle, quantization excluded"}


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
        tot = {"selected": 0, "hits": 0, "misses": 0, "h2d_bytes": 0}
        for t in range(warmup):
            m.step(qsteps[t], stats=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(warmup, n):
            st = m.step(qsteps[t], stats=True)
            for k2 in tot:
                tot[k2] += st[k2]
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        return {"workload": w.name, "store": "host_pinned", "query_process": "AR(1) rho=0.9",
                "steps": steps, "warmup": warmup, "ms_per_step": dt * 1e3, "steps_per_s": 1.0 / dt,
                "hit_rate": tot["hits"] / max(tot["selected"], 1),
                "h2d_bytes_per_step": tot["h2d_bytes"] / steps}
    finally:
        m.close()


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama8b_128k")
    ap.add_argument("--tier", choices=["device", "host"], default="device")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the decode step is measured on one GPU's share "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)

    import torch
    from selective_kv_cache_amd import binding as B
    from selective_kv_cache_amd import workloads as W
    torch.cuda.set_device(0)
    w = W.WORKLOADS[args.workload]
    tier = B.SF_TIER_DEVICE if args.tier == "device" else B.SF_TIER_HOST_PINNED
    log(f"setup {w.name}: {w.layers} layers, ctx {w.seq_lengths()[:4]}, tier {args.tier}")
    model = Model(w, tier)
    log("timing steps")
    ms = time_steps(model, args.steps, args.warmup)
    log(f"{ms:.3f} ms/step; timing the score and attention kernels")
    kt = time_kernels(model, max(2, args.steps // 4))
    model.close()
    del model

    step_bytes = algorithmic_bytes(w, w.seq_lengths()) * w.layers
    kb = kernel_bytes(w, w.seq_lengths())
    dom = max(("score", "attend"), key=lambda k: kt[k])
    gbps = {k: kb[k] / (kt[k] * 1e-3) / 1e9 for k in kb}
    rec = {
        "metric": METRIC, "value": 1e3 / ms, "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "ctx": w.ctx or list(w.ctx_range),
                   "layers": w.layers, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "base_bits": w.base_bits, "refine_bits": w.refine_bits,
                   "top_t": w.top_t, "refinement_store": args.tier},
        "step_algorithmic_bytes": step_bytes,
        "step_hbm_gbps": step_bytes / (ms * 1e-3) / 1e9,
        "step_frac_of_peak": step_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "roofline": {"bound": "hbm", "achieved": gbps[dom], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": gbps[dom] / PEAK_HBM_GBPS, "traffic": None, "kernel": dom,
                     "bytes_per_launch": kb[dom], "avg_launch_ms": kt[dom],
                     "kernels": {k: {"bytes_per_launch": kb[k], "avg_launch_ms": kt[k],
                                     "median_launch_ms": kt[k + "_median"], "achieved_gbps": gbps[k]}
                                 for k in kb}},
    }
    if not args.no_secondary:
        sec = {}
        w2 = W.WORKLOADS["llama8b_32k"]
        log("secondary: llama8b_32k")
        m2 = Model(w2, B.SF_TIER_DEVICE)
        ms2 = time_steps(m2, args.steps, args.warmup)
        m2.close()
        del m2
        b2 = algorithmic_bytes(w2, w2.seq_lengths()) * w2.layers
        sec["llama8b_32k"] = {"steps_per_s": 1e3 / ms2, "ms_per_step": ms2,
                              "step_hbm_gbps": b2 / (ms2 * 1e-3) / 1e9,
                              "step_frac_of_peak": b2 / (ms2 * 1e-3) / 1e9 / PEAK_HBM_GBPS}
        if w.host_store:
            log("secondary: host-pinned store")
            sec["host_store"] = host_tier_run(w, max(4, args.steps // 2), 2)
        rec["secondary"] = sec
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a bounded sample)")
        rec["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

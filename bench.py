#!/usr/bin/env python
"""Decode-attention benchmark of the KV-cache refinement decode step on one GPU.

A step is one decode step of every layer of the workload: for each of the 32
layers, score all cached tokens from the resident base key codes, select the
top-T tokens per KV head, refine their K/V with the stored refinement bits,
and attend over all tokens (one sf_decode_step per layer, in layer order).
Inputs are seeded synthetic K/V/q of the named head geometry, resident in HBM
before timing starts.

Prints ONE JSON line: steps/s (whole job), the step's algorithmic HBM GB/s,
a roofline record of the dominant kernel (the single-launch decode kernel, or
the score or attention pass of the five-kernel form) timed live with HIP
events, the CPU oracle timed on a bounded sample on the host, and secondary
measurements (the five-kernel form beside the single launch; 32K context; the
multi-step run's shape (3-bit codes, 8,192 tokens) on the device tier; the
16-sequence batch over distinct layers; host-pinned refinement store over 64
AR(1) steps: cold and warm step time, hit rate and bytes fetched; the
multi-step reuse run; the weight-side refinement GEMV at the Llama-3.1-8B
projection shapes).
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


def fused_bytes(w, lens):
    """The single-launch form moves every algorithmic byte of the layer in its
    one kernel."""
    return {"fused": algorithmic_bytes(w, lens)}


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

    def __init__(self, w, tier, layers=None, multi_pass=False):
        import torch
        from selective_kv_cache_amd import binding as B
        from selective_kv_cache_amd import workloads as W
        from selective_kv_cache_amd.kvcache import Decoder, LayerCache
        self.w = w
        self.lens = w.seq_lengths()
        self.off = W.seq_offsets(self.lens)
        self.L = w.layers if layers is None else layers
        self.multi_pass = multi_pass
        g = B.geom(w.head_dim, w.n_q_heads, w.n_kv_heads, w.base_bits, w.refine_bits)
        ntot = int(self.off[-1])
        self.caches = []
        # one query buffer for all layers ([L][B][Hq][D]); a step reads it in
        # place, so new queries are copied in between steps
        self.qbuf = torch.empty((self.L, w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
        for l in range(self.L):
            c = LayerCache(g, ntot, tier=tier, max_seqs=w.batch, cache_slots=w.cache_slots())
            k, v = W.layer_kv(w, l, device="cuda")
            c.append(k, v, 0)
            del k, v
            self.caches.append(c)
            self.qbuf[l].copy_(torch.as_tensor(W.query(w, l)))
        self.qs = [self.qbuf[l] for l in range(self.L)]
        torch.cuda.synchronize()
        self.dec = Decoder(g, self.off, w.top_t)
        self.outs = [torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
                     for _ in range(self.L)]

    def ar1_queries(self, n_steps, rho=0.9):
        """[n_steps][L][B][Hq][D] queries following the AR(1) process per layer
        (selections then change from step to step but overlap)."""
        import torch
        from selective_kv_cache_amd import workloads as W
        wq = W.Workload(**{**self.w.__dict__, "rho": rho})
        per = np.stack([W.queries(wq, l, n_steps) for l in range(self.L)], axis=1)
        return torch.as_tensor(per, device="cuda")

    def step(self, qs=None, events=None, stats=False):
        acc = {"selected": 0, "hits": 0, "misses": 0, "h2d_bytes": 0}
        for l in range(self.L):
            ev = events[l] if events is not None else None
            res = self.dec.step(self.caches[l], (qs or self.qs)[l], out=self.outs[l], events=ev,
                                want_stats=stats, multi_pass=self.multi_pass)
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


def time_graph(graph, steps, warmup, model=None, qseq=None):
    """Exactly `steps` back-to-back graph replays, synchronized on both sides,
    with a HIP event between consecutive ones: (mean ms per step over the
    whole timed region, per-step ms).  With ``qseq`` ([warmup + steps][L]...)
    each replay is preceded by the copy of that step's queries into the
    model's query buffer (inside the timed region)."""
    import torch
    for i in range(warmup):
        if qseq is not None:
            model.qbuf.copy_(qseq[i])
        graph.replay()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        if qseq is not None:
            model.qbuf.copy_(qseq[warmup + i])
        graph.replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return evs[0].elapsed_time(evs[-1]) / steps, per


def gemv_record(calls=32, reps=10):
    """Weight-side refinement GEMV (sf_w_gemv) at the Llama-3.1-8B projection
    shapes: 3-bit resident weights, 4-bit refinements, k = 32 of every 1,024
    input channels.  `calls` calls, each on its own activation vector (so
    each selects anew), captured back to back in one HIP graph; the time per
    call is the replay time over `calls`.  Algorithmic bytes per call: base
    codes, (lo, delta) scales, the selected channels' refinement columns, x,
    y and the selection."""
    import torch
    from selective_kv_cache_amd import binding as B
    from selective_kv_cache_amd import workloads as W
    out = {}
    b, r, top_k, chunk = 3, 4, 32, 1024
    for name, (m, k) in sorted(W.PROJECTIONS.items()):
        g = B.wgeom(m, k, b, r, top_k, chunk)
        w = torch.as_tensor(W.projection_weights(800, m, k), device="cuda")
        codes = torch.empty((m, k // 128, 16 * b), dtype=torch.uint8, device="cuda")
        scales = torch.empty((m, k // 128, 2), dtype=torch.float32, device="cuda")
        cols = torch.empty((k, m * r // 8), dtype=torch.uint8, device="cuda")
        scratch = torch.empty(m * k * r // 8, dtype=torch.uint8, device="cuda")
        B.sf_w_quantize(g, w, codes, scales, cols, scratch)
        torch.cuda.synchronize()
        del w, scratch
        nchunks = (k + chunk - 1) // chunk
        n_sel = nchunks * top_k
        xs = [torch.as_tensor(W.projection_input(800, k, step=i, n_outlier=12), device="cuda") for i in range(calls)]
        ys = [torch.empty(m, device="cuda") for _ in range(calls)]
        sels = [torch.empty(n_sel, dtype=torch.int32, device="cuda") for _ in range(calls)]
        ws = torch.zeros(B.sf_w_gemv_workspace_words(g), dtype=torch.int32, device="cuda")
        for i in range(calls):
            B.sf_w_gemv(g, codes, scales, cols, xs[i], ys[i], sels[i], ws)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(calls):
                B.sf_w_gemv(g, codes, scales, cols, xs[i], ys[i], sels[i], ws)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        assert int(ws[-1].item()) == 0, "a GEMV wait expired"
        us = e0.elapsed_time(e1) * 1e3 / (reps * calls)
        nbytes = m * k * b // 8 + m * (k // 128) * 8 + n_sel * m * r // 8 + k * 4 + m * 4 + n_sel * 4
        traffic = measured_traffic(None, os.path.join(ROOT, "profiles", "weight_gemv_llama8b_projections.md"))
        out[name] = {"m": m, "k": k, "base_bits": b, "refine_bits": r, "top_k": top_k, "chunk": chunk,
                     "us_per_call": us, "algorithmic_bytes": nbytes, "gbps": nbytes / (us * 1e-6) / 1e9,
                     "frac_of_peak": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS,
                     "traffic": traffic.get(name),
                     "timing": f"{calls} calls on distinct activations in one HIP graph, {reps} replays"}
        del graph, xs, ys, sels, codes, scales, cols
        torch.cuda.empty_cache()
    return out


def achievable_read_gbps(nbytes=4 << 30):
    """Streaming read bandwidth of the box: the library's plain read kernel
    (sf_stream_read) over a 4 GiB buffer, the best of a few launch widths;
    context for the peak, not a measurement of the decode path."""
    import torch
    from selective_kv_cache_amd import binding as B
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    best = {}
    for blocks in (1024, 2048, 4096, 8192):
        for _ in range(2):
            B.sf_stream_read(x, nbytes, 0xDEADBEEF, sink, blocks)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            B.sf_stream_read(x, nbytes, 0xDEADBEEF, sink, blocks)
        e1.record()
        torch.cuda.synchronize()
        best[blocks] = x_bytes_per_ms(nbytes, e0.elapsed_time(e1) / 5)
    del x
    return max(best.values()), best


def source_hash():
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "selective_kv_cache_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, path=None):
    """HBM bytes per launch of each kernel from the committed counter summary
    (rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by a copy of known size), or {}
    when there is none or it was taken on other library sources."""
    path = path or os.path.join(ROOT, "profiles", f"decode_step_{workload}_hbm_traffic.md")
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


def time_kernels(model, steps, names=KERNELS):
    """Average duration of each kernel of the step, from a pair of HIP events
    around every launch: the start event is recorded just before the kernel's
    dispatch, the stop event completes with it (both created without the
    system-scope fence, so no cache write-back is added), and
    elapsed(start, stop) is the kernel's time as it ran inside the step."""
    import torch
    from selective_kv_cache_amd.binding import TimingEvent
    evs = [[tuple((TimingEvent(), TimingEvent()) for _ in names) for _ in range(model.L)]
           for _ in range(steps)]
    torch.cuda.synchronize()
    # hold the stream with a spin kernel while the host queues every timed
    # launch, so that the kernels run back to back instead of waiting on the
    # host (each launch costs the host more than some kernels take)
    torch.cuda._sleep(50_000_000)
    for s in range(steps):
        model.step(events=evs[s])
    torch.cuda.synchronize()
    dur = {k: [] for k in names}
    for row in evs:
        for quint in row:
            for k, (e0, e1) in zip(names, quint):
                dur[k].append(e0.elapsed_ms(e1))
            for e0, e1 in quint:
                e0.close()
                e1.close()
    out = {}
    for k in names:
        out[k] = float(np.mean(dur[k]))
        out[k + "_median"] = float(np.median(dur[k]))
    return out


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rate(w, layers, heads, off, min_s, max_s):
    """Seconds per whole layer of the oracle, timed over the given layers'
    (sequence, KV head) units in turn until at least min_s (at most max_s)."""
    import oracle.kv_oracle as O
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
    return dt * len(heads) / done, dt, done, full


def cpu_baseline(w, min_s=8.0, max_s=15.0, n_layers=3):
    """The oracle timed on the host on a bounded sample: the decode of the
    first n_layers layers (all KV heads of every sequence), layer after layer
    and again until at least min_s of timed work (stopping at max_s), scaled
    to whole-model steps/s; once with the BLAS thread pool at one thread and
    once with every core the process may use."""
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
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
    except Exception:
        threadpool_limits = None
    res = {}
    for label, nthreads in (("all_cores", cores), ("one_core", 1)):
        if threadpool_limits is not None:
            with threadpool_limits(limits=nthreads):
                layer_s, dt, done, full = _oracle_rate(w, layers, heads, off, min_s, max_s)
        else:
            layer_s, dt, done, full = _oracle_rate(w, layers, heads, off, min_s, max_s)
        res[label] = {"steps_per_s": 1.0 / (layer_s * w.layers), "threads": nthreads, "timed_s": dt,
                      "units": done, "whole_layers": full}
    return {"value": res["all_cores"]["steps_per_s"], "unit": "steps/s", "cores": cores, "kind": "oracle",
            "cpu_model": _cpu_model(), "one_core_value": res["one_core"]["steps_per_s"], "runs": res,
            "sample": f"layers 0-{len(layers) - 1} of {w.name}, in turn: the (sequence, KV head) units of each "
                      f"layer timed until {min_s:.0f} s (at most {max_s:.0f} s) of work, scaled to {w.layers} "
                      f"layers; numpy fp64 oracle (BLAS threads: all {cores} cores the process may use, then 1), "
                      f"quantization excluded"}


def host_tier_run(w, steps=64):
    """Host-pinned refinement store + device cache over `steps` steps of an
    AR(1) query process (rho = 0.9, selections overlap from step to step),
    from empty caches: the 32-layer step (lookup, fetch over the link and the
    five kernels per layer; no host synchronization, the LRU stamp advanced
    on the device) captured as one HIP graph and replayed once per step with
    that step's queries copied in before it, every replay timed on its own;
    then the same steps with eager launches; then the same queries again from
    empty caches with statistics for the hit rate and link bytes of each
    step.  Cold = the first step, warm = the second half."""
    import torch
    from selective_kv_cache_amd import binding as B
    m = Model(w, B.SF_TIER_HOST_PINNED)
    half = steps // 2

    def timed(run):
        for c in m.caches:
            c.clear_cache()
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        for t in range(steps):
            m.qbuf.copy_(qseq[t])
            evs[t].record()
            run()
        evs[steps].record()
        torch.cuda.synchronize()
        return [evs[t].elapsed_time(evs[t + 1]) for t in range(steps)]

    try:
        qseq = m.ar1_queries(steps)
        m.step()                     # leaves the workspace histograms clear
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            m.step()
        torch.cuda.synchronize()
        per = timed(graph.replay)
        del graph
        per_eager = timed(m.step)
        for c in m.caches:
            c.clear_cache()
        st = []
        for t in range(steps):
            m.qbuf.copy_(qseq[t])
            st.append(m.step(stats=True))
        warm = st[half:]
        sel_w = sum(x["selected"] for x in warm)
        return {"workload": w.name, "store": "host_pinned", "query_process": "AR(1) rho=0.9", "steps": steps,
                "launch": "hip_graph", "from": "empty caches",
                "cold_ms_per_step": per[0], "warm_ms_per_step": float(np.mean(per[half:])),
                "warm_steps_per_s": 1e3 / float(np.mean(per[half:])), "all_steps_ms_mean": float(np.mean(per)),
                "eager_cold_ms_per_step": per_eager[0], "eager_warm_ms_per_step": float(np.mean(per_eager[half:])),
                "cold_hit_rate": st[0]["hits"] / max(st[0]["selected"], 1),
                "warm_hit_rate": sum(x["hits"] for x in warm) / max(sel_w, 1),
                "cold_h2d_bytes": st[0]["h2d_bytes"],
                "warm_h2d_bytes_per_step": float(np.mean([x["h2d_bytes"] for x in warm])),
                "warm": f"steps {half}-{steps - 1}"}
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


def headline(w, tier, steps, warmup, multi_pass=False):
    """steps/s of the workload: eager launches with fixed queries, then the
    step captured as a HIP graph and replayed under AR(1) queries (copied into
    the query buffer before each replay, inside the timed region), then each
    kernel timed with event pairs.  Returns (record, per-kernel times, form)."""
    import torch
    from selective_kv_cache_amd import binding as B
    model = Model(w, tier, multi_pass=multi_pass)
    try:
        form = model.dec.form(model.caches[0], multi_pass=multi_pass)
        ms_eager = time_steps(model, steps, warmup)
        rec = {"eager_ms_per_step": ms_eager, "kernels_per_layer": form}
        if tier == B.SF_TIER_DEVICE:
            qseq = model.ar1_queries(warmup + steps)
            graph = capture_step(model)
            ms, per = time_graph(graph, steps, warmup, model, qseq)
            del graph
            rec.update(ms_per_step=ms, launch="hip_graph", query_process="AR(1) rho=0.9, new queries every step",
                       ms_per_step_p50=float(np.percentile(per, 50)),
                       ms_per_step_p10=float(np.percentile(per, 10)),
                       ms_per_step_p90=float(np.percentile(per, 90)))
        else:
            rec.update(ms_per_step=ms_eager, launch="eager", query_process="fixed per layer")
        names = ("fused",) if form == 1 else KERNELS
        kt = time_kernels(model, max(2, steps // 4), names)
        assert model.dec.check() == B.SF_OK, "a bounded wait expired"
        return rec, kt, form
    finally:
        model.close()


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama8b_128k")
    ap.add_argument("--tier", choices=["device", "host"], default="device")
    ap.add_argument("--multi-pass", action="store_true", help="the five-kernel form for the headline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--gemv", action="store_true",
                    help="only the weight-side GEMV record (one JSON line), for profiling it alone")
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
    if args.gemv:
        print(json.dumps({"weight_gemv": gemv_record()}), flush=True)
        return
    w = W.WORKLOADS[args.workload]
    tier = B.SF_TIER_DEVICE if args.tier == "device" else B.SF_TIER_HOST_PINNED
    log(f"setup {w.name}: {w.layers} layers, ctx {w.seq_lengths()[:4]}, tier {args.tier}")
    hl, kt, form = headline(w, tier, args.steps, args.warmup, args.multi_pass)
    ms = hl["ms_per_step"]
    log(f"{ms:.3f} ms/step ({hl['launch']}, {form} kernel(s) per layer); kernels {kt}")
    lens = w.seq_lengths()
    step_bytes = algorithmic_bytes(w, lens) * w.layers
    kb = fused_bytes(w, lens) if form == 1 else kernel_bytes(w, lens)
    dom = max(kb, key=lambda k: kt[k])
    gbps = {k: kb[k] / (kt[k] * 1e-3) / 1e9 for k in kb}
    traffic = measured_traffic(w.name).get(dom + "_decode" if form == 1 else dom + "_mfma")
    rec = {
        "metric": METRIC, "value": 1e3 / ms, "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "ctx": w.ctx or list(w.ctx_range),
                   "layers": w.layers, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "base_bits": w.base_bits, "refine_bits": w.refine_bits,
                   "top_t": w.top_t, "refinement_store": args.tier, "launch": hl["launch"],
                   "query_process": hl["query_process"], "kernels_per_layer": form},
        "ms_per_step_p50": hl.get("ms_per_step_p50"), "ms_per_step_p10": hl.get("ms_per_step_p10"),
        "ms_per_step_p90": hl.get("ms_per_step_p90"), "eager_ms_per_step": hl["eager_ms_per_step"],
        "step_algorithmic_bytes": step_bytes,
        "step_hbm_gbps": step_bytes / (ms * 1e-3) / 1e9,
        "step_frac_of_peak": step_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "roofline": {"bound": "hbm", "achieved": gbps[dom], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": gbps[dom] / PEAK_HBM_GBPS, "traffic": traffic, "kernel": dom,
                     "bytes_per_launch": kb[dom], "avg_launch_ms": kt[dom],
                     "kernels": {k: {"bytes_per_launch": kb[k], "avg_launch_ms": kt[k],
                                     "median_launch_ms": kt[k + "_median"], "achieved_gbps": gbps[k]}
                                 for k in kb},
                     "other_kernels_avg_ms": {k: kt[k] for k in kt if k not in kb and not k.endswith("_median")},
                     "event_timing": "start/stop HIP event pair around each launch, in this run"},
    }
    if not args.no_secondary:
        sec = {}
        if form == 1:
            log(f"secondary: {w.name}, the five-kernel form")
            hm, ktm, _ = headline(w, tier, args.steps, args.warmup, multi_pass=True)
            sec["multi_pass"] = {"ms_per_step": hm["ms_per_step"], "steps_per_s": 1e3 / hm["ms_per_step"],
                                 "launch": hm["launch"], "kernels_avg_ms": {k: ktm[k] for k in KERNELS}}
        w2 = W.WORKLOADS["llama8b_32k"]
        log("secondary: llama8b_32k")
        h2, kt2, f2 = headline(w2, B.SF_TIER_DEVICE, args.steps, args.warmup)
        b2 = algorithmic_bytes(w2, w2.seq_lengths()) * w2.layers
        sec["llama8b_32k"] = {"steps_per_s": 1e3 / h2["ms_per_step"], "ms_per_step": h2["ms_per_step"],
                              "launch": h2["launch"], "kernels_per_layer": f2,
                              "kernels_avg_ms": {k: v for k, v in kt2.items() if not k.endswith("_median")},
                              "step_hbm_gbps": b2 / (h2["ms_per_step"] * 1e-3) / 1e9,
                              "step_frac_of_peak": b2 / (h2["ms_per_step"] * 1e-3) / 1e9 / PEAK_HBM_GBPS}
        w5 = W.WORKLOADS["llama8b_reuse"]
        log("secondary: llama8b_reuse shape on the device tier (3-bit base codes)")
        h5, kt5, f5 = headline(w5, B.SF_TIER_DEVICE, args.steps, args.warmup)
        l5 = w5.seq_lengths()
        b5 = algorithmic_bytes(w5, l5) * w5.layers
        kb5 = kernel_bytes(w5, l5)
        sec["llama8b_reuse_device"] = {
            "steps_per_s": 1e3 / h5["ms_per_step"], "ms_per_step": h5["ms_per_step"],
            "us_per_layer": 1e3 * h5["ms_per_step"] / w5.layers, "launch": h5["launch"],
            "kernels_per_layer": f5, "ctx": int(l5[0]), "base_bits": w5.base_bits, "refine_bits": w5.refine_bits,
            "top_t": w5.top_t, "kernels_avg_ms": {k: v for k, v in kt5.items() if not k.endswith("_median")},
            "kernels_gbps": {k: x_bytes_per_ms(kb5[k], kt5[k]) for k in kb5},
            "step_hbm_gbps": b5 / (h5["ms_per_step"] * 1e-3) / 1e9,
            "step_frac_of_peak": b5 / (h5["ms_per_step"] * 1e-3) / 1e9 / PEAK_HBM_GBPS}
        w4 = W.Workload(**{**W.WORKLOADS["qwen8b_b16"].__dict__, "layers": 4})
        log("secondary: qwen8b_b16 over 4 distinct layers")
        h4, kt4, f4 = headline(w4, B.SF_TIER_DEVICE, args.steps, args.warmup)
        ms4 = min(h4["ms_per_step"], h4["eager_ms_per_step"]) / w4.layers
        b4 = algorithmic_bytes(w4, w4.seq_lengths())
        sec["qwen8b_b16"] = {"layer_steps_per_s": 1e3 / ms4, "ms_per_layer_step": ms4,
                             "layers_timed": w4.layers, "working_set_bytes": b4 * w4.layers,
                             "launch": "hip_graph" if h4["ms_per_step"] <= h4["eager_ms_per_step"] else "eager",
                             "kernels_per_layer": f4, "batch": w4.batch, "tokens": int(sum(w4.seq_lengths())),
                             "kernels_avg_ms": {k: v for k, v in kt4.items() if not k.endswith("_median")},
                             "step_hbm_gbps": b4 / (ms4 * 1e-3) / 1e9,
                             "step_frac_of_peak": b4 / (ms4 * 1e-3) / 1e9 / PEAK_HBM_GBPS}
        if w.host_store:
            log("secondary: host-pinned store, 64 AR(1) steps from empty caches")
            sec["host_store"] = host_tier_run(w, 64)
        log("secondary: multi-step reuse run (llama8b_reuse)")
        sec["reuse"] = reuse_record(W.WORKLOADS["llama8b_reuse"])
        log("secondary: weight-side refinement GEMV")
        sec["weight_gemv"] = gemv_record()
        rec["secondary"] = sec
    rd, rd_all = achievable_read_gbps()
    rec["achievable_read_gbps"] = rd
    rec["achievable_read"] = {"kernel": "sf_stream_read", "bytes": 4 << 30, "gbps_by_blocks": rd_all}
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a bounded sample)")
        rec["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

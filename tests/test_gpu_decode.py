"""GPU parity: the HIP decode path against the oracle on the same seeded inputs.

Bit-exact: packed base codes, refinement codes, (lo, delta) scales, and the
selection whenever the oracle's boundary is not within 1e-4 of a tie.
Scores within an fp32 evaluation bound; outputs within 2e-3 max abs.
"""
import numpy as np
import pytest

import oracle.kv_oracle as O
import parity as P
from selective_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu


def _case(w, top_t=None, layer=0, heads=None, dup=None, flat_rows=(), tier=0, multi_pass=False):
    lens = w.seq_lengths()
    off = W.seq_offsets(lens)
    k, v = W.layer_kv(w, layer)
    if dup is not None:
        dup(k, v)
    for t in flat_rows:
        k[t] = 0.75
        v[t] = -1.5
    q = W.query(w, layer)
    t = w.top_t if top_t is None else top_t
    print(f"case {w.name}: lens={lens[:4]}.. b={w.base_bits} r={w.refine_bits} T={t} G={w.group}", flush=True)
    run = P.run_gpu(w, k, v, q, off, t, tier=tier, multi_pass=multi_pass)
    stats = P.compare_layer(w, k, v, q, off, t, run, heads=heads)
    print(stats, flush=True)
    return run, stats


def test_tiny_reference_layer():
    _case(W.WORKLOADS["tiny_1k"])


SMALL = [
    dict(ctx=1000, n_q_heads=8, n_kv_heads=2, top_t=37),                       # ragged tail
    dict(ctx=3000, n_q_heads=8, n_kv_heads=2, base_bits=3, refine_bits=2, top_t=100),
    dict(ctx=2049, n_q_heads=4, n_kv_heads=1, base_bits=4, refine_bits=4, top_t=300),
    dict(ctx=777, n_q_heads=2, n_kv_heads=2, top_t=50),                        # G = 1
    dict(ctx=1500, n_q_heads=4, n_kv_heads=2, top_t=64),                       # G = 2
    dict(ctx=1300, n_q_heads=8, n_kv_heads=1, top_t=64),                       # G = 8
    dict(ctx=900, base_bits=2, refine_bits=0, top_t=64),                       # no refinement bits
    dict(ctx=900, top_t=0),                                                    # nothing selected
    dict(ctx=300, top_t=512),                                                  # N < T: all selected
    dict(ctx=256, top_t=256),                                                  # N == T
    dict(ctx=1, top_t=4),                                                      # one token
    dict(ctx=5000, refine_bits=8, top_t=256, n_q_heads=8, n_kv_heads=2),
    dict(ctx=20_000, n_q_heads=32, n_kv_heads=8, base_bits=3, refine_bits=2, top_t=2048),  # 64-token selected blocks
    dict(ctx=300_000, n_q_heads=2, n_kv_heads=1, top_t=1000),                 # > 64 selection chunks
    dict(ctx=600_000, n_q_heads=2, n_kv_heads=1, top_t=3000),                 # bitmap beyond LDS
    dict(ctx=777, n_q_heads=2, n_kv_heads=2, base_bits=3, refine_bits=2, top_t=50),   # 3-bit, G = 1
    dict(ctx=1500, n_q_heads=4, n_kv_heads=2, base_bits=3, refine_bits=4, top_t=64),  # 3-bit, G = 2
    dict(ctx=1300, n_q_heads=8, n_kv_heads=1, base_bits=3, refine_bits=2, top_t=64),  # 3-bit, G = 8
    dict(ctx=33, n_q_heads=8, n_kv_heads=2, base_bits=3, refine_bits=8, top_t=7),     # 3-bit, one chunk + 1
    dict(ctx=9000, n_q_heads=16, n_kv_heads=2, refine_bits=4, top_t=300),             # G = 8, several splits
    dict(ctx=1111, n_q_heads=2, n_kv_heads=2, base_bits=4, refine_bits=2, top_t=90),  # 4-bit, G = 1
    dict(ctx=5000, n_q_heads=16, n_kv_heads=2, base_bits=4, refine_bits=4, top_t=256), # 4-bit, G = 8
]


def test_base_pass_precision():
    """Every token at base precision (T = 0), so the whole result comes from
    the base pass's matrix-core P.V product: within 1e-4 of the oracle.  The
    2-bit codes enter that product at fp16 mantissa bits >= 4; with codes at
    bit 0 its error on this case was 2.5e-4 (measured 1.8e-5 after)."""
    _, st = _case(W.small(cfg_id=228, ctx=1000, top_t=0))
    assert st["max_out_err"] <= 1e-4, st


def test_base_pass_precision_3bit():
    """The same with 3-bit base codes: every token through the matrix-core
    P.V with the codes cut from two dwords by a funnel shift and placed at
    fp16 mantissa bits 4-9."""
    _, st = _case(W.small(cfg_id=229, ctx=1000, base_bits=3, refine_bits=2, top_t=0))
    assert st["max_out_err"] <= 1e-4, st


def test_base_pass_precision_4bit():
    """The same with 4-bit base codes (dword n of a row holds row n's 8 codes,
    placed at fp16 mantissa bits 4-7)."""
    _, st = _case(W.small(cfg_id=231, ctx=1000, base_bits=4, refine_bits=4, top_t=0))
    assert st["max_out_err"] <= 1e-4, st


def test_base_pass_precision_group8():
    """The same for groups of 8 query heads: two heads per softmax lane and
    the 16 weight columns (hi and lo parts of 8 heads) filling the P.V
    product."""
    _, st = _case(W.small(cfg_id=230, ctx=1000, n_q_heads=16, n_kv_heads=2, top_t=0))
    assert st["max_out_err"] <= 1e-4, st


@pytest.mark.parametrize("form", ["single", "multi"])
@pytest.mark.parametrize("i", range(len(SMALL)), ids=[",".join(f"{k}={v}" for k, v in o.items()) for o in SMALL])
def test_small_shapes(i, form):
    """Each shape through the single-launch form (where it applies: 2-bit base
    codes, groups of 1, 2 or 4, work-groups resident at once; the others take
    the five kernels anyway) and through the five-kernel form."""
    _case(W.small(cfg_id=220 + i, **SMALL[i]), multi_pass=form == "multi")


def test_varlen_batch():
    w = W.small("varlen", cfg_id=210, batch=3, n_q_heads=8, n_kv_heads=2, refine_bits=8, top_t=200)
    lens = [700, 1500, 129]
    off = W.seq_offsets(lens)
    k, v = W.layer_kv(w, 0, n_tok=int(off[-1]))
    q = W.query(w, 0)
    run = P.run_gpu(w, k, v, q, off, w.top_t)
    P.compare_layer(w, k, v, q, off, w.top_t, run)


def test_ties_at_the_cut_go_to_the_lower_index():
    w = W.small(cfg_id=300, ctx=600, top_t=50)
    k, v = W.layer_kv(w, 0)
    q = W.query(w, 0)
    oc = O.quantize_cache(k, v, w.base_bits, w.refine_bits)
    s = O.token_scores(q[0], O.dequant_base(O._rows(oc.k, 0, 0, 600)))
    pivot = int(np.argsort(-s, kind="stable")[w.top_t - 1])         # the T-th ranked token
    rng = np.random.default_rng(1)
    dst = rng.choice(np.setdiff1d(np.arange(600), [pivot]), size=25, replace=False)
    W.duplicate_rows(k, v, [pivot] * 25, dst)                       # 26 exact ties straddle the cut
    off = W.seq_offsets([600])
    run = P.run_gpu(w, k, v, q, off, w.top_t)
    stats = P.compare_layer(w, k, v, q, off, w.top_t, run)
    assert stats["selections_differing"] == 0
    tied = np.sort(np.concatenate([[pivot], dst]))
    chosen = np.intersect1d(run.sel[0, 0], tied)
    assert 0 < chosen.size < tied.size
    assert np.array_equal(chosen, tied[:chosen.size])              # the lowest indices of the tie win


def test_flat_rows_and_all_equal_scores():
    w = W.small(cfg_id=301, ctx=700, top_t=40)
    _case(w, flat_rows=(3, 100, 699))
    # every key identical: all scores tie, the selection is tokens 0..T-1
    k, v = W.layer_kv(w, 0)
    k[:] = k[5]
    q = W.query(w, 0)
    off = W.seq_offsets([700])
    run = P.run_gpu(w, k, v, q, off, w.top_t)
    P.compare_layer(w, k, v, q, off, w.top_t, run)
    assert np.array_equal(run.sel[0, 0], np.arange(w.top_t))


def _near_equal_keys(k, v):
    # every key close to one row: more than 2,048 tokens share the level-1
    # boundary bin, so the single launch settles them by its histogram levels
    k[:] = k[5] + 1e-3 * k


def _pivot_ties(k, v):
    # 40 exact copies of one row spread over the context
    rng = np.random.default_rng(7)
    dst = rng.choice(np.arange(1, k.shape[0]), size=40, replace=False)
    W.duplicate_rows(k, v, [0] * 40, dst)


def _all_equal(k, v):
    k[:] = k[5]


SELECT_CASES = {
    "random": (dict(ctx=20000, top_t=500), None),
    "pivot_ties": (dict(ctx=9000, top_t=300), _pivot_ties),
    "near_equal": (dict(ctx=6000, top_t=300), _near_equal_keys),
    "all_equal": (dict(ctx=5000, top_t=100), _all_equal),
}


@pytest.mark.parametrize("case", list(SELECT_CASES))
def test_single_launch_selects_as_the_five_kernel_form(case):
    """Both forms take the exact top-T of the same fp32 keys, ties to the
    lower index, so their selections are identical (the single launch through
    its candidate list, or through its histogram levels when the level-1
    boundary bin holds more than 2,048 tokens)."""
    over, dup = SELECT_CASES[case]
    w = W.small(cfg_id=304, **over)
    off = W.seq_offsets(w.seq_lengths())
    k, v = W.layer_kv(w, 0)
    if dup is not None:
        dup(k, v)
    q = W.query(w, 0)
    print(f"case {case}: {over}", flush=True)
    a = P.run_gpu(w, k, v, q, off, w.top_t)
    b = P.run_gpu(w, k, v, q, off, w.top_t, multi_pass=True)
    assert np.array_equal(a.scores.view(np.uint32), b.scores.view(np.uint32))
    assert np.array_equal(a.sel, b.sel)
    assert float(np.abs(a.out - b.out).max()) < 1e-4
    P.compare_layer(w, k, v, q, off, w.top_t, a)


def test_deterministic_repeat():
    w = W.small(cfg_id=302, ctx=5000, n_q_heads=8, n_kv_heads=2, top_t=128)
    lens = w.seq_lengths()
    off = W.seq_offsets(lens)
    k, v = W.layer_kv(w, 0)
    q = W.query(w, 0)
    a = P.run_gpu(w, k, v, q, off, w.top_t)
    b = P.run_gpu(w, k, v, q, off, w.top_t)
    assert np.array_equal(a.out.view(np.uint32), b.out.view(np.uint32))
    assert np.array_equal(a.sel, b.sel)


def test_consecutive_steps_share_one_workspace():
    # each step clears the selection histogram for the next one; a stale
    # count would move the cut of a later step
    w = W.small("steps", cfg_id=303, batch=2, n_q_heads=8, n_kv_heads=2, top_t=96, rho=0.5)
    off = W.seq_offsets([2500, 1100])
    k, v = W.layer_kv(w, 0, n_tok=int(off[-1]))
    qs = W.queries(w, 0, 4)
    runs = P.run_gpu_steps(w, k, v, qs, off, w.top_t)
    for q, run in zip(qs, runs):
        P.compare_layer(w, k, v, q, off, w.top_t, run, codec=False)


def test_graph_replay_matches_eager():
    # the device-tier step launches kernels only, so it can be captured; every
    # replay, with eager steps and synchronisations in between, must equal the
    # eager result bit for bit
    import torch
    from selective_kv_cache_amd.kvcache import Decoder, LayerCache
    w = W.small("graph", cfg_id=304, batch=2, n_q_heads=8, n_kv_heads=2, refine_bits=4, top_t=100)
    off = W.seq_offsets([3000, 1200])
    g = P.geom_of(w)
    caches, qs = [], []
    try:
        for layer in range(2):
            c = LayerCache(g, int(off[-1]))
            k, v = W.layer_kv(w, layer, n_tok=int(off[-1]))
            c.append(torch.as_tensor(k, device="cuda"), torch.as_tensor(v, device="cuda"), 0)
            caches.append(c)
            qs.append(torch.as_tensor(W.query(w, layer), device="cuda"))
        dec = Decoder(g, off, w.top_t)
        outs = [torch.empty((2, 8, 128), dtype=torch.float32, device="cuda") for _ in range(2)]
        sels = [torch.empty((2, 2, w.top_t), dtype=torch.int32, device="cuda") for _ in range(2)]

        def step():
            for layer in range(2):
                dec.step(caches[layer], qs[layer], out=outs[layer], sel_out=sels[layer])

        step()
        torch.cuda.synchronize()
        want = [o.cpu().numpy().copy() for o in outs]
        want_sel = [x.cpu().numpy().copy() for x in sels]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for rep in range(3):
            for o in outs:
                o.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            for layer in range(2):
                assert np.array_equal(outs[layer].cpu().numpy().view(np.uint32), want[layer].view(np.uint32)), rep
                assert np.array_equal(sels[layer].cpu().numpy(), want_sel[layer]), rep
            step()                      # eager work between replays
            torch.cuda.synchronize()
            for layer in range(2):
                assert np.array_equal(outs[layer].cpu().numpy().view(np.uint32), want[layer].view(np.uint32))
        del graph
    finally:
        for c in caches:
            c.close()


def test_host_tier_matches_device_tier_and_cache_simulation():
    """Host-pinned store + device refinement cache over several steps of an
    AR(1) query process: outputs bit-identical to the device-resident store,
    and hits/misses equal to the oracle's cache simulation."""
    import torch
    from selective_kv_cache_amd import binding as B
    from selective_kv_cache_amd.kvcache import Decoder, LayerCache
    w = W.small("reuse", cfg_id=303, ctx=3000, n_q_heads=8, n_kv_heads=2, base_bits=3, refine_bits=2,
                top_t=128, rho=0.9)
    g = P.geom_of(w)
    off = W.seq_offsets([3000])
    k, v = W.layer_kv(w, 0)
    qs = W.queries(w, 0, 6)
    dev = LayerCache(g, 3000, tier=B.SF_TIER_DEVICE)
    host = LayerCache(g, 3000, tier=B.SF_TIER_HOST_PINNED, max_seqs=1, cache_slots=2 * w.top_t)
    try:
        kd, vd = torch.as_tensor(k, device="cuda"), torch.as_tensor(v, device="cuda")
        dev.append(kd, vd, 0)
        host.append(kd, vd, 0)
        dec = Decoder(g, off, w.top_t)
        sims = [O.CacheSim(2 * w.top_t) for _ in range(w.n_kv_heads)]
        sel = torch.empty((1, w.n_kv_heads, w.top_t), dtype=torch.int32, device="cuda")
        for t in range(qs.shape[0]):
            qd = torch.as_tensor(qs[t], device="cuda")
            o_dev = dec.step(dev, qd, multi_pass=True).cpu().numpy()
            o_host, st = dec.step(host, qd, sel_out=sel, want_stats=True)
            o_host = o_host.cpu().numpy()
            assert np.array_equal(o_dev.view(np.uint32), o_host.view(np.uint32)), t
            hits = misses = 0
            for h in range(w.n_kv_heads):
                hh, mm = sims[h].step(sel[0, h].cpu().numpy(), t)
                hits, misses = hits + hh, misses + mm
            assert (st["hits"], st["misses"]) == (hits, misses), (t, st, hits, misses)
            assert st["h2d_bytes"] == O.fetched_bytes(misses, w.head_dim, w.refine_bits)
            print(t, st, flush=True)
        # a cold cache misses on the whole selection and still gives the same output
        host.clear_cache()
        o_host, st = dec.step(host, qd, want_stats=True)
        assert st["misses"] == st["selected"] and st["hits"] == 0
        assert np.array_equal(o_dev.view(np.uint32), o_host.cpu().numpy().view(np.uint32))
    finally:
        dev.close()
        host.close()


def test_host_tier_graph_replays_match_eager():
    """The host-tier step (cache lookup, fetch of the misses over the link,
    the five kernels) captured as a HIP graph and replayed under an AR(1)
    query process: every replay's output bit-identical to the same step
    launched eagerly on an identical store, and the caches left in the same
    state (the LRU stamp advances on the device, so replays age the cache as
    eager steps do)."""
    import torch
    from selective_kv_cache_amd import binding as B
    from selective_kv_cache_amd.kvcache import Decoder, LayerCache
    w = W.small("hostgraph", cfg_id=310, ctx=3000, n_q_heads=8, n_kv_heads=2, refine_bits=4, top_t=128, rho=0.9)
    g = P.geom_of(w)
    off = W.seq_offsets([3000])
    k, v = W.layer_kv(w, 0)
    qs = W.queries(w, 0, 10)
    stores = [LayerCache(g, 3000, tier=B.SF_TIER_HOST_PINNED, max_seqs=1, cache_slots=w.top_t + 64)
              for _ in range(2)]
    try:
        kd, vd = torch.as_tensor(k, device="cuda"), torch.as_tensor(v, device="cuda")
        decs = []
        for c in stores:
            c.append(kd, vd, 0)
            decs.append(Decoder(g, off, w.top_t))
        qbuf = torch.as_tensor(qs[0], device="cuda").clone()
        obuf = torch.empty((1, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
        for c, d in zip(stores, decs):            # the same warm-up step on both
            d.step(c, qbuf)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            decs[1].step(stores[1], qbuf, out=obuf)
        torch.cuda.synchronize()
        for c in stores:
            c.clear_cache()
        torch.cuda.synchronize()
        for t in range(qs.shape[0] - 1):
            qd = torch.as_tensor(qs[t], device="cuda")
            o_eager = decs[0].step(stores[0], qd).cpu().numpy()
            qbuf.copy_(qd)
            graph.replay()
            torch.cuda.synchronize()
            o_graph = obuf.cpu().numpy()
            assert np.array_equal(o_eager.view(np.uint32), o_graph.view(np.uint32)), t
        qd = torch.as_tensor(qs[-1], device="cuda")
        st = [d.step(c, qd, want_stats=True)[1] for c, d in zip(stores, decs)]
        assert st[0]["hits"] == st[1]["hits"] and st[0]["misses"] == st[1]["misses"], st
        assert 0 < st[0]["hits"] < st[0]["selected"], st
        del graph
    finally:
        for c in stores:
            c.close()


def test_append_steps_host_tier():
    """Multi-step reuse run, reduced: each step appends one token (quantized on
    the GPU, its refinement rows put in the pinned store) and decodes over the
    grown context with an AR(1) query.  Every step: codes, scales and
    refinement rows of all tokens so far, scores, selection and output against
    the oracle on the same tokens; host-tier output bit-identical to the
    device tier's; hits and misses equal to the oracle's cache simulation."""
    import torch
    from selective_kv_cache_amd import binding as B
    from selective_kv_cache_amd.kvcache import Decoder, LayerCache
    w = W.small("reuse5", cfg_id=305, ctx=2000, n_q_heads=8, n_kv_heads=2, base_bits=3, refine_bits=2,
                top_t=128, rho=0.9)
    steps, n0 = 6, 2000
    g = P.geom_of(w)
    k, v = W.layer_kv(w, 0)
    qs = W.queries(w, 0, steps)
    dev = LayerCache(g, n0 + steps, tier=B.SF_TIER_DEVICE)
    host = LayerCache(g, n0 + steps, tier=B.SF_TIER_HOST_PINNED, max_seqs=1, cache_slots=2 * w.top_t)
    try:
        cuda = lambda x: torch.as_tensor(x, device="cuda")
        kr, vr = dev.append(cuda(k), cuda(v), 0, keep_refine=True)
        host.append(cuda(k), cuda(v), 0)
        sims = [O.CacheSim(2 * w.top_t) for _ in range(w.n_kv_heads)]
        for t in range(steps):
            ka, va = W.appended_kv(w, 0, t)
            kra, vra = dev.append(cuda(ka), cuda(va), n0 + t, keep_refine=True)
            host.append(cuda(ka), cuda(va), n0 + t)
            kr, vr = torch.cat([kr, kra], 1), torch.cat([vr, vra], 1)
            k, v = np.concatenate([k, ka]), np.concatenate([v, va])
            n = n0 + t + 1
            off = W.seq_offsets([n])
            dec = Decoder(g, off, w.top_t)
            q = cuda(qs[t])
            sel = torch.full((1, w.n_kv_heads, w.top_t), -7, dtype=torch.int32, device="cuda")
            scores = torch.empty((w.n_kv_heads, n), dtype=torch.float32, device="cuda")
            o_dev = dec.step(dev, q, sel_out=sel, scores_out=scores, multi_pass=True)
            o_host, st = dec.step(host, q, want_stats=True)
            torch.cuda.synchronize()
            assert np.array_equal(o_dev.cpu().numpy().view(np.uint32), o_host.cpu().numpy().view(np.uint32)), t
            cpu = lambda x: x.cpu().numpy()
            run = P.GpuRun(out=cpu(o_dev), sel=cpu(sel), scores=cpu(scores), k_codes=cpu(dev.k_codes),
                           v_codes=cpu(dev.v_codes), k_scales=cpu(dev.k_scales), v_scales=cpu(dev.v_scales),
                           k_ref=cpu(kr), v_ref=cpu(vr))
            stats = P.compare_layer(w, k, v, qs[t], off, w.top_t, run)
            hits = misses = 0
            for h in range(w.n_kv_heads):
                hh, mm = sims[h].step(run.sel[0, h], t)
                hits, misses = hits + hh, misses + mm
            assert (st["hits"], st["misses"]) == (hits, misses), (t, st, hits, misses)
            assert st["h2d_bytes"] == O.fetched_bytes(misses, w.head_dim, w.refine_bits)
            print(t, n, st, stats, flush=True)
    finally:
        dev.close()
        host.close()


def test_skip_misses_host_tier():
    """Policy "skip" on a miss over AR(1) steps, a token appended before each:
    the output against the oracle with only the cache's hits refined (the
    misses at base precision), hits and misses as the oracle's cache
    simulation, and, at a step where nothing misses (the last query
    repeated), bit-identical to the "wait" policy."""
    import torch
    from selective_kv_cache_amd import binding as B
    from selective_kv_cache_amd.kvcache import Decoder, LayerCache
    w = W.small("skip", cfg_id=306, ctx=2500, n_q_heads=8, n_kv_heads=2, base_bits=2, refine_bits=4,
                top_t=128, rho=0.9)
    steps, n0 = 5, 2500
    g = P.geom_of(w)
    k, v = W.layer_kv(w, 0)
    qs = W.queries(w, 0, steps)
    qs = np.concatenate([qs, qs[-1:]])                     # the last query again: every selected token cached
    mk = lambda: LayerCache(g, n0 + steps + 1, tier=B.SF_TIER_HOST_PINNED, max_seqs=1,
                            cache_slots=2 * w.top_t)
    wait, skip = mk(), mk()
    try:
        cuda = lambda x: torch.as_tensor(x, device="cuda")
        for c in (wait, skip):
            c.append(cuda(k), cuda(v), 0)
        sims = [O.CacheSim(2 * w.top_t) for _ in range(w.n_kv_heads)]
        n = n0
        for t in range(qs.shape[0]):
            if t < steps:
                ka, va = W.appended_kv(w, 0, t)
                for c in (wait, skip):
                    c.append(cuda(ka), cuda(va), n)
                k, v = np.concatenate([k, ka]), np.concatenate([v, va])
                n += 1
            dec = Decoder(g, W.seq_offsets([n]), w.top_t)
            q = cuda(qs[t])
            sel = torch.full((1, w.n_kv_heads, w.top_t), -7, dtype=torch.int32, device="cuda")
            o_wait = dec.step(wait, q).cpu().numpy()
            o_skip, st = dec.step(skip, q, sel_out=sel, want_stats=True, skip_misses=True)
            o_skip, sel = o_skip.cpu().numpy(), sel.cpu().numpy()
            oc = O.quantize_cache(k, v, w.base_bits, w.refine_bits)
            hits = misses = 0
            worst = 0.0
            for h in range(w.n_kv_heads):
                hit_toks, miss_toks = sims[h].step_tokens(sel[0, h], t)
                hits, misses = hits + len(hit_toks), misses + len(miss_toks)
                qg = qs[t][0, h * w.group:(h + 1) * w.group]
                ref = O.decode_head(qg, O._rows(oc.k, h, 0, n), O._rows(oc.v, h, 0, n), w.top_t,
                                    sel=sel[0, h], refined=np.asarray(hit_toks, dtype=np.int64))
                worst = max(worst, float(np.abs(o_skip[0, h * w.group:(h + 1) * w.group] - ref.out).max()))
            assert worst <= P.OUT_ATOL, (t, worst)
            assert (st["hits"], st["misses"]) == (hits, misses), (t, st, hits, misses)
            if misses == 0:
                assert np.array_equal(o_skip.view(np.uint32), o_wait.view(np.uint32)), t
            print(t, n, st, "max err", worst, "vs wait", float(np.abs(o_skip - o_wait).max()), flush=True)
        assert misses == 0                                    # the repeated query hit everything
    finally:
        wait.close()
        skip.close()


def test_host_tier_rewrite_invalidates_cached_rows():
    """Rewriting tokens whose refinement rows the device cache holds (the same
    K, new V stored over them, so the selection stays the same): the next step
    misses exactly on the rewritten selected tokens and refetches them, and its
    output equals a device-tier store holding the rewritten rows, bit for bit."""
    import torch
    from selective_kv_cache_amd import binding as B
    from selective_kv_cache_amd.kvcache import Decoder, LayerCache
    w = W.small("rewrite", cfg_id=307, ctx=1500, n_q_heads=8, n_kv_heads=2, base_bits=2, refine_bits=4,
                top_t=96)
    g = P.geom_of(w)
    k, v = W.layer_kv(w, 0)
    q = W.query(w, 0)
    dev = LayerCache(g, 1500, tier=B.SF_TIER_DEVICE)
    host = LayerCache(g, 1500, tier=B.SF_TIER_HOST_PINNED, max_seqs=1, cache_slots=2 * w.top_t)
    try:
        cuda = lambda x: torch.as_tensor(x, device="cuda")
        for c in (dev, host):
            c.append(cuda(k), cuda(v), 0)
        dec = Decoder(g, W.seq_offsets([1500]), w.top_t)
        sel = torch.empty((1, w.n_kv_heads, w.top_t), dtype=torch.int32, device="cuda")
        dec.step(host, cuda(q), sel_out=sel)                 # caches the selection's rows
        chosen = np.unique(sel.cpu().numpy())
        lo, hi = int(chosen[0]), int(chosen[0]) + 64            # a run of tokens, some of them cached
        rng = np.random.default_rng(11)
        v2 = v.copy()
        v2[lo:hi] = rng.standard_normal(v2[lo:hi].shape).astype(np.float32)
        for c in (dev, host):
            c.append(cuda(k[lo:hi]), cuda(v2[lo:hi]), lo)
        sel_np = sel.cpu().numpy()[0]
        rewritten = sum(int(((sel_np[h] >= lo) & (sel_np[h] < hi)).sum()) for h in range(w.n_kv_heads))
        o_dev = dec.step(dev, cuda(q), multi_pass=True).cpu().numpy()
        o_host, st = dec.step(host, cuda(q), want_stats=True)
        assert rewritten > 0 and st["misses"] == rewritten, (rewritten, st)
        assert np.array_equal(o_dev.view(np.uint32), o_host.cpu().numpy().view(np.uint32))
    finally:
        dev.close()
        host.close()


@pytest.mark.slow
@pytest.mark.timeout(600)
@pytest.mark.parametrize("form", ["single", "multi"])
@pytest.mark.parametrize("name", ["llama8b_32k", "llama8b_128k", "qwen8b_b16"])
def test_full_size_layer_all_heads(name, form):
    """Full-size layer in the benchmark's launch configuration (the single
    launch where it applies; the five kernels with "multi"); the oracle checks
    every (sequence, KV head) pair: codes and scales bit-exact, scores,
    selection and output."""
    w = W.WORKLOADS[name]
    off = W.seq_offsets(w.seq_lengths())
    k, v = W.layer_kv(w, 0)
    q = W.query(w, 0)
    print(f"full size {name} ({form}): tokens={int(off[-1])}", flush=True)
    run = P.run_gpu(w, k, v, q, off, w.top_t, multi_pass=form == "multi")
    st = P.compare_layer(w, k, v, q, off, w.top_t, run)
    print(st, flush=True)
    assert st["units"] == w.batch * w.n_kv_heads


def _two_seq_host_run(w, lens, steps, skip=False):
    """A 2-sequence batch over AR(1) steps on a host-pinned store (2 batch
    positions) beside a device-tier store: per step, hits and misses against
    the oracle's cache simulation of every (sequence, KV head), outputs against
    the oracle (only the hits refined under the skip policy), and, under
    "wait", bit-identical to the device tier."""
    import torch
    from selective_kv_cache_amd import binding as B
    from selective_kv_cache_amd.kvcache import Decoder, LayerCache
    g = P.geom_of(w)
    off = W.seq_offsets(lens)
    n = int(off[-1])
    k, v = W.layer_kv(w, 0, n_tok=n)
    qs = W.queries(w, 0, steps)
    dev = LayerCache(g, n, tier=B.SF_TIER_DEVICE)
    host = LayerCache(g, n, tier=B.SF_TIER_HOST_PINNED, max_seqs=2, cache_slots=2 * w.top_t)
    cuda = lambda x: torch.as_tensor(x, device="cuda")
    try:
        for c in (dev, host):
            c.append(cuda(k), cuda(v), 0)
        dec = Decoder(g, off, w.top_t)
        oc = O.quantize_cache(k, v, w.base_bits, w.refine_bits)
        sims = {(s, h): O.CacheSim(2 * w.top_t) for s in range(2) for h in range(w.n_kv_heads)}
        for t in range(steps):
            q = cuda(qs[t])
            sel = torch.full((2, w.n_kv_heads, w.top_t), -7, dtype=torch.int32, device="cuda")
            scores = torch.empty((w.n_kv_heads, n), dtype=torch.float32, device="cuda")
            o_dev = dec.step(dev, q, sel_out=sel, scores_out=scores, multi_pass=True).cpu().numpy()
            sel_np = sel.cpu().numpy()
            o_host, st = dec.step(host, q, want_stats=True, skip_misses=skip)
            o_host = o_host.cpu().numpy()
            run = P.GpuRun(out=o_dev, sel=sel_np, scores=scores.cpu().numpy(), k_codes=None, v_codes=None,
                           k_scales=None, v_scales=None, k_ref=None, v_ref=None)
            P.compare_layer(w, k, v, qs[t], off, w.top_t, run, codec=False)
            hits = misses = 0
            worst = 0.0
            for s in range(2):
                a, e = int(off[s]), int(off[s + 1])
                tn = min(w.top_t, e - a)
                for h in range(w.n_kv_heads):
                    hit_toks, miss_toks = sims[(s, h)].step_tokens(sel_np[s, h, :tn], t)
                    hits, misses = hits + len(hit_toks), misses + len(miss_toks)
                    if skip:
                        qg = qs[t][s, h * w.group:(h + 1) * w.group]
                        ref = O.decode_head(qg, O._rows(oc.k, h, a, e), O._rows(oc.v, h, a, e), w.top_t,
                                            sel=sel_np[s, h, :tn], refined=np.asarray(hit_toks, dtype=np.int64))
                        worst = max(worst, float(np.abs(o_host[s, h * w.group:(h + 1) * w.group] - ref.out).max()))
            assert (st["hits"], st["misses"]) == (hits, misses), (t, st, hits, misses)
            assert st["h2d_bytes"] == O.fetched_bytes(misses, w.head_dim, w.refine_bits)
            if skip:
                assert worst <= P.OUT_ATOL, (t, worst)
            else:
                assert np.array_equal(o_dev.view(np.uint32), o_host.view(np.uint32)), t
            print(t, st, flush=True)
        assert B.sf_store_check(host.store) == B.SF_OK
        return dev, host, k, v, qs, off
    except BaseException:
        dev.close()
        host.close()
        raise


def test_host_tier_two_sequences_and_reorder():
    """Two sequences on a host-pinned store (the cache of each batch position
    checked against its own simulation), then the second sequence alone at
    batch position 0 without clearing the cache: its tokens are cached only in
    position 1's cache, so every selected token misses; the output still equals
    the device tier's bit for bit and the tables stay consistent."""
    import torch
    from selective_kv_cache_amd import binding as B
    from selective_kv_cache_amd.kvcache import Decoder
    w = W.small("reuse2", cfg_id=308, batch=2, n_q_heads=8, n_kv_heads=2, base_bits=2, refine_bits=4,
                top_t=96, rho=0.9)
    dev, host, k, v, qs, off = _two_seq_host_run(w, [1500, 2100], 4)
    try:
        g = P.geom_of(w)
        dec = Decoder(g, [int(off[1]), int(off[2])], w.top_t)
        q = torch.as_tensor(qs[-1][1:2], device="cuda")
        o_dev = dec.step(dev, q, multi_pass=True).cpu().numpy()
        o_host, st = dec.step(host, q, want_stats=True)
        assert st["misses"] == st["selected"] and st["hits"] == 0, st
        assert np.array_equal(o_dev.view(np.uint32), o_host.cpu().numpy().view(np.uint32))
        assert B.sf_store_check(host.store) == B.SF_OK
        o_host2, st2 = dec.step(host, q, want_stats=True)       # now cached at position 0
        assert st2["misses"] == 0, st2
        assert np.array_equal(o_dev.view(np.uint32), o_host2.cpu().numpy().view(np.uint32))
    finally:
        dev.close()
        host.close()


def test_skip_misses_two_sequences():
    w = W.small("skip2", cfg_id=309, batch=2, n_q_heads=8, n_kv_heads=2, base_bits=2, refine_bits=2,
                top_t=64, rho=0.9)
    dev, host, *_ = _two_seq_host_run(w, [1800, 900], 4, skip=True)
    dev.close()
    host.close()


def test_store_pitch_must_match_the_caches():
    """A store whose capacity differs from the caches' pitch is refused before
    anything is launched (the kernels index the store with that pitch)."""
    import torch
    from selective_kv_cache_amd import binding as B
    from selective_kv_cache_amd.kvcache import Decoder, LayerCache
    w = W.small("pitch", cfg_id=310, ctx=500, n_q_heads=4, n_kv_heads=1, top_t=32)
    g = P.geom_of(w)
    for tier in (B.SF_TIER_DEVICE, B.SF_TIER_HOST_PINNED):
        c = LayerCache(g, 600, tier=tier, max_seqs=1, cache_slots=64)
        other = B.sf_store_create(g, 512, 1, tier, 64)
        try:
            dec = Decoder(g, [0, 500], w.top_t)
            q = torch.zeros((1, 4, 128), dtype=torch.float32, device="cuda")
            out = torch.full((1, 4, 128), 7.0, dtype=torch.float32, device="cuda")
            with pytest.raises(B.SfError) as ei:
                B.sf_decode_step(g, seq_off_host=dec.seq_off, seq_off_dev=dec.seq_off_dev, q=q,
                                 k_codes=c.k_codes, k_scales=c.k_scales, v_codes=c.v_codes, v_scales=c.v_scales,
                                 cap=c.cap, store=other, top_t=w.top_t, out=out, workspace=dec.workspace)
            assert ei.value.status == B.SF_ERR_INVALID_ARG
            torch.cuda.synchronize()
            assert bool((out == 7.0).all())                    # nothing was written
        finally:
            B.sf_store_destroy(other)
            c.close()


def test_refused_allocation_is_oom():
    """Allocations the device cannot hold are refused with SF_ERR_OOM and leave
    nothing allocated: a device-tier store of 2 TiB of refinement rows, and a
    host-tier store whose small pinned store succeeds but whose device cache
    (60,000 batch positions x 8 heads x 4,096 slots x 256 B) cannot be held, so
    the pinned memory already taken is released again.  A normal store still
    works afterwards.  (Pinned host memory itself is not pushed to its limit:
    that limit depends on the host.)"""
    from selective_kv_cache_amd import binding as B
    g = B.geom(128, 32, 8, 2, 8)
    with pytest.raises(B.SfError) as ei:
        B.sf_store_create(g, 1 << 30, 1, B.SF_TIER_DEVICE, 0)  # 2 x 8 x 2^30 x 128 B
    assert ei.value.status == B.SF_ERR_OOM
    with pytest.raises(B.SfError) as ei:
        B.sf_store_create(g, 1024, 60000, B.SF_TIER_HOST_PINNED, 4096)
    assert ei.value.status == B.SF_ERR_OOM
    h = B.sf_store_create(g, 1024, 1, B.SF_TIER_HOST_PINNED, 64)
    B.sf_store_destroy(h)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_reuse_run_stated_shape():
    """The multi-step reuse workload at its stated shape, layer 0: 32 query /
    8 KV heads, 3-bit base codes, 2 refinement bits, T = 512, 8,192 tokens
    growing by one per step over 256 steps, AR(1) queries (rho = 0.9), the
    refinement store in pinned host memory with 2T cache slots per head.
    Every step: the appended token's codes, scales and refinement rows
    bit-exact, every head's scores, selection and output against the oracle
    (composed step by step: its quantizer on the appended rows, then its
    scoring, top-T and attention), and hits, misses and link bytes against the
    oracle's cache simulation."""
    import torch
    from selective_kv_cache_amd import binding as B
    from selective_kv_cache_amd.kvcache import Decoder, LayerCache
    w = W.WORKLOADS["llama8b_reuse"]
    g = P.geom_of(w)
    n0, steps, hkv, G, T = w.ctx, w.steps, w.n_kv_heads, w.group, w.top_t
    cap = n0 + steps
    k, v = W.layer_kv(w, 0)
    qs = W.queries(w, 0, steps)
    host = LayerCache(g, cap, tier=B.SF_TIER_HOST_PINNED, max_seqs=1, cache_slots=2 * T)
    cuda = lambda x: torch.as_tensor(x, device="cuda")
    try:
        host.append(cuda(k), cuda(v), 0)
        oc = O.quantize_cache(k, v, w.base_bits, w.refine_bits)
        # the oracle's rows for the whole run, filled as tokens are appended
        kq = {f: np.zeros((hkv, cap) + getattr(oc.k, f).shape[2:], getattr(oc.k, f).dtype)
              for f in ("lo", "delta", "fine", "base", "refine")}
        vq = {f: np.zeros_like(a) for f, a in kq.items()}
        for f in kq:
            kq[f][:, :n0] = getattr(oc.k, f)
            vq[f][:, :n0] = getattr(oc.v, f)
        rows = lambda d, h, n, a=0: O.QuantRows(**{f: d[f][h, a:n] for f in d}, b=w.base_bits, r=w.refine_bits)
        kb = np.zeros((hkv, cap, w.head_dim))
        vb = np.zeros((hkv, cap, w.head_dim))
        for h in range(hkv):
            kb[h, :n0] = O.dequant_base(rows(kq, h, n0))
            vb[h, :n0] = O.dequant_base(rows(vq, h, n0))
        sims = [O.CacheSim(2 * T) for _ in range(hkv)]
        dec = Decoder(g, [0, n0 + 1], T)
        worst_out, differ = 0.0, 0
        for t in range(steps):
            n = n0 + t + 1
            ka, va = W.appended_kv(w, 0, t)
            kr, vr = host.append(cuda(ka), cuda(va), n - 1, keep_refine=True)
            oa = O.quantize_cache(ka, va, w.base_bits, w.refine_bits)
            for f in kq:
                kq[f][:, n - 1] = getattr(oa.k, f)[:, 0]
                vq[f][:, n - 1] = getattr(oa.v, f)[:, 0]
            assert np.array_equal(host.k_codes[:, n - 1].cpu().numpy(), O.pack_bits(oa.k.base[:, 0], w.base_bits))
            assert np.array_equal(host.v_codes[:, n - 1].cpu().numpy(), O.pack_bits(oa.v.base[:, 0], w.base_bits))
            ksc = host.k_scales[:, n - 1].cpu().numpy()
            assert np.array_equal(ksc[:, 0].view(np.uint32), oa.k.lo[:, 0].view(np.uint32))
            assert np.array_equal(ksc[:, 1].view(np.uint32), oa.k.delta[:, 0].view(np.uint32))
            assert np.array_equal(kr.cpu().numpy()[:, 0], O.pack_bits(oa.k.refine[:, 0], w.refine_bits))
            assert np.array_equal(vr.cpu().numpy()[:, 0], O.pack_bits(oa.v.refine[:, 0], w.refine_bits))
            for h in range(hkv):
                kb[h, n - 1] = O.dequant_base(rows(kq, h, n, n - 1))[0]
                vb[h, n - 1] = O.dequant_base(rows(vq, h, n, n - 1))[0]
            dec.set_offsets([0, n])
            sel = torch.full((1, hkv, T), -7, dtype=torch.int32, device="cuda")
            scores = torch.empty((hkv, n), dtype=torch.float32, device="cuda")
            out, st = dec.step(host, cuda(qs[t]), sel_out=sel, scores_out=scores, want_stats=True)
            out, sel, scores = out.cpu().numpy(), sel.cpu().numpy(), scores.cpu().numpy()
            hits = misses = 0
            for h in range(hkv):
                qg = qs[t][0, h * G:(h + 1) * G]
                s_or = O.token_scores(qg, kb[h, :n])
                tol = P.score_tolerance(qg, rows(kq, h, n))
                assert np.all(np.abs(scores[h].astype(np.float64) - s_or) <= tol), (t, h)
                same = P.check_selection(sel[0, h], scores[h], s_or, T)
                differ += 0 if same else 1
                chosen = sel[0, h, :min(T, n)].astype(np.int64)
                k_star, v_star = kb[h, :n].copy(), vb[h, :n].copy()
                k_star[chosen] = O.dequant_refined(O._take(rows(kq, h, n), chosen))
                v_star[chosen] = O.dequant_refined(O._take(rows(vq, h, n), chosen))
                ref = O.attend(qg, k_star, v_star)
                err = float(np.abs(out[0, h * G:(h + 1) * G] - ref).max())
                assert err <= P.OUT_ATOL, (t, h, err)
                worst_out = max(worst_out, err)
                hh, mm = sims[h].step(chosen, t)
                hits, misses = hits + hh, misses + mm
            assert (st["hits"], st["misses"]) == (hits, misses), (t, st, hits, misses)
            assert st["h2d_bytes"] == O.fetched_bytes(misses, w.head_dim, w.refine_bits)
            if t % 32 == 0 or t == steps - 1:
                print(f"step {t} n={n} {st} worst_out={worst_out:.2e} sel_differ={differ}", flush=True)
        assert B.sf_store_check(host.store) == B.SF_OK
    finally:
        host.close()


@pytest.mark.slow
def test_full_size_host_tier_128k():
    """The 128K layer with its refinement store in pinned host memory, as the
    long-context workload keeps it, over two AR(1) steps in the benchmark's
    launch configuration: outputs bit-identical to the device-resident store,
    hits and misses equal to the oracle's cache simulation."""
    import torch
    from selective_kv_cache_amd import binding as B
    from selective_kv_cache_amd.kvcache import Decoder, LayerCache
    w0 = W.WORKLOADS["llama8b_128k"]
    w = W.Workload(**{**w0.__dict__, "rho": 0.9})
    g = P.geom_of(w)
    n = w.ctx
    k, v = W.layer_kv(w, 0, device="cuda")
    qs = W.queries(w, 0, 2)
    dev = LayerCache(g, n, tier=B.SF_TIER_DEVICE)
    host = LayerCache(g, n, tier=B.SF_TIER_HOST_PINNED, max_seqs=1, cache_slots=2 * w.top_t)
    try:
        dev.append(k, v, 0)
        host.append(k, v, 0)
        del k, v
        dec = Decoder(g, W.seq_offsets([n]), w.top_t)
        sims = [O.CacheSim(2 * w.top_t) for _ in range(w.n_kv_heads)]
        sel = torch.empty((1, w.n_kv_heads, w.top_t), dtype=torch.int32, device="cuda")
        for t in range(qs.shape[0]):
            q = torch.as_tensor(qs[t], device="cuda")
            o_dev = dec.step(dev, q, multi_pass=True).cpu().numpy()
            o_host, st = dec.step(host, q, sel_out=sel, want_stats=True)
            assert np.array_equal(o_dev.view(np.uint32), o_host.cpu().numpy().view(np.uint32)), t
            s_np = sel.cpu().numpy()[0]
            hits = misses = 0
            for h in range(w.n_kv_heads):
                hh, mm = sims[h].step(s_np[h], t)
                hits, misses = hits + hh, misses + mm
            assert (st["hits"], st["misses"]) == (hits, misses), (t, st, hits, misses)
            assert st["h2d_bytes"] == O.fetched_bytes(misses, w.head_dim, w.refine_bits)
            print(t, st, flush=True)
    finally:
        dev.close()
        host.close()

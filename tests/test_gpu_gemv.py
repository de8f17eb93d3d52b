"""GPU parity of the weight-side refinement GEMV (sf_w_quantize, sf_w_gemv)
against the oracle (oracle/gemv_oracle.py): base codes, scales and the
column-major refinement codes bit-exact, the selected channels identical,
y within the fp32 accumulation bound below.

Tolerance: the kernel sums, per output row, at most 32 products per segment,
then at most K/32/64 + 6 partial sums per lane and across the wavefront, plus
the correction of the selected channels: a depth of at most 32 + 4 + 6 + 2
additions for K <= 15,360 (the correction adds per thread, 8 slots per row,
then 8 LDS atomics).  With unit roundoff u = 2^-24 the error of such a sum is
below (depth + 4) u times the sum of the magnitudes it adds, here bounded by
sum_j (|lo| + 2^b delta) |x_j| over the row's groups plus delta |x_c| over the
selected channels.  The test allows 1e-5 of that bound, about 3x the
worst-case figure for a depth of 48 and far above the typical error."""
import numpy as np
import pytest

import oracle.gemv_oracle as G
import oracle.kv_oracle as O
from selective_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu

REL = 1e-5


def _gpu_quantize(w_np, b, r, top_k, chunk):
    import torch
    from selective_kv_cache_amd import binding as B
    m, k = w_np.shape
    g = B.wgeom(m, k, b, r, top_k, chunk)
    dev = "cuda"
    t = dict(codes=torch.empty((m, k // 128, 16 * b), dtype=torch.uint8, device=dev),
             scales=torch.empty((m, k // 128, 2), dtype=torch.float32, device=dev),
             cols=torch.empty((k, m * r // 8), dtype=torch.uint8, device=dev))
    w = torch.as_tensor(w_np, device=dev)
    scratch = torch.empty(m * k * r // 8, dtype=torch.uint8, device=dev)
    B.sf_w_quantize(g, w, t["codes"], t["scales"], t["cols"], scratch)
    torch.cuda.synchronize()
    del w, scratch
    return g, t


def _workspace(g):
    import torch
    from selective_kv_cache_amd import binding as B
    return torch.zeros(B.sf_w_gemv_workspace_words(g), dtype=torch.int32, device="cuda")


def _gpu_gemv(g, t, x_np, ws=None):
    import torch
    from selective_kv_cache_amd import binding as B
    nchunks = (g.k + g.chunk - 1) // g.chunk
    kout = min(g.top_k, g.chunk)
    x = torch.as_tensor(x_np, device="cuda")
    y = torch.full((g.m,), float("nan"), dtype=torch.float32, device="cuda")
    sel = torch.full((max(nchunks * kout, 1),), -7, dtype=torch.int32, device="cuda")
    ws = _workspace(g) if ws is None else ws
    B.sf_w_gemv(g, t["codes"], t["scales"], t["cols"], x, y, sel, ws)
    torch.cuda.synchronize()
    assert int(ws[-1]) == 0, "a wait for the selection expired"
    return y.cpu().numpy(), sel.cpu().numpy()[:nchunks * kout]


def _check_codes(t, qw, rows, b, r):
    """Packed base codes, (lo, delta) and the refinement columns of `rows`."""
    q = qw.q
    m_s, ng, _ = q.base.shape
    k = ng * 128
    codes = t["codes"][rows].cpu().numpy() if rows is not None else t["codes"].cpu().numpy()
    scales = t["scales"][rows].cpu().numpy() if rows is not None else t["scales"].cpu().numpy()
    assert np.array_equal(codes, O.pack_bits(q.base, b)), "packed base codes"
    assert np.array_equal(scales[..., 0].view(np.uint32), q.lo.view(np.uint32)), "lo"
    assert np.array_equal(scales[..., 1].view(np.uint32), q.delta.view(np.uint32)), "delta"
    cols = t["cols"].cpu().numpy()                  # [k][m r / 8]
    if rows is None:
        rows = np.arange(cols.shape[1] * 8 // r)
    # row i's code in channel c's column: bits [i r, i r + r) of that column
    got = np.zeros((k, len(rows)), dtype=np.uint32)
    for j in range(r):
        bit = np.asarray(rows, dtype=np.int64) * r + j
        got |= ((cols[:, bit >> 3] >> (bit & 7).astype(np.uint8)) & 1).astype(np.uint32) << j
    assert np.array_equal(got, q.refine.reshape(m_s, k).T), "refinement columns"


def _check_gemv(y, sel, qw, x, b, top_k, chunk, rows=None):
    y_ref, sel_ref = G.gemv(qw, x, top_k, chunk)
    k = x.shape[0]
    kout = min(top_k, chunk)
    # selection: chunk by chunk, ascending, padded with -1 past a short last chunk
    want = np.full(((k + chunk - 1) // chunk) * kout, -1, dtype=np.int64)
    pos = 0
    for c, c0 in enumerate(range(0, k, chunk)):
        n = min(top_k, min(chunk, k - c0))
        want[c * kout:c * kout + n] = sel_ref[pos:pos + n]
        pos += n
    if kout:
        assert np.array_equal(sel.astype(np.int64), want), "selected channels"
    q = qw.q
    ax = np.abs(x.astype(np.float64)).reshape(-1, 128)
    mag = (np.abs(q.lo)[..., None] + np.ldexp(1.0, b) * q.delta[..., None]) * ax[None]
    bound = mag.reshape(mag.shape[0], -1).sum(1)
    if sel_ref.size:
        dl = q.delta.reshape(q.delta.shape[0], -1)[:, sel_ref // 128].astype(np.float64)
        bound += (dl * np.abs(x[sel_ref].astype(np.float64))).sum(1)
    yy = y if rows is None else y[rows]
    err = np.abs(yy.astype(np.float64) - y_ref)
    assert np.all(np.isfinite(yy)), "every row written"
    worst = float((err / bound).max())
    assert worst <= REL, f"relative-to-bound error {worst:.2e}"
    return worst


CASES = [
    # (m, k, b, r, top_k, chunk, n_outlier, ties)
    (96, 2688, 3, 4, 32, 1024, 8, 40),       # the page's k = 32 of 1,024 on 3-bit weights, ragged last chunk
    (64, 1024, 2, 3, 100, 1000, 4, 16),      # r straddles bytes; last chunk (24) shorter than top_k
    (32, 512, 4, 8, 0, 1024, 2, 0),          # nothing refined: the base product
    (128, 1280, 2, 1, 256, 256, 2, 0),       # everything refined
    (256, 4096, 4, 2, 7, 512, 16, 64),       # several chunks, many ties
    (32, 15360, 3, 4, 32, 1024, 24, 32),     # the largest k
    (64, 128, 2, 2, 3, 4096, 0, 5),          # one group, a chunk longer than k
]


@pytest.mark.parametrize("case", CASES, ids=[f"m{c[0]}k{c[1]}b{c[2]}r{c[3]}t{c[4]}c{c[5]}" for c in CASES])
def test_gemv_matches_oracle(case):
    m, k, b, r, top_k, chunk, n_out, ties = case
    print(f"gemv case {case}", flush=True)
    w = W.projection_weights(500 + m + k, m, k)
    x = W.projection_input(500 + k, k, n_outlier=n_out, ties=ties)
    qw = G.quantize_weights(w, b, r)
    g, t = _gpu_quantize(w, b, r, top_k, chunk)
    _check_codes(t, qw, None, b, r)
    y, sel = _gpu_gemv(g, t, x)
    worst = _check_gemv(y, sel, qw, x, b, top_k, chunk)
    print(f"worst error / bound {worst:.2e}", flush=True)


@pytest.mark.parametrize("bits", [(b, r) for b in (2, 3, 4) for r in range(1, 9)])
def test_gemv_every_width(bits):
    b, r = bits
    m, k = 64, 640
    w = W.projection_weights(600 + 10 * b + r, m, k)
    x = W.projection_input(600 + r, k, n_outlier=3, ties=6)
    qw = G.quantize_weights(w, b, r)
    g, t = _gpu_quantize(w, b, r, 20, 300)
    _check_codes(t, qw, None, b, r)
    y, sel = _gpu_gemv(g, t, x)
    _check_gemv(y, sel, qw, x, b, 20, 300)


def test_gemv_steps_reuse_the_quantized_weights():
    # the resident weights are quantized once; each step brings a new x and
    # refines its own channels
    m, k, b, r = 160, 2048, 3, 4
    w = W.projection_weights(700, m, k)
    qw = G.quantize_weights(w, b, r)
    g, t = _gpu_quantize(w, b, r, 32, 1024)
    ws = _workspace(g)            # one workspace for every step
    sels = []
    for step in range(4):
        x = W.projection_input(700, k, step=step, n_outlier=4)
        y, sel = _gpu_gemv(g, t, x, ws)
        _check_gemv(y, sel, qw, x, b, 32, 1024)
        sels.append(sel)
    assert not np.array_equal(sels[0], sels[1])


@pytest.mark.parametrize("name", sorted(W.PROJECTIONS))
def test_gemv_full_size_sampled_rows(name):
    # Llama-3.1-8B projection shapes at 3-bit weights, 4-bit refinements,
    # k = 32 of 1,024: selection in full, codes and y on 97 sampled rows
    # (the quantizer and the product are row-independent)
    m, k = W.PROJECTIONS[name]
    b, r, top_k, chunk = 3, 4, 32, 1024
    print(f"gemv full size {name} m={m} k={k}", flush=True)
    w = W.projection_weights(800, m, k)
    x = W.projection_input(800, k, n_outlier=12, ties=8)
    g, t = _gpu_quantize(w, b, r, top_k, chunk)
    y, sel = _gpu_gemv(g, t, x)
    rows = np.unique(np.concatenate([[0, 31, 32, m - 1], np.random.default_rng(5).choice(m, 93, replace=False)]))
    qw = G.quantize_weights(w[rows], b, r)
    _check_codes(t, qw, rows, b, r)
    worst = _check_gemv(y, sel, qw, x, b, top_k, chunk, rows=rows)
    print(f"worst error / bound {worst:.2e}", flush=True)


def test_gemv_argument_checks():
    import torch
    from selective_kv_cache_amd import binding as B
    g, t = _gpu_quantize(W.projection_weights(900, 32, 256), 2, 2, 4, 128)
    x = torch.zeros(256, device="cuda")
    y = torch.empty(32, device="cuda")
    sel = torch.empty(8, dtype=torch.int32, device="cuda")
    ws = torch.zeros(16, dtype=torch.int32, device="cuda")
    for bad in (B.wgeom(33, 256, 2, 2, 4, 128), B.wgeom(32, 200, 2, 2, 4, 128), B.wgeom(32, 256, 5, 2, 4, 128),
                B.wgeom(32, 256, 2, 9, 4, 128), B.wgeom(32, 256, 2, 2, 200, 128), B.wgeom(32, 256, 2, 2, 4, 0)):
        with pytest.raises(B.SfError):
            B.sf_w_gemv(bad, t["codes"], t["scales"], t["cols"], x, y, sel, ws)
    with pytest.raises(B.SfError):
        B.sf_w_gemv(B.wgeom(32, 15488, 2, 2, 4, 128), t["codes"], t["scales"], t["cols"], x, y, sel, ws)
    with pytest.raises(B.SfError):        # x not 16-byte aligned
        B.sf_w_gemv(g, t["codes"], t["scales"], t["cols"], x[1:], y, sel, ws)


def test_gemv_graph_replays_follow_new_inputs():
    # the call's epoch lives on the device: a captured call replayed with new
    # activations (copied into the captured buffer between replays, with
    # eager work and synchronization in between) selects and sums anew
    import torch
    from selective_kv_cache_amd import binding as B
    m, k, b, r, top_k, chunk = 192, 3072, 3, 4, 32, 1024
    w = W.projection_weights(950, m, k)
    qw = G.quantize_weights(w, b, r)
    g, t = _gpu_quantize(w, b, r, top_k, chunk)
    ws = _workspace(g)
    x = torch.zeros(k, device="cuda")
    y = torch.empty(m, device="cuda")
    sel = torch.empty(3 * top_k, dtype=torch.int32, device="cuda")
    x.copy_(torch.as_tensor(W.projection_input(950, k, step=99), device="cuda"))
    B.sf_w_gemv(g, t["codes"], t["scales"], t["cols"], x, y, sel, ws)     # eager warm-up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            B.sf_w_gemv(g, t["codes"], t["scales"], t["cols"], x, y, sel, ws, stream=s)
    torch.cuda.synchronize()
    for step in range(4):
        xn = W.projection_input(950, k, step=step, n_outlier=3)
        x.copy_(torch.as_tensor(xn, device="cuda"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(ws[-1]) == 0
        _check_gemv(y.cpu().numpy(), sel.cpu().numpy(), qw, xn, b, top_k, chunk)
        # an eager call between replays shares the workspace
        y2, sel2 = _gpu_gemv(g, t, xn, ws)
        assert np.array_equal(sel2, sel.cpu().numpy()) and np.array_equal(y2, y.cpu().numpy())

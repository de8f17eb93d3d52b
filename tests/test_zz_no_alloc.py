"""sf_decode_step_noalloc (the decode step on the library's own device scratch,
for callers that cannot allocate) against sf_decode_step with a workspace of
its own: same inputs, bit-identical outputs, selections and scores, on two
calls in a row, the second with a smaller input; a step needing more scratch
than the library holds is refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest

import parity as P
from selective_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu


def _step_both(w, lens, cfg_layer=0):
    import torch
    from selective_kv_cache_amd import binding as B
    from selective_kv_cache_amd.kvcache import Decoder, LayerCache
    g = P.geom_of(w)
    off = W.seq_offsets(lens)
    n = int(off[-1])
    k, v = W.layer_kv(w, cfg_layer, n_tok=n)
    q = torch.as_tensor(W.query(w, cfg_layer), device="cuda")
    cache = LayerCache(g, n, tier=B.SF_TIER_DEVICE)
    try:
        cache.append(torch.as_tensor(k, device="cuda"), torch.as_tensor(v, device="cuda"), 0)
        dec = Decoder(g, off, w.top_t)
        res = []
        for noalloc in (False, True):
            out = torch.full((len(lens), w.n_q_heads, w.head_dim), float("nan"), device="cuda")
            sel = torch.full((len(lens), w.n_kv_heads, w.top_t), -7, dtype=torch.int32, device="cuda")
            scores = torch.full((w.n_kv_heads, n), float("nan"), device="cuda")
            B.sf_decode_step(g, seq_off_host=dec.seq_off, seq_off_dev=dec.seq_off_dev, q=q,
                             k_codes=cache.k_codes, k_scales=cache.k_scales, v_codes=cache.v_codes,
                             v_scales=cache.v_scales, cap=cache.cap, store=cache.store, top_t=w.top_t, out=out,
                             workspace=None if noalloc else dec.workspace, sel_out=sel, scores_out=scores,
                             noalloc=noalloc)
            torch.cuda.synchronize()
            res.append((out.cpu().numpy(), sel.cpu().numpy(), scores.cpu().numpy()))
        (o0, s0, c0), (o1, s1, c1) = res
        print(f"{w.name} lens={lens}: max |noalloc - workspace| = {np.abs(o1 - o0).max()}", flush=True)
        assert np.array_equal(o0.view(np.uint32), o1.view(np.uint32))
        assert np.array_equal(s0, s1)
        assert np.array_equal(c0.view(np.uint32), c1.view(np.uint32))
        # and both within the oracle's bar
        run = P.GpuRun(out=o1, sel=s1, scores=c1, k_codes=None, v_codes=None, k_scales=None, v_scales=None,
                       k_ref=None, v_ref=None)
        P.compare_layer(w, k, v, W.query(w, cfg_layer), off, w.top_t, run, codec=False)
    finally:
        cache.close()


def test_noalloc_matches_workspace_step_twice_second_smaller():
    big = W.small("noalloc_big", cfg_id=400, batch=2, n_q_heads=8, n_kv_heads=2, refine_bits=4, top_t=100)
    _step_both(big, [3000, 1200])
    small = W.small("noalloc_small", cfg_id=401, batch=1, n_q_heads=4, n_kv_heads=1, refine_bits=2, top_t=40)
    _step_both(small, [700])


def test_noalloc_refuses_steps_beyond_its_scratch():
    import torch
    from selective_kv_cache_amd import binding as B
    g = B.geom(128, 32, 8, 2, 4)
    n = 400_000                                              # needs more than the scratch holds
    need = B.sf_decode_workspace_size(g, 1, n, n, 0)
    assert need > B.sf_decode_noalloc_max_bytes()
    off = np.asarray([0, n], dtype=np.int64)
    off_dev = torch.as_tensor(off, device="cuda")
    out = torch.full((1, 32, 128), 3.0, device="cuda")
    dummy = torch.zeros(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.SfError) as ei:
        B.sf_decode_step(g, seq_off_host=off, seq_off_dev=off_dev, q=dummy, k_codes=dummy, k_scales=dummy,
                         v_codes=dummy, v_scales=dummy, cap=n, store=None, top_t=0, out=out, workspace=None,
                         noalloc=True)
    assert ei.value.status == B.SF_ERR_UNSUPPORTED
    assert "scratch" in B.load().sf_last_error_string().decode()
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())

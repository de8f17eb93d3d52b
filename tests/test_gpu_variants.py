"""GPU parity of the decode step's comparison variants against the oracle's
(oracle/kv_variants.py): unselected tokens left out, the selection's 16-bit
rows (and both: sparse attention), the score by the attention a token
receives, and fp16 scale storage.  Outputs within 2e-3 max abs; codes and
scales bit-exact; selections equal or differing only near the T-th score."""
import numpy as np
import pytest

import oracle.kv_oracle as O
import oracle.kv_variants as V
import parity as P
from selective_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu


def _run(w, k, v, q, off, t, variant=0, fp16_scales=False, rows16=False):
    from selective_kv_cache_amd import binding as B
    import torch
    from selective_kv_cache_amd.kvcache import Decoder, LayerCache
    g = P.geom_of(w)
    ntot = int(off[-1])
    cache = LayerCache(g, ntot, fp16_scales=fp16_scales, rows16=rows16)
    try:
        cache.append(torch.as_tensor(k, device="cuda"), torch.as_tensor(v, device="cuda"), 0)
        dec = Decoder(g, off, t)
        sel = torch.full((dec.batch, w.n_kv_heads, t), -7, dtype=torch.int32, device="cuda")
        scores = torch.empty((w.n_kv_heads, ntot), dtype=torch.float32, device="cuda")
        out = dec.step(cache, torch.as_tensor(q, device="cuda"), sel_out=sel, scores_out=scores, variant=variant)
        torch.cuda.synchronize()
        assert dec.check() == B.SF_OK
        form = B.sf_decode_form(g, off, t, cache.store, variant)
        return dict(out=out.cpu().numpy(), sel=sel.cpu().numpy(), scores=scores.cpu().numpy(),
                    k_codes=cache.k_codes.cpu().numpy(), k_scales=cache.k_scales.cpu().numpy(),
                    v_codes=cache.v_codes.cpu().numpy(), v_scales=cache.v_scales.cpu().numpy(), form=form)
    finally:
        cache.close()


def _compare(w, k, v, q, off, t, run, score="max", drop=False, rows16=False, oc=None):
    """Every (sequence, KV head): scores, selection, output against the
    oracle variant (on the GPU's selection when it differs near a tie)."""
    oc = oc or O.quantize_cache(k, v, w.base_bits, w.refine_bits)
    g = w.group
    worst = 0.0
    for s in range(len(off) - 1):
        a, e = int(off[s]), int(off[s + 1])
        for h in range(w.n_kv_heads):
            qg = q[s, h * g:(h + 1) * g]
            kc, vc = O._rows(oc.k, h, a, e), O._rows(oc.v, h, a, e)
            k16 = k[a:e, h] if rows16 else None
            v16 = v[a:e, h] if rows16 else None
            ref = V.decode_head_variant(qg, kc, vc, t, score=score, drop=drop, k16=k16, v16=v16)
            gs = run["scores"][h, a - int(off[0]):e - int(off[0])].astype(np.float64)
            if score == "softmax_sum":
                assert np.all(np.abs(gs - ref.scores) <= 1e-4 * ref.scores + 1e-9), "summed-probability scores"
            else:
                tol = P.score_tolerance(qg, kc)
                assert np.all(np.abs(gs - ref.scores) <= tol), "scores"
            tn = min(t, e - a)
            got = run["sel"][s, h, :tn]
            if not np.array_equal(got, ref.sel):
                # valid only as the top-T of the GPU's own scores, differing near the T-th
                assert np.array_equal(got, O.select_top_t(gs, t))
                s_t = np.sort(ref.scores)[::-1][tn - 1]
                diff = np.setxor1d(got, ref.sel)
                assert np.all(np.abs(ref.scores[diff] - s_t) <= 1e-4 * abs(s_t)), diff[:8]
                ref = _on_selection(qg, kc, vc, got, drop, k16, v16)
            err = float(np.abs(run["out"][s, h * g:(h + 1) * g].astype(np.float64) - ref.out).max())
            assert err <= P.OUT_ATOL, f"output error {err} at {(s, h)}"
            worst = max(worst, err)
    return worst


def _on_selection(qg, kc, vc, sel, drop, k16, v16):
    k_star, v_star = O.dequant_base(kc), O.dequant_base(vc)
    if k16 is not None:
        k_star[sel], v_star[sel] = V.rows_fp16(k16[sel]), V.rows_fp16(v16[sel])
    else:
        k_star[sel] = O.dequant_refined(O._take(kc, sel))
        v_star[sel] = O.dequant_refined(O._take(vc, sel))
    if drop:
        k_star, v_star = k_star[sel], v_star[sel]
    return O.HeadResult(scores=None, sel=sel, out=O.attend(qg, k_star, v_star))


CASES = [
    dict(ctx=3000, n_q_heads=8, n_kv_heads=2, top_t=100),                 # G = 4, ragged tail
    dict(ctx=1100, n_q_heads=2, n_kv_heads=2, top_t=37, refine_bits=4),   # G = 1
    dict(batch=3, ctx=0, ctx_range=(300, 900), n_q_heads=4, n_kv_heads=2, top_t=50),   # varlen batch, G = 2
    dict(ctx=2500, n_q_heads=8, n_kv_heads=2, top_t=80, base_bits=3, refine_bits=2),   # 3-bit base codes
    dict(ctx=1700, n_q_heads=4, n_kv_heads=2, top_t=60, base_bits=4, refine_bits=4),   # 4-bit base codes
]


def _inputs(i):
    w = W.small(cfg_id=400 + i, **CASES[i])
    off = W.seq_offsets(w.seq_lengths())
    k, v = W.layer_kv(w, 0, n_tok=int(off[-1]))
    q = W.query(w, 0)
    return w, k, v, q, off


@pytest.mark.parametrize("i", range(len(CASES)))
@pytest.mark.parametrize("name", ["drop", "rows16", "sparse", "softmax_score", "softmax_drop"])
def test_variant_matches_oracle(name, i):
    from selective_kv_cache_amd import binding as B
    w, k, v, q, off = _inputs(i)
    t = w.top_t
    flags = {"drop": B.SF_DECODE_DROP_UNSELECTED, "rows16": B.SF_DECODE_ROWS16,
             "sparse": B.SF_DECODE_DROP_UNSELECTED | B.SF_DECODE_ROWS16,
             "softmax_score": B.SF_DECODE_SCORE_SOFTMAX,
             "softmax_drop": B.SF_DECODE_SCORE_SOFTMAX | B.SF_DECODE_DROP_UNSELECTED}[name]
    rows16 = bool(flags & B.SF_DECODE_ROWS16)
    print(f"variant {name} case {CASES[i]}", flush=True)
    run = _run(w, k, v, q, off, t, variant=flags, rows16=rows16)
    assert run["form"] == 5
    worst = _compare(w, k, v, q, off, t, run, score="softmax_sum" if flags & B.SF_DECODE_SCORE_SOFTMAX else "max",
                     drop=bool(flags & B.SF_DECODE_DROP_UNSELECTED), rows16=rows16)
    print(f"max output error {worst:.2e}", flush=True)


def test_softmax_score_selects_differently_from_max():
    # the summed-probability score is not the max logit in disguise: on this
    # layer the two selections differ (and each matches its oracle)
    from selective_kv_cache_amd import binding as B
    w, k, v, q, off = _inputs(0)
    a = _run(w, k, v, q, off, w.top_t)
    b = _run(w, k, v, q, off, w.top_t, variant=B.SF_DECODE_SCORE_SOFTMAX)
    assert not np.array_equal(a["sel"], b["sel"])


@pytest.mark.parametrize("bits", [(2, 2), (2, 4), (3, 2)])
def test_fp16_scales_codec_and_step(bits):
    b, r = bits
    w = W.small(cfg_id=410, ctx=2000, n_q_heads=8, n_kv_heads=2, top_t=64, base_bits=b, refine_bits=r)
    off = W.seq_offsets(w.seq_lengths())
    k, v = W.layer_kv(w, 0, n_tok=int(off[-1]))
    q = W.query(w, 0)
    run = _run(w, k, v, q, off, w.top_t, fp16_scales=True)
    kq = V.quantize_rows_fp16_scales(np.swapaxes(k, 0, 1), b, r)
    vq = V.quantize_rows_fp16_scales(np.swapaxes(v, 0, 1), b, r)
    n = int(off[-1])
    for gpu_codes, gpu_scales, qr in ((run["k_codes"], run["k_scales"], kq), (run["v_codes"], run["v_scales"], vq)):
        assert np.array_equal(gpu_codes[:, :n], O.pack_bits(qr.base, b)), "packed base codes"
        assert np.array_equal(gpu_scales[:, :n, 0].view(np.uint32), qr.lo.view(np.uint32)), "lo"
        assert np.array_equal(gpu_scales[:, :n, 1].view(np.uint32), qr.delta.view(np.uint32)), "delta"
    _compare(w, k, v, q, off, w.top_t, run, oc=O.QuantCache(kq, vq))


def test_variant_argument_checks():
    from selective_kv_cache_amd import binding as B
    w, k, v, q, off = _inputs(0)
    # 16-bit rows without the rows, and dropping with nothing selected, are refused
    with pytest.raises(B.SfError):
        _run(w, k, v, q, off, w.top_t, variant=B.SF_DECODE_ROWS16, rows16=False)
    with pytest.raises(B.SfError):
        _run(w, k, v, q, off, 0, variant=B.SF_DECODE_DROP_UNSELECTED)

"""Pins of the oracle's variants (score by the attention a token receives,
16-bit rows, unselected tokens left out, KL of the attention, fp16 scales)
against hand-derived values, closed forms and a library attention routine;
planted mistakes in the variants must fail some pin."""
import json
import math
import os

import numpy as np
import pytest

import oracle.kv_oracle as O
import oracle.kv_variants as V

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _sdpa(q, k, v):
    import torch
    qt = torch.as_tensor(np.asarray(q, np.float64))[None]
    kt = torch.as_tensor(np.asarray(k, np.float64))[None]
    vt = torch.as_tensor(np.asarray(v, np.float64))[None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0].numpy()


def _softmax_torch(logits):
    import torch
    return torch.softmax(torch.as_tensor(np.asarray(logits, np.float64)), dim=-1).numpy()


def _fp16_exact_rows(seed, n, d):
    # multiples of 1/8 in [-4, 4): exact in fp16, so a 16-bit row is the row
    rng = np.random.default_rng(seed)
    return (rng.integers(-32, 32, size=(n, d)) / 8.0).astype(np.float32)


# --------------------------------------------------------------------- pins

def pin_softmax_sum_toy():
    g = _golden("softmax_sum_toy.json")
    q = np.asarray(g["q"], np.float32)
    k = np.asarray(g["k"], np.float64)
    np.testing.assert_allclose(V.token_scores_softmax_sum(q, k), g["softmax_sum"], rtol=0, atol=1e-7)
    np.testing.assert_allclose(O.token_scores(q, k), g["max_logit"], rtol=0, atol=1e-7)
    for t, want in g["select_softmax_sum"].items():
        assert O.select_top_t(V.token_scores_softmax_sum(q, k), int(t)).tolist() == want
    for t, want in g["select_max"].items():
        assert O.select_top_t(O.token_scores(q, k), int(t)).tolist() == want


def pin_softmax_sum_library_and_invariants():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((4, 16)).astype(np.float32)
    k = rng.standard_normal((50, 16))
    s = V.token_scores_softmax_sum(q, k)
    want = _softmax_torch(q.astype(np.float64) @ k.T / 4.0).sum(axis=0)
    np.testing.assert_allclose(s, want, rtol=1e-12, atol=0)
    assert abs(s.sum() - 4.0) < 1e-12                        # each head's probabilities sum to 1
    # one query head: the probability is monotone in the logit, so the
    # selection is the max-logit score's
    s1 = V.token_scores_softmax_sum(q[:1], k)
    assert np.array_equal(O.select_top_t(s1, 7), O.select_top_t(O.token_scores(q[:1], k), 7))


def pin_fp16_rows():
    g = _golden("fp16_scales_toy.json")
    assert float(V.rows_fp16(np.float32(0.7))) == g["fp16_of_0_7"]
    x = _fp16_exact_rows(5, 4, 8)
    assert np.array_equal(V.rows_fp16(x), x.astype(np.float64))


def pin_fp16_scales_toy():
    g = _golden("fp16_scales_toy.json")
    qr = V.quantize_rows_fp16_scales(np.asarray(g["x"], np.float32), g["b"], g["r"])
    assert qr.lo.tolist() == g["lo"] and qr.delta.tolist() == g["delta"]
    assert qr.fine.tolist() == g["fine"]
    assert qr.base.tolist() == g["base"] and qr.refine.tolist() == g["refine"]


def pin_fp16_scales_bounds():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((400, 128)).astype(np.float32)
    x[:, [3, 50, 99]] *= 8
    for b, r in ((2, 2), (2, 4), (3, 2)):
        qr = V.quantize_rows_fp16_scales(x, b, r)
        lo, d = qr.lo, qr.delta
        assert np.array_equal(lo.astype(np.float16).astype(np.float32), lo)       # fp16 values
        assert np.array_equal(d.astype(np.float16).astype(np.float32), d)
        assert np.all(lo <= x.min(axis=1))                                       # range covered
        assert np.all(lo.astype(np.float64) + d.astype(np.float64) * 2 ** b >= x.max(axis=1) * (1 - 2e-7))
        assert qr.fine.max() <= 2 ** (b + r) - 1
        assert np.array_equal(qr.base, qr.fine >> r)
        err = np.abs(O.dequant_refined(qr) - x.astype(np.float64))
        sub = d.astype(np.float64)[:, None] / 2 ** r
        assert np.all(err <= sub * (0.5 + 1e-5) + 1e-6)                          # within half a sub-bin


def pin_kl_closed_forms():
    assert abs(V.kl_divergence([0.5, 0.5], [0.25, 0.75]) - 0.5 * math.log(4 / 3)) < 1e-15
    assert abs(V.kl_divergence([1.0, 0.0], [0.5, 0.5]) - math.log(2)) < 1e-15
    p = np.asarray([0.1, 0.2, 0.7])
    assert V.kl_divergence(p, p) == 0.0


def pin_drop_and_fetch16_library():
    # fp16-exact rows: the 16-bit entries are the rows themselves
    k = _fp16_exact_rows(21, 40, 8)
    v = _fp16_exact_rows(22, 40, 8)
    q = np.random.default_rng(23).standard_normal((2, 8)).astype(np.float32)
    kc, vc = O.quantize_rows(k, 2, 2), O.quantize_rows(v, 2, 2)
    # every token fetched at 16 bits: textbook attention over the rows
    full = V.decode_head_variant(q, kc, vc, 40, k16=k, v16=v)
    np.testing.assert_allclose(full.out, _sdpa(q, k, v), rtol=0, atol=1e-12)
    # 16-bit rows of the selection, the others left out: attention over the
    # selected rows alone
    res = V.decode_head_variant(q, kc, vc, 9, drop=True, k16=k, v16=v)
    sel = res.sel
    assert sel.size == 9
    np.testing.assert_allclose(res.out, _sdpa(q, k[sel], v[sel]), rtol=0, atol=1e-12)
    # the others at base precision: the base rows for them
    mixed = V.decode_head_variant(q, kc, vc, 9, k16=k, v16=v)
    kb, vb = O.dequant_base(kc), O.dequant_base(vc)
    kb[sel], vb[sel] = k[sel], v[sel]
    np.testing.assert_allclose(mixed.out, _sdpa(q, kb, vb), rtol=0, atol=1e-12)


def pin_sparse_kl_closed_form():
    # exact rows left alone on the selection: p_sparse = p_full restricted and
    # renormalised, so KL(sparse || full) = -ln(p_full(S))
    k = _fp16_exact_rows(31, 64, 8)
    q = np.random.default_rng(32).standard_normal((1, 8)).astype(np.float32)
    p_full = V.attention_probs(q, k.astype(np.float64))
    sel = np.asarray([1, 5, 9, 20, 33])
    p_sparse = V.attention_probs(q, k.astype(np.float64), keep=sel)
    assert abs(V.kl_divergence(p_sparse, p_full)[0] + math.log(p_full[0, sel].sum())) < 1e-12


def pin_study_limits():
    rng = np.random.default_rng(41)
    k = rng.standard_normal((256, 128)).astype(np.float32)
    q = rng.standard_normal((4, 128)).astype(np.float32)
    res = V.study_head(q, k, 2, 4, 256)          # every token refined, 64 16-bit rows
    for m in res.values():
        assert m >= 0.0
    # nested refinement of every token at 14 bits is near full precision;
    # more refined tokens never hurt here
    fine = V.study_head(q, k, 2, 12, 256)["nested"]
    assert fine < 1e-7
    assert V.study_head(q, k, 2, 4, 32)["nested"] >= res["nested"]
    assert V.matched_rows(2048, 4) == 512 and V.matched_rows(2048, 8) == 1024
    # a budget of 256 16-bit rows keeps every token: sparse attention is then
    # SpeCache with every token fetched
    both = V.study_head(q, k, 2, 8, 512)
    assert abs(both["sparse"] - both["fetch16"]) < 1e-15


PINS = [pin_softmax_sum_toy, pin_softmax_sum_library_and_invariants, pin_fp16_rows, pin_fp16_scales_toy,
        pin_fp16_scales_bounds, pin_kl_closed_forms, pin_drop_and_fetch16_library, pin_sparse_kl_closed_form,
        pin_study_limits]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


def _fails_some_pin():
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            return True
    return False


# planted mistakes (on the CPU): each must make some pin fail

def _mut_softmax_unnormalised(q, k):
    qg = np.asarray(q, np.float64)
    lg = qg @ np.asarray(k, np.float64).T / np.sqrt(qg.shape[-1])
    return np.exp(lg - lg.max(axis=1, keepdims=True)).sum(axis=0)


def _mut_softmax_sum_of_logits(q, k):
    qg = np.asarray(q, np.float64)
    return (qg @ np.asarray(k, np.float64).T / np.sqrt(qg.shape[-1])).sum(axis=0)


def _mut_fp16_truncate(x):
    x = np.asarray(x, np.float32)
    h = x.astype(np.float16)
    down = np.where(h.astype(np.float32) > x, np.nextafter(h, np.float16(-np.inf)), h)
    return down.astype(np.float64)


_orig_variant = V.decode_head_variant


def _mut_drop_ignored(q, kc, vc, t, score="max", drop=False, k16=None, v16=None):
    return _orig_variant(q, kc, vc, t, score=score, drop=False, k16=k16, v16=v16)


def _mut_kl_swapped(p, q):
    p, q = np.asarray(p, np.float64), np.asarray(q, np.float64)
    return np.where(q > 0, q * (np.log(np.where(q > 0, q, 1)) - np.log(np.where(q > 0, p, 1))), 0).sum(axis=-1)


def _mut_fp16_lo_nearest(x, b, r):
    x = np.asarray(x, np.float32)
    f = b + r
    lo = x.min(axis=-1).astype(np.float16).astype(np.float32)
    rng = (x.max(axis=-1) - lo).astype(np.float32)
    d = V._fp16_up((rng * np.float32(2.0 ** -b)).astype(np.float32))
    u = (x - lo[..., None]) / (d * np.float32(2.0 ** -r))[..., None]
    fine = np.clip(np.floor(u), 0, 2 ** f - 1).astype(np.uint16)
    return O.QuantRows(lo=lo, delta=d, fine=fine, base=(fine >> r).astype(np.uint16),
                       refine=(fine & ((1 << r) - 1)).astype(np.uint16), b=b, r=r)


def _mut_matched_rows_k_only(t, r):
    return (t * r) // 8


MUTATIONS = [
    ("token_scores_softmax_sum", _mut_softmax_unnormalised),
    ("token_scores_softmax_sum", _mut_softmax_sum_of_logits),
    ("rows_fp16", _mut_fp16_truncate),
    ("decode_head_variant", _mut_drop_ignored),
    ("kl_divergence", _mut_kl_swapped),
    ("quantize_rows_fp16_scales", _mut_fp16_lo_nearest),
    ("matched_rows", _mut_matched_rows_k_only),
]


@pytest.mark.parametrize("name,fn", MUTATIONS, ids=[f"{n}:{f.__name__}" for n, f in MUTATIONS])
def test_pins_catch_planted_mistakes(monkeypatch, name, fn):
    monkeypatch.setattr(V, name, fn)
    assert _fails_some_pin(), f"no pin failed with {fn.__name__} planted in {name}"


def test_accuracy_study_runs_small():
    # the study script at a small size: every KL is finite and >= 0, and
    # refining T tokens improves on the base-only cache
    import dataclasses
    import accuracy_study as S
    from selective_kv_cache_amd import workloads as W
    w = dataclasses.replace(W.WORKLOADS["llama8b_32k"], top_t=64)
    res = S.study(w, 4, layers=(0,), heads=(0, 1), n_tok=4096)
    assert all(np.isfinite(v) and v >= 0 for v in res.values())
    assert res["nested"] < res["base_only"]

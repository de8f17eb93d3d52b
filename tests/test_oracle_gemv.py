"""Pins of the weight-side refinement GEMV oracle (oracle/gemv_oracle.py):
the page's worked example, library products at the two ends of the refined
share, brute-force channel selection, the closed-form error bound; planted
mistakes must fail some pin."""
import json
import os

import numpy as np
import pytest

import oracle.gemv_oracle as GO
import oracle.kv_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _weights(seed, m, k):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((m, k)).astype(np.float32) * np.float32(0.02)
    w[:, rng.choice(k, size=k // 64, replace=False)] *= np.float32(6.0)    # outlier input channels
    x = rng.standard_normal(k).astype(np.float32)
    x[rng.choice(k, size=k // 32, replace=False)] *= np.float32(10.0)     # large activations
    return w, x


def pin_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "gemv_worked_example.json")))
    got = GO.bits_per_weight(g["k_top"], g["chunk"], g["refine_bits"], g["base_bits"])
    assert got["share"] == g["share"] and round(got["share"], 3) == g["share_printed"]
    assert got["extra_bits"] == g["extra_bits"] and got["touched_bits"] == g["touched_bits"]
    assert got["bf16_over_payload"] == g["bf16_over_payload"]
    # a shorter last chunk: 2,048 + 512 channels, k = 32 each -> 96 / 2,560
    assert GO.bits_per_weight(32, 1024, 4, 3, k_in=2560)["share"] == 96 / 2560


def pin_selection_bruteforce():
    x = np.asarray([0.5, -2.0, 2.0, 1.0, -1.0, 0.1, 3.0, -3.0, 0.2], np.float32)
    # chunks of 4: |x| = (.5 2 2 1), (1 .1 3 3), (.2); ties to the lower index
    assert GO.select_channels(x, 2, chunk=4).tolist() == [1, 2, 6, 7, 8]
    assert GO.select_channels(x, 1, chunk=4).tolist() == [1, 6, 8]
    rng = np.random.default_rng(2)
    y = rng.standard_normal(300).astype(np.float32)
    got = GO.select_channels(y, 5, chunk=100)
    for c0 in (0, 100, 200):
        seg = np.abs(y[c0:c0 + 100])
        want = sorted(range(c0, c0 + 100), key=lambda i: (-abs(float(y[i])), i))[:5]
        assert got[(c0 // 100) * 5:(c0 // 100) * 5 + 5].tolist() == sorted(want)
        assert seg.max() == abs(y[got[(c0 // 100) * 5:(c0 // 100) * 5 + 5]]).max()


def pin_ends_are_library_products():
    w, x = _weights(3, 64, 2048)
    qw = GO.quantize_weights(w, 3, 4)
    # the groups are kv_oracle's rows of 128
    ref = O.quantize_rows(w.reshape(64, 16, 128), 3, 4)
    wb, wr = O.dequant_base(ref).reshape(64, 2048), O.dequant_refined(ref).reshape(64, 2048)
    x64 = x.astype(np.float64)
    y0, s0 = GO.gemv(qw, x, 0)
    assert s0.size == 0 and np.allclose(y0, wb @ x64, rtol=1e-12, atol=1e-12)
    y1, s1 = GO.gemv(qw, x, 1024)
    assert s1.size == 2048 and np.allclose(y1, wr @ x64, rtol=1e-12, atol=1e-12)
    # in between: exactly the selected columns refined
    y, s = GO.gemv(qw, x, 32)
    wm = wb.copy()
    wm[:, s] = wr[:, s]
    assert np.allclose(y, wm @ x64, rtol=1e-12, atol=1e-12)


def pin_error_bound():
    w, x = _weights(5, 32, 4096)
    b, r = 3, 4
    qw = GO.quantize_weights(w, b, r)
    x64 = x.astype(np.float64)
    exact = w.astype(np.float64) @ x64
    d = np.repeat(qw.q.delta.astype(np.float64), 128, axis=1)          # [M][K] group deltas
    for kt in (0, 32, 256):
        y, sel = GO.gemv(qw, x, kt)
        half = d / 2.0
        half[:, sel] = d[:, sel] / 2 ** (r + 1)
        bound = (half * np.abs(x64)[None, :]).sum(axis=1)
        assert np.all(np.abs(y - exact) <= bound * (1 + 1e-6) + 1e-9)
    # refining the largest activations shrinks the bound most
    y32, sel32 = GO.gemv(qw, x, 32)
    rng = np.random.default_rng(6)
    other = np.sort(np.concatenate([rng.choice(np.arange(c, c + 1024), 32, replace=False) for c in range(0, 4096, 1024)]))
    gain = lambda s: (d[:, s] * (0.5 - 2.0 ** -(r + 1)) * np.abs(x64[s])[None, :]).sum()
    assert gain(sel32) >= gain(other)


PINS = [pin_worked_example, pin_selection_bruteforce, pin_ends_are_library_products, pin_error_bound]


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


def _mut_select_high_index(x, k_top, chunk=1024):
    a = np.abs(np.asarray(x, np.float32)).astype(np.float64)
    out = []
    for c0 in range(0, a.shape[0], chunk):
        seg = a[c0:c0 + chunk]
        order = np.lexsort((-np.arange(seg.shape[0]), -seg))
        out.append(np.sort(order[:min(k_top, seg.shape[0])]) + c0)
    return np.concatenate(out).astype(np.int64)


def _mut_select_smallest(x, k_top, chunk=1024):
    a = np.abs(np.asarray(x, np.float32))
    out = []
    for c0 in range(0, a.shape[0], chunk):
        out.append(np.sort(np.argsort(a[c0:c0 + chunk], kind="stable")[:k_top]) + c0)
    return np.concatenate(out).astype(np.int64)


_orig_gemv = GO.gemv


def _mut_gemv_refine_all(qw, x, k_top, chunk=1024):
    y, sel = _orig_gemv(qw, x, chunk, chunk)
    return y, GO.select_channels(x, k_top, chunk)


def _mut_bits_no_r(k_top, chunk, r, b, k_in=None):
    share = k_top / chunk
    return {"share": share, "extra_bits": share, "touched_bits": b + share, "bf16_over_payload": 16.0 / share}


def _mut_dequant_swapped(qw, refined):
    x = O.dequant_base(qw.q) if refined else O.dequant_refined(qw.q)
    return x.reshape(x.shape[0], -1)


MUTATIONS = [("select_channels", _mut_select_high_index), ("select_channels", _mut_select_smallest),
             ("gemv", _mut_gemv_refine_all), ("bits_per_weight", _mut_bits_no_r),
             ("dequant_weights", _mut_dequant_swapped)]


@pytest.mark.parametrize("name,fn", MUTATIONS, ids=[f"{n}:{f.__name__}" for n, f in MUTATIONS])
def test_pins_catch_planted_mistakes(monkeypatch, name, fn):
    monkeypatch.setattr(GO, name, fn)
    assert _fails_some_pin(), f"no pin failed with {fn.__name__} planted in {name}"

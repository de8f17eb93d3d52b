"""Accuracy study at matched key-plus-value bit budgets (page "StrataFlux --
Selective precision streaming -- What does it mean?", paragraph "What travels
over the link ..." and the comparison table): KL(approx || full precision)
of the attention distribution for nested refinement with r = 4 or 8 extra
bits on T tokens, against fetching complete 16-bit rows for T r / 16 tokens
(the others at base precision, "SpeCache") and against sparse attention on
those T r / 16 tokens (the others left out), on the synthetic caches of the
32K and 128K workloads.  Uses the oracle (oracle/kv_variants.py), whose
variants the GPU flags match (tests/test_gpu_variants.py).

    python tests/accuracy_study.py            # prints a markdown table
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle.kv_variants as V  # noqa: E402
from selective_kv_cache_amd import workloads as W  # noqa: E402

METHODS = ("base_only", "nested", "fetch16", "sparse")


def study(w: W.Workload, r: int, layers=(0, 1), heads=None, n_tok=None):
    """Mean KL per method over the given layers and KV heads of workload w
    (base bits w.base_bits, T = w.top_t nested tokens, r extra bits)."""
    n = n_tok or w.seq_lengths()[0]
    g = w.group
    acc = {m: [] for m in METHODS}
    for layer in layers:
        k, _ = W.layer_kv(w, layer, n_tok=n)
        q = W.query(w, layer)
        for h in (heads if heads is not None else range(w.n_kv_heads)):
            res = V.study_head(q[0, h * g:(h + 1) * g], k[:, h], w.base_bits, r, w.top_t)
            for m in METHODS:
                acc[m].append(res[m])
    return {m: float(np.mean(v)) for m, v in acc.items()}


def main():
    rows = []
    for name in ("llama8b_32k", "llama8b_128k"):
        w = W.WORKLOADS[name]
        for r in (4, 8):
            res = study(w, r)
            rows.append((name, w.seq_lengths()[0], w.top_t, r, V.matched_rows(w.top_t, r), res))
    print("| workload | tokens | T nested | r | T 16-bit | base only | nested | 16-bit rows (SpeCache) | sparse |")
    print("|---|---|---|---|---|---|---|---|---|")
    for name, n, t, r, t16, res in rows:
        print(f"| {name} | {n} | {t} | {r} | {t16} | {res['base_only']:.3e} | {res['nested']:.3e} | "
              f"{res['fetch16']:.3e} | {res['sparse']:.3e} |")


if __name__ == "__main__":
    main()

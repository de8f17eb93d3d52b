"""CPU oracle of the decode step's variants and of the accuracy study.
TEST INFRASTRUCTURE ONLY: like kv_oracle, only the test-suite, the smoke check
and the benchmark's CPU-baseline leg may import it; the product path never
does, and the two share no code.

Pages, cited as in kv_oracle (EXPLAINER = "StrataFlux -- Selective precision
streaming -- What does it mean?"):

* EXPLAINER, paragraph "Which tiles count ...": tokens are scored by the
  attention they receive -> the score variant "softmax_sum" (V1).
* EXPLAINER, paragraph "What travels over the link ..." and the comparison
  table (rows "Sparse attention (top-k, Quest)", "SpeCache (16-bit
  fetching)", "StrataFlux"): at matched key-plus-value bit budgets, nested
  refinement with 4 or 8 extra bits per element is compared with fetching
  complete 16-bit entries for the selected tokens and with sparse attention,
  which leaves the unselected tokens out; quality is the KL divergence of the
  attention -> V2 (16-bit rows), V3 (drop unselected), V4 (KL), V5 (budgets).
* The scale storage is not fixed by the pages; V6 stores (lo, delta) in fp16.

Readings (each stated at its step):
* V1: the attention a token receives from query head h is its softmax
  probability over the sequence's tokens, computed from the base keys; the
  group's score is the sum over its G query heads.
* V2: a 16-bit entry is the fp32 row rounded to IEEE fp16 (nearest, ties to
  even).
* V3: tokens left out take no part in the softmax (the selected tokens'
  weights are renormalised among themselves).
* V4: KL(approx || full) of each query head's attention distribution over the
  sequence's tokens, with "full" the fp32 K/V in fp64 arithmetic; mean over
  query heads.  This direction stays finite when tokens are left out.
* V5: matched budget = the same bits crossing the link per decode step and KV
  head: T_nested * D * r * 2 = T_16 * D * 16 * 2 (K and V rows), so a 16-bit
  method fetches T_16 = T_nested * r / 16 rows.
* V6: fp16 scales: lo is rounded down to fp16 and delta_b = (max - lo) 2^-b
  rounded up, so the stored range still covers the row; codes are computed in
  fp32 against those values.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from oracle import kv_oracle as O


# ---------------------------------------------------------------------------
# V1: score = the attention each token receives, summed over the GQA group
# (EXPLAINER, "Which tiles count").  fp64.
# ---------------------------------------------------------------------------

def token_scores_softmax_sum(q_group: np.ndarray, k_base: np.ndarray) -> np.ndarray:
    """q_group [G][D], k_base [N][D] -> scores [N]: sum over the G query heads
    of softmax over tokens of q_h . k_i / sqrt(D)."""
    qg = np.asarray(q_group, dtype=np.float64)
    d = qg.shape[-1]
    logits = (qg @ np.asarray(k_base, dtype=np.float64).T) / np.sqrt(d)   # [G][N]
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return p.sum(axis=0)


# ---------------------------------------------------------------------------
# V2: 16-bit entries (comparison table, rows "Sparse attention" and
# "SpeCache"): the selected tokens' complete rows in fp16.
# ---------------------------------------------------------------------------

def rows_fp16(x: np.ndarray) -> np.ndarray:
    """fp32 rows rounded to fp16 (nearest even), returned as fp64 values."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float64)


# ---------------------------------------------------------------------------
# V3: one (sequence, KV head) under a variant.  `score` is "max" (the step's
# default, kv_oracle O3) or "softmax_sum" (V1).  The selected tokens take
# their refined values (nested refinement, kv_oracle O2) or, with `k16`/`v16`
# given ([N][D] fp32 rows of the head), their fp16 rows; with `drop` the
# unselected tokens are left out of the softmax, else they take part at base
# precision.
# ---------------------------------------------------------------------------

def decode_head_variant(q_group: np.ndarray, kc: O.QuantRows, vc: O.QuantRows, t: int, score: str = "max",
                        drop: bool = False, k16: Optional[np.ndarray] = None,
                        v16: Optional[np.ndarray] = None) -> O.HeadResult:
    k_hat = O.dequant_base(kc)
    v_hat = O.dequant_base(vc)
    if score == "max":
        s = O.token_scores(q_group, k_hat)
    elif score == "softmax_sum":
        s = token_scores_softmax_sum(q_group, k_hat)
    else:
        raise ValueError(score)
    sel = O.select_top_t(s, t)
    k_star, v_star = k_hat.copy(), v_hat.copy()
    if sel.size:
        if k16 is not None:
            k_star[sel] = rows_fp16(np.asarray(k16)[sel])
            v_star[sel] = rows_fp16(np.asarray(v16)[sel])
        else:
            k_star[sel] = O.dequant_refined(O._take(kc, sel))
            v_star[sel] = O.dequant_refined(O._take(vc, sel))
    if drop:
        k_star, v_star = k_star[sel], v_star[sel]
    return O.HeadResult(scores=s, sel=sel, out=O.attend(q_group, k_star, v_star))


# ---------------------------------------------------------------------------
# V4: the attention distribution and its KL divergence from full precision.
# ---------------------------------------------------------------------------

def attention_probs(q_group: np.ndarray, k_star: np.ndarray, keep: Optional[np.ndarray] = None) -> np.ndarray:
    """[G][N] softmax over tokens of q_h . k_i / sqrt(D) (fp64); tokens not in
    `keep` (indices) get probability 0."""
    qg = np.asarray(q_group, dtype=np.float64)
    logits = (qg @ np.asarray(k_star, np.float64).T) / np.sqrt(qg.shape[-1])
    if keep is not None:
        mask = np.full(logits.shape[1], -np.inf)
        mask[np.asarray(keep, dtype=np.int64)] = 0.0
        logits = logits + mask
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    return p / p.sum(axis=1, keepdims=True)


def kl_divergence(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """KL(p || q) = sum_i p_i ln(p_i / q_i) per row, 0 ln 0 = 0 (fp64)."""
    p = np.asarray(p, np.float64)
    q = np.asarray(q, np.float64)
    terms = np.where(p > 0, p * (np.log(np.where(p > 0, p, 1.0)) - np.log(np.where(p > 0, q, 1.0))), 0.0)
    return terms.sum(axis=-1)


def study_head(q_group: np.ndarray, k_fp32: np.ndarray, b: int, r: int, t_nested: int):
    """KL(approx || full) of one (sequence, KV head) for the three methods at
    the matched budget (V5): nested refinement with r extra bits for T_nested
    tokens; 16-bit rows for T_16 = T_nested * r / 16 tokens with the others at
    base precision ("SpeCache"); the same T_16 16-bit rows with the others
    left out ("sparse").  Also the static base-only cache (nothing fetched).
    The selection is the step's (max-logit score from the base keys).  The
    attention distribution depends on the keys alone.
    Returns {method: mean KL over the group's query heads}."""
    k = np.asarray(k_fp32, np.float32)
    kc = O.quantize_rows(k, b, r)
    k_hat = O.dequant_base(kc)
    p_full = attention_probs(q_group, k.astype(np.float64))
    s = O.token_scores(q_group, k_hat)
    t16 = matched_rows(t_nested, r)
    out = {}
    out["base_only"] = kl_divergence(attention_probs(q_group, k_hat), p_full).mean()
    sel = O.select_top_t(s, t_nested)
    k_n = k_hat.copy()
    k_n[sel] = O.dequant_refined(O._take(kc, sel))
    out["nested"] = kl_divergence(attention_probs(q_group, k_n), p_full).mean()
    sel16 = O.select_top_t(s, t16)
    k_s = k_hat.copy()
    k_s[sel16] = rows_fp16(k[sel16])
    out["fetch16"] = kl_divergence(attention_probs(q_group, k_s), p_full).mean()
    out["sparse"] = kl_divergence(attention_probs(q_group, k_s, keep=sel16), p_full).mean()
    return out


def matched_rows(t_nested: int, r: int) -> int:
    """V5: 16-bit rows fetched at the budget of T_nested rows of r bits."""
    return (t_nested * r) // 16


# ---------------------------------------------------------------------------
# V6: fp16 scale storage (4 bytes per row instead of 8).
# ---------------------------------------------------------------------------

def _fp16_down(x: np.ndarray) -> np.ndarray:
    """Largest fp16 value <= x (x finite fp32), as fp32."""
    x = np.asarray(x, np.float32)
    h = x.astype(np.float16).astype(np.float32)          # nearest
    lower = np.nextafter(x.astype(np.float16), np.float16(-np.inf)).astype(np.float32)
    return np.where(h > x, lower, h).astype(np.float32)


def _fp16_up(x: np.ndarray) -> np.ndarray:
    """Smallest fp16 value >= x (x finite fp32, >= 0), as fp32."""
    x = np.asarray(x, np.float32)
    h = x.astype(np.float16).astype(np.float32)
    upper = np.nextafter(x.astype(np.float16), np.float16(np.inf)).astype(np.float32)
    return np.where(h < x, upper, h).astype(np.float32)


def quantize_rows_fp16_scales(x: np.ndarray, b: int, r: int) -> O.QuantRows:
    """kv_oracle O1 with (lo, delta_b) stored in fp16 (V6): lo = the row
    minimum rounded down to fp16, delta_b = (max - lo) 2^-b rounded up to
    fp16 (the range measured from the stored lo, so that lo + 2^b delta_b
    reaches the maximum), codes from one fp32 subtraction and one fp32
    division by delta_b 2^-r, clamped to [0, 2^(b+r) - 1]."""
    x = np.asarray(x, dtype=np.float32)
    f = b + r
    lo = _fp16_down(x.min(axis=-1))
    rng = (x.max(axis=-1) - lo).astype(np.float32)           # from the stored lo
    delta_b = _fp16_up((rng * np.float32(2.0 ** -b)).astype(np.float32))
    delta_f = (delta_b * np.float32(2.0 ** -r)).astype(np.float32)
    flat = delta_f == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        u = (x - lo[..., None]) / delta_f[..., None]
    u = np.where(flat[..., None], np.float32(0), u)
    fine = np.clip(np.floor(u), 0, 2 ** f - 1).astype(np.uint16)
    return O.QuantRows(lo=lo, delta=delta_b, fine=fine, base=(fine >> r).astype(np.uint16),
                       refine=(fine & ((1 << r) - 1)).astype(np.uint16), b=b, r=r)

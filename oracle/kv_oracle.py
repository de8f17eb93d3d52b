"""CPU oracle for the KV-cache refinement decode step.  TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The product path (the HIP library and its Python binding)
never calls it, and shares no code, table or constant with it.

It is a plain, slow, obviously correct restatement of what the method computes,
written from the StrataFlux pages:

* page "StrataFlux -- Selective precision streaming -- What does it mean?"
  (learnaivisually.com explainer), cited below as EXPLAINER with the paragraph:
  - "Think about how a map app ..."  (resident low-bit KV cache, refinement bits
    in host RAM)                                            -> tiers
  - "Which tiles count ..."  (score every cached token from the resident
    low-bit keys, refine the top tokens per KV head, the set a GQA group of
    query heads shares; unselected tokens still take part at low precision)
                                                            -> O3, O4, O5
  - "What travels over the link ..." (nested quantization: fetched bits
    subdivide the bin the resident code names; 2-bit code + 2 fetched bits =
    4-bit resolution)                                       -> O1, O2
  - "The map app also loads tiles ..." (fetched bits are kept and reused
    across steps because selections repeat)                  -> O6
  - comparison table, row "StrataFlux" (only the refinement bits of the
    selected tokens cross the link; unselected data gets the low-bit value)
* page "StrataFlux: Memory-Hierarchy-Native Low-Bit LLM Inference" (arXiv
  abstract as listed by readsearch.ai), cited as ABSTRACT: 2-3-bit KV cache,
  reuse of fetched precision across decoding steps.

Where the pages leave a step open, the reading taken is stated at the step.
Arithmetic: the quantizer runs in fp32 exactly as defined (one rounded
subtraction and one correctly rounded division per element); dequantization,
dot products and the softmax run in fp64, and outputs are cast to fp32.

Pinned by tests/test_oracle.py (hand-derived toy example in tests/golden/,
closed-form bounds, brute force on tiny inputs, textbook attention at T=0 and
convergence to full-precision attention as the refinement width grows).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


# ---------------------------------------------------------------------------
# O1 / O2: nested quantization of one row (EXPLAINER, "What travels over the
# link"): a b-bit code names one of 2^b equal bins of the row's range; r fetched
# bits split that bin into 2^r equal sub-bins, so base + refinement together
# have the resolution of a (b+r)-bit code.
# Readings: the range is [min, max] of the row over head_dim (asymmetric); the
# maximum element falls in the top bin; values sit at bin (sub-bin) centres; a
# row whose sub-bin width is 0 (max == min) has all codes 0 and decodes to min.
# Inputs must be finite with a finite range.
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class QuantRows:
    """Quantized rows.  Arrays share the leading shape of the input rows."""

    lo: np.ndarray       # fp32, row minimum
    delta: np.ndarray    # fp32, base bin width (max - min) / 2^b
    fine: np.ndarray     # uint16, (b+r)-bit code of each element
    base: np.ndarray     # uint16, b-bit base code = fine >> r
    refine: np.ndarray   # uint16, r-bit refinement code = fine & (2^r - 1)
    b: int
    r: int


def quantize_rows(x: np.ndarray, b: int, r: int) -> QuantRows:
    """Quantize each row (last axis) with a b-bit base code and r refinement bits."""
    x = np.asarray(x, dtype=np.float32)
    f = b + r
    lo = x.min(axis=-1)
    hi = x.max(axis=-1)
    rng = (hi - lo).astype(np.float32)                       # one fp32 subtraction
    delta_b = (rng * np.float32(2.0 ** -b)).astype(np.float32)   # exact scaling
    delta_f = (rng * np.float32(2.0 ** -f)).astype(np.float32)   # sub-bin width
    flat = delta_f == 0          # max == min (or a range too small to split)
    with np.errstate(divide="ignore", invalid="ignore"):
        u = (x - lo[..., None]) / delta_f[..., None]         # fp32, correctly rounded
    u = np.where(flat[..., None], np.float32(0), u)
    fine = np.minimum(np.floor(u), 2 ** f - 1).astype(np.uint16)
    base = (fine >> r).astype(np.uint16)
    refine = (fine & ((1 << r) - 1)).astype(np.uint16)
    return QuantRows(lo=lo.astype(np.float32), delta=delta_b, fine=fine,
                     base=base, refine=refine, b=b, r=r)


def dequant_base(qr: QuantRows) -> np.ndarray:
    """Base-precision value: centre of the bin the base code names (fp64)."""
    lo = qr.lo.astype(np.float64)[..., None]
    d = qr.delta.astype(np.float64)[..., None]
    return lo + (qr.base.astype(np.float64) + 0.5) * d


def dequant_refined(qr: QuantRows) -> np.ndarray:
    """Refined value: centre of the sub-bin the r fetched bits name inside the
    bin of the base code (fp64).  lo + c*delta + (s + 1/2)*delta/2^r."""
    lo = qr.lo.astype(np.float64)[..., None]
    d = qr.delta.astype(np.float64)[..., None]
    c = qr.base.astype(np.float64)
    s = qr.refine.astype(np.float64)
    return lo + c * d + (s + 0.5) * d / float(2 ** qr.r)


# ---------------------------------------------------------------------------
# Packing.  The pages fix no byte layout; the reading taken: each row's codes
# form one little-endian bitstream, element d occupying bits [w*d, w*d + w).
# ---------------------------------------------------------------------------

def pack_bits(codes: np.ndarray, w: int) -> np.ndarray:
    """Pack the last axis of ``codes`` (w-bit integers) LSB-first into bytes."""
    codes = np.asarray(codes)
    n = codes.shape[-1]
    if w == 0:
        return np.zeros(codes.shape[:-1] + (0,), dtype=np.uint8)
    if (n * w) % 8:
        raise ValueError("row length times width must be a whole number of bytes")
    bits = (codes[..., :, None].astype(np.uint32) >> np.arange(w, dtype=np.uint32)) & 1
    bits = bits.reshape(codes.shape[:-1] + (n * w,)).astype(np.uint8)
    return np.packbits(bits, axis=-1, bitorder="little")


def unpack_bits(packed: np.ndarray, w: int, n: int) -> np.ndarray:
    """Inverse of :func:`pack_bits`: n codes of w bits per row."""
    packed = np.asarray(packed, dtype=np.uint8)
    if w == 0:
        return np.zeros(packed.shape[:-1] + (n,), dtype=np.uint8)
    bits = np.unpackbits(packed, axis=-1, bitorder="little")[..., : n * w]
    bits = bits.reshape(packed.shape[:-1] + (n, w)).astype(np.uint32)
    return (bits << np.arange(w, dtype=np.uint32)).sum(axis=-1).astype(np.uint16)


# ---------------------------------------------------------------------------
# A quantized KV cache of one layer, head-major: [n_kv_heads][n_tok][D].
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class QuantCache:
    k: QuantRows
    v: QuantRows

    @property
    def n_tok(self) -> int:
        return self.k.base.shape[1]


def quantize_cache(k_tok_major: np.ndarray, v_tok_major: np.ndarray, b: int, r: int) -> QuantCache:
    """Quantize token-major [n_tok][Hkv][D] K and V into a head-major cache."""
    k = np.ascontiguousarray(np.swapaxes(np.asarray(k_tok_major, np.float32), 0, 1))
    v = np.ascontiguousarray(np.swapaxes(np.asarray(v_tok_major, np.float32), 0, 1))
    return QuantCache(quantize_rows(k, b, r), quantize_rows(v, b, r))


def _rows(qr: QuantRows, head: int, t0: int, t1: int) -> QuantRows:
    return QuantRows(lo=qr.lo[head, t0:t1], delta=qr.delta[head, t0:t1],
                     fine=qr.fine[head, t0:t1], base=qr.base[head, t0:t1],
                     refine=qr.refine[head, t0:t1], b=qr.b, r=qr.r)


# ---------------------------------------------------------------------------
# O3: score every cached token against the current query from the resident
# low-bit keys (EXPLAINER, "Which tiles count").  Reading: the score of token i
# for KV head k is the maximum over the query heads of k's GQA group of the
# scaled logit q_h . Khat_i / sqrt(D); query head h belongs to KV head
# floor(h / G).  Base keys are used whatever refinement may be cached.
# ---------------------------------------------------------------------------

def token_scores(q_group: np.ndarray, k_base: np.ndarray) -> np.ndarray:
    """q_group [G][D], k_base [N][D] (dequantized base keys) -> scores [N] fp64."""
    qg = np.asarray(q_group, dtype=np.float64)
    d = qg.shape[-1]
    logits = (qg @ np.asarray(k_base, dtype=np.float64).T) / np.sqrt(d)   # [G][N]
    return logits.max(axis=0)


# ---------------------------------------------------------------------------
# O4: the T highest-scoring tokens per KV head (EXPLAINER, "Which tiles
# count").  Reading: ties at the cut go to the lower token index; with N <= T
# every token is selected.  Output in ascending token order.
# ---------------------------------------------------------------------------

def select_top_t(scores: np.ndarray, t: int) -> np.ndarray:
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    idx = np.arange(n)
    order = np.lexsort((idx, -s))          # primary: score descending; then index
    return np.sort(order[: min(t, n)]).astype(np.int64)


# ---------------------------------------------------------------------------
# O5: attention over all cached tokens; the selected tokens use their refined
# keys and values, the others their base-precision values (EXPLAINER, "Which
# tiles count": unselected data still takes part at low precision; comparison
# table, row "StrataFlux").  Reading: plain softmax attention with scale
# 1/sqrt(D), no mask, K taken as already position-encoded.
# ---------------------------------------------------------------------------

def attend(q_group: np.ndarray, k_star: np.ndarray, v_star: np.ndarray) -> np.ndarray:
    """q_group [G][D], k_star/v_star [N][D] (fp64 values) -> out [G][D] fp64."""
    qg = np.asarray(q_group, dtype=np.float64)
    d = qg.shape[-1]
    logits = (qg @ np.asarray(k_star, np.float64).T) / np.sqrt(d)         # [G][N]
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    return (p @ np.asarray(v_star, np.float64)) / p.sum(axis=1, keepdims=True)


@dataclasses.dataclass
class HeadResult:
    scores: np.ndarray    # [N] fp64
    sel: np.ndarray       # ascending token indices, length min(T, N)
    out: np.ndarray       # [G][D] fp64


def decode_head(q_group: np.ndarray, kc: QuantRows, vc: QuantRows, t: int,
                sel: Optional[np.ndarray] = None, refined: Optional[np.ndarray] = None) -> HeadResult:
    """One (sequence, KV head): score, select, refine the selection, attend.

    ``kc``/``vc`` hold the head's rows [N][D].  ``sel`` overrides the
    selection (used to check the attention step for another valid selection
    when two selections differ only at a tie within the allowed tolerance).
    ``refined`` (O8, the skip policy) names the selected tokens whose
    refinement is at hand; the others take part at base precision.  By
    default every selected token is refined."""
    k_hat = dequant_base(kc)
    v_hat = dequant_base(vc)
    s = token_scores(q_group, k_hat)
    sel = select_top_t(s, t) if sel is None else np.sort(np.asarray(sel, dtype=np.int64))
    ref = sel if refined is None else np.sort(np.asarray(refined, dtype=np.int64))
    k_star = k_hat.copy()
    v_star = v_hat.copy()
    if ref.size:
        k_star[ref] = dequant_refined(_take(kc, ref))
        v_star[ref] = dequant_refined(_take(vc, ref))
    return HeadResult(scores=s, sel=sel, out=attend(q_group, k_star, v_star))


def _take(qr: QuantRows, rows: np.ndarray) -> QuantRows:
    return QuantRows(lo=qr.lo[rows], delta=qr.delta[rows], fine=qr.fine[rows],
                     base=qr.base[rows], refine=qr.refine[rows], b=qr.b, r=qr.r)


def decode_step(q: np.ndarray, cache: QuantCache, seq_off: Sequence[int], t: int,
                heads: Optional[Sequence[Tuple[int, int]]] = None) -> Dict[Tuple[int, int], HeadResult]:
    """Decode one layer for a packed batch.

    q [B][Hq][D]; ``cache`` head-major over the packed tokens; sequence s owns
    tokens [seq_off[s], seq_off[s+1]).  Returns {(seq, kv_head): HeadResult};
    ``heads`` restricts the work to some (seq, kv_head) pairs.
    """
    q = np.asarray(q, dtype=np.float32)
    n_b, n_q, _ = q.shape
    n_kv = cache.k.base.shape[0]
    g = n_q // n_kv
    res = {}
    todo = heads if heads is not None else [(s, h) for s in range(n_b) for h in range(n_kv)]
    for s, h in todo:
        t0, t1 = int(seq_off[s]), int(seq_off[s + 1])
        res[(s, h)] = decode_head(q[s, h * g:(h + 1) * g], _rows(cache.k, h, t0, t1),
                                  _rows(cache.v, h, t0, t1), t)
    return res


# ---------------------------------------------------------------------------
# O6: reuse of fetched refinement bits across decode steps (EXPLAINER, "The
# map app also loads tiles": fetched bits are kept and reused because
# selections repeat; ABSTRACT: fetched precision is reused across decoding
# steps).  Reading: one cache of C slots per (sequence, KV head); a selected
# token already resident is a hit; each miss is fetched (K and V refinement
# rows) and installed in a free slot, else in place of the resident that is not
# selected now and was selected longest ago (lower token index first); every
# selected token is stamped with the current step.  Policy on a miss: wait.
# ---------------------------------------------------------------------------

class CacheSim:
    def __init__(self, n_slots: int):
        self.n_slots = n_slots
        self.slot_tok = np.full(n_slots, -1, dtype=np.int64)
        self.stamp = np.full(n_slots, -1, dtype=np.int64)

    def residents(self) -> set:
        return {int(x) for x in self.slot_tok if x >= 0}

    def step(self, sel: np.ndarray, t: int) -> Tuple[int, int]:
        """Apply one step's selection; returns (hits, misses)."""
        hits, misses = self.step_tokens(sel, t)
        return len(hits), len(misses)

    def step_tokens(self, sel: np.ndarray, t: int) -> Tuple[List[int], List[int]]:
        """Apply one step's selection; returns the hit and the missed tokens
        (ascending).  Under the skip policy (O8) the hits are the tokens that
        step refines."""
        sel = [int(x) for x in np.sort(np.asarray(sel))]
        if len(sel) > self.n_slots:
            raise ValueError("cache smaller than the selection")
        where = {int(tok): i for i, tok in enumerate(self.slot_tok) if tok >= 0}
        sel_set = set(sel)
        hits = [x for x in sel if x in where]
        misses = [x for x in sel if x not in where]
        for x in hits:
            self.stamp[where[x]] = t
        free = [i for i in range(self.n_slots) if self.slot_tok[i] < 0]
        evictable = [i for i in range(self.n_slots)
                     if self.slot_tok[i] >= 0 and int(self.slot_tok[i]) not in sel_set]
        evictable.sort(key=lambda i: (self.stamp[i], self.slot_tok[i]))
        victims = free + evictable
        for x, slot in zip(misses, victims):
            self.slot_tok[slot] = x
            self.stamp[slot] = t
        return hits, misses


# ---------------------------------------------------------------------------
# O8: policy on a miss (EXPLAINER, "The map app also loads tiles ...": on a
# miss the runtime may wait for the bits, or use the low-bit value now while
# the bits are loaded for later steps).  "wait" is O6 with every selected
# token refined.  "skip": the step refines only the hits of O6's lookup; the
# misses take part at base precision and are installed in the cache all the
# same (they are there at the next step): decode_head(..., refined=hits).
# ---------------------------------------------------------------------------

def fetched_bytes(misses: int, head_dim: int, r: int) -> int:
    """Bytes that cross the link for ``misses`` tokens: K and V refinement rows."""
    return misses * 2 * head_dim * r // 8

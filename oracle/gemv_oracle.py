"""CPU oracle of the weight-side refinement GEMV.  TEST INFRASTRUCTURE ONLY:
only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import it; the product path never does, and the two share no code.

Page "StrataFlux -- Selective precision streaming -- What does it mean?"
(EXPLAINER):
* paragraph "Think about how a map app ...": weights resident at 2-4 bits;
* paragraph "Which tiles count ...": a projection's error is the sum of each
  input channel's activation times that channel's weight error, so the input
  channels are split into chunks of 1,024 and the k channels with the largest
  activation magnitude in each chunk are refined at this step;
* paragraph "What travels over the link ...": the fetched bits subdivide the
  bin the resident code names (nested quantization);
* the worked example (k = 32 of 1,024 channels, 4-bit refinement values,
  3-bit resident weights): 3.1 % of the columns fetched, 0.125 extra bits per
  weight on average, 3.125 bits per weight touched, a BF16 copy 128 times the
  refinement payload.

Readings:
* W1: the weights y = W x, W of M output rows and K input channels, are
  quantized along each output row in groups of 128 input channels with the
  nested quantizer of kv_oracle (O1: b-bit base code, r refinement bits, fp32
  (lo, delta) per group).  (The pages fit the weight refinements on a
  calibration set; that needs data and is out of scope: the refinement here
  is the nested code itself.)
* W2: per chunk of 1,024 input channels (the last chunk may be shorter), the
  k channels of largest |x|, ties to the lower channel index.
* W3: y = sum over channels of (refined column if selected, else base column)
  times x, in fp64.
* W4: bits per weight fetched = (selected channels / K) * r; the resident
  weights' b bits per weight are read every step as well.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from oracle import kv_oracle as O

GROUP = 128      # input channels per quantization group (W1)


@dataclasses.dataclass
class QuantWeights:
    q: O.QuantRows   # rows = (output row, group): shape [M][K/128] leading, 128 codes each


def quantize_weights(w: np.ndarray, b: int, r: int) -> QuantWeights:
    """W1: [M][K] fp32 (K a multiple of 128) -> per (row, group) nested codes."""
    w = np.asarray(w, np.float32)
    m, k = w.shape
    assert k % GROUP == 0
    return QuantWeights(O.quantize_rows(w.reshape(m, k // GROUP, GROUP), b, r))


def dequant_weights(qw: QuantWeights, refined: bool) -> np.ndarray:
    """[M][K] fp64 base (bin centres) or refined (sub-bin centres) weights."""
    x = O.dequant_refined(qw.q) if refined else O.dequant_base(qw.q)
    return x.reshape(x.shape[0], -1)


def select_channels(x: np.ndarray, k_top: int, chunk: int = 1024) -> np.ndarray:
    """W2: ascending indices of the k largest |x| of each chunk (ties to the
    lower index)."""
    a = np.abs(np.asarray(x, np.float32)).astype(np.float64)
    out = []
    for c0 in range(0, a.shape[0], chunk):
        seg = a[c0:c0 + chunk]
        idx = np.arange(seg.shape[0])
        order = np.lexsort((idx, -seg))
        out.append(np.sort(order[:min(k_top, seg.shape[0])]) + c0)
    return np.concatenate(out).astype(np.int64) if out else np.zeros(0, np.int64)


def gemv(qw: QuantWeights, x: np.ndarray, k_top: int, chunk: int = 1024):
    """W3: (y [M] fp64, selected channels)."""
    x64 = np.asarray(x, np.float32).astype(np.float64)
    sel = select_channels(x, k_top, chunk)
    w = dequant_weights(qw, refined=False)
    if sel.size:
        w[:, sel] = dequant_weights(qw, refined=True)[:, sel]
    return w @ x64, sel


def bits_per_weight(k_top: int, chunk: int, r: int, b: int, k_in: int = None) -> dict:
    """W4 for one projection: share of columns fetched, extra (fetched) bits
    per weight, bits per weight the step touches, and the ratio of a BF16
    copy of every weight to the refinement payload.  With k_in given, the
    shorter last chunk is counted exactly."""
    if k_in is None:
        share = k_top / chunk
    else:
        full, rest = divmod(k_in, chunk)
        share = (full * min(k_top, chunk) + min(k_top, rest)) / k_in
    extra = share * r
    return {"share": share, "extra_bits": extra, "touched_bits": b + extra, "bf16_over_payload": 16.0 / extra}

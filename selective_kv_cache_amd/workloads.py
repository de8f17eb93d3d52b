"""Seeded synthetic decode workloads.

This module only draws random inputs: it holds none of the method's
arithmetic (no quantization, scoring, selection or attention).  The HIP path,
the CPU oracle, the tests and the benchmark all take their inputs from here.

Shapes follow the head geometry the StrataFlux pages evaluate on
(Llama-3.1-8B: 32 query heads / 8 KV heads, Qwen3-8B: the same attention
geometry; head_dim 128) and the context lengths they quote (up to 128K).
Values are standard normal with a few key channels scaled up, standing in for
the outlier channels the explainer page mentions ("outlier channels hurt
quantization", page "StrataFlux -- Selective precision streaming -- What does
it mean?", paragraph on which tiles count).  No dataset or trained weight is
used: none is available.

Seeds: every draw comes from ``numpy.random.default_rng(SeedSequence([cfg_id,
layer, stream, step]))`` with stream 0 = K, 1 = V, 2 = outlier channels,
3 = query, 4 = appended tokens, 5 = sequence lengths, 6 = projection
weights, 7 = projection activations.  A torch variant draws
the large per-layer K/V tensors directly on a GPU (``torch.Generator`` seeded
from the same tuple); its numbers differ from numpy's, so any comparison must
feed one draw to both sides.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

STREAM_K, STREAM_V, STREAM_OUTLIER, STREAM_Q, STREAM_APPEND, STREAM_LEN, STREAM_W, STREAM_X = range(8)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One decode workload.  Token counts are per sequence."""

    name: str
    cfg_id: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    base_bits: int
    refine_bits: int
    top_t: int
    layers: int
    ctx: int = 0                      # fixed context (0 when lengths are drawn)
    ctx_range: Tuple[int, int] = (0, 0)   # inclusive range for drawn lengths
    n_outlier: int = 3                # outlier key channels per KV head
    outlier_scale: float = 8.0
    fixed_outliers: Tuple[int, ...] = ()  # same channels for every head when set
    host_store: bool = False          # refinement store in pinned host memory
    steps: int = 1                    # decode steps (multi-step reuse run)
    rho: float = 0.0                  # AR(1) coefficient of the query process
    cache_slots_factor: int = 2       # device refinement cache: slots = factor*T

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def seq_lengths(self) -> List[int]:
        if self.ctx:
            return [self.ctx] * self.batch
        rng = _rng(self.cfg_id, 0, STREAM_LEN, 0)
        lo, hi = self.ctx_range
        return [int(x) for x in rng.integers(lo, hi, size=self.batch, endpoint=True)]

    def cache_slots(self) -> int:
        return self.cache_slots_factor * self.top_t


WORKLOADS: Dict[str, Workload] = {
    # tiny single-layer parity reference
    "tiny_1k": Workload("tiny_1k", 1, batch=1, n_q_heads=4, n_kv_heads=1, head_dim=128,
                        base_bits=2, refine_bits=2, top_t=64, layers=1, ctx=1024,
                        n_outlier=4, fixed_outliers=(9, 42, 77, 118)),
    # Llama-3.1-8B attention layer, 32K context
    "llama8b_32k": Workload("llama8b_32k", 2, batch=1, n_q_heads=32, n_kv_heads=8,
                            head_dim=128, base_bits=2, refine_bits=2, top_t=512,
                            layers=32, ctx=32768),
    # Llama-3.1-8B, 128K context, refinement store in pinned host memory
    "llama8b_128k": Workload("llama8b_128k", 3, batch=1, n_q_heads=32, n_kv_heads=8,
                             head_dim=128, base_bits=2, refine_bits=4, top_t=2048,
                             layers=32, ctx=131072, host_store=True),
    # Qwen3-8B-shaped batched decode, per-sequence contexts 4K..16K
    "qwen8b_b16": Workload("qwen8b_b16", 4, batch=16, n_q_heads=32, n_kv_heads=8,
                           head_dim=128, base_bits=2, refine_bits=8, top_t=256,
                           layers=1, ctx_range=(4096, 16384)),
    # multi-step reuse: 8K context growing by one token per step, AR(1) queries
    "llama8b_reuse": Workload("llama8b_reuse", 5, batch=1, n_q_heads=32, n_kv_heads=8,
                              head_dim=128, base_bits=3, refine_bits=2, top_t=512,
                              layers=32, ctx=8192, host_store=True, steps=256, rho=0.9),
}


def _rng(cfg_id: int, layer: int, stream: int, step: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg_id, layer, stream, step]))


def _torch_seed(cfg_id: int, layer: int, stream: int, step: int) -> int:
    h = hashlib.sha256(f"{cfg_id}/{layer}/{stream}/{step}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def outlier_channels(w: Workload, layer: int) -> np.ndarray:
    """[n_kv_heads][n_outlier] key channels scaled by ``outlier_scale``."""
    if w.fixed_outliers:
        return np.tile(np.asarray(w.fixed_outliers, dtype=np.int64), (w.n_kv_heads, 1))
    rng = _rng(w.cfg_id, layer, STREAM_OUTLIER, 0)
    return np.stack([rng.choice(w.head_dim, size=w.n_outlier, replace=False)
                     for _ in range(w.n_kv_heads)]).astype(np.int64)


def layer_kv(w: Workload, layer: int, n_tok: Optional[int] = None,
             device=None, head_slice: Optional[slice] = None):
    """K and V of one layer, token-major ``[n_tok][n_kv_heads][head_dim]`` fp32.

    ``n_tok`` defaults to the sum of the sequence lengths (sequences packed in
    order).  With ``device`` set, the draw is made by torch on that device.
    ``head_slice`` keeps only some KV heads (host draw only; the full draw is
    made first so the values do not depend on the slice).
    """
    if n_tok is None:
        n_tok = sum(w.seq_lengths())
    shape = (n_tok, w.n_kv_heads, w.head_dim)
    ch = outlier_channels(w, layer)
    if device is not None:
        import torch
        out = []
        for stream in (STREAM_K, STREAM_V):
            g = torch.Generator(device=device)
            g.manual_seed(_torch_seed(w.cfg_id, layer, stream, 0))
            out.append(torch.randn(shape, generator=g, device=device, dtype=torch.float32))
        k, v = out
        for h in range(w.n_kv_heads):
            idx = torch.as_tensor(ch[h], device=device)
            k[:, h, idx] *= w.outlier_scale
        return k, v
    k = _rng(w.cfg_id, layer, STREAM_K, 0).standard_normal(shape, dtype=np.float32)
    v = _rng(w.cfg_id, layer, STREAM_V, 0).standard_normal(shape, dtype=np.float32)
    for h in range(w.n_kv_heads):
        k[:, h, ch[h]] *= np.float32(w.outlier_scale)
    if head_slice is not None:
        k = np.ascontiguousarray(k[:, head_slice])
        v = np.ascontiguousarray(v[:, head_slice])
    return k, v


def appended_kv(w: Workload, layer: int, step: int) -> Tuple[np.ndarray, np.ndarray]:
    """The one token appended at decode ``step``: K, V of shape [1][Hkv][D]."""
    rng = _rng(w.cfg_id, layer, STREAM_APPEND, step)
    kv = rng.standard_normal((2, 1, w.n_kv_heads, w.head_dim), dtype=np.float32)
    k, v = kv[0].copy(), kv[1].copy()
    ch = outlier_channels(w, layer)
    for h in range(w.n_kv_heads):
        k[:, h, ch[h]] *= np.float32(w.outlier_scale)
    return k, v


def query(w: Workload, layer: int, step: int = 0) -> np.ndarray:
    """Query of one layer at one step, ``[batch][n_q_heads][head_dim]`` fp32."""
    return queries(w, layer, step + 1)[step]


def queries(w: Workload, layer: int, n_steps: int) -> np.ndarray:
    """Queries of steps 0..n_steps-1, ``[n_steps][batch][n_q_heads][head_dim]`` fp32.

    With ``rho > 0`` they follow a stationary AR(1) process over steps:
    q_0 ~ N(0, I) and q_t = rho*q_{t-1} + sqrt(1 - rho^2)*eps_t, eps_t ~ N(0, I).
    With ``rho == 0`` every step draws a fresh N(0, I) query.
    """
    shape = (w.batch, w.n_q_heads, w.head_dim)
    out = np.empty((n_steps,) + shape, dtype=np.float32)
    q = _rng(w.cfg_id, layer, STREAM_Q, 0).standard_normal(shape)
    c = np.sqrt(1.0 - w.rho * w.rho)
    for t in range(n_steps):
        if t:
            eps = _rng(w.cfg_id, layer, STREAM_Q, t).standard_normal(shape)
            q = w.rho * q + c * eps if w.rho > 0.0 else eps
        out[t] = q
    return out


def seq_offsets(lengths: Sequence[int]) -> np.ndarray:
    off = np.zeros(len(lengths) + 1, dtype=np.int64)
    off[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return off


def small(name: str = "tiny", **over) -> Workload:
    """A reduced workload for parity tests (same structure, smaller sizes)."""
    base = dict(cfg_id=100, batch=1, n_q_heads=4, n_kv_heads=1, head_dim=128,
                base_bits=2, refine_bits=2, top_t=64, layers=1, ctx=1024)
    base.update(over)
    return Workload(name, **base)


def duplicate_rows(k: np.ndarray, v: np.ndarray, src: Sequence[int], dst: Sequence[int]) -> None:
    """Copy token rows ``src`` onto ``dst`` in place: exact score ties."""
    k[list(dst)] = k[list(src)]
    v[list(dst)] = v[list(src)]


# Projection shapes of Llama-3.1-8B (hidden 4,096, MLP 14,336): (output rows,
# input channels) of the gate/up projection and of the down projection.
PROJECTIONS: Dict[str, Tuple[int, int]] = {
    "llama8b_up": (14336, 4096),
    "llama8b_down": (4096, 14336),
}


def projection_weights(cfg_id: int, m: int, k: int) -> np.ndarray:
    """[m][k] fp32 weights, normal with standard deviation 1/sqrt(k)."""
    rng = _rng(cfg_id, 0, STREAM_W, 0)
    return (rng.standard_normal((m, k), dtype=np.float32) / np.float32(np.sqrt(k))).astype(np.float32)


def projection_input(cfg_id: int, k: int, step: int = 0, n_outlier: int = 0, outlier_scale: float = 8.0,
                     ties: int = 0) -> np.ndarray:
    """[k] fp32 activations: standard normal, ``n_outlier`` channels scaled by
    ``outlier_scale`` (heavy activation channels), and ``ties`` channels made
    to share one magnitude (with random signs) so that selections must break
    ties by index."""
    rng = _rng(cfg_id, 0, STREAM_X, step)
    x = rng.standard_normal(k, dtype=np.float32)
    if n_outlier:
        x[rng.choice(k, size=min(n_outlier, k), replace=False)] *= np.float32(outlier_scale)
    if ties:
        idx = rng.choice(k, size=min(ties, k), replace=False)
        mag = np.float32(np.quantile(np.abs(x), 0.97))
        x[idx] = np.where(rng.random(idx.size) < 0.5, -mag, mag).astype(np.float32)
    return x


"""Device buffers of one layer's resident KV cache and its refinement store.

Marshalling only: allocates torch tensors in the layouts include/sf_kv.h
documents and forwards to the C entry points (quantization, store, decode).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from . import binding as B


class LayerCache:
    """Codes and scales of K and V for one layer ([Hkv][cap][...]) plus the
    refinement store.  ``tier`` is binding.SF_TIER_DEVICE or SF_TIER_HOST_PINNED."""

    def __init__(self, g: B.sf_geom, cap: int, device="cuda", tier: int = B.SF_TIER_DEVICE,
                 max_seqs: int = 1, cache_slots: int = 0, fp16_scales: bool = False, rows16: bool = False):
        """``fp16_scales``: scales quantized as fp16 values (SF_QUANT_FP16_SCALES);
        ``rows16``: also keep the appended K and V rows as fp16 ([2][Hkv][cap][D],
        the complete 16-bit entries the SF_DECODE_ROWS16 comparison fetches)."""
        self.g, self.cap, self.device, self.tier = g, cap, torch.device(device), tier
        self.quant_flags = B.SF_QUANT_FP16_SCALES if fp16_scales else 0
        hkv, d, b, r = g.n_kv_heads, g.head_dim, g.base_bits, g.refine_bits
        mk = lambda shape, dt: torch.empty(shape, dtype=dt, device=self.device)
        self.k_codes = mk((hkv, cap, d * b // 8), torch.uint8)
        self.v_codes = mk((hkv, cap, d * b // 8), torch.uint8)
        self.k_scales = mk((hkv, cap, 2), torch.float32)
        self.v_scales = mk((hkv, cap, 2), torch.float32)
        self.store = B.sf_store_create(g, cap, max_seqs, tier, cache_slots) if r > 0 else None
        self.rows16 = mk((2, hkv, cap, d), torch.float16) if rows16 else None

    def append(self, k: torch.Tensor, v: torch.Tensor, tok_begin: int, keep_refine: bool = False):
        """Quantize token-major [n][Hkv][D] fp32 K and V into tokens
        [tok_begin, tok_begin + n) and put their refinement rows in the store.
        Returns the refinement rows (K, V) when ``keep_refine``."""
        n = k.shape[0]
        r = self.g.refine_bits
        hkv, d = self.g.n_kv_heads, self.g.head_dim
        out = []
        for x, codes, scales, which in ((k, self.k_codes, self.k_scales, B.SF_K),
                                        (v, self.v_codes, self.v_scales, B.SF_V)):
            x = x.contiguous()
            rr = torch.empty((hkv, n, d * r // 8), dtype=torch.uint8, device=self.device) if r else None
            B.sf_kv_quantize(self.g, x, n, tok_begin, self.cap, codes, scales, rr, flags=self.quant_flags)
            if r:
                B.sf_refine_store(self.store, which, rr, tok_begin, n)
            if self.rows16 is not None:
                self.rows16[which, :, tok_begin:tok_begin + n] = x.transpose(0, 1).to(torch.float16)
            out.append(rr)
        return tuple(out) if keep_refine else None

    def clear_cache(self):
        if self.store is not None:
            B.sf_store_clear_cache(self.store)

    def close(self):
        if self.store is not None:
            B.sf_store_destroy(self.store)
            self.store = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Decoder:
    """Workspace and offsets for decode steps of one batch shape."""

    def __init__(self, g: B.sf_geom, seq_off: Sequence[int], top_t: int, device="cuda"):
        self.g, self.top_t = g, top_t
        self.device = torch.device(device)
        self.seq_off = np.asarray(seq_off, dtype=np.int64)
        lens = np.diff(self.seq_off)
        self.batch = len(lens)
        self.total = int(self.seq_off[-1] - self.seq_off[0])
        self.max_seq = int(lens.max())
        self.seq_off_dev = torch.as_tensor(self.seq_off, device=self.device)
        nbytes = B.sf_decode_workspace_size(g, self.batch, self.total, self.max_seq, top_t)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self._hist_clean = False   # a successful step leaves the workspace histogram zero

    def form(self, cache: "LayerCache", multi_pass: bool = False) -> int:
        """Kernels per step (1: single launch, 5) for this cache."""
        return B.sf_decode_form(self.g, self.seq_off, self.top_t, cache.store,
                                B.SF_DECODE_MULTI_PASS if multi_pass else 0)

    def check(self) -> int:
        """sf_decode_check on this decoder's workspace (synchronizes)."""
        return B.sf_decode_check(self.workspace)

    def set_offsets(self, seq_off: Sequence[int]) -> None:
        """Point the decoder at new sequence offsets (a context that grew).
        The workspace is reallocated, with a quarter to spare, only when the
        new shape needs more; a reallocated workspace starts uncleared."""
        self.seq_off = np.asarray(seq_off, dtype=np.int64)
        lens = np.diff(self.seq_off)
        batch = len(lens)
        self.total = int(self.seq_off[-1] - self.seq_off[0])
        self.max_seq = int(lens.max())
        if batch != self.batch:
            self.batch = batch
            self._hist_clean = False
        if self.seq_off_dev.numel() == self.seq_off.size:
            src = torch.as_tensor(self.seq_off)
            if self.device.type == "cuda":
                # from pinned memory, stream-ordered: a copy from pageable
                # memory would wait for every launch queued before it
                self.seq_off_dev.copy_(src.pin_memory(), non_blocking=True)
            else:
                self.seq_off_dev.copy_(src)
        else:
            self.seq_off_dev = torch.as_tensor(self.seq_off, device=self.device)
        nbytes = B.sf_decode_workspace_size(self.g, self.batch, self.total, self.max_seq, self.top_t)
        if nbytes > self.workspace.numel():
            self.workspace = torch.empty(nbytes + nbytes // 4, dtype=torch.uint8, device=self.device)
            self._hist_clean = False

    def step(self, cache: LayerCache, q: torch.Tensor, out: Optional[torch.Tensor] = None,
             sel_out: Optional[torch.Tensor] = None, scores_out: Optional[torch.Tensor] = None,
             want_stats: bool = False, events=None, stream=None, skip_misses: bool = False,
             multi_pass: bool = False, variant: int = 0):
        """One decode step of one layer.  ``skip_misses``: policy "skip" on
        a refinement-cache miss (SF_DECODE_SKIP_MISSES); ``multi_pass``: the
        five-kernel form even where the single launch applies; ``variant``:
        SF_DECODE_DROP_UNSELECTED | SF_DECODE_ROWS16 | SF_DECODE_SCORE_SOFTMAX
        (the 16-bit rows are the cache's)."""
        if out is None:
            out = torch.empty((self.batch, self.g.n_q_heads, self.g.head_dim), dtype=torch.float32,
                              device=self.device)
        flags = B.SF_DECODE_HIST_CLEAN if self._hist_clean else 0
        if skip_misses:
            flags |= B.SF_DECODE_SKIP_MISSES
        if multi_pass:
            flags |= B.SF_DECODE_MULTI_PASS
        flags |= variant
        self._hist_clean = False
        st = B.sf_decode_step(self.g, seq_off_host=self.seq_off, seq_off_dev=self.seq_off_dev, q=q,
                              k_codes=cache.k_codes, k_scales=cache.k_scales, v_codes=cache.v_codes,
                              v_scales=cache.v_scales, cap=cache.cap, store=cache.store,
                              top_t=self.top_t, out=out, workspace=self.workspace, sel_out=sel_out,
                              scores_out=scores_out, want_stats=want_stats, events=events,
                              stream=stream, flags=flags,
                              rows16=cache.rows16 if variant & B.SF_DECODE_ROWS16 else None)
        self._hist_clean = True
        return (out, st) if want_stats else out

// The split-K combine of the five-kernel form.
//
// Page "StrataFlux -- Selective precision streaming -- What does it mean?",
// paragraph "Which tiles count ...": every token takes part in attention;
// unselected ones at the low-bit base value.  The attention pass
// (attend_mfma, sf_mfma.hip) has work-groups of two kinds:
//   blockIdx.x <  n_sel_blk : refined terms of p.sel_blk_tok selected tokens
//                             (selected_block, sf_attend_common.h);
//   blockIdx.x >= n_sel_blk : one split of tokens at base precision, with the
//                             selected tokens left out.
// Both write partials (m, l, acc[D]); combine merges those of a (sequence,
// query head).  The selection is known before that pass, so every token
// enters exactly one partial, with its final logit and value.
#include <math.h>

#include "sf_attend_common.h"

namespace sfk {

// combine: grid (B * Hq, 4); a work-group takes 32 of the head's 128 output
// elements.  Every partial's weight e^{m_x - M} is staged in LDS first, so the
// accumulation reads of different partials are independent of each other.
template <bool Batched>
__global__ void __launch_bounds__(256) combine(DecodeParams p) {
  __shared__ float red[4];
  __shared__ float ew[kCombineMax], lw[kCombineMax];
  __shared__ float snum[8][32];
  const int s = blockIdx.x / p.hq, h = blockIdx.x % p.hq;
  const int kvh = h / p.grp, hg = h % p.grp;
  const int tid = threadIdx.x, dl = tid & 31, sl = tid >> 5;
  const int d = blockIdx.y * 32 + dl;
  // partials of the sequences before s: base splits bb, selected blocks sb
  // (the Batched form, up to 63 sequences: lane i reads sequence i's length,
  // one memory round trip)
  int sb = 0, bb = 0;
  if (Batched && p.batch < 64) {
    const int lane = tid & 63;
    const bool in = lane < s;
    const int64_t n = in ? p.seq_off[lane + 1] - p.seq_off[lane] : 0;
    const uint32_t nb = in && !p.drop ? (uint32_t)((n + p.split - 1) / p.split) : 0u;
    const uint32_t ns = in && p.use_refine ? (uint32_t)(((n < p.top_t ? n : p.top_t) + p.sel_blk_tok - 1) / p.sel_blk_tok)
                                          : 0u;
    bb = (int)__builtin_amdgcn_readlane(wave_inclusive_scan(nb), 63);
    sb = (int)__builtin_amdgcn_readlane(wave_inclusive_scan(ns), 63);
  } else {
    for (int i = 0; i < s; ++i) {
      const int64_t n = seq_at(p, i + 1) - seq_at(p, i);
      if (!p.drop) bb += (int)((n + p.split - 1) / p.split);
      if (p.use_refine) sb += (int)(((n < p.top_t ? n : p.top_t) + p.sel_blk_tok - 1) / p.sel_blk_tok);
    }
  }
  const int64_t n = seq_at(p, s + 1) - seq_at(p, s);
  const int nb = p.drop ? 0 : (int)((n + p.split - 1) / p.split);   // left out: no base partials
  const int ns = p.use_refine ? (int)(((n < p.top_t ? n : p.top_t) + p.sel_blk_tok - 1) / p.sel_blk_tok) : 0;
  const int64_t stride = (int64_t)p.grp * kPartStride;
  const float* base = p.part + (int64_t)kvh * (p.n_sel_blk + p.n_split) * stride + hg * kPartStride;
  const int np = ns + nb;
  auto row = [&](int x) { return x < ns ? base + (sb + x) * stride : base + (p.n_sel_blk + bb + x - ns) * stride; };
  // every load at once: thread (sl, dl)'s first kPre accumulator values, and
  // the (m, l) of the partials it scans; the weights e^{m_x - M} follow in LDS
  constexpr int kPre = 16;
  float av[kPre];
#pragma unroll
  for (int k = 0; k < kPre; ++k) {
    const int x = sl + 8 * k;
    av[k] = x < np ? row(x)[d] : 0.f;
  }
  float M = -INFINITY;
  for (int x = tid; x < np; x += 256) {
    const float* r = row(x);
    const float mx = r[kHeadDim];
    ew[x] = mx;
    lw[x] = r[kHeadDim + 1];
    M = fmaxf(M, mx);
  }
  M = wave_max_dpp(M);
  if ((tid & 63) == 0) red[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float den = 0.f;
  for (int x = tid; x < np; x += 256) {
    const float mx = ew[x];
    const float e = mx == -INFINITY ? 0.f : expf(mx - M);   // -inf: a split whose tokens were all selected
    ew[x] = e;
    den = fmaf(e, lw[x], den);
  }
  den = wave_sum_dpp(den);
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = den;
  float num = 0.f;
#pragma unroll
  for (int k = 0; k < kPre; ++k) {
    const int x = sl + 8 * k;
    if (x < np) num = fmaf(ew[x], av[k], num);
  }
  for (int x = sl + 8 * kPre; x < np; x += 8) num = fmaf(ew[x], row(x)[d], num);
  snum[sl][dl] = num;
  __syncthreads();
  if (sl == 0) {
    float x = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) x += snum[i][dl];
    p.out[((int64_t)s * p.hq + h) * kHeadDim + d] = x / (red[0] + red[1] + red[2] + red[3]);
  }
}

void launch_combine(const DecodeParams& p, hipStream_t st, KernelEvents ev) {
  if (p.batch > 1)
    sf_launch(combine<true>, dim3(p.batch * p.hq, kHeadDim / 32), dim3(256), st, ev, p);
  else
    sf_launch(combine<false>, dim3(p.batch * p.hq, kHeadDim / 32), dim3(256), st, ev, p);
}

}  // namespace sfk

// Attention pass (portable VALU form) and the split-K combine.
//
// Page "StrataFlux -- Selective precision streaming -- What does it mean?",
// paragraph "Which tiles count ...": every token takes part in attention;
// unselected ones at the low-bit base value.  The work-groups of this kernel
// are of two kinds:
//   blockIdx.x <  n_sel_blk : refined terms of p.sel_blk_tok selected tokens
//                             (selected_block, sf_attend_common.h);
//   blockIdx.x >= n_sel_blk : one split of tokens at base precision, with the
//                             selected tokens left out.
// Both write partials (m, l, acc[D]); combine merges those of a (sequence,
// query head).  The selection is known before this pass, so every token
// enters exactly one partial, with its final logit and value.
//
// This form computes the inner products on the VALU; it serves base codes of
// 3 and 4 bits and GQA groups of 8; sf_mfma.hip holds the matrix-core form.
#include <math.h>

#include "sf_attend_common.h"

namespace sfk {

// One split at base precision: 4 wavefronts, tiles of 64 tokens (one per
// lane); K rows go through the lane's LDS row so the 128-element loop can
// stay rolled.
template <int BB, int G>
struct ValuLds {
  float qs[G][kHeadDim];
  float qsum[G];
  uint32_t kt[4][64][4 * BB + 1];
  uint32_t vt[4][64][4 * BB + 1];
  float2 vsc[4][64];
  float pt[4][G][64];
  float mw[4][G], lw[4][G];
  float accw[4][G][kHeadDim];
};

template <int BB, int G>
__device__ inline void base_split_valu(const DecodeParams& p, int split, int kvh, uint8_t* smem) {
  constexpr int W = 4 * BB;
  using Lds = ValuLds<BB, G>;
  Lds& s = *reinterpret_cast<Lds*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int64_t lo, hi;
  int first;
  const int seq = locate_unit(p, p.split, split, false, lo, hi, first);
  const int64_t a = seq_at(p, seq);
  const int64_t sk = (int64_t)seq * p.hkv + kvh;
  const uint32_t* bm = p.bitmap + sk * p.bm_words;
  const bool masked = p.use_refine != 0;

  for (int i = tid; i < G * kHeadDim; i += 256)
    s.qs[i / kHeadDim][i % kHeadDim] = p.q[((int64_t)seq * p.hq + kvh * G) * kHeadDim + i];
  __syncthreads();
  if (tid < G) {
    float acc = 0.f;
    for (int d = 0; d < kHeadDim; ++d) acc += s.qs[tid][d];
    s.qsum[tid] = acc;
  }
  __syncthreads();

  float m[G], l[G], acc[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
    acc[h][0] = acc[h][1] = 0.f;
  }
  const uint8_t* kbase = p.kc + (int64_t)kvh * p.cap * (16 * BB);
  const uint8_t* vbase = p.vc + (int64_t)kvh * p.cap * (16 * BB);
  const float2* ksc = reinterpret_cast<const float2*>(p.ks) + (int64_t)kvh * p.cap;
  const float2* vscg = reinterpret_cast<const float2*>(p.vs) + (int64_t)kvh * p.cap;
  const int niter = (int)((hi - lo + 255) / 256);
  const int vpos = 2 * lane * BB, vwi = vpos >> 5, vsh = vpos & 31;
  uint32_t* myk = s.kt[wid][lane];
  uint32_t* myv = s.vt[wid][lane];
  for (int it = 0; it < niter; ++it) {
    const int64_t li = lo + (int64_t)it * 256 + wid * 64 + lane;
    const int64_t tok = a + li;
    const bool valid = li < hi && !(masked && ((bm[li >> 5] >> (li & 31)) & 1u));
    float2 sk2 = make_float2(0.f, 0.f), sv2 = make_float2(0.f, 0.f);
    if (valid) {
      const uint4* ks4 = reinterpret_cast<const uint4*>(kbase + tok * (16 * BB));
      const uint4* vs4 = reinterpret_cast<const uint4*>(vbase + tok * (16 * BB));
#pragma unroll
      for (int w = 0; w < BB; ++w) {
        const uint4 u = ks4[w], v = vs4[w];
        myk[4 * w] = u.x; myk[4 * w + 1] = u.y; myk[4 * w + 2] = u.z; myk[4 * w + 3] = u.w;
        myv[4 * w] = v.x; myv[4 * w + 1] = v.y; myv[4 * w + 2] = v.z; myv[4 * w + 3] = v.w;
      }
      sk2 = ksc[tok];
      sv2 = vscg[tok];
    } else {
#pragma unroll
      for (int w = 0; w < W; ++w) myk[w] = myv[w] = 0u;
    }
    myk[W] = myv[W] = 0u;
    s.vsc[wid][lane] = sv2;
    float dot[G];
#pragma unroll
    for (int h = 0; h < G; ++h) dot[h] = 0.f;
#pragma unroll 4
    for (int d = 0; d < kHeadDim; ++d) {
      const float c = (float)code_at<BB>(myk, d);
#pragma unroll
      for (int h = 0; h < G; ++h) dot[h] = fmaf(s.qs[h][d], c, dot[h]);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float lg = (sk2.x * s.qsum[h] + sk2.y * (dot[h] + 0.5f * s.qsum[h])) * kRsqrtD;
      const float mt = wave_max(valid ? lg : -INFINITY);
      const float mn = fmaxf(m[h], mt);
      float pj = 0.f;
      if (mn != -INFINITY) {
        const float alpha = expf(m[h] - mn);
        pj = valid ? expf(lg - mn) : 0.f;
        l[h] = l[h] * alpha + pj;
        acc[h][0] *= alpha;
        acc[h][1] *= alpha;
        m[h] = mn;
      }
      s.pt[wid][h][lane] = pj;
    }
    wave_barrier();
    for (int j = 0; j < 64; ++j) {
      const uint64_t win = (uint64_t)s.vt[wid][j][vwi] | ((uint64_t)s.vt[wid][j][vwi + 1] << 32);
      const uint32_t two = (uint32_t)(win >> vsh);
      const float2 sc = s.vsc[wid][j];
      const float v0 = fmaf((float)(two & ((1u << BB) - 1u)) + 0.5f, sc.y, sc.x);
      const float v1 = fmaf((float)((two >> BB) & ((1u << BB) - 1u)) + 0.5f, sc.y, sc.x);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float w = s.pt[wid][h][j];
        acc[h][0] = fmaf(w, v0, acc[h][0]);
        acc[h][1] = fmaf(w, v1, acc[h][1]);
      }
    }
    wave_barrier();
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float ls = wave_sum(l[h]);
    if (lane == 0) {
      s.mw[wid][h] = m[h];
      s.lw[wid][h] = ls;
    }
    s.accw[wid][h][2 * lane] = acc[h][0];
    s.accw[wid][h][2 * lane + 1] = acc[h][1];
  }
  __syncthreads();
  float* part = p.part + ((int64_t)kvh * (p.n_sel_blk + p.n_split) + p.n_sel_blk + split) * G * kPartStride;
  write_partial<G, 4>(part, s.mw, s.lw, s.accw);
}

template <int BB, int G>
__global__ void __launch_bounds__(256) attend_valu(DecodeParams p) {
  __shared__ __align__(16) uint8_t smem[cmax(sizeof(SelLds<BB, G, 4, 16>), sizeof(ValuLds<BB, G>))];
  if ((int)blockIdx.x < p.n_sel_blk)
    selected_block_any<BB, G, 4, false>(p, blockIdx.x, blockIdx.y, smem);
  else
    base_split_valu<BB, G>(p, blockIdx.x - p.n_sel_blk, blockIdx.y, smem);
}

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

template <int BB>
static bool attend_g(const DecodeParams& p, dim3 grid, hipStream_t st, KernelEvents ev) {
  switch (p.grp) {
    case 1: sf_launch(attend_valu<BB, 1>, grid, dim3(256), st, ev, p); return true;
    case 2: sf_launch(attend_valu<BB, 2>, grid, dim3(256), st, ev, p); return true;
    case 4: sf_launch(attend_valu<BB, 4>, grid, dim3(256), st, ev, p); return true;
    case 8: sf_launch(attend_valu<BB, 8>, grid, dim3(256), st, ev, p); return true;
  }
  return false;
}

bool launch_attend_mfma(const DecodeParams& p, dim3 grid, hipStream_t st, KernelEvents ev);

bool launch_attend(const DecodeParams& p, dim3 grid, hipStream_t st, KernelEvents ev) {
  if (launch_attend_mfma(p, grid, st, ev)) return true;
  switch (p.b) {
    case 2: return attend_g<2>(p, grid, st, ev);
    case 3: return attend_g<3>(p, grid, st, ev);
    case 4: return attend_g<4>(p, grid, st, ev);
  }
  return false;
}

void launch_combine(const DecodeParams& p, hipStream_t st, KernelEvents ev) {
  if (p.batch > 1)
    sf_launch(combine<true>, dim3(p.batch * p.hq, kHeadDim / 32), dim3(256), st, ev, p);
  else
    sf_launch(combine<false>, dim3(p.batch * p.hq, kHeadDim / 32), dim3(256), st, ev, p);
}

}  // namespace sfk

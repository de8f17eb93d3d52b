// Token scoring from the resident base key codes.
//
// Page "StrataFlux -- Selective precision streaming -- What does it mean?",
// paragraph "Which tiles count ...": every cached token is scored by the
// attention it receives, computed from the resident low-bit keys.  The score
// of token i for KV head k is the maximum, over the query heads of k's GQA
// group, of the scaled logit q_h . Khat_i / sqrt(D).
//
// Folded dequantization: with Khat = lo + (c + 1/2) * delta,
//   q . Khat = lo * sum(q) + delta * (q . c + sum(q) / 2),
// so only the integer codes enter the inner products.
//
// Besides the scores, each work-group adds the top 12 bits of every score's
// order-preserving key into a per-(sequence, KV head) histogram (LDS first,
// then one global atomic per non-empty bin), the first radix level of the
// top-T selection.
#include <math.h>

#include "sf_decode_kernels.h"

namespace sfk {

constexpr float kRsqrtD = 0.08838834764831845f;   // 1 / sqrt(128)

// Work-group of 256 threads over one split of `score_split` tokens; one token
// per thread per iteration.
template <int BB, int G>
__global__ void __launch_bounds__(256) score_valu(DecodeParams p) {
  constexpr int W = 4 * BB;
  __shared__ float qs[G][kHeadDim];
  __shared__ float qsum[G];
  __shared__ uint32_t lhist[kHistBins];
  __shared__ uint32_t krow[256][W + 1];     // each thread's current K row

  const int tid = threadIdx.x;
  const int kvh = blockIdx.y;
  int64_t lo, hi;
  int first;
  const int seq = locate_unit(p, p.score_split, blockIdx.x, false, lo, hi, first);
  const int64_t a = seq_at(p, seq);
  for (int i = tid; i < G * kHeadDim; i += 256)
    qs[i / kHeadDim][i % kHeadDim] = p.q[((int64_t)seq * p.hq + kvh * G) * kHeadDim + i];
  const bool hist = p.top_t > 0;   // no selection, no histogram
  for (int i = tid; i < kHistBins; i += 256) lhist[i] = 0u;
  __syncthreads();
  if (tid < G) {
    float s = 0.f;
    for (int d = 0; d < kHeadDim; ++d) s += qs[tid][d];
    qsum[tid] = s;
  }
  __syncthreads();
  const uint8_t* kbase = p.kc + (int64_t)kvh * p.cap * (16 * BB);
  const float2* ksc = reinterpret_cast<const float2*>(p.ks) + (int64_t)kvh * p.cap;
  float* scores = p.scores + (int64_t)kvh * p.ntot + (a - p.off0);
  uint32_t* kw = krow[tid];
  for (int64_t i = lo + tid; i < hi; i += 256) {
    const int64_t tok = a + i;
    const uint4* src = reinterpret_cast<const uint4*>(kbase + tok * (16 * BB));
#pragma unroll
    for (int w = 0; w < BB; ++w) {
      const uint4 u = src[w];
      kw[4 * w] = u.x; kw[4 * w + 1] = u.y; kw[4 * w + 2] = u.z; kw[4 * w + 3] = u.w;
    }
    kw[W] = 0u;
    const float2 sk = ksc[tok];
    float dot[G];
#pragma unroll
    for (int h = 0; h < G; ++h) dot[h] = 0.f;
#pragma unroll 4
    for (int d = 0; d < kHeadDim; ++d) {
      const float c = (float)code_at<BB>(kw, d);
#pragma unroll
      for (int h = 0; h < G; ++h) dot[h] = fmaf(qs[h][d], c, dot[h]);
    }
    float best = -INFINITY;
#pragma unroll
    for (int h = 0; h < G; ++h)
      best = fmaxf(best, (sk.x * qsum[h] + sk.y * (dot[h] + 0.5f * qsum[h])) * kRsqrtD);
    scores[i] = best;
    if (hist) atomicAdd(&lhist[score_key(best) >> (32 - kHistBits)], 1u);
  }
  if (!hist) return;
  __syncthreads();
  uint32_t* gh = p.hist + ((int64_t)seq * p.hkv + kvh) * kHistBins;   // level-1 histogram
  for (int i = tid; i < kHistBins; i += 256) {
    const uint32_t c = lhist[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

template <int BB>
static bool score_g(const DecodeParams& p, dim3 grid, hipStream_t st, KernelEvents ev) {
  switch (p.grp) {
    case 1: sf_launch(score_valu<BB, 1>, grid, dim3(256), st, ev, p); return true;
    case 2: sf_launch(score_valu<BB, 2>, grid, dim3(256), st, ev, p); return true;
    case 4: sf_launch(score_valu<BB, 4>, grid, dim3(256), st, ev, p); return true;
    case 8: sf_launch(score_valu<BB, 8>, grid, dim3(256), st, ev, p); return true;
  }
  return false;
}

bool launch_score_mfma(const DecodeParams& p, dim3 grid, hipStream_t st, KernelEvents ev);

bool launch_score(const DecodeParams& p, dim3 grid, hipStream_t st, KernelEvents ev) {
  if (launch_score_mfma(p, grid, st, ev)) return true;
  switch (p.b) {
    case 2: return score_g<2>(p, grid, st, ev);
    case 3: return score_g<3>(p, grid, st, ev);
    case 4: return score_g<4>(p, grid, st, ev);
  }
  return false;
}

}  // namespace sfk

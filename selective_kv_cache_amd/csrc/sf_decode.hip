// The decode step (sf_decode_step): score, select, refine, attend.
//
// Method: page "StrataFlux -- Selective precision streaming -- What does it
// mean?", paragraph "Which tiles count ...": every cached token is scored by
// the attention it receives, computed from the resident low-bit keys; the
// highest-scoring tokens of each KV head (the set its GQA group of query heads
// shares) are refined; everything not selected still takes part at low
// precision.  Paragraph "What travels over the link ...": refinement bits
// subdivide the bin the base code names.
//
// Kernel sequence on the caller's stream (one layer):
//   zero_words          clear the histogram and counters of the step
//   score_attn          one pass over the base K and V codes of every token:
//                       base logits of the G query heads, the token score
//                       (max over the group), a histogram of the scores'
//                       order-preserving keys, and split-K online-softmax
//                       partials (m, l, acc[D]) of base-precision attention
//   select_top_t        per (sequence, KV head): threshold bin from the
//                       histogram, bitmap of tokens above it, candidates in
//                       it; the last work-group resolves the boundary exactly
//                       (score desc, token asc) and lists the selection
//   [host tier: cache lookup, fetch of the misses, install]
//   refine_correct      per selected token: refined and base logits/values;
//                       correction partials  sum e^{l~-m} v~ - e^{l^-m} v^
//   combine             merge base partials and corrections per query head
//
// Attention over all tokens with refined selected rows equals base attention
// plus, for each selected token, (refined term - base term) in both the
// numerator and the softmax denominator; the combine merges both sets of
// partials under one running maximum.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "sf_decode_kernels.h"

namespace sfk {

constexpr float kRsqrtD = 0.08838834764831845f;   // 1 / sqrt(128)

__global__ void zero_words(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// ---------------------------------------------------------------------------
// score_attn: grid (n_split, hkv), 4 wavefronts; each wavefront takes tiles of
// 64 tokens (one per lane) of the block's split.
// ---------------------------------------------------------------------------
template <int BB, int G>
__global__ void __launch_bounds__(256) score_attn_valu(DecodeParams p) {
  constexpr int W = 4 * BB;
  __shared__ float qs[G][kHeadDim];
  __shared__ float qsum[G];
  __shared__ uint32_t lhist[kHistBins];
  __shared__ uint32_t vt[4][64][W + 1];
  __shared__ float2 vsc[4][64];
  __shared__ float pt[4][G][64];
  __shared__ float mw[4][G], lw[4][G];
  __shared__ float accw[4][G][kHeadDim];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int kvh = blockIdx.y;
  int64_t lo, hi;
  int first;
  const int seq = locate_unit(p.seq_off, p.batch, p.split, blockIdx.x, false, 0, lo, hi, first);
  const int64_t a = p.seq_off[seq];
  const int64_t t0 = a + lo, t1 = a + hi;

  for (int i = tid; i < G * kHeadDim; i += 256)
    qs[i / kHeadDim][i % kHeadDim] = p.q[((int64_t)seq * p.hq + kvh * G) * kHeadDim + i];
  for (int i = tid; i < kHistBins; i += 256) lhist[i] = 0u;
  __syncthreads();
  if (tid < G) {
    float s = 0.f;
    for (int d = 0; d < kHeadDim; ++d) s += qs[tid][d];
    qsum[tid] = s;
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
  float* scores = p.scores + (int64_t)kvh * p.ntot;

  const int niter = (int)((t1 - t0 + 255) / 256);
  const int vpos = 2 * lane * BB, vwi = vpos >> 5, vsh = vpos & 31;
  for (int it = 0; it < niter; ++it) {
    const int64_t tok = t0 + (int64_t)it * 256 + wid * 64 + lane;
    const bool valid = tok < t1;
    uint32_t kw[W + 1];
    float2 sk = make_float2(0.f, 0.f);
    if (valid) {
      const uint4* src = reinterpret_cast<const uint4*>(kbase + tok * (16 * BB));
#pragma unroll
      for (int i = 0; i < BB; ++i) {
        const uint4 u = src[i];
        kw[4 * i] = u.x; kw[4 * i + 1] = u.y; kw[4 * i + 2] = u.z; kw[4 * i + 3] = u.w;
      }
      sk = ksc[tok];
    } else {
#pragma unroll
      for (int i = 0; i < W; ++i) kw[i] = 0u;
    }
    kw[W] = 0u;
    float dot[G];
#pragma unroll
    for (int h = 0; h < G; ++h) dot[h] = 0.f;
#pragma unroll
    for (int d = 0; d < kHeadDim; ++d) {
      const float c = (float)code_at<BB>(kw, d);
#pragma unroll
      for (int h = 0; h < G; ++h) dot[h] = fmaf(qs[h][d], c, dot[h]);
    }
    float lg[G];
    float best = -INFINITY;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      lg[h] = (sk.x * qsum[h] + sk.y * (dot[h] + 0.5f * qsum[h])) * kRsqrtD;
      best = fmaxf(best, lg[h]);
    }
    if (valid) {
      scores[tok - p.off0] = best;
      atomicAdd(&lhist[score_key(best) >> (32 - kHistBits)], 1u);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mt = wave_max(valid ? lg[h] : -INFINITY);
      const float mn = fmaxf(m[h], mt);
      float pj = 0.f;
      if (mn != -INFINITY) {
        const float alpha = expf(m[h] - mn);
        pj = valid ? expf(lg[h] - mn) : 0.f;
        l[h] = l[h] * alpha + pj;
        acc[h][0] *= alpha;
        acc[h][1] *= alpha;
        m[h] = mn;
      }
      pt[wid][h][lane] = pj;
    }
    if (valid) {
      const uint4* src = reinterpret_cast<const uint4*>(vbase + tok * (16 * BB));
#pragma unroll
      for (int i = 0; i < BB; ++i) {
        const uint4 u = src[i];
        vt[wid][lane][4 * i] = u.x; vt[wid][lane][4 * i + 1] = u.y;
        vt[wid][lane][4 * i + 2] = u.z; vt[wid][lane][4 * i + 3] = u.w;
      }
      vsc[wid][lane] = vscg[tok];
    } else {
#pragma unroll
      for (int i = 0; i < W; ++i) vt[wid][lane][i] = 0u;
      vsc[wid][lane] = make_float2(0.f, 0.f);
    }
    vt[wid][lane][W] = 0u;
    wave_barrier();
    for (int j = 0; j < 64; ++j) {
      const uint64_t win = (uint64_t)vt[wid][j][vwi] | ((uint64_t)vt[wid][j][vwi + 1] << 32);
      const uint32_t two = (uint32_t)(win >> vsh);
      const float c0 = (float)(two & ((1u << BB) - 1u));
      const float c1 = (float)((two >> BB) & ((1u << BB) - 1u));
      const float2 sc = vsc[wid][j];
      const float v0 = fmaf(c0 + 0.5f, sc.y, sc.x);
      const float v1 = fmaf(c1 + 0.5f, sc.y, sc.x);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float w = pt[wid][h][j];
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
      mw[wid][h] = m[h];
      lw[wid][h] = ls;
    }
    accw[wid][h][2 * lane] = acc[h][0];
    accw[wid][h][2 * lane + 1] = acc[h][1];
  }
  __syncthreads();
  float* part = p.part + ((int64_t)kvh * p.n_split + blockIdx.x) * G * kPartStride;
  for (int i = tid; i < G * kHeadDim; i += 256) {
    const int h = i / kHeadDim, d = i % kHeadDim;
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mw[w][h]);
    float A = 0.f, L = 0.f;
    for (int w = 0; w < 4; ++w) {
      if (mw[w][h] == -INFINITY) continue;
      const float e = expf(mw[w][h] - M);
      A += e * accw[w][h][d];
      L += e * lw[w][h];
    }
    part[h * kPartStride + d] = A;
    if (d == 0) {
      part[h * kPartStride + kHeadDim] = M;
      part[h * kPartStride + kHeadDim + 1] = L;
    }
  }
  uint32_t* gh = p.hist + ((int64_t)seq * p.hkv + kvh) * kHistBins;
  for (int i = tid; i < kHistBins; i += 256) {
    const uint32_t c = lhist[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

// ---------------------------------------------------------------------------
// select_top_t: grid (n_sel_chunk, hkv), 256 threads.
// ---------------------------------------------------------------------------
__device__ inline uint64_t cand_value(uint2 c) {
  // low 20 key bits (the top 12 are the threshold bin) over the inverted token
  // index: a larger value ranks first, and no two candidates are equal
  return ((uint64_t)(c.x & 0xFFFFFu) << 32) | (uint64_t)(0xFFFFFFFFu - c.y);
}

__global__ void __launch_bounds__(256) select_top_t(DecodeParams p) {
  __shared__ uint32_t sh_hist[kHistBins];
  __shared__ uint32_t sh_part[256];
  __shared__ uint32_t rh[256];
  __shared__ int sh_b1, sh_need, sh_last, sh_d, sh_exact;
  __shared__ uint32_t sh_cnt[256];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int kvh = blockIdx.y;
  int64_t lo, hi;
  int first;
  const int seq = locate_unit(p.seq_off, p.batch, p.sel_chunk, blockIdx.x, false, 0, lo, hi, first);
  const int64_t a = p.seq_off[seq];
  const int64_t n = p.seq_off[seq + 1] - a;
  const int64_t tn = n < p.top_t ? n : (int64_t)p.top_t;
  const bool all = (tn == n);
  const int64_t sk = (int64_t)seq * p.hkv + kvh;
  uint32_t* bm = p.bitmap + sk * p.bm_words;
  const float* sc = p.scores + (int64_t)kvh * p.ntot + (a - p.off0);

  if (!all) {
    const uint32_t* gh = p.hist + sk * kHistBins;
    uint32_t part = 0;
    for (int i = 0; i < kHistBins / 256; ++i) {
      const uint32_t c = gh[tid * (kHistBins / 256) + i];
      sh_hist[tid * (kHistBins / 256) + i] = c;
      part += c;
    }
    sh_part[tid] = part;
    __syncthreads();
    if (tid == 0) {
      uint32_t cum = 0;
      int t = 255;
      for (; t > 0 && cum + sh_part[t] < (uint32_t)tn; --t) cum += sh_part[t];
      int b = t * (kHistBins / 256) + (kHistBins / 256) - 1;
      for (; b > t * (kHistBins / 256) && cum + sh_hist[b] < (uint32_t)tn; --b) cum += sh_hist[b];
      sh_b1 = b;
      sh_need = (int)((uint32_t)tn - cum);
    }
    __syncthreads();
  }
  const uint32_t b1 = all ? 0u : (uint32_t)sh_b1;
  for (int64_t base = lo; base < hi; base += 256) {
    const int64_t i = base + tid;
    const bool valid = i < hi;
    bool s = false, cnd = false;
    uint32_t key = 0;
    if (valid) {
      if (all) {
        s = true;
      } else {
        key = score_key(sc[i]);
        const uint32_t bin = key >> (32 - kHistBits);
        s = bin > b1;
        cnd = bin == b1;
      }
    }
    const uint64_t bal = __ballot(s);
    if (lane == 0) {
      const int64_t w = (base + wid * 64) >> 5;
      bm[w] = (uint32_t)bal;
      bm[w + 1] = (uint32_t)(bal >> 32);
    }
    const uint64_t cb = __ballot(cnd);
    if (cb) {
      uint32_t at = 0;
      if (lane == 0) at = atomicAdd(&p.counters[sk * 4 + 0], (uint32_t)__popcll(cb));
      at = __shfl(at, 0);
      if (cnd) {
        const uint32_t off = (uint32_t)__popcll(cb & ((1ull << lane) - 1ull));
        p.cand[sk * p.max_seq + at + off] = make_uint2(key, (uint32_t)i);
      }
    }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t nchunks = (uint32_t)((n + p.sel_chunk - 1) / p.sel_chunk);
    sh_last = atomicAdd(&p.counters[sk * 4 + 1], 1u) == nchunks - 1u;
  }
  __syncthreads();
  if (!sh_last) return;
  __threadfence();

  if (!all) {
    // Exact boundary: radix select over the candidates' 56-bit values, 8 bits
    // per pass, until the remaining need is met by a whole digit bucket.
    const uint32_t ncand = __atomic_load_n(&p.counters[sk * 4 + 0], __ATOMIC_RELAXED);
    const uint2* cand = p.cand + sk * p.max_seq;
    uint32_t need = (uint32_t)sh_need;
    uint64_t prefix = 0, mask = 0;
    for (int shift = 48; shift >= 0; shift -= 8) {
      rh[tid] = 0u;
      __syncthreads();
      for (uint32_t c = tid; c < ncand; c += 256) {
        const uint64_t v = cand_value(cand[c]);
        if ((v & mask) == prefix) atomicAdd(&rh[(v >> shift) & 0xFFu], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        uint32_t cum = 0;
        int d = 255;
        for (; d > 0 && cum + rh[d] < need; --d) cum += rh[d];
        sh_d = d;
        sh_need = (int)(need - cum);
        sh_exact = (rh[d] == need - cum);
      }
      __syncthreads();
      prefix |= (uint64_t)sh_d << shift;
      mask |= 0xFFull << shift;
      need = (uint32_t)sh_need;
      if (sh_exact) break;
      __syncthreads();
    }
    for (uint32_t c = tid; c < ncand; c += 256) {
      const uint2 cv = cand[c];
      if ((cand_value(cv) & mask) >= prefix) atomicOr(&bm[cv.y >> 5], 1u << (cv.y & 31u));
    }
    __threadfence_block();
    __syncthreads();
  }

  // List the selection in ascending token order.
  const int64_t nw = (n + 31) >> 5;
  const int64_t per = (nw + 255) / 256;
  const int64_t w0 = tid * per, w1 = w0 + per < nw ? w0 + per : nw;
  uint32_t cnt = 0;
  for (int64_t w = w0; w < w1; ++w) cnt += __popc(bm[w]);
  sh_cnt[tid] = cnt;
  __syncthreads();
  if (tid == 0) {
    uint32_t run = 0;
    for (int t = 0; t < 256; ++t) {
      const uint32_t c = sh_cnt[t];
      sh_cnt[t] = run;
      run += c;
    }
  }
  __syncthreads();
  int32_t* sel = p.sel + sk * p.top_t;
  int32_t* selo = p.sel_out ? p.sel_out + sk * p.top_t : nullptr;
  uint32_t pos = sh_cnt[tid];
  for (int64_t w = w0; w < w1; ++w) {
    uint32_t bits = bm[w];
    while (bits) {
      const int bit = __ffs(bits) - 1;
      bits &= bits - 1u;
      const int32_t idx = (int32_t)((w << 5) + bit);
      if (pos < (uint32_t)p.top_t) {
        sel[pos] = idx;
        if (selo) selo[pos] = idx;
      }
      ++pos;
    }
  }
  for (int64_t j = tn + tid; j < p.top_t; j += 256) {
    sel[j] = -1;
    if (selo) selo[j] = -1;
  }
}

// ---------------------------------------------------------------------------
// refine_correct: grid (n_corr, hkv), 4 wavefronts of 64 selected tokens.
// ---------------------------------------------------------------------------
template <int BB, int G>
__global__ void __launch_bounds__(256) refine_correct(DecodeParams p) {
  constexpr int W = 4 * BB;
  __shared__ float qs[G][kHeadDim];
  __shared__ float qsum[G];
  __shared__ uint32_t vt[4][64][W + 1];
  __shared__ uint32_t vr[4][64][33];
  __shared__ float2 vsc[4][64];
  __shared__ float wt[4][G][64], wh[4][G][64];
  __shared__ float mred[4][G];
  __shared__ float lw[4][G];
  __shared__ float accw[4][G][kHeadDim];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int kvh = blockIdx.y;
  int64_t lo, hi;
  int first;
  const int seq = locate_unit(p.seq_off, p.batch, p.corr_chunk, blockIdx.x, true, p.top_t, lo, hi, first);
  const int64_t a = p.seq_off[seq];
  const int64_t sk = (int64_t)seq * p.hkv + kvh;
  const int r = p.r, rb = p.rb, rw = rb >> 2;
  const float sub = __builtin_ldexpf(1.0f, -r);

  for (int i = tid; i < G * kHeadDim; i += 256)
    qs[i / kHeadDim][i % kHeadDim] = p.q[((int64_t)seq * p.hq + kvh * G) * kHeadDim + i];
  __syncthreads();
  if (tid < G) {
    float s = 0.f;
    for (int d = 0; d < kHeadDim; ++d) s += qs[tid][d];
    qsum[tid] = s;
  }
  __syncthreads();

  const int64_t j = lo + tid;
  const bool valid = j < hi;
  int64_t tok = 0;
  const uint8_t* kref = nullptr;
  const uint8_t* vref = nullptr;
  if (valid) {
    tok = a + p.sel[sk * p.top_t + j];
    if (p.ref_rows) {
      kref = p.ref_rows + (((int64_t)0 * p.hkv + kvh) * p.cap + tok) * rb;
      vref = p.ref_rows + (((int64_t)1 * p.hkv + kvh) * p.cap + tok) * rb;
    } else {
      int32_t slot = p.tok_slot[(int64_t)kvh * p.cap + tok];
      slot = slot < 0 ? 0 : slot;   // installed by the lookup; never negative when consistent
      const uint8_t* base = p.cache_data + ((sk * p.slots + slot) * 2) * (int64_t)rb;
      kref = base;
      vref = base + rb;
    }
  }
  // this lane's K rows (base + refinement) go through its own LDS row
  uint32_t* myb = vt[wid][lane];
  uint32_t* myr = vr[wid][lane];
  for (int i = 0; i <= W; ++i) myb[i] = 0u;
  for (int i = 0; i < 33; ++i) myr[i] = 0u;
  float2 sk2 = make_float2(0.f, 0.f);
  if (valid) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(p.kc + ((int64_t)kvh * p.cap + tok) * (16 * BB));
    for (int i = 0; i < W; ++i) myb[i] = src[i];
    const uint32_t* rs = reinterpret_cast<const uint32_t*>(kref);
    for (int i = 0; i < rw; ++i) myr[i] = rs[i];
    sk2 = reinterpret_cast<const float2*>(p.ks)[(int64_t)kvh * p.cap + tok];
  }
  float dc[G], ds[G];
#pragma unroll
  for (int h = 0; h < G; ++h) dc[h] = ds[h] = 0.f;
  const uint32_t rmask = (1u << r) - 1u;
#pragma unroll 4
  for (int d = 0; d < kHeadDim; ++d) {
    const float c = (float)code_at<BB>(myb, d);
    const int pos = d * r, wi = pos >> 5, sh = pos & 31;
    const uint64_t win = (uint64_t)myr[wi] | ((uint64_t)myr[wi + 1] << 32);
    const float sv = (float)((uint32_t)(win >> sh) & rmask);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      dc[h] = fmaf(qs[h][d], c, dc[h]);
      ds[h] = fmaf(qs[h][d], sv, ds[h]);
    }
  }
  float lb[G], lr[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float base = sk2.x * qsum[h];
    lb[h] = (base + sk2.y * (dc[h] + 0.5f * qsum[h])) * kRsqrtD;
    lr[h] = (base + sk2.y * (dc[h] + (ds[h] + 0.5f * qsum[h]) * sub)) * kRsqrtD;
    const float mv = wave_max(valid ? fmaxf(lb[h], lr[h]) : -INFINITY);
    if (lane == 0) mred[wid][h] = mv;
  }
  __syncthreads();
  float acc[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float M = fmaxf(fmaxf(mred[0][h], mred[1][h]), fmaxf(mred[2][h], mred[3][h]));
    const float e1 = valid ? expf(lr[h] - M) : 0.f;
    const float e0 = valid ? expf(lb[h] - M) : 0.f;
    wt[wid][h][lane] = e1;
    wh[wid][h][lane] = e0;
    const float ls = wave_sum(e1 - e0);
    if (lane == 0) lw[wid][h] = ls;
    acc[h][0] = acc[h][1] = 0.f;
  }
  // stage this wavefront's V rows
  wave_barrier();
  for (int i = 0; i <= W; ++i) vt[wid][lane][i] = 0u;
  for (int i = 0; i < 33; ++i) vr[wid][lane][i] = 0u;
  vsc[wid][lane] = make_float2(0.f, 0.f);
  if (valid) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(p.vc + ((int64_t)kvh * p.cap + tok) * (16 * BB));
    for (int i = 0; i < W; ++i) vt[wid][lane][i] = src[i];
    const uint32_t* rs = reinterpret_cast<const uint32_t*>(vref);
    for (int i = 0; i < rw; ++i) vr[wid][lane][i] = rs[i];
    vsc[wid][lane] = reinterpret_cast<const float2*>(p.vs)[(int64_t)kvh * p.cap + tok];
  }
  wave_barrier();
  const int cpos = 2 * lane * BB, cwi = cpos >> 5, csh = cpos & 31;
  const int rpos = 2 * lane * r, rwi = rpos >> 5, rsh = rpos & 31;
  for (int jj = 0; jj < 64; ++jj) {
    const uint64_t cwin = (uint64_t)vt[wid][jj][cwi] | ((uint64_t)vt[wid][jj][cwi + 1] << 32);
    const uint32_t cc = (uint32_t)(cwin >> csh);
    const uint64_t rwin = (uint64_t)vr[wid][jj][rwi] | ((uint64_t)vr[wid][jj][rwi + 1] << 32);
    const uint32_t rr = (uint32_t)(rwin >> rsh);
    const float c0 = (float)(cc & ((1u << BB) - 1u)), c1 = (float)((cc >> BB) & ((1u << BB) - 1u));
    const float s0 = (float)(rr & rmask), s1 = (float)((rr >> r) & rmask);
    const float2 sc = vsc[wid][jj];
    const float vb0 = fmaf(c0 + 0.5f, sc.y, sc.x), vb1 = fmaf(c1 + 0.5f, sc.y, sc.x);
    const float vr0 = fmaf((s0 + 0.5f) * sub, sc.y, fmaf(c0, sc.y, sc.x));
    const float vr1 = fmaf((s1 + 0.5f) * sub, sc.y, fmaf(c1, sc.y, sc.x));
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float w1 = wt[wid][h][jj], w0 = wh[wid][h][jj];
      acc[h][0] = fmaf(w1, vr0, fmaf(-w0, vb0, acc[h][0]));
      acc[h][1] = fmaf(w1, vr1, fmaf(-w0, vb1, acc[h][1]));
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    accw[wid][h][2 * lane] = acc[h][0];
    accw[wid][h][2 * lane + 1] = acc[h][1];
  }
  __syncthreads();
  float* corr = p.corr + ((int64_t)kvh * p.n_corr + blockIdx.x) * G * kPartStride;
  for (int i = tid; i < G * kHeadDim; i += 256) {
    const int h = i / kHeadDim, d = i % kHeadDim;
    corr[h * kPartStride + d] = accw[0][h][d] + accw[1][h][d] + accw[2][h][d] + accw[3][h][d];
    if (d == 0) {
      corr[h * kPartStride + kHeadDim] =
          fmaxf(fmaxf(mred[0][h], mred[1][h]), fmaxf(mred[2][h], mred[3][h]));
      corr[h * kPartStride + kHeadDim + 1] = lw[0][h] + lw[1][h] + lw[2][h] + lw[3][h];
    }
  }
}

// ---------------------------------------------------------------------------
// combine: one work-group of 128 threads per (sequence, query head).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(128) combine(DecodeParams p, int use_corr) {
  const int s = blockIdx.x / p.hq, h = blockIdx.x % p.hq;
  const int kvh = h / p.grp, hg = h % p.grp, d = threadIdx.x;
  int sb = 0, cb = 0;
  for (int i = 0; i < s; ++i) {
    const int64_t n = p.seq_off[i + 1] - p.seq_off[i];
    sb += (int)((n + p.split - 1) / p.split);
    const int64_t tn = n < p.top_t ? n : p.top_t;
    cb += (int)((tn + p.corr_chunk - 1) / p.corr_chunk);
  }
  const int64_t n = p.seq_off[s + 1] - p.seq_off[s];
  const int se = sb + (int)((n + p.split - 1) / p.split);
  const int64_t tn = n < p.top_t ? n : p.top_t;
  const int ce = use_corr ? cb + (int)((tn + p.corr_chunk - 1) / p.corr_chunk) : cb;
  const float* part = p.part + (int64_t)kvh * p.n_split * p.grp * kPartStride;
  const float* corr = p.corr + (int64_t)kvh * p.n_corr * p.grp * kPartStride;
  float M = -INFINITY;
  for (int x = sb; x < se; ++x) M = fmaxf(M, part[(x * p.grp + hg) * kPartStride + kHeadDim]);
  for (int x = cb; x < ce; ++x) M = fmaxf(M, corr[(x * p.grp + hg) * kPartStride + kHeadDim]);
  float num = 0.f, den = 0.f;
  for (int x = sb; x < se; ++x) {
    const float* pp = part + (x * p.grp + hg) * kPartStride;
    const float e = expf(pp[kHeadDim] - M);
    num += e * pp[d];
    den += e * pp[kHeadDim + 1];
  }
  for (int x = cb; x < ce; ++x) {
    const float* pp = corr + (x * p.grp + hg) * kPartStride;
    const float e = expf(pp[kHeadDim] - M);
    num += e * pp[d];
    den += e * pp[kHeadDim + 1];
  }
  p.out[((int64_t)s * p.hq + h) * kHeadDim + d] = num / den;
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int32_t choose_split(int64_t total_tokens, int32_t n_kv_heads) {
  const int64_t work = total_tokens * n_kv_heads;
  int32_t s = 256;
  while (s < 2048 && work / s > 2048) s *= 2;
  return s;
}

constexpr int32_t kSelChunk = 4096;
constexpr int32_t kCorrChunk = 256;

Carve carve(const sf_geom& g, int32_t batch, int64_t total_tokens, int64_t max_seq_tokens,
            int32_t top_t, int32_t n_split_bound, int32_t n_corr_bound) {
  const int grp = g.n_q_heads / g.n_kv_heads;
  const int64_t hkv = g.n_kv_heads;
  const int64_t bm_words = ((max_seq_tokens + 255) / 256) * 8;
  Carve c{};
  size_t at = 0;
  c.scores = at; at += align256((size_t)hkv * total_tokens * 4);
  c.hist = at; at += align256((size_t)batch * hkv * kHistBins * 4);
  c.counters = at; at += align256((size_t)batch * hkv * 4 * 4);
  c.cand = at; at += align256((size_t)batch * hkv * max_seq_tokens * 8);
  c.bitmap = at; at += align256((size_t)batch * hkv * bm_words * 4);
  c.sel = at; at += align256((size_t)batch * hkv * (top_t > 0 ? top_t : 1) * 4);
  c.part = at; at += align256((size_t)hkv * n_split_bound * grp * kPartStride * 4);
  c.corr = at; at += align256((size_t)hkv * (n_corr_bound > 0 ? n_corr_bound : 1) * grp * kPartStride * 4);
  c.miss = at; at += align256((size_t)batch * hkv * (2 * ((top_t > 0 ? top_t : 1) + 1) + 1) * 4);
  c.total = at;
  return c;
}

static int32_t split_bound(int64_t total, int32_t batch, int32_t split) {
  return (int32_t)(total / split + batch);
}
static int32_t corr_bound(int32_t batch, int32_t top_t) {
  return batch * ((top_t + kCorrChunk - 1) / kCorrChunk);
}

template <int BB, int G>
static void launch_kernel(bool score, const DecodeParams& p, dim3 grid, hipStream_t st) {
  if (score)
    hipLaunchKernelGGL((score_attn_valu<BB, G>), grid, dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((refine_correct<BB, G>), grid, dim3(256), 0, st, p);
}

template <int BB>
static bool dispatch_g(int grp, bool score, const DecodeParams& p, dim3 grid, hipStream_t st) {
  switch (grp) {
    case 1: launch_kernel<BB, 1>(score, p, grid, st); return true;
    case 2: launch_kernel<BB, 2>(score, p, grid, st); return true;
    case 4: launch_kernel<BB, 4>(score, p, grid, st); return true;
    case 8: launch_kernel<BB, 8>(score, p, grid, st); return true;
  }
  return false;
}

// score == true: score_attn; false: refine_correct.
static bool dispatch(bool score, const DecodeParams& p, dim3 grid, hipStream_t st) {
  switch (p.b) {
    case 2: return dispatch_g<2>(p.grp, score, p, grid, st);
    case 3: return dispatch_g<3>(p.grp, score, p, grid, st);
    case 4: return dispatch_g<4>(p.grp, score, p, grid, st);
  }
  return false;
}

}  // namespace sfk

using namespace sfk;

// Host-tier fetch (sf_store.hip): lookup, copy of the misses, install.
sf_status sf_store_fetch(sf_store store, const DecodeParams& p, int32_t* miss_dev, hipStream_t st,
                         sf_step_stats* stats);

extern "C" sf_status sf_decode_workspace_size(const sf_geom* geom, int32_t batch, int64_t total_tokens,
                                              int64_t max_seq_tokens, int32_t top_t, size_t* bytes) {
  clear_error();
  sf_status s = sf_check_geom(geom);
  if (s != SF_OK) return s;
  if (!bytes || batch <= 0 || total_tokens <= 0 || max_seq_tokens <= 0 || top_t < 0 ||
      max_seq_tokens > total_tokens)
    return SF_ERR_INVALID_ARG;
  if (max_seq_tokens > 0x7fffffffLL) return SF_ERR_UNSUPPORTED;
  const int32_t split = choose_split(total_tokens, geom->n_kv_heads);
  *bytes = carve(*geom, batch, total_tokens, max_seq_tokens, top_t, split_bound(total_tokens, batch, split),
                 corr_bound(batch, top_t)).total;
  return SF_OK;
}

extern "C" sf_status sf_decode_step(const sf_geom* geom, const sf_decode_args* a, void* stream) {
  clear_error();
  sf_status s = sf_check_geom(geom);
  if (s != SF_OK) return s;
  if (!a || a->batch <= 0 || !a->seq_off_host || !a->seq_off_dev || !a->q || !a->k_codes ||
      !a->k_scales || !a->v_codes || !a->v_scales || !a->out || !a->workspace || a->cap <= 0 ||
      a->top_t < 0 || a->flags != 0 || (!a->score_events[0] != !a->score_events[1]))
    return SF_ERR_INVALID_ARG;
  const int32_t B = a->batch;
  const int64_t* off = a->seq_off_host;
  if (off[0] < 0) return SF_ERR_INVALID_ARG;
  int64_t max_seq = 0;
  for (int i = 0; i < B; ++i) {
    const int64_t n = off[i + 1] - off[i];
    if (n <= 0) return SF_ERR_INVALID_ARG;   // softmax over an empty set is undefined
    max_seq = std::max(max_seq, n);
  }
  if (off[B] > a->cap) return SF_ERR_INVALID_ARG;
  if (max_seq > 0x7fffffffLL) return SF_ERR_UNSUPPORTED;
  const int64_t total = off[B] - off[0];
  const bool refine = a->top_t > 0 && geom->refine_bits > 0;
  if (refine) {
    if (!a->store) return SF_ERR_INVALID_ARG;
    const sf_store_s* st = a->store;
    if (st->g.head_dim != geom->head_dim || st->g.n_kv_heads != geom->n_kv_heads ||
        st->g.refine_bits != geom->refine_bits || st->cap < off[B])
      return SF_ERR_INVALID_ARG;
    if (st->tier == SF_TIER_HOST_PINNED && (B > st->max_seqs || a->top_t > st->slots))
      return SF_ERR_INVALID_ARG;
  }
  const int32_t split = choose_split(total, geom->n_kv_heads);
  const Carve c = carve(*geom, B, total, max_seq, a->top_t, split_bound(total, B, split),
                        corr_bound(B, a->top_t));
  if (a->workspace_bytes < c.total) return SF_ERR_INVALID_ARG;

  int32_t n_split = 0, n_sel = 0, n_corr = 0;
  for (int i = 0; i < B; ++i) {
    const int64_t n = off[i + 1] - off[i];
    n_split += (int32_t)((n + split - 1) / split);
    n_sel += (int32_t)((n + kSelChunk - 1) / kSelChunk);
    const int64_t tn = std::min<int64_t>(n, a->top_t);
    n_corr += (int32_t)((tn + kCorrChunk - 1) / kCorrChunk);
  }

  uint8_t* ws = static_cast<uint8_t*>(a->workspace);
  DecodeParams p{};
  p.batch = B;
  p.hq = geom->n_q_heads;
  p.hkv = geom->n_kv_heads;
  p.grp = geom->n_q_heads / geom->n_kv_heads;
  p.b = geom->base_bits;
  p.r = geom->refine_bits;
  p.top_t = a->top_t;
  p.split = split;
  p.sel_chunk = kSelChunk;
  p.corr_chunk = kCorrChunk;
  p.n_split = n_split;
  p.n_corr = n_corr;
  p.bm_words = (int32_t)(((max_seq + 255) / 256) * 8);
  p.cap = a->cap;
  p.ntot = total;
  p.off0 = off[0];
  p.max_seq = max_seq;
  p.seq_off = a->seq_off_dev;
  p.q = a->q;
  p.kc = a->k_codes;
  p.ks = a->k_scales;
  p.vc = a->v_codes;
  p.vs = a->v_scales;
  p.scores = a->scores_out ? a->scores_out : reinterpret_cast<float*>(ws + c.scores);
  p.hist = reinterpret_cast<uint32_t*>(ws + c.hist);
  p.counters = reinterpret_cast<uint32_t*>(ws + c.counters);
  p.cand = reinterpret_cast<uint2*>(ws + c.cand);
  p.bitmap = reinterpret_cast<uint32_t*>(ws + c.bitmap);
  p.sel = reinterpret_cast<int32_t*>(ws + c.sel);
  p.sel_out = a->sel_out;
  p.part = reinterpret_cast<float*>(ws + c.part);
  p.corr = reinterpret_cast<float*>(ws + c.corr);
  p.out = a->out;
  if (refine) {
    sf_store_s* st = a->store;
    p.rb = st->row_bytes;
    p.slots = st->slots;
    if (st->tier == SF_TIER_DEVICE) {
      p.ref_rows = st->dev_rows;
    } else {
      p.cache_data = st->cache_data;
      p.tok_slot = st->tok_slot;
    }
  }

  hipStream_t hs = (hipStream_t)stream;
  const int64_t nzero = (c.counters + (size_t)B * p.hkv * 16 - c.hist) / 4;
  hipLaunchKernelGGL(zero_words, dim3((unsigned)std::min<int64_t>((nzero + 255) / 256, 1024)), dim3(256), 0, hs,
                     reinterpret_cast<uint32_t*>(ws + c.hist), nzero);
  SF_LAUNCH_CHECK("zero_words");
  if (a->score_events[0]) SF_HIP_CHECK(hipEventRecord((hipEvent_t)a->score_events[0], hs));
  if (!dispatch(true, p, dim3(n_split, p.hkv), hs)) return SF_ERR_UNSUPPORTED;
  SF_LAUNCH_CHECK("score_attn");
  if (a->score_events[1]) SF_HIP_CHECK(hipEventRecord((hipEvent_t)a->score_events[1], hs));
  if (a->top_t > 0) {
    hipLaunchKernelGGL(select_top_t, dim3(n_sel, p.hkv), dim3(256), 0, hs, p);
    SF_LAUNCH_CHECK("select_top_t");
  }
  if (a->stats) {
    memset(a->stats, 0, sizeof(*a->stats));
    int64_t sel = 0;
    for (int i = 0; i < B; ++i) sel += std::min<int64_t>(off[i + 1] - off[i], a->top_t);
    a->stats->selected = sel * p.hkv;
  }
  if (refine) {
    if (a->store->tier == SF_TIER_HOST_PINNED) {
      s = sf_store_fetch(a->store, p, reinterpret_cast<int32_t*>(ws + c.miss), hs, a->stats);
      if (s != SF_OK) return s;
      if (a->stats) a->stats->hits = a->stats->selected - a->stats->misses;
    }
    if (!dispatch(false, p, dim3(n_corr, p.hkv), hs)) return SF_ERR_UNSUPPORTED;
    SF_LAUNCH_CHECK("refine_correct");
  }
  hipLaunchKernelGGL(combine, dim3(B * p.hq), dim3(128), 0, hs, p, refine ? 1 : 0);
  SF_LAUNCH_CHECK("combine");
  return SF_OK;
}

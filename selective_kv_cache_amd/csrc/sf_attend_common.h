// Pieces shared by the attention kernels: the selected-token work-group and
// the per-wavefront partial merge.
//
// Page "StrataFlux -- Selective precision streaming -- What does it mean?",
// paragraph "What travels over the link ...": a selected element is
//   lo + c * delta + (s + 1/2) * delta / 2^r
// (the r fetched bits name a sub-bin of the base code's bin).  Attention runs
// over all tokens; the selected tokens' terms are computed here with their
// refined keys and values, the other tokens' terms by the base pass, each
// into partials (m, l, acc[D]) that only ever add positive weights.
#pragma once

#include "sf_decode_kernels.h"

namespace sfk {

constexpr float kRsqrtD = 0.08838834764831845f;   // 1 / sqrt(128)

constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }

// Refinement row (rb bytes) of token `tok`: K when which == 0, V when 1.
__device__ inline const uint32_t* refine_row(const DecodeParams& p, int64_t sk, int kvh, int64_t tok, int which) {
  if (p.ref_rows)
    return reinterpret_cast<const uint32_t*>(p.ref_rows + (((int64_t)which * p.hkv + kvh) * p.cap + tok) * p.rb);
  int32_t slot = p.tok_slot[(int64_t)kvh * p.cap + tok];
  slot = slot < 0 ? 0 : slot;   // installed by the lookup; never negative when consistent
  return reinterpret_cast<const uint32_t*>(p.cache_data + ((sk * p.slots + slot) * 2 + which) * (int64_t)p.rb);
}

// Dot products of one quarter of head_dim (32 elements) with the G query
// heads: base codes (BB bits), refinement codes (R bits), and the sum of the
// query elements.
template <int BB, int R, int G>
__device__ inline void quarter_dots(const uint32_t* kb, const uint32_t* kr, const float* qs, int qd, float* dc,
                                    float* ds, float* dq) {
#pragma unroll
  for (int h = 0; h < G; ++h) dc[h] = ds[h] = dq[h] = 0.f;
#pragma unroll
  for (int d = 0; d < 32; ++d) {
    const float c = (float)code_at<BB>(kb, d);
    const float s = (float)code_at<R>(kr, d);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float qv = qs[h * kHeadDim + qd * 32 + d];
      dc[h] = fmaf(qv, c, dc[h]);
      ds[h] = fmaf(qv, s, ds[h]);
      dq[h] += qv;
    }
  }
}

// The refinement-code part alone: q . s over one quarter of head_dim, and the
// sum of the query elements.
template <int R, int G>
__device__ inline void quarter_dots_ref(const uint32_t* kr, const float* qs, int qd, float* ds, float* dq) {
#pragma unroll
  for (int h = 0; h < G; ++h) ds[h] = dq[h] = 0.f;
#pragma unroll
  for (int d = 0; d < 32; ++d) {
    const float s = (float)code_at<R>(kr, d);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float qv = qs[h * kHeadDim + qd * 32 + d];
      ds[h] = fmaf(qv, s, ds[h]);
      dq[h] += qv;
    }
  }
}

// Sum over the four lanes of a quad (DPP quad permutes).
__device__ inline float quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
}

// Merge the NW wavefronts' (m, l, acc) of a work-group into one partial.
// mw/lw [NW][G], accw [NW][R >= G][D] in LDS (rows past G unused); called by
// all 64 NW threads after a barrier.
template <int G, int NW, int R = G>
__device__ inline void write_partial(float* part, const float (*mw)[G], const float (*lw)[G],
                                     const float (*accw)[R][kHeadDim]) {
  for (int i = threadIdx.x; i < G * kHeadDim; i += 64 * NW) {
    const int h = i / kHeadDim, d = i % kHeadDim;
    float M = -INFINITY;
    for (int w = 0; w < NW; ++w) M = fmaxf(M, mw[w][h]);
    float A = 0.f, L = 0.f;
    if (M != -INFINITY) {
      for (int w = 0; w < NW; ++w) {
        if (mw[w][h] == -INFINITY) continue;
        const float e = expf(mw[w][h] - M);
        A += e * accw[w][h][d];
        L += e * lw[w][h];
      }
    }
    part[h * kPartStride + d] = A;
    if (d == 0) {
      part[h * kPartStride + kHeadDim] = M;
      part[h * kPartStride + kHeadDim + 1] = L;
    }
  }
}

// write_partial for waves that share one maximum (mall[w][h] equal for all w):
// the accumulators and sums add without rescaling.
template <int G, int NW>
__device__ inline void write_partial_shared(float* part, const float (*mall)[G], const float (*lw)[G],
                                            const float (*accw)[G][kHeadDim]) {
  for (int i = threadIdx.x; i < G * kHeadDim; i += 64 * NW) {
    const int h = i / kHeadDim, d = i % kHeadDim;
    float A = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      A += accw[w][h][d];
      L += lw[w][h];
    }
    part[h * kPartStride + d] = A;
    if (d == 0) {
      part[h * kPartStride + kHeadDim] = mall[0][h];
      part[h * kPartStride + kHeadDim + 1] = L;
    }
  }
}

// Selected tokens of one (sequence, KV head): 16 NW of them per work-group
// (p.sel_blk_tok), NW wavefronts x 16 tokens, 4 lanes (a quarter of head_dim
// each) per token.  Writes the partial of the refined terms.
template <int BB, int G, int NW>
struct SelLds {
  float qs[G][kHeadDim];
  uint32_t vt[NW][16][4 * BB + 1];
  uint32_t vr[NW][16][33];
  float2 vsc[NW][16];
  float wt[NW][G][16];
  float mred[NW][G], mall[NW][G], lw[NW][G];
  float accw[NW][G][kHeadDim];
};

//
// With LG, the score pass left every token's base logits (log2 units) in
// p.logits, and the refined logit is that base logit plus the refinement's
// change: with sub = 2^-r,
//   refined - base = delta / sqrt(D) * (sub * (q . s) + (sub - 1) * sum(q) / 2),
// so the K base codes are not read again.
template <int BB, int G, int NW, bool LG>
__device__ inline void selected_block(const DecodeParams& p, int blk, int kvh, uint8_t* smem) {
  constexpr int W = 4 * BB;
  using Lds = SelLds<BB, G, NW>;
  Lds& s = *reinterpret_cast<Lds*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int tk = lane >> 2, qd = lane & 3;
  int64_t lo, hi;
  int first;
  const int seq = locate_unit(p, 16 * NW, blk, true, lo, hi, first);
  const int64_t a = seq_at(p, seq);
  const int64_t sk = (int64_t)seq * p.hkv + kvh;
  const int r = p.r;
  const float sub = __builtin_ldexpf(1.0f, -r);
  const uint32_t rmask = (1u << r) - 1u;

  // the query and the token's index, then every row of the token at once:
  // K and V codes, their refinement rows and scales (two dependent memory
  // round trips in all)
  for (int i = tid; i < G * kHeadDim; i += 64 * NW)
    s.qs[i / kHeadDim][i % kHeadDim] = p.q[((int64_t)seq * p.hq + kvh * G) * kHeadDim + i];
  const int64_t j = lo + wid * 16 + tk;
  const bool valid = j < hi;
  const int64_t tok = valid ? a + p.sel[sk * p.top_t + j] : 0;
  uint32_t kb[BB], kr[9], vb[BB], vr[8];
  float lgb[G];                   // base logits from the score pass (LG)
  float2 ksc = make_float2(0.f, 0.f), vsc = make_float2(0.f, 0.f);
#pragma unroll
  for (int h = 0; h < G; ++h) lgb[h] = 0.f;
#pragma unroll
  for (int i = 0; i < BB; ++i) kb[i] = vb[i] = 0u;
#pragma unroll
  for (int i = 0; i < 9; ++i) kr[i] = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) vr[i] = 0u;
  if (valid) {
    const int64_t row = (int64_t)kvh * p.cap + tok;
    const uint32_t* srck = reinterpret_cast<const uint32_t*>(p.kc + row * (16 * BB)) + qd * BB;
    const uint32_t* srcv = reinterpret_cast<const uint32_t*>(p.vc + row * (16 * BB)) + qd * BB;
    const uint32_t* rk = refine_row(p, sk, kvh, tok, 0) + qd * r;
    const uint32_t* rv = refine_row(p, sk, kvh, tok, 1) + qd * r;
    if (LG) {
      const float* lgs = p.logits + ((int64_t)kvh * p.ntot + (tok - p.off0)) * G;
#pragma unroll
      for (int h = 0; h < G; ++h) lgb[h] = lgs[h];
    }
#pragma unroll
    for (int i = 0; i < BB; ++i) {
      if (!LG) kb[i] = srck[i];
      vb[i] = srcv[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      kr[i] = i < r ? rk[i] : 0u;
      vr[i] = i < r ? rv[i] : 0u;
    }
    ksc = reinterpret_cast<const float2*>(p.ks)[row];
    vsc = reinterpret_cast<const float2*>(p.vs)[row];
  }
  __syncthreads();
  float dc[G], ds[G], dq[G];
  if (LG) {
    switch (r) {
      case 1: quarter_dots_ref<1, G>(kr, &s.qs[0][0], qd, ds, dq); break;
      case 2: quarter_dots_ref<2, G>(kr, &s.qs[0][0], qd, ds, dq); break;
      case 3: quarter_dots_ref<3, G>(kr, &s.qs[0][0], qd, ds, dq); break;
      case 4: quarter_dots_ref<4, G>(kr, &s.qs[0][0], qd, ds, dq); break;
      case 5: quarter_dots_ref<5, G>(kr, &s.qs[0][0], qd, ds, dq); break;
      case 6: quarter_dots_ref<6, G>(kr, &s.qs[0][0], qd, ds, dq); break;
      case 7: quarter_dots_ref<7, G>(kr, &s.qs[0][0], qd, ds, dq); break;
      default: quarter_dots_ref<8, G>(kr, &s.qs[0][0], qd, ds, dq); break;
    }
  } else {
    switch (r) {
      case 1: quarter_dots<BB, 1, G>(kb, kr, &s.qs[0][0], qd, dc, ds, dq); break;
      case 2: quarter_dots<BB, 2, G>(kb, kr, &s.qs[0][0], qd, dc, ds, dq); break;
      case 3: quarter_dots<BB, 3, G>(kb, kr, &s.qs[0][0], qd, dc, ds, dq); break;
      case 4: quarter_dots<BB, 4, G>(kb, kr, &s.qs[0][0], qd, dc, ds, dq); break;
      case 5: quarter_dots<BB, 5, G>(kb, kr, &s.qs[0][0], qd, dc, ds, dq); break;
      case 6: quarter_dots<BB, 6, G>(kb, kr, &s.qs[0][0], qd, dc, ds, dq); break;
      case 7: quarter_dots<BB, 7, G>(kb, kr, &s.qs[0][0], qd, dc, ds, dq); break;
      default: quarter_dots<BB, 8, G>(kb, kr, &s.qs[0][0], qd, dc, ds, dq); break;
    }
  }
  float lr[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float qsum = quad_sum(dq[h]);
    if (LG)
      lr[h] = fmaf(lgb[h], 0.6931471805599453f,
                   ksc.y * kRsqrtD * fmaf(sub, quad_sum(ds[h]), 0.5f * (sub - 1.0f) * qsum));
    else
      lr[h] = (ksc.x * qsum + ksc.y * (quad_sum(dc[h]) + (quad_sum(ds[h]) + 0.5f * qsum) * sub)) * kRsqrtD;
    const float mv = wave_max_dpp(valid ? lr[h] : -INFINITY);
    if (lane == 0) s.mred[wid][h] = mv;
  }
  {
    uint32_t* dstb = &s.vt[wid][tk][qd * BB];
    uint32_t* dstr = &s.vr[wid][tk][qd * r];
#pragma unroll
    for (int i = 0; i < BB; ++i) dstb[i] = vb[i];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < r) dstr[i] = vr[i];
    if (qd == 0) {
      s.vsc[wid][tk] = vsc;
      s.vt[wid][tk][W] = 0u;
      s.vr[wid][tk][4 * r] = 0u;
    }
  }
  __syncthreads();
  float acc[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float M = s.mred[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s.mred[w][h]);
    const float e = valid ? expf(lr[h] - M) : 0.f;
    if (qd == 0) s.wt[wid][h][tk] = e;
    const float ls = wave_sum_dpp(qd == 0 ? e : 0.f);
    if (lane == 0) {
      s.lw[wid][h] = ls;
      s.mall[wid][h] = M;       // all waves share the work-group maximum
    }
    acc[h][0] = acc[h][1] = 0.f;
  }
  wave_barrier();
  const int cpos = 2 * lane * BB, cwi = cpos >> 5, csh = cpos & 31;
  const int rpos = 2 * lane * r, rwi = rpos >> 5, rsh = rpos & 31;
  for (int jj = 0; jj < 16; ++jj) {
    const uint64_t cwin = (uint64_t)s.vt[wid][jj][cwi] | ((uint64_t)s.vt[wid][jj][cwi + 1] << 32);
    const uint32_t cc = (uint32_t)(cwin >> csh);
    const uint64_t rwin = (uint64_t)s.vr[wid][jj][rwi] | ((uint64_t)s.vr[wid][jj][rwi + 1] << 32);
    const uint32_t rr = (uint32_t)(rwin >> rsh);
    const float c0 = (float)(cc & ((1u << BB) - 1u)), c1 = (float)((cc >> BB) & ((1u << BB) - 1u));
    const float s0 = (float)(rr & rmask), s1 = (float)((rr >> r) & rmask);
    const float2 sc = s.vsc[wid][jj];
    const float v0 = fmaf((s0 + 0.5f) * sub, sc.y, fmaf(c0, sc.y, sc.x));
    const float v1 = fmaf((s1 + 0.5f) * sub, sc.y, fmaf(c1, sc.y, sc.x));
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float w = s.wt[wid][h][jj];
      acc[h][0] = fmaf(w, v0, acc[h][0]);
      acc[h][1] = fmaf(w, v1, acc[h][1]);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    s.accw[wid][h][2 * lane] = acc[h][0];
    s.accw[wid][h][2 * lane + 1] = acc[h][1];
  }
  __syncthreads();
  float* part = p.part + ((int64_t)kvh * (p.n_sel_blk + p.n_split) + blk) * G * kPartStride;
  write_partial_shared<G, NW>(part, s.mall, s.lw, s.accw);
}

}  // namespace sfk

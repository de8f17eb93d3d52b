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
// Host tier: the token's global cache slot (installed by the lookup of this
// step).  A slot outside this (sequence, KV head)'s cache means the tables are
// inconsistent: the store's error word records it (sf_store_check reports it)
// and the first slot of the cache is read instead.
__device__ inline const uint32_t* refine_row(const DecodeParams& p, int64_t sk, int kvh, int64_t tok, int which) {
  if (p.ref_rows)
    return reinterpret_cast<const uint32_t*>(p.ref_rows + (((int64_t)which * p.hkv + kvh) * p.cap + tok) * p.rb);
  int64_t gs = p.tok_slot[(int64_t)kvh * p.cap + tok];
  if (gs < sk * p.slots || gs >= (sk + 1) * p.slots) {
    if (p.store_err) atomicOr(p.store_err, 1);
    gs = sk * p.slots;
  }
  return reinterpret_cast<const uint32_t*>(p.cache_data + (gs * 2 + which) * (int64_t)p.rb);
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

// Selected tokens of one (sequence, KV head): NW wavefronts x TPW tokens per
// work-group (p.sel_blk_tok = NW TPW).  The rows of a wave's TPW tokens are
// loaded by 4 lanes per token (a quarter row each) into LDS; the logits are
// computed by LPT = 64 / TPW lanes per token, each over EPL = 128 / LPT
// elements (fewer tokens per wave: shorter chains per lane); P.V takes 2
// output elements per lane over the wave's tokens.  Writes the partial of the
// refined terms.
template <int BB, int G, int NW, int TPW>
struct SelLds {
  float qs[G][kHeadDim];
  uint32_t kq[NW][TPW][33];          // K refinement rows (r <= 8: 32 words + a zero word)
  uint32_t kbq[NW][TPW][4 * BB + 1]; // K base codes (when the logits are recomputed)
  uint32_t vt[NW][TPW][4 * BB + 1];
  uint32_t vr[NW][TPW][33];
  float2 vsc[NW][TPW], ksc[NW][TPW];
  float hsub[NW][TPW];               // 2^-r, or 1 for a skipped miss (base precision)
  float lgt[NW][TPW][G];             // base logits from the score pass
  float wt[NW][G][TPW];
  float mred[NW][G], mall[NW][G], lw[NW][G];
  float accw[NW][G][kHeadDim];
};

// The EPL codes (W bits each) from element e0 of an LDS row, shifted so that
// the first one sits at bit 0 of the returned words (EPL W <= 256 bits).
template <int W, int EPL>
__device__ inline void row_window(const uint32_t* row, int e0, uint32_t (&out)[EPL * W / 32 + 1]) {
  const int bit = e0 * W, wo = bit >> 5, sh = bit & 31;
#pragma unroll
  for (int j = 0; j < EPL * W / 32 + 1; ++j) {
    const uint32_t lo = row[wo + j], hi = j + 1 < EPL * W / 32 + 1 || sh ? row[wo + j + 1] : 0u;
    out[j] = sh ? (lo >> sh) | (hi << (32 - sh)) : lo;
  }
}

// Sum over the LPT lanes of a token (LPT = 4: a quad, 8: two quads, 16: a DPP
// row); every lane of the group receives it.
template <int LPT>
__device__ inline float token_sum(float x) {
  x = quad_sum(x);
  if constexpr (LPT == 8) {
    // the other quad of the eight lanes (swizzle: lane ^ 4)
    x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x101F));
  }
  if constexpr (LPT == 16) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
  }
  return x;
}

// Dot products of lane's EPL elements [e0, e0 + EPL) with the G query heads:
// base codes (BB bits, when !LG), refinement codes (R bits) and the query
// sum.
template <int BB, int R, int G, int EPL, bool LG>
__device__ inline void lane_dots(const uint32_t* kbrow, const uint32_t* krrow, const float* qs, int e0, float* dc,
                                 float* ds, float* dq) {
  uint32_t kb[EPL * BB / 32 + 1], kr[EPL * R / 32 + 1];
  if (!LG) row_window<BB, EPL>(kbrow, e0, kb);
  row_window<R, EPL>(krrow, e0, kr);
#pragma unroll
  for (int h = 0; h < G; ++h) dc[h] = ds[h] = dq[h] = 0.f;
#pragma unroll
  for (int d = 0; d < EPL; ++d) {
    const float sv = (float)code_at<R>(kr, d);
    const float cv = LG ? 0.f : (float)code_at<BB>(kb, d);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float qv = qs[h * kHeadDim + e0 + d];
      if (!LG) dc[h] = fmaf(qv, cv, dc[h]);
      ds[h] = fmaf(qv, sv, ds[h]);
      dq[h] += qv;
    }
  }
}

//
// With LG, the score pass left every token's base logits (log2 units) in
// p.logits, and the refined logit is that base logit plus the refinement's
// change: with sub = 2^-r,
//   refined - base = delta / sqrt(D) * (sub * (q . s) + (sub - 1) * sum(q) / 2),
// so the K base codes are not read again.
template <int BB, int G, int NW, bool LG, int TPW, bool Batched = false>
__device__ inline void selected_block(const DecodeParams& p, int blk, int kvh, uint8_t* smem) {
  constexpr int W = 4 * BB, LPT = 64 / TPW, EPL = kHeadDim / LPT;
  static_assert(TPW == 4 || TPW == 16, "4 or 16 lanes per token");
  using Lds = SelLds<BB, G, NW, TPW>;
  Lds& s = *reinterpret_cast<Lds*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int64_t lo, hi;
  int first;
  const int seq = locate_unit<Batched>(p, NW * TPW, blk, true, lo, hi, first);
  const int64_t a = seq_at(p, seq);
  const int64_t sk = (int64_t)seq * p.hkv + kvh;
  const int r = p.r;
  const float sub = __builtin_ldexpf(1.0f, -r);
  const uint32_t rmask = (1u << r) - 1u;

  // the query and the tokens' indices, then every row of the tokens at once
  // (two dependent memory round trips): lane (tl, qd) < 4 TPW loads quarter
  // qd of token tl's rows
  for (int i = tid; i < G * kHeadDim; i += 64 * NW)
    s.qs[i / kHeadDim][i % kHeadDim] = p.q[((int64_t)seq * p.hq + kvh * G) * kHeadDim + i];
  {
    const int tl = lane >> 2, qd = lane & 3;
    const int64_t j = lo + wid * TPW + tl;
    const bool loader = lane < 4 * TPW;
    const bool valid = loader && j < hi;
    // a selected token marked as ~token (a refinement-cache miss under the
    // skip policy) takes part at base precision: no refinement rows, and
    // its sub-bin factor 1 with zero codes gives the bin centre
    const int32_t e = valid ? p.sel[sk * p.top_t + j] : 0;
    const bool refined = e >= 0;
    const int64_t tok = a + (e >= 0 ? e : ~e);
    uint32_t kb[BB], kr[8], vb[BB], vr[8];
    float lg[G];
    float2 ksc = make_float2(0.f, 0.f), vsc = make_float2(0.f, 0.f);
#pragma unroll
    for (int i = 0; i < BB; ++i) kb[i] = vb[i] = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) kr[i] = vr[i] = 0u;
#pragma unroll
    for (int h = 0; h < G; ++h) lg[h] = 0.f;
    if (valid) {
      const int64_t row = (int64_t)kvh * p.cap + tok;
      const uint32_t* srck = reinterpret_cast<const uint32_t*>(p.kc + row * (16 * BB)) + qd * BB;
      const uint32_t* srcv = reinterpret_cast<const uint32_t*>(p.vc + row * (16 * BB)) + qd * BB;
      const uint32_t* rk = refined ? refine_row(p, sk, kvh, tok, 0) + qd * r : nullptr;
      const uint32_t* rv = refined ? refine_row(p, sk, kvh, tok, 1) + qd * r : nullptr;
      if (LG) {
        const float* lgs = p.logits + ((int64_t)kvh * p.ntot + (tok - p.off0)) * G;
#pragma unroll
        for (int h = 0; h < G; ++h) lg[h] = lgs[h];
      }
#pragma unroll
      for (int i = 0; i < BB; ++i) {
        if (!LG) kb[i] = srck[i];
        vb[i] = srcv[i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        kr[i] = refined && i < r ? rk[i] : 0u;
        vr[i] = refined && i < r ? rv[i] : 0u;
      }
      ksc = reinterpret_cast<const float2*>(p.ks)[row];
      vsc = reinterpret_cast<const float2*>(p.vs)[row];
    }
    if (loader) {
#pragma unroll
      for (int i = 0; i < BB; ++i) {
        s.kbq[wid][tl][qd * BB + i] = kb[i];
        s.vt[wid][tl][qd * BB + i] = vb[i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < r) {
          s.kq[wid][tl][qd * r + i] = kr[i];
          s.vr[wid][tl][qd * r + i] = vr[i];
        }
      if (qd == 0) {
        s.kbq[wid][tl][W] = s.vt[wid][tl][W] = 0u;
        for (int i = 4 * r; i < 33; ++i) s.kq[wid][tl][i] = s.vr[wid][tl][i] = 0u;
        s.ksc[wid][tl] = ksc;
        s.vsc[wid][tl] = vsc;
        s.hsub[wid][tl] = refined ? sub : 1.0f;
#pragma unroll
        for (int h = 0; h < G; ++h) s.lgt[wid][tl][h] = lg[h];
      }
    }
  }
  __syncthreads();

  // the logits: lane (tc, e) over elements [e EPL, e EPL + EPL) of token tc
  const int tc = lane / LPT, e0 = (lane % LPT) * EPL;
  const bool valid = lo + wid * TPW + tc < hi;
  float dc[G], ds[G], dq[G];
  const uint32_t* kbrow = &s.kbq[wid][tc][0];
  const uint32_t* krrow = &s.kq[wid][tc][0];
  switch (r) {
    case 1: lane_dots<BB, 1, G, EPL, LG>(kbrow, krrow, &s.qs[0][0], e0, dc, ds, dq); break;
    case 2: lane_dots<BB, 2, G, EPL, LG>(kbrow, krrow, &s.qs[0][0], e0, dc, ds, dq); break;
    case 3: lane_dots<BB, 3, G, EPL, LG>(kbrow, krrow, &s.qs[0][0], e0, dc, ds, dq); break;
    case 4: lane_dots<BB, 4, G, EPL, LG>(kbrow, krrow, &s.qs[0][0], e0, dc, ds, dq); break;
    case 5: lane_dots<BB, 5, G, EPL, LG>(kbrow, krrow, &s.qs[0][0], e0, dc, ds, dq); break;
    case 6: lane_dots<BB, 6, G, EPL, LG>(kbrow, krrow, &s.qs[0][0], e0, dc, ds, dq); break;
    case 7: lane_dots<BB, 7, G, EPL, LG>(kbrow, krrow, &s.qs[0][0], e0, dc, ds, dq); break;
    default: lane_dots<BB, 8, G, EPL, LG>(kbrow, krrow, &s.qs[0][0], e0, dc, ds, dq); break;
  }
  const float2 ksc = s.ksc[wid][tc];
  const float hs = s.hsub[wid][tc];
  float lr[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float qsum = token_sum<LPT>(dq[h]);
    if (LG)
      lr[h] = fmaf(s.lgt[wid][tc][h], 0.6931471805599453f,
                   ksc.y * kRsqrtD * fmaf(hs, token_sum<LPT>(ds[h]), 0.5f * (hs - 1.0f) * qsum));
    else
      lr[h] = (ksc.x * qsum + ksc.y * (token_sum<LPT>(dc[h]) + (token_sum<LPT>(ds[h]) + 0.5f * qsum) * hs)) *
              kRsqrtD;
    const float mv = wave_max_dpp(valid ? lr[h] : -INFINITY);
    if (lane == 0) s.mred[wid][h] = mv;
  }
  __syncthreads();
  float acc[G][2];
  const bool lead = lane % LPT == 0;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float M = s.mred[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s.mred[w][h]);
    const float ew = valid ? expf(lr[h] - M) : 0.f;
    if (lead) s.wt[wid][h][tc] = ew;
    const float ls = wave_sum_dpp(lead ? ew : 0.f);
    if (lane == 0) {
      s.lw[wid][h] = ls;
      s.mall[wid][h] = M;       // all waves share the work-group maximum
    }
    acc[h][0] = acc[h][1] = 0.f;
  }
  wave_barrier();
  const int cpos = 2 * lane * BB, cwi = cpos >> 5, csh = cpos & 31;
  const int rpos = 2 * lane * r, rwi = rpos >> 5, rsh = rpos & 31;
#pragma unroll 4
  for (int jj = 0; jj < TPW; ++jj) {
    const uint64_t cwin = (uint64_t)s.vt[wid][jj][cwi] | ((uint64_t)s.vt[wid][jj][cwi + 1] << 32);
    const uint32_t cc = (uint32_t)(cwin >> csh);
    const uint64_t rwin = (uint64_t)s.vr[wid][jj][rwi] | ((uint64_t)s.vr[wid][jj][rwi + 1] << 32);
    const uint32_t rr = (uint32_t)(rwin >> rsh);
    const float c0 = (float)(cc & ((1u << BB) - 1u)), c1 = (float)((cc >> BB) & ((1u << BB) - 1u));
    const float s0 = (float)(rr & rmask), s1 = (float)((rr >> r) & rmask);
    const float2 sc = s.vsc[wid][jj];
    const float hj = s.hsub[wid][jj];
    const float v0 = fmaf((s0 + 0.5f) * hj, sc.y, fmaf(c0, sc.y, sc.x));
    const float v1 = fmaf((s1 + 0.5f) * hj, sc.y, fmaf(c1, sc.y, sc.x));
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

// Selected tokens of one (sequence, KV head) with their complete 16-bit K
// and V rows (the comparison variant of page "StrataFlux -- Selective
// precision streaming -- What does it mean?", table row "SpeCache (16-bit
// fetching)"): the work-group takes p.sel_blk_tok tokens of the selection,
// wavefront w the tokens w, w + NW, ...; lane l holds elements 2l and 2l + 1.
// The same partial as selected_block (natural-log maximum shared by the
// work-group).
template <int G, int NW>
struct Sel16Lds {
  float lg[kSelBlkTok][G];
  float mred[NW][G], mall[NW][G], lw[NW][G];
  float accw[NW][G][kHeadDim];
};

template <int G, int NW, bool Batched = false>
__device__ inline void selected16_block(const DecodeParams& p, int blk, int kvh, uint8_t* smem) {
  using Lds = Sel16Lds<G, NW>;
  Lds& s = *reinterpret_cast<Lds*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int64_t lo, hi;
  int first;
  const int seq = locate_unit<Batched>(p, p.sel_blk_tok, blk, true, lo, hi, first);
  const int64_t a = seq_at(p, seq);
  const int64_t sk = (int64_t)seq * p.hkv + kvh;
  const int n = (int)(hi - lo);                     // <= p.sel_blk_tok <= kSelBlkTok
  const float* qg = p.q + ((int64_t)seq * p.hq + kvh * G) * kHeadDim;
  float q0[G], q1[G], mloc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    q0[h] = qg[h * kHeadDim + 2 * lane];
    q1[h] = qg[h * kHeadDim + 2 * lane + 1];
    mloc[h] = -INFINITY;
  }
  auto token = [&](int j) {
    const int32_t e = p.sel[sk * p.top_t + lo + j];
    return a + (e >= 0 ? e : ~e);
  };
  for (int j = wid; j < n; j += NW) {
    const _Float16* kr = p.rows16 + ((int64_t)kvh * p.cap + token(j)) * kHeadDim;
    const float k0 = (float)kr[2 * lane], k1 = (float)kr[2 * lane + 1];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float l = wave_sum_dpp(fmaf(q0[h], k0, q1[h] * k1)) * kRsqrtD;
      if (lane == 0) s.lg[j][h] = l;
      mloc[h] = fmaxf(mloc[h], l);
    }
  }
  if (lane == 0)
#pragma unroll
    for (int h = 0; h < G; ++h) s.mred[wid][h] = mloc[h];
  __syncthreads();
  float M[G], l[G], acc[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    M[h] = s.mred[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) M[h] = fmaxf(M[h], s.mred[w][h]);
    l[h] = acc[h][0] = acc[h][1] = 0.f;
  }
  for (int j = wid; j < n; j += NW) {
    const _Float16* vr = p.rows16 + (((int64_t)p.hkv + kvh) * p.cap + token(j)) * kHeadDim;
    const float v0 = (float)vr[2 * lane], v1 = (float)vr[2 * lane + 1];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float w = expf(s.lg[j][h] - M[h]);
      l[h] += w;
      acc[h][0] = fmaf(w, v0, acc[h][0]);
      acc[h][1] = fmaf(w, v1, acc[h][1]);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    s.accw[wid][h][2 * lane] = acc[h][0];
    s.accw[wid][h][2 * lane + 1] = acc[h][1];
    if (lane == 0) {
      s.lw[wid][h] = l[h];
      s.mall[wid][h] = M[h];
    }
  }
  __syncthreads();
  float* part = p.part + ((int64_t)kvh * (p.n_sel_blk + p.n_split) + blk) * G * kPartStride;
  write_partial_shared<G, NW>(part, s.mall, s.lw, s.accw);
}

// The selected block's shape chosen on the host: p.sel_blk_tok = NW TPW.
template <int BB, int G, int NW, bool LG, bool Batched = false>
__device__ inline void selected_block_any(const DecodeParams& p, int blk, int kvh, uint8_t* smem) {
  static_assert(sizeof(Sel16Lds<G, NW>) <= sizeof(SelLds<BB, G, NW, 4>), "fits the selected blocks' LDS");
  if (p.rows16)
    selected16_block<G, NW, Batched>(p, blk, kvh, smem);
  else if (p.sel_blk_tok == NW * 4)
    selected_block<BB, G, NW, LG, 4, Batched>(p, blk, kvh, smem);
  else
    selected_block<BB, G, NW, LG, 16, Batched>(p, blk, kvh, smem);
}

}  // namespace sfk

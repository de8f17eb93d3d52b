// Per-KV-head top-T selection (the "refine the highest-scoring tokens for
// each KV head" step of the page "StrataFlux -- Selective precision streaming
// -- What does it mean?", paragraph "Which tiles count ...").
//
// Order: score descending, then token index ascending (ties at the cut go to
// the lower index); with N <= T every token is selected.  Scores are compared
// through their order-preserving 32-bit keys (sfk::score_key).
//
// Three radix levels of the key, all exact:
//   level 1 (bits 31..20): histogram built by the score kernel;
//   select_scan (many work-groups per (sequence, KV head), one chunk of
//     kSelChunk tokens each): derive the boundary bin b1, write the chunk's
//     selection-bitmap words for tokens above b1, and copy the chunk's
//     tokens inside b1 (candidates) into the chunk's own segment of the
//     candidate buffer with their count;
//   select_resolve (one work-group per (sequence, KV head)): histogram the
//     candidates' level-2 digit (bits 19..8), find the boundary b2, mark the
//     candidates above it and resolve those left in (b1, b2) by (key bits 7..0
//     descending, token ascending) with an LDS radix select; then list the
//     selection in ascending token order.
// The kernel boundary orders the two phases: no global atomics, no fences.
#include "sf_decode_kernels.h"

namespace sfk {

constexpr int kResThreads = 1024;
constexpr int kFinMax = 4096;   // level-3 candidates kept in LDS
constexpr int kRankMax = 128;   // up to this many, level 3 ranks directly

// 40-bit rank value of a level-3 candidate: low key byte over the inverted
// token index (larger ranks first; no two candidates are equal).
__device__ inline uint64_t fin_value(uint2 c) {
  return ((uint64_t)(c.x & 0xFFu) << 32) | (uint64_t)(0xFFFFFFFFu - c.y);
}

template <bool Batched>
__global__ void __launch_bounds__(kSelThreads) select_scan(DecodeParams p) {
  __shared__ __align__(16) uint32_t h[kHistBins];
  __shared__ int sh_bin;
  __shared__ uint32_t sh_need, sh_cnt;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int kvh = blockIdx.y;
  int64_t lo, hi;
  int first;
  const int seq = locate_unit<Batched>(p, p.sel_chunk, blockIdx.x, false, lo, hi, first);
  const int chunk = blockIdx.x - first;
  const int64_t a = seq_at(p, seq);
  const int64_t n = seq_at(p, seq + 1) - a;
  const int64_t tn = n < p.top_t ? n : (int64_t)p.top_t;
  const bool all = (tn == n);
  const int64_t sk = (int64_t)seq * p.hkv + kvh;
  uint32_t* bm = p.bitmap + sk * p.bm_words;
  const float* sc = p.scores + (int64_t)kvh * p.ntot + (a - p.off0);
  uint2* cand = p.cand + sk * p.max_seq + lo;     // this chunk's segment
  // the chunk's scores are loaded first, so that their latency overlaps the
  // boundary search below
  constexpr int kPer = kSelChunk / kSelThreads;
  float sv[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int64_t i = lo + j * kSelThreads + tid;
    sv[j] = (!all && i < hi) ? sc[i] : 0.f;
  }

  if (!all) {
    // the level-1 histogram in 16-byte pieces, every load issued before the
    // first LDS store
    static_assert(kHistBins == 8 * kSelThreads, "two 16-byte pieces per thread");
    const uint4* h1 = reinterpret_cast<const uint4*>(p.hist + sk * kHistBins);
    const uint4 x0 = h1[tid], x1 = h1[tid + kSelThreads];
    reinterpret_cast<uint4*>(h)[tid] = x0;
    reinterpret_cast<uint4*>(h)[tid + kSelThreads] = x1;
    if (tid == 0) sh_cnt = 0u;
    __syncthreads();
    find_threshold_wave<kHistBins>(h, (uint32_t)tn, &sh_bin, &sh_need);
  }
  const uint32_t b1 = all ? 0u : (uint32_t)sh_bin;
  // bitmap words of the tokens above b1; the candidates' ballots are kept so
  // that each wavefront reserves its candidate slots with one LDS atomic
  uint64_t cbal[kPer];
  uint32_t ckey[kPer];
  uint32_t wave_cnt = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int64_t base = lo + j * kSelThreads;
    const int64_t i = base + tid;
    const bool valid = i < hi;
    bool s = false, cnd = false;
    uint32_t key = 0;
    if (valid) {
      if (all) {
        s = true;
      } else {
        key = score_key(sv[j]);
        const uint32_t bin = key >> (32 - kHistBits);
        s = bin > b1;
        cnd = bin == b1;
      }
    }
    const uint64_t bal = __ballot(s);
    if (lane == 0 && base < hi) {
      const int64_t w = (base + wid * 64) >> 5;
      bm[w] = (uint32_t)bal;
      bm[w + 1] = (uint32_t)(bal >> 32);
    }
    cbal[j] = __ballot(cnd);
    ckey[j] = key;
    wave_cnt += (uint32_t)__popcll(cbal[j]);
  }
  if (wave_cnt) {
    uint32_t at = 0;
    if (lane == 0) at = atomicAdd(&sh_cnt, wave_cnt);
    at = __builtin_amdgcn_readlane(at, 0);
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if ((cbal[j] >> lane) & 1ull)
        cand[at + (uint32_t)__popcll(cbal[j] & below)] = make_uint2(ckey[j], (uint32_t)(lo + j * kSelThreads + tid));
      at += (uint32_t)__popcll(cbal[j]);
    }
  }
  __syncthreads();
  if (tid == 0) {
    p.counters[sk * p.cnt_stride + chunk] = all ? 0u : sh_cnt;
    if (chunk == 0 && !all) {   // the level-1 boundary, for the resolve kernel
      p.counters[sk * p.cnt_stride + p.cnt_stride - 2] = b1;
      p.counters[sk * p.cnt_stride + p.cnt_stride - 1] = sh_need;
    }
  }
}

// Candidate j of a (sequence, KV head): segments of the chunks laid end to end
// (prefix offsets in LDS, binary search over at most kMaxSelChunks entries).
__device__ inline uint2 cand_at(const uint2* cand, const uint32_t* segoff, int nch, int32_t chunk_len, uint32_t j) {
  int lo = 0, hi = nch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (segoff[mid] <= j) lo = mid; else hi = mid - 1;
  }
  return cand[(int64_t)lo * chunk_len + (j - segoff[lo])];
}

constexpr int kLdsBitmapWords = 16384;   // bitmaps up to 512K tokens are kept in LDS
constexpr int kCandLds = 4096;           // candidates kept in LDS
constexpr int kBmQuads = kLdsBitmapWords / 4 / kResThreads;   // 16-byte bitmap pieces per thread
// Candidates loaded before their counts are known: the first kSpecCand of
// each of the first kSpecChunks chunks (kResThreads / kSpecChunks threads per
// chunk, two each).
constexpr int kSpecChunks = 32, kSpecCand = 64;
static_assert(kSpecChunks * kSpecCand == 2 * kResThreads, "two speculative candidates per thread");

__global__ void __launch_bounds__(kResThreads) select_resolve(DecodeParams p) {
  __shared__ __align__(16) uint32_t h[kHistBins];
  __shared__ uint32_t scan_lds[kResThreads / 64];
  __shared__ uint32_t rh[256];
  __shared__ uint2 cl[kCandLds];
  __shared__ uint2 fin[kFinMax];
  __shared__ uint32_t segoff[kMaxSelChunks + 1];
  __shared__ __align__(16) uint32_t lbm[kLdsBitmapWords];
  __shared__ int sh_bin;
  __shared__ uint32_t sh_need, sh_fin, sh_spill;
  static_assert(kMaxSelChunks <= kResThreads, "one chunk count per thread");

  const int tid = threadIdx.x;
  const int64_t sk = blockIdx.x;
  uint32_t* gbm = p.bitmap + sk * p.bm_words;
  const uint2* cand = p.cand + sk * p.max_seq;
  const uint32_t* cnts = p.counters + sk * p.cnt_stride;
  // Everything this kernel reads from the scan is loaded up front, before the
  // sequence's length is known (every read is inside the per-head areas):
  // the chunks' candidate counts, the level-1 boundary, the bitmap words.
  const bool in_lds = p.bm_words <= kLdsBitmapWords;
  const int nqb = p.bm_words >> 2;   // bm_words is a multiple of 16
  uint4 bq[kBmQuads];
  if (in_lds) {
    const uint4* g4 = reinterpret_cast<const uint4*>(gbm);
#pragma unroll
    for (int k = 0; k < kBmQuads; ++k) {
      const int qi = tid + k * kResThreads;
      bq[k] = qi < nqb ? g4[qi] : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  uint32_t my_cnt = tid < p.cnt_stride - 2 ? cnts[tid] : 0u;
  const uint32_t need1 = cnts[p.cnt_stride - 1];
  const int sp_c = tid / (kResThreads / kSpecChunks), sp_i = tid % (kResThreads / kSpecChunks);
  uint2 spec[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int64_t at = (int64_t)sp_c * p.sel_chunk + sp_i + k * (kResThreads / kSpecChunks);
    spec[k] = (sp_c < p.cnt_stride - 2 && at < p.max_seq) ? cand[at] : make_uint2(0u, 0u);
  }

  const int seq = (int)(sk / p.hkv);
  const int64_t a = seq_at(p, seq);
  const int64_t n = seq_at(p, seq + 1) - a;
  const int64_t tn = n < p.top_t ? n : (int64_t)p.top_t;
  const bool all = (tn == n);
  const int nch = (int)((n + p.sel_chunk - 1) / p.sel_chunk);
  const int64_t nw = (n + 31) >> 5;
  uint32_t* bm = in_lds ? lbm : gbm;
  my_cnt = (!all && tid < nch) ? my_cnt : 0u;

  // the level-1 histogram is cleared for the next step
  uint32_t* h1 = p.hist + sk * kHistBins;
  for (int i = tid; i < kHistBins; i += kResThreads) {
    h1[i] = 0u;
    h[i] = 0u;
  }
  if (in_lds) {
    uint4* l4 = reinterpret_cast<uint4*>(lbm);
#pragma unroll
    for (int k = 0; k < kBmQuads; ++k) {
      const int qi = tid + k * kResThreads;
      if (qi < nqb) l4[qi] = bq[k];
    }
  }
  if (!all) {
    // segment offsets: exclusive prefix of the per-chunk candidate counts;
    // sh_spill says whether some candidate lies outside the speculative loads
    if (nch <= 64) {
      if (tid < 64) {
        const uint32_t inc = wave_inclusive_scan(my_cnt);
        if (tid < nch) segoff[tid] = inc - my_cnt;
        if (tid == nch - 1) segoff[nch] = inc;
        const uint64_t big = __ballot(my_cnt > (uint32_t)kSpecCand);
        if (tid == 0) sh_spill = (big != 0 || nch > kSpecChunks) ? 1u : 0u;
      }
    } else {
      uint32_t tot;
      const uint32_t run = block_exclusive_scan<kResThreads>(my_cnt, scan_lds, tot);
      if (tid < nch) segoff[tid] = run;
      if (tid == 0) {
        segoff[nch] = tot;
        sh_spill = 1u;
      }
    }
    if (tid == 0) sh_fin = 0u;
    __syncthreads();
    const uint32_t ncand = segoff[nch];
    const bool cand_lds = ncand <= (uint32_t)kCandLds;
    // level 2: histogram of the candidates' middle 12 key bits (candidates
    // are copied to LDS on the way)
    if (!sh_spill) {
      // every candidate is among the speculative loads (and fits in LDS)
      const uint32_t cc = sp_c < nch ? segoff[sp_c + 1] - segoff[sp_c] : 0u;
      const uint32_t o = sp_c < nch ? segoff[sp_c] : 0u;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t i = sp_i + k * (kResThreads / kSpecChunks);
        if (i < cc) {
          cl[o + i] = spec[k];
          atomicAdd(&h[(spec[k].x >> 8) & 0xFFFu], 1u);
        }
      }
    } else {
      // candidate j found by a search over the segment offsets; loads in
      // groups of four
      for (uint32_t j0 = tid; j0 < ncand; j0 += 4 * kResThreads) {
        uint2 cv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t j = j0 + k * kResThreads;
          cv[k] = j < ncand ? cand_at(cand, segoff, nch, p.sel_chunk, j) : make_uint2(0u, 0u);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t j = j0 + k * kResThreads;
          if (j < ncand) {
            if (cand_lds) cl[j] = cv[k];
            atomicAdd(&h[(cv[k].x >> 8) & 0xFFFu], 1u);
          }
        }
      }
    }
    __syncthreads();
    find_threshold_wave<kHistBins>(h, need1, &sh_bin, &sh_need);
    const uint32_t b2 = (uint32_t)sh_bin, need2 = sh_need;
    auto cget = [&](uint32_t j) -> uint2 { return cand_lds ? cl[j] : cand_at(cand, segoff, nch, p.sel_chunk, j); };
    for (uint32_t j = tid; j < ncand; j += kResThreads) {
      const uint2 cv = cget(j);
      const uint32_t mid = (cv.x >> 8) & 0xFFFu;
      if (mid > b2) {
        atomicOr(&bm[cv.y >> 5], 1u << (cv.y & 31u));
      } else if (mid == b2) {
        const uint32_t k = atomicAdd(&sh_fin, 1u);
        if (k < kFinMax) fin[k] = cv;
      }
    }
    __syncthreads();
    const uint32_t m = sh_fin;
    // level 3: the need2 largest (low key byte, inverted token) among the
    // candidates sharing the top 24 key bits; radix over 40 bits, 8 per pass
    auto get = [&](uint32_t j, bool& ok) -> uint64_t {
      if (m <= kFinMax) {
        ok = true;
        return fin_value(fin[j]);
      }
      const uint2 cv = cget(j);
      ok = ((cv.x >> 8) & 0xFFFu) == b2;
      return fin_value(cv);
    };
    const uint32_t cnt = m <= kFinMax ? m : ncand;
    if (m <= (uint32_t)kRankMax) {
      // few left: rank each by counting the larger ones (all values differ)
      if (tid < (int)m) {
        const uint64_t v = fin_value(fin[tid]);
        uint32_t rank = 0;
        for (uint32_t k = 0; k < m; ++k) rank += fin_value(fin[k]) > v ? 1u : 0u;
        if (rank < need2) atomicOr(&bm[fin[tid].y >> 5], 1u << (fin[tid].y & 31u));
      }
    } else {
      uint64_t prefix = 0, mask = 0;
      uint32_t need = need2;
      for (int shift = 32; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += kResThreads) rh[i] = 0u;
        __syncthreads();
        for (uint32_t j = tid; j < cnt; j += kResThreads) {
          bool ok;
          const uint64_t v = get(j, ok);
          if (ok && (v & mask) == prefix) atomicAdd(&rh[(v >> shift) & 0xFFu], 1u);
        }
        __syncthreads();
        const uint32_t mine = tid < 256 ? rh[255 - tid] : 0u;
        uint32_t tot;
        const uint32_t above = block_exclusive_scan<kResThreads>(mine, scan_lds, tot);
        if (tid < 256 && above < need && need <= above + mine) {
          sh_bin = 255 - tid;
          sh_need = need - above;
        }
        __syncthreads();
        const int d = sh_bin;
        const uint32_t left = sh_need;
        const bool whole = rh[d] == left;     // the bucket is taken entirely
        prefix |= (uint64_t)d << shift;
        mask |= 0xFFull << shift;
        need = left;
        __syncthreads();
        if (whole) break;
      }
      for (uint32_t j = tid; j < cnt; j += kResThreads) {
        bool ok;
        const uint64_t v = get(j, ok);
        const uint32_t tok = m <= kFinMax ? fin[j].y : cget(j).y;
        if (ok && (v & mask) >= prefix) atomicOr(&bm[tok >> 5], 1u << (tok & 31u));
      }
    }
  }
  __syncthreads();

  // List the selection in ascending token order; the final bitmap goes back
  // to global memory for the attention pass.
  int32_t* sel = p.sel + sk * p.top_t;
  int32_t* selo = p.sel_out ? p.sel_out + sk * p.top_t : nullptr;
  uint32_t pos = 0;
  auto emit = [&](uint32_t bits, int64_t w) {
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
  };
  uint32_t tot;
  if (in_lds) {
    // thread t: 16-byte pieces [t qp, (t + 1) qp) of the bitmap (qp <= kBmQuads);
    // the pieces' words past the sequence's last word hold no bits
    const int nq = (int)((nw + 3) >> 2);
    const int qp = (nq + kResThreads - 1) / kResThreads;
    const uint4* l4 = reinterpret_cast<const uint4*>(lbm);
    uint4* g4 = reinterpret_cast<uint4*>(gbm);
    uint4 mine[kBmQuads];
    uint32_t cnt = 0;
#pragma unroll
    for (int k = 0; k < kBmQuads; ++k) {
      const int qi = tid * qp + k;
      mine[k] = (k < qp && qi < nq) ? l4[qi] : make_uint4(0u, 0u, 0u, 0u);
      cnt += __popc(mine[k].x) + __popc(mine[k].y) + __popc(mine[k].z) + __popc(mine[k].w);
    }
    pos = block_exclusive_scan<kResThreads>(cnt, scan_lds, tot);
#pragma unroll
    for (int k = 0; k < kBmQuads; ++k) {
      const int qi = tid * qp + k;
      if (k < qp && qi < nq) {
        g4[qi] = mine[k];
        emit(mine[k].x, 4 * (int64_t)qi);
        emit(mine[k].y, 4 * (int64_t)qi + 1);
        emit(mine[k].z, 4 * (int64_t)qi + 2);
        emit(mine[k].w, 4 * (int64_t)qi + 3);
      }
    }
  } else {
    const int64_t per = (nw + kResThreads - 1) / kResThreads;
    const int64_t w0 = tid * per < nw ? tid * per : nw;
    const int64_t w1 = w0 + per < nw ? w0 + per : nw;
    uint32_t cnt = 0;
    for (int64_t w = w0; w < w1; ++w) cnt += __popc(bm[w]);
    pos = block_exclusive_scan<kResThreads>(cnt, scan_lds, tot);
    for (int64_t w = w0; w < w1; ++w) emit(bm[w], w);
  }
  for (int64_t j = tn + tid; j < p.top_t; j += kResThreads) {
    sel[j] = -1;
    if (selo) selo[j] = -1;
  }
}

void launch_select(const DecodeParams& p, dim3 grid, hipStream_t st, KernelEvents scan_ev, KernelEvents resolve_ev) {
  if (p.batch > 1)
    sf_launch(select_scan<true>, grid, dim3(kSelThreads), st, scan_ev, p);
  else
    sf_launch(select_scan<false>, grid, dim3(kSelThreads), st, scan_ev, p);
  sf_launch(select_resolve, dim3(p.batch * p.hkv), dim3(kResThreads), st, resolve_ev, p);
}

}  // namespace sfk

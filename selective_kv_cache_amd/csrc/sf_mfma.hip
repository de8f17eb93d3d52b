// Matrix-core (CDNA4 MFMA) forms of the score pass and of the base attention
// pass, for 2-, 3- and 4-bit base codes and GQA groups of 1, 2, 4 or 8 query
// heads (a group of 8 takes two tiles of 4 heads in the logit product and
// two heads per lane in the softmax; its 16 weight columns, hi and lo parts,
// fill the P.V product's 16).
//
// Logits (page "StrataFlux -- Selective precision streaming -- What does it
// mean?", paragraph "Which tiles count ...": scores from the resident low-bit
// keys).  With Khat = lo + (c + 1/2) * delta,
//   q . Khat = (lo + delta/2) * sum(q) + delta * (q . c),
// and q . c is an integer-code dot product.  Each query head is written as
// s * (d0 + d1/254 + d2/254^2 + d3/254^3) with int8 digits dk, so q . c is
// four exact int32 dot products: one v_mfma_i32_16x16x64_i8 tile holds
// 4 heads x 4 digits (rows) against 16 tokens (columns), two tiles per 128
// elements.  Lane l of the result then holds the four digit sums of head
// l/16 for token l%16.
//
// Values (paragraph "Which tiles count": unselected tokens take part at base
// precision).  sum_i p_i * vhat_i = sum_i p_i (lo_i + delta_i/2)
//                                   + sum_i (p_i delta_i) c_i,
// the first term a per-head scalar, the second a [heads x tokens] x
// [tokens x 128] product on v_mfma_f32_16x16x32_f16: the weights p*delta go in
// as fp16 hi + lo pieces (22 significant bits), the 2-bit codes as fp16
// subnormals taken from the packed bits with a shift and a mask (a code c at
// mantissa bit k reads as c * 2^(k-24), exactly; the power of two is undone
// per tile).  Every code is placed at bit k >= 4: measured on gfx950, the
// product's sums lose precision on the smallest subnormals (codes at bit 0
// gave errors near 1e-4 of the result, bit 2 near 2e-5, bits 4-8 the fp32
// level, 1e-6).  The codes of 8 tokens at one element are gathered with one
// v_perm_b32 per token pair, so the packed rows are read as they are stored.
//
// 3-bit codes straddle dword boundaries.  Row n of a P.V tile stands for
// elements 8n + tt (tile tt), so the lane of row n needs the 24-bit group of
// codes 8n .. 8n + 7 of each of its tokens: bits 24n .. 24n + 23 of the row,
// taken from two dwords with one funnel shift (v_alignbit_b32).  Two byte
// permutes pair the groups of two tokens (codes 0-3 and 4-7 of each in the
// two halves), and a shift and a mask per code put it at mantissa bit 4-7.
// The logit product takes a lane's 32 codes (96 bits) as four such groups,
// each half spread to one code per byte (decode_b3).
#include <math.h>
#include <stddef.h>

#include <type_traits>

#include "sf_attend_common.h"
#include "sf_mfma_common.h"

namespace sfk {

// ---------------------------------------------------------------------------
// Score pass: grid (n_score_split, hkv), NW wavefronts.  Each wave streams
// 32-token chunks (two logit tiles) of its split through an LDS ring; the
// per-head logits go to the logits buffer for the attention pass, their
// maximum over the group to the scores and the level-1 histogram.
// ---------------------------------------------------------------------------
constexpr int kSRing = 4;                      // stages per wavefront

template <int BB>
struct SStage {
  uint8_t k[32 * 16 * BB];                     // one 32-token chunk's K rows, as stored
  float2 ks[32];
};

template <int G, int NW, bool Batched, int BB = 2>
__global__ void __launch_bounds__(64 * NW) score_mfma(DecodeParams p) {
  static_assert(NW >= 4, "waves 0-3 prepare the query digits");
  static_assert(BB >= 2 && BB <= 4, "2-, 3- or 4-bit codes");
  constexpr int RB = 16 * BB;                    // bytes of a packed row
  constexpr int kSRingLoads = BB == 2 ? 2 : 3;   // direct loads per stage
  constexpr int SR = BB == 4 ? 3 : kSRing;       // stages per wavefront (4-bit: 3, so the ring fits the LDS)
  using SSt = SStage<BB>;
  constexpr int NT = G > 4 ? 2 : 1;              // tiles of 4 query heads
  static_assert(G <= 4 || G == 8, "groups of 1, 2, 4 or 8 query heads");
  __shared__ QPrepN<4 * NT> qp;
  __shared__ uint32_t lhist[kHistBins];
  __shared__ SSt ring[NW][SR];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kvh = blockIdx.y;
  int64_t lo, hi;
  int first;
  const int seq = locate_unit<Batched>(p, p.score_split, blockIdx.x, false, lo, hi, first);
  const float2 qx = load_query<G>(p.q + ((int64_t)seq * p.hq + kvh * G) * kHeadDim);
  const int64_t a = seq_at(p, seq);
  const int64_t t0 = (int64_t)kvh * p.cap + a + lo;            // first token row of the split
  const int nsp = (int)(hi - lo);
  const int nchunks = (nsp + 31) / 32;
  const int nmine = nchunks > wid ? (nchunks - wid + NW - 1) / NW : 0;
  // stage i <- chunk wid + NW i of the wave's own chunks: lane L loads bytes
  // 16L .. 16L + 15 of the chunk's K rows (2-bit: half L&1 of row L/2; 3-bit:
  // lanes L < 32 also bytes 1024 + 16L ..) and scale word L; the resources
  // end at the split's end (tokens past it read as zeros)
  const rsrc_t rK = make_rsrc(p.kc + t0 * RB, (uint32_t)nsp * (uint32_t)RB);
  const rsrc_t rS = make_rsrc(p.ks + t0 * 2, (uint32_t)nsp * 8u);
  const uint32_t oK = 16u * (uint32_t)lane, oS = 4u * (uint32_t)lane;
  auto issue = [&](int i, SSt& st) {
    const uint32_t c = (uint32_t)(wid + NW * i);
    bdma16(rK, oK, c * (32u * RB), st.k);
    if (BB == 4 || (BB == 3 && lane < 32)) bdma16(rK, oK + 1024u, c * (32u * RB), st.k + 1024);
    bdma4(rS, oS, c * 256u, st.ks);
  };
  // no selection, no histogram; the summed-probability score builds its own
  const bool hist = p.top_t > 0 && p.score_mode == 0;
  for (int i = tid; i < kHistBins; i += 64 * NW) lhist[i] = 0u;
#pragma unroll
  for (int k = 0; k < SR - 1; ++k)
    if (k < nmine) issue(k, ring[wid][k]);
  v4i aq[2 * NT];                                 // A operands: tile tl's k-halves in aq[2 tl], aq[2 tl + 1]
  if constexpr (NT == 2)
    prep_query8<BB>(qx, qp, aq);
  else
    prep_query<G, BB>(qx, qp, aq[0], aq[1]);
  // logits in log2 units (1/sqrt(D) and log2(e) folded into the per-head
  // constants): the attention pass's softmax takes them as they are; lane
  // (t, hl) holds head hl of each tile (hl and 4 + hl)
  constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
  const int t = lane & 15, hl = lane >> 4;
  float scale[NT], sumq[NT];
#pragma unroll
  for (int tl = 0; tl < NT; ++tl) {
    scale[tl] = qp.scale[4 * tl + (hl < G ? hl : 0)] * (kRsqrtD * kLog2e);
    sumq[tl] = qp.sumq[4 * tl + (hl < G ? hl : 0)] * (kRsqrtD * kLog2e);
  }
  float* scores = p.scores + (int64_t)kvh * p.ntot + (a - p.off0) + lo;
  float* lgo = p.logits + ((int64_t)kvh * p.ntot + (a - p.off0) + lo) * G;
  const uint32_t ring0 = lds_addr(&ring[wid][0]);
  // the lane's 32 codes of token t: bytes 8 hl .. (2-bit) or 12 hl .. (3-bit)
  const uint32_t aK = ring0 + (uint32_t)(t * RB + 4 * BB * hl);
  const uint32_t aS = ring0 + (uint32_t)(offsetof(SSt, ks) + 8 * t);
  const int hx = hl >> 1;                         // the tile a lane writes the score of
  const uint32_t hist0 = lds_addr(&lhist[0]);
  auto body = [&](auto kc, int i) {
    constexpr int k = decltype(kc)::value;        // stage of chunk i
    constexpr int OFF = k * (int)sizeof(SSt);
    if (i + SR - 1 < nmine) issue(i + SR - 1, ring[wid][(k + SR - 1) % SR]);
    // this wave's loads complete in order: stage i is in once no more than
    // the stages issued after it are outstanding (stores only add to the count)
    wait_stages<kSRingLoads, SR - 1>(min(SR - 1, nmine - 1 - i));
    const int c = wid + NW * i;
    uint32_t kw[2][4];
    uint64_t ks[2];
    if constexpr (BB == 2) {
      uint64_t k0, k1;
      asm volatile(
          "ds_read_b64 %0, %4 offset:%6\n\t"
          "ds_read_b64 %1, %4 offset:%7\n\t"
          "ds_read_b64 %2, %5 offset:%6\n\t"
          "ds_read_b64 %3, %5 offset:%8\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(k0), "=&v"(k1), "=&v"(ks[0]), "=&v"(ks[1])
          : "v"(aK), "v"(aS), "n"(OFF), "n"(OFF + 16 * RB), "n"(OFF + 128)
          : "memory");
      kw[0][0] = (uint32_t)k0;
      kw[0][1] = (uint32_t)(k0 >> 32);
      kw[1][0] = (uint32_t)k1;
      kw[1][1] = (uint32_t)(k1 >> 32);
      kw[0][2] = kw[1][2] = kw[0][3] = kw[1][3] = 0u;
    } else if constexpr (BB == 4) {
      v4u k0, k1;
      asm volatile(
          "ds_read_b128 %0, %4 offset:%6\n\t"
          "ds_read_b128 %1, %4 offset:%7\n\t"
          "ds_read_b64 %2, %5 offset:%6\n\t"
          "ds_read_b64 %3, %5 offset:%8\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(k0), "=&v"(k1), "=&v"(ks[0]), "=&v"(ks[1])
          : "v"(aK), "v"(aS), "n"(OFF), "n"(OFF + 16 * RB), "n"(OFF + 128)
          : "memory");
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        kw[0][x] = k0[x];
        kw[1][x] = k1[x];
      }
    } else {
      asm volatile(
          "ds_read_b32 %0, %8 offset:%10\n\t"
          "ds_read_b32 %1, %8 offset:%11\n\t"
          "ds_read_b32 %2, %8 offset:%12\n\t"
          "ds_read_b32 %3, %8 offset:%13\n\t"
          "ds_read_b32 %4, %8 offset:%14\n\t"
          "ds_read_b32 %5, %8 offset:%15\n\t"
          "ds_read_b64 %6, %9 offset:%10\n\t"
          "ds_read_b64 %7, %9 offset:%16\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(kw[0][0]), "=&v"(kw[0][1]), "=&v"(kw[0][2]), "=&v"(kw[1][0]), "=&v"(kw[1][1]), "=&v"(kw[1][2]),
            "=&v"(ks[0]), "=&v"(ks[1])
          : "v"(aK), "v"(aS), "n"(OFF), "n"(OFF + 4), "n"(OFF + 8), "n"(OFF + 16 * RB), "n"(OFF + 16 * RB + 4),
            "n"(OFF + 16 * RB + 8), "n"(OFF + 128)
          : "memory");
      kw[0][3] = kw[1][3] = 0u;
    }
    const bool full = 32 * c + 32 <= nsp;         // every token of the chunk inside the split
    float lg[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      v4i b0, b1;
      if constexpr (BB == 2)
        decode_b2(kw[j][0], kw[j][1], b0, b1);
      else if constexpr (BB == 3)
        decode_b3(kw[j][0], kw[j][1], kw[j][2], b0, b1);
      else
        decode_b4(kw[j][0], kw[j][1], kw[j][2], kw[j][3], b0, b1);
      const int rel = 32 * c + 16 * j + t;
      float xm = -INFINITY;
#pragma unroll
      for (int tl = 0; tl < NT; ++tl) {
        v4i D = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq[2 * tl], b0, v4i{0, 0, 0, 0}, 0, 0, 0);
        D = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq[2 * tl + 1], b1, D, 0, 0, 0);
        const float x = logit_scaled(D, __builtin_bit_cast(float2, ks[j]), scale[tl], sumq[tl]);
        xm = fmaxf(xm, hl < G ? x : -INFINITY);
        if (hl < G && (full || rel < nsp)) store_through(&lgo[rel * G + 4 * tl + hl], x);   // kept for the attention pass
      }
      lg[j] = xm;
    }
    // maximum over the heads, two tiles at once: lane (t, hl) keeps tile
    // hl/2 (token 16 (hl/2) + t)
    const float y = max_two_tiles(lg[0], lg[1]);
    const int rel = 32 * c + 16 * hx + t;
    if ((hl & 1) == 0 && (full || rel < nsp)) {
      const float sc = y * kLn2;                  // the score in natural units
      store_through(&scores[rel], sc);
      if (hist) lds_add_u32(hist0 + 4u * (score_key(sc) >> (32 - kHistBits)), 1u);
    }
  };
  for (int i = 0; i < nmine; i += SR) {
    progress_priority(nmine - i, nmine);
    ring_round<SR>(body, i, nmine);
  }
  __builtin_amdgcn_s_setprio(0);
  // the histogram adds (asm, not waited for) complete before the barrier
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  if (!hist) return;
  __syncthreads();
  uint32_t* gh = p.hist + ((int64_t)seq * p.hkv + kvh) * kHistBins;   // level-1 histogram
  for (int i = tid; i < kHistBins; i += 64 * NW) {
    const uint32_t c = lhist[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

// ---------------------------------------------------------------------------
// Score variant: the attention a token receives (page "StrataFlux --
// Selective precision streaming -- What does it mean?", paragraph "Which
// tiles count ..."), the sum over the group of each query head's softmax
// probability over the sequence's tokens, from the logits (log2 units) the
// score pass left.  softmax_stats: per score unit, each head's maximum and
// sum of 2^(logit - maximum); softmax_scores: the sequence's normalisers
// from its units' pairs, then the unit's scores and the level-1 histogram.
// One work-group of 256 threads per (score unit, KV head), as the score pass.
// ---------------------------------------------------------------------------

template <int N>
__device__ inline void block_max_sum(float (&m)[N], float* red, bool take_max) {
  // every thread ends with the block's maximum (take_max) or sum of each value
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float v = take_max ? wave_max_dpp(m[i]) : wave_sum_dpp(m[i]);
    if (lane == 0) red[wid * N + i] = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float v = red[i];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) v = take_max ? fmaxf(v, red[w * N + i]) : v + red[w * N + i];
    m[i] = v;
  }
  __syncthreads();
}

template <int G, bool Batched>
__global__ void __launch_bounds__(256) softmax_stats(DecodeParams p) {
  __shared__ float red[4 * G];
  const int kvh = blockIdx.y;
  int64_t lo, hi;
  int first;
  const int seq = locate_unit<Batched>(p, p.score_split, blockIdx.x, false, lo, hi, first);
  const int64_t a = seq_at(p, seq);
  const float* lg = p.logits + ((int64_t)kvh * p.ntot + (a - p.off0) + lo) * G;
  const int n = (int)(hi - lo);
  float m[G], z[G];
#pragma unroll
  for (int h = 0; h < G; ++h) m[h] = -INFINITY;
  for (int i = threadIdx.x; i < n; i += blockDim.x)
#pragma unroll
    for (int h = 0; h < G; ++h) m[h] = fmaxf(m[h], lg[i * G + h]);
  block_max_sum<G>(m, red, true);
#pragma unroll
  for (int h = 0; h < G; ++h) z[h] = 0.f;
  for (int i = threadIdx.x; i < n; i += blockDim.x)
#pragma unroll
    for (int h = 0; h < G; ++h) z[h] += __builtin_amdgcn_exp2f(lg[i * G + h] - m[h]);
  block_max_sum<G>(z, red, false);
  if (threadIdx.x == 0)
#pragma unroll
    for (int h = 0; h < G; ++h) p.sstat[((int64_t)kvh * p.n_score_split + blockIdx.x) * G + h] = make_float2(m[h], z[h]);
}

template <int G, bool Batched>
__global__ void __launch_bounds__(256) softmax_scores(DecodeParams p) {
  __shared__ float red[4 * G];
  __shared__ uint32_t lhist[kHistBins];
  const int kvh = blockIdx.y;
  int64_t lo, hi;
  int first;
  const int seq = locate_unit<Batched>(p, p.score_split, blockIdx.x, false, lo, hi, first);
  const int64_t a = seq_at(p, seq);
  const int64_t n_s = seq_at(p, seq + 1) - a;
  const int nu = (int)((n_s + p.score_split - 1) / p.score_split);   // the sequence's units
  const float2* st = p.sstat + ((int64_t)kvh * p.n_score_split + first) * G;
  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) lhist[i] = 0u;
  // the normalisers: M = max of the units' maxima, Z = sum of z_u 2^(m_u - M)
  float M[G], Z[G];
#pragma unroll
  for (int h = 0; h < G; ++h) M[h] = -INFINITY;
  for (int u = threadIdx.x; u < nu; u += blockDim.x)
#pragma unroll
    for (int h = 0; h < G; ++h) M[h] = fmaxf(M[h], st[u * G + h].x);
  block_max_sum<G>(M, red, true);
#pragma unroll
  for (int h = 0; h < G; ++h) Z[h] = 0.f;
  for (int u = threadIdx.x; u < nu; u += blockDim.x)
#pragma unroll
    for (int h = 0; h < G; ++h) Z[h] += st[u * G + h].y * __builtin_amdgcn_exp2f(st[u * G + h].x - M[h]);
  block_max_sum<G>(Z, red, false);
  float rz[G];
#pragma unroll
  for (int h = 0; h < G; ++h) rz[h] = 1.0f / Z[h];
  const float* lg = p.logits + ((int64_t)kvh * p.ntot + (a - p.off0) + lo) * G;
  float* scores = p.scores + (int64_t)kvh * p.ntot + (a - p.off0) + lo;
  const int n = (int)(hi - lo);
  const bool hist = p.top_t > 0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    float sc = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) sc = fmaf(__builtin_amdgcn_exp2f(lg[i * G + h] - M[h]), rz[h], sc);
    scores[i] = sc;
    if (hist) atomicAdd(&lhist[score_key(sc) >> (32 - kHistBits)], 1u);
  }
  if (!hist) return;
  __syncthreads();
  uint32_t* gh = p.hist + ((int64_t)seq * p.hkv + kvh) * kHistBins;   // level-1 histogram
  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) {
    const uint32_t c = lhist[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

template <bool Batched>
static bool launch_softmax_scores_b(const DecodeParams& p, dim3 grid, hipStream_t st) {
  switch (p.grp) {
    case 1:
      hipLaunchKernelGGL((softmax_stats<1, Batched>), grid, dim3(256), 0, st, p);
      hipLaunchKernelGGL((softmax_scores<1, Batched>), grid, dim3(256), 0, st, p);
      return true;
    case 2:
      hipLaunchKernelGGL((softmax_stats<2, Batched>), grid, dim3(256), 0, st, p);
      hipLaunchKernelGGL((softmax_scores<2, Batched>), grid, dim3(256), 0, st, p);
      return true;
    case 4:
      hipLaunchKernelGGL((softmax_stats<4, Batched>), grid, dim3(256), 0, st, p);
      hipLaunchKernelGGL((softmax_scores<4, Batched>), grid, dim3(256), 0, st, p);
      return true;
  }
  return false;
}

bool launch_softmax_scores(const DecodeParams& p, dim3 grid, hipStream_t st) {
  return p.batch > 1 ? launch_softmax_scores_b<true>(p, grid, st) : launch_softmax_scores_b<false>(p, grid, st);
}

// The base pass streams its split through a per-wavefront ring of LDS stages
// filled by direct global->LDS loads (global_load_lds: lane i's 16 or 4 bytes
// land at stage offset 16*i or 4*i), so the loads in flight hold no
// registers.  One stage is one 32-token chunk: the per-head logits the score
// pass left, V codes (1 KiB, as stored) and V scales (256 B).  K is not read
// again.
constexpr int kRing = 4;                       // stages per wavefront; kRing - 1 chunks in flight

template <int G, int BB = 2>
struct Stage {
  float lg[32 * G];
  uint8_t v[32 * 16 * BB];
  float2 vs[32];
};

template <int G, int NW, int BB = 2>
struct MfmaLds {
  alignas(16) _Float16 wt[NW][2 * G][32];   // per wave: P.V weights [column][kappa]: hi parts, then lo parts
  alignas(16) _Float16 wzero[8];            // weight columns >= 2G read zeros
  float mw[NW][G], lw[NW][G];
  union {
    Stage<G, BB> ring[NW][kRing];
    float accw[NW][2 * G][kHeadDim + 1];    // after the stream: per-wave P.V, hi and lo columns
                                            // (rows padded by a word: the 16 columns one write spans hit different banks)
  } u;
};

// One lane's operands of a stage.  The LDS reads are written in asm: a read
// the compiler sees makes it wait for every direct load in flight (it cannot
// tell the ring stages apart), which would serialise the stream.  The block
// waits for its own reads before it ends, so every output is complete.  OFF
// is the stage's byte offset in the wave's ring (an immediate of each read).
struct StageRegs {
  float lg[2];             // logits of tokens t, 16 + t for head hl
  uint64_t vsc[2];         // (lo, delta) of tokens t, 16 + t
  uint32_t vw[8];          // V dword vdw of tokens 4rg+v (vw[2v]) and 16+4rg+v (vw[2v+1])
};

template <int G, int OFF>
__device__ inline void read_stage(uint32_t aL, uint32_t aS, const uint32_t (&aV)[4], StageRegs& r) {
  asm volatile(
      "ds_read_b32 %0, %12 offset:%18\n\t"
      "ds_read_b32 %1, %12 offset:%19\n\t"
      "ds_read_b64 %2, %13 offset:%18\n\t"
      "ds_read_b64 %3, %13 offset:%20\n\t"
      "ds_read_b32 %4, %14 offset:%18\n\t"
      "ds_read_b32 %5, %14 offset:%21\n\t"
      "ds_read_b32 %6, %15 offset:%18\n\t"
      "ds_read_b32 %7, %15 offset:%21\n\t"
      "ds_read_b32 %8, %16 offset:%18\n\t"
      "ds_read_b32 %9, %16 offset:%21\n\t"
      "ds_read_b32 %10, %17 offset:%18\n\t"
      "ds_read_b32 %11, %17 offset:%21\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r.lg[0]), "=&v"(r.lg[1]), "=&v"(r.vsc[0]), "=&v"(r.vsc[1]), "=&v"(r.vw[0]), "=&v"(r.vw[1]),
        "=&v"(r.vw[2]), "=&v"(r.vw[3]), "=&v"(r.vw[4]), "=&v"(r.vw[5]), "=&v"(r.vw[6]), "=&v"(r.vw[7])
      : "v"(aL), "v"(aS), "v"(aV[0]), "v"(aV[1]), "v"(aV[2]), "v"(aV[3]), "n"(OFF), "n"(OFF + 16 * G * 4),
        "n"(OFF + 128), "n"(OFF + 512)
      : "memory");
}

// The 3-bit form: the two dwords holding row n's 24-bit group of each of
// the lane's 8 tokens (4rg + v: vw[4v], vw[4v + 1]; 16 + 4rg + v: vw[4v + 2],
// vw[4v + 3]).  aV points at the first dword of token 4rg's group.  Row 15's
// group lies in the row's last dword alone; its second read (the next row's
// first dword, or for token 31 the stage's first scale word) stays inside
// the stage and its value is shifted out.
struct StageRegs3 {
  float lg[2];
  uint64_t vsc[2];
  uint32_t vw[16];
};

template <int G, int OFF>
__device__ inline void read_stage3(uint32_t aL, uint32_t aS, uint32_t aV, StageRegs3& r) {
  constexpr int RB = 48, T16 = 16 * RB;
  asm volatile(
      "ds_read_b32 %0, %20 offset:%23\n\t"
      "ds_read_b32 %1, %20 offset:%24\n\t"
      "ds_read_b64 %2, %21 offset:%23\n\t"
      "ds_read_b64 %3, %21 offset:%25\n\t"
      "ds_read_b32 %4, %22 offset:%23\n\t"
      "ds_read_b32 %5, %22 offset:%26\n\t"
      "ds_read_b32 %6, %22 offset:%27\n\t"
      "ds_read_b32 %7, %22 offset:%28\n\t"
      "ds_read_b32 %8, %22 offset:%29\n\t"
      "ds_read_b32 %9, %22 offset:%30\n\t"
      "ds_read_b32 %10, %22 offset:%31\n\t"
      "ds_read_b32 %11, %22 offset:%32\n\t"
      "ds_read_b32 %12, %22 offset:%33\n\t"
      "ds_read_b32 %13, %22 offset:%34\n\t"
      "ds_read_b32 %14, %22 offset:%35\n\t"
      "ds_read_b32 %15, %22 offset:%36\n\t"
      "ds_read_b32 %16, %22 offset:%37\n\t"
      "ds_read_b32 %17, %22 offset:%38\n\t"
      "ds_read_b32 %18, %22 offset:%39\n\t"
      "ds_read_b32 %19, %22 offset:%40\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r.lg[0]), "=&v"(r.lg[1]), "=&v"(r.vsc[0]), "=&v"(r.vsc[1]), "=&v"(r.vw[0]), "=&v"(r.vw[1]),
        "=&v"(r.vw[2]), "=&v"(r.vw[3]), "=&v"(r.vw[4]), "=&v"(r.vw[5]), "=&v"(r.vw[6]), "=&v"(r.vw[7]),
        "=&v"(r.vw[8]), "=&v"(r.vw[9]), "=&v"(r.vw[10]), "=&v"(r.vw[11]), "=&v"(r.vw[12]), "=&v"(r.vw[13]),
        "=&v"(r.vw[14]), "=&v"(r.vw[15])
      : "v"(aL), "v"(aS), "v"(aV), "n"(OFF), "n"(OFF + 16 * G * 4), "n"(OFF + 128), "n"(OFF + 4),
        "n"(OFF + T16), "n"(OFF + T16 + 4), "n"(OFF + RB), "n"(OFF + RB + 4), "n"(OFF + T16 + RB),
        "n"(OFF + T16 + RB + 4), "n"(OFF + 2 * RB), "n"(OFF + 2 * RB + 4), "n"(OFF + T16 + 2 * RB),
        "n"(OFF + T16 + 2 * RB + 4), "n"(OFF + 3 * RB), "n"(OFF + 3 * RB + 4), "n"(OFF + T16 + 3 * RB),
        "n"(OFF + T16 + 3 * RB + 4)
      : "memory");
}

// The 4-bit form: dword n of each of the lane's 8 tokens' rows (row n's 8
// codes; 4rg + v: vw[2v], 16 + 4rg + v: vw[2v + 1]).  aV points at dword n of
// token 4rg's row.
template <int OFF>
__device__ inline void read_vrows4(uint32_t aV, uint32_t (&vw)[8]) {
  constexpr int RB = 64, T16 = 16 * RB;
  asm volatile(
      "ds_read_b32 %0, %8 offset:%9\n\t"
      "ds_read_b32 %1, %8 offset:%10\n\t"
      "ds_read_b32 %2, %8 offset:%11\n\t"
      "ds_read_b32 %3, %8 offset:%12\n\t"
      "ds_read_b32 %4, %8 offset:%13\n\t"
      "ds_read_b32 %5, %8 offset:%14\n\t"
      "ds_read_b32 %6, %8 offset:%15\n\t"
      "ds_read_b32 %7, %8 offset:%16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(vw[0]), "=&v"(vw[1]), "=&v"(vw[2]), "=&v"(vw[3]), "=&v"(vw[4]), "=&v"(vw[5]), "=&v"(vw[6]),
        "=&v"(vw[7])
      : "v"(aV), "n"(OFF), "n"(OFF + T16), "n"(OFF + RB), "n"(OFF + T16 + RB), "n"(OFF + 2 * RB),
        "n"(OFF + T16 + 2 * RB), "n"(OFF + 3 * RB), "n"(OFF + T16 + 3 * RB)
      : "memory");
}

template <int G, int NW, bool Batched, int BB = 2>
__device__ inline void base_split_mfma(const DecodeParams& p, int split, int kvh, uint8_t* smem) {
  static_assert(BB >= 2 && BB <= 4, "2-, 3- or 4-bit codes");
  static_assert(G <= 4 || G == 8, "groups of 1, 2, 4 or 8 query heads");
  constexpr int NS = G > 4 ? 2 : 1;                // query heads per logit lane: hl (and 4 + hl)
  constexpr int RB = 16 * BB;                      // bytes of a packed row
  constexpr int kRingLoads = BB == 2 ? 3 : 4;      // direct loads per stage (3- and 4-bit rows: two V loads)
  using Lds = MfmaLds<G, NW, BB>;
  using St = Stage<G, BB>;
  Lds& s = *reinterpret_cast<Lds*>(smem);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  int64_t lo, hi;
  int first;
  const int seq = locate_unit<Batched>(p, p.split, split, false, lo, hi, first);
  const int64_t a = seq_at(p, seq);
  const int64_t sk = (int64_t)seq * p.hkv + kvh;
  const bool masked = p.use_refine != 0;
  const int64_t t0 = (int64_t)kvh * p.cap + a + lo;            // first token row of the split
  const int nsp = (int)(hi - lo);                               // tokens of the split (<= 4096)
  const int nchunks = (nsp + 31) / 32;
  const int nmine = nchunks > wid ? (nchunks - wid + NW - 1) / NW : 0;   // chunks wid, wid+NW, ...

  // Stage i of this wave <- chunk wid + NW*i.  Lane L loads the scale word L
  // of the chunk (token L/2), lanes L < 8G the logits' bytes [16L, 16L+16),
  // and 2-bit codes: half L&1 of V row (L/2) ^ ((L/8) & 3): row r of the
  // chunk sits at stage row r ^ ((r/4) & 3), so that the four rows one P.V
  // read takes (4rg + v, rg = 0..3) fall in different LDS banks; 3-bit codes:
  // bytes 16L .. 16L + 15 of the chunk's rows as stored (and lanes L < 32
  // bytes 1024 + 16L ..; rows 48 bytes apart already spread the four rows
  // over the banks).  The resources end at the split's end: tokens past it
  // read as zeros.
  const rsrc_t rV = make_rsrc(p.vc + t0 * RB, (uint32_t)nsp * (uint32_t)RB);
  const rsrc_t rS = make_rsrc(p.vs + t0 * 2, (uint32_t)nsp * 8u);
  const rsrc_t rL = make_rsrc(p.logits + ((int64_t)kvh * p.ntot + (a - p.off0) + lo) * G, (uint32_t)nsp * G * 4u);
  const uint32_t oV =
      BB == 2 ? (uint32_t)(((lane >> 1) ^ ((lane >> 3) & 3)) * 32 + 16 * (lane & 1)) : 16u * (uint32_t)lane;
  const uint32_t oS = 4u * (uint32_t)lane, oL = 16u * (uint32_t)lane;
  auto issue = [&](int i, St& st) {
    const uint32_t c = (uint32_t)(wid + NW * i);
    if (lane < 8 * G) bdma16(rL, oL, c * (32u * G * 4u), st.lg);
    bdma16(rV, oV, c * (32u * RB), st.v);
    if (BB == 4 || (BB == 3 && lane < 32)) bdma16(rV, oV + 1024u, c * (32u * RB), st.v + 1024);
    bdma4(rS, oS, c * 256u, st.vs);
  };
#pragma unroll
  for (int k = 0; k < kRing - 1; ++k)
    if (k < nmine) issue(k, s.u.ring[wid][k]);

  for (int i = lane; i < 2 * G * 32; i += 64) (&s.wt[wid][0][0])[i] = (_Float16)0.f;
  if (tid < 8) s.wzero[tid] = (_Float16)0.f;
  // selection words of the split (one per chunk) in two registers: lane L
  // holds those of chunks L and 64 + L; splits start on a word boundary
  constexpr int kMaxSplitWords = 4096 / 32;
  static_assert(kMaxSplitWords <= 128, "two words per lane");
  const uint32_t* bmw = p.bitmap + sk * p.bm_words + (lo >> 5);
  const uint32_t sw0 = masked && lane < nchunks ? bmw[lane] : 0u;
  const uint32_t sw1 = masked && 64 + lane < nchunks ? bmw[64 + lane] : 0u;
  __syncthreads();
  const int t = lane & 15, hl = lane >> 4;        // logit layout: token t (and 16 + t), head hl
  const int n = lane & 15, rg = lane >> 4;        // P.V layout: column n, k-group rg
  const int hlc = hl < G ? hl : 0;
  // v_perm_b32 selector: half (n & 1) of each of two dwords
  const uint32_t hsel = 2u * (uint32_t)(n & 1);
  const uint32_t psel = hsel | ((hsel + 1u) << 8) | ((hsel + 4u) << 16) | ((hsel + 5u) << 24);
  const int vdw = n >> 1;                         // dword of the V row holding elements 8n..8n+7

  // LDS addresses of this lane's stage operands (stage 0; the stage's offset
  // is an immediate of each read).  P.V k index kappa = 2u + j stands for
  // token 16j + u, so lane (n, rg) takes tokens 4rg..4rg+3 and
  // 16+4rg..16+4rg+3, and a logit lane's two weights are adjacent.  Weight
  // column h < G holds head h's hi parts, column G + h its lo parts, so one
  // product per tile takes both.
  const uint32_t ring0 = lds_addr(&s.u.ring[wid][0]);
  const uint32_t wtR = n < 2 * G ? lds_addr(&s.wt[wid][n][8 * rg]) : lds_addr(&s.wzero[0]);
  uint32_t wtHi[NS], wtLo[NS];
#pragma unroll
  for (int q = 0; q < NS; ++q) {
    wtHi[q] = lds_addr(&s.wt[wid][4 * q + hlc][2 * t]);
    wtLo[q] = lds_addr(&s.wt[wid][G + 4 * q + hlc][2 * t]);
  }
  const uint32_t aL = ring0 + (uint32_t)(offsetof(St, lg) + 4 * (t * G + hlc));
  const uint32_t aS = ring0 + (uint32_t)(offsetof(St, vs) + 8 * t);
  uint32_t aV[4];                                 // 2-bit: token 4rg + v at stage row 4rg + (v ^ rg)
#pragma unroll
  for (int v = 0; v < 4; ++v) aV[v] = ring0 + (uint32_t)(offsetof(St, v) + (4 * rg + (v ^ rg)) * 32 + 4 * vdw);
  // 3-bit: row n's group (bits 24n ..) starts in dword 3n/4 at bit 24n % 32
  const uint32_t aV3 = ring0 + (uint32_t)(offsetof(St, v) + 4 * rg * RB + 4 * ((3 * n) >> 2));
  // 4-bit: row n's group is dword n of the row
  const uint32_t aV4 = ring0 + (uint32_t)(offsetof(St, v) + 4 * rg * RB + 4 * n);
  const uint32_t gsh = (uint32_t)((24 * n) & 31);
  // rows hl < G hold heads; the others take no part
  const uint64_t rows = G >= 4 ? ~0ull : (1ull << (16 * (G & 3))) - 1ull;
  const float ninf = -INFINITY;

  // running maximum: a finite floor below every logit until a token takes
  // part, so exp2(logit - m) is 0 (not NaN) for the -inf of tokens left out
  constexpr float kFloor = -1e30f;
  constexpr int kSlack = 6;                       // weights up to 2^kSlack (log2 units of the reference)
  float m[NS], lsum[NS], t1[NS];
#pragma unroll
  for (int q = 0; q < NS; ++q) {
    m[q] = kFloor;
    lsum[q] = t1[q] = 0.f;
  }
  int sexp = 127;                                 // weight scale 2^sexp; 127 = not set yet
  float wsc = 1.0f;                               // 2^sexp once set
  v4f acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};

  auto body = [&](auto kc, int i) {
    constexpr int k = decltype(kc)::value;        // stage of chunk i
    if (i + kRing - 1 < nmine) issue(i + kRing - 1, s.u.ring[wid][(k + kRing - 1) % kRing]);
    // this wave's loads complete in order: stage i is in once no more than
    // the stages issued after it are outstanding
    wait_stages<kRingLoads, kRing - 1>(min(kRing - 1, nmine - 1 - i));
    const int c = wid + NW * i;
    const int rem = nsp - 32 * c;                 // tokens of this chunk inside the split
    // the chunk's tokens that take part (unmarked, inside the split) as lane
    // masks: bit l of mk[j] for lane l = (row, t): token 16 j + t
    uint32_t vm = ~(uint32_t)__builtin_amdgcn_readlane((int)(c < 64 ? sw0 : sw1), c & 63);
    if (rem < 32) vm &= (1u << rem) - 1u;
    const uint32_t y0 = (vm & 0xFFFFu) | (vm << 16), y1 = (vm >> 16) | (vm & 0xFFFF0000u);
    const uint64_t mk[2] = {((uint64_t)y0 | ((uint64_t)y0 << 32)) & rows, ((uint64_t)y1 | ((uint64_t)y1 << 32)) & rows};
    StageRegs R;
    [[maybe_unused]] StageRegs3 R3;
    if constexpr (BB == 2) {
      read_stage<G, k * (int)sizeof(St)>(aL, aS, aV, R);
    } else if constexpr (BB == 4) {
      // the logits and scales as in the 2-bit read (its V reads go to the
      // first row, unused), then the rows' dwords n
      read_stage<G, k * (int)sizeof(St)>(aL, aS, aV, R);
      read_vrows4<k * (int)sizeof(St)>(aV4, R.vw);
    } else {
      read_stage3<G, k * (int)sizeof(St)>(aL, aS, aV3, R3);
      R.lg[0] = R3.lg[0];
      R.lg[1] = R3.lg[1];
      R.vsc[0] = R3.vsc[0];
      R.vsc[1] = R3.vsc[1];
    }
    // head 4 + hl's logits (groups of 8)
    float lgB[2] = {0.f, 0.f};
    if constexpr (NS == 2) {
      constexpr int OFF = k * (int)sizeof(St);
      asm volatile(
          "ds_read_b32 %0, %2 offset:%3\n\t"
          "ds_read_b32 %1, %2 offset:%4\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(lgB[0]), "=&v"(lgB[1])
          : "v"(aL), "n"(OFF + 16), "n"(OFF + 16 * G * 4 + 16)
          : "memory");
    }
    // logits (log2 units, as the score pass kept them); -inf where the token
    // takes no part
    float lg[NS][2];
    float2 vsc[2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      lg[0][jj] = lane_select(mk[jj], R.lg[jj], ninf);
      if constexpr (NS == 2) lg[NS - 1][jj] = lane_select(mk[jj], lgB[jj], ninf);
      vsc[jj] = __builtin_bit_cast(float2, R.vsc[jj]);
    }
    // online softmax with a lazy reference: m moves (and the sums are
    // rescaled) only when a logit exceeds it by more than kSlack, so the
    // weights stay below 2^kSlack and most chunks need no row maximum
    float xm[NS], mnew[NS];
    bool grow = false;
#pragma unroll
    for (int q = 0; q < NS; ++q) {
      xm[q] = fmaxf(lg[q][0], lg[q][1]);
      grow = grow || __ballot(xm[q] > m[q] + kSlack) != 0ull;
    }
#pragma unroll
    for (int q = 0; q < NS; ++q) mnew[q] = grow ? fmaxf(m[q], row16_max_dpp(xm[q])) : m[q];
    // weight scale: keep delta * 2^sexp below 2^(14 - kSlack) over the
    // chunk; the chunk's largest delta is needed only when one reaches it
    float dmax = fmaxf(lane_select(mk[0], vsc[0].y, 0.f), lane_select(mk[1], vsc[1].y, 0.f));
    int need = sexp;
    if (__ballot(dmax > 0.f && (sexp == 127 || dmax >= __builtin_ldexpf(1.0f, 14 - kSlack - sexp))) != 0ull) {
      dmax = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_max(dmax))));
      int e2;
      frexpf(dmax, &e2);
      need = 14 - kSlack - e2;   // wave-uniform, and so is sexp
    }
    if (grow || need < sexp) {
      float alpha[NS];
#pragma unroll
      for (int q = 0; q < NS; ++q) {
        alpha[q] = mnew[q] > m[q] ? __builtin_amdgcn_exp2f(m[q] - mnew[q]) : 1.f;   // 0 from the floor
        lsum[q] *= alpha[q];
        t1[q] *= alpha[q];
      }
      // column n < 2G: head n % G (lane group (n % G) % 4, slot (n % G) / 4)
      const int hc = n < 2 * G ? n % G : 0;
      float f = lane_value(alpha[0], 0);
#pragma unroll
      for (int h = 1; h < G; ++h) {
        // read with every lane active (a lane read inside the selection
        // could run where lane 16 h is off)
        const float ah = lane_value(alpha[h / 4], 16 * (h % 4));
        f = hc == h ? ah : f;
      }
      if (need < sexp) {
        if (sexp != 127) f = __builtin_ldexpf(f, need - sexp);
        sexp = need;
        wsc = __builtin_ldexpf(1.0f, sexp);
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) acc[jj] *= f;
#pragma unroll
      for (int q = 0; q < NS; ++q) m[q] = mnew[q];
    }
    // weights as fp16 hi + lo (truncated hi, exact remainder): 22 bits, the
    // two parts in separate columns of one product
#pragma unroll
    for (int q = 0; q < NS; ++q) {
      float wv[2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const float pk = __builtin_amdgcn_exp2f(lg[q][jj] - m[q]);   // exp2(-inf) = 0: tokens left out
        lsum[q] += pk;
        t1[q] = fmaf(pk, fmaf(0.5f, vsc[jj].y, vsc[jj].x), t1[q]);
        wv[jj] = pk * (vsc[jj].y * wsc);
      }
      const auto whi = __builtin_amdgcn_cvt_pkrtz(wv[0], wv[1]);
      const auto wlo = __builtin_amdgcn_cvt_pkrtz(wv[0] - (float)whi[0], wv[1] - (float)whi[1]);
      if (4 * q + hl < G) {
        lds_write_u32(wtHi[q], __builtin_bit_cast(uint32_t, whi));
        lds_write_u32(wtLo[q], __builtin_bit_cast(uint32_t, wlo));
      }
    }
    const v8h bw = lds_read_v8h(wtR);
    if constexpr (BB == 2) {
      const uint32_t* vw = R.vw;
      // each 16-bit half of P holds the 8 codes (2 bits each, code tt at bit
      // 2tt) of one token; code tt goes in at mantissa bit code_bit(tt) >= 4:
      // codes 0-1 from P << 4, 2-4 from P, 5-7 from P >> 6 (the masks keep
      // each half's own bits)
      uint32_t P[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) P[v] = __builtin_amdgcn_perm(vw[2 * v + 1], vw[2 * v], psel);
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const uint32_t msk = 0x00030003u << code_bit(tt);
        v4u av;
#pragma unroll
        for (int v = 0; v < 4; ++v) av[v] = (tt < 2 ? P[v] << 4 : tt < 5 ? P[v] : P[v] >> 6) & msk;
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, av), bw, acc[tt], 0, 0, 0);
      }
    } else if constexpr (BB == 4) {
      // row n's 8 codes are dword n of each row: P03 pairs the two tokens'
      // low halves (codes 0-3 at bits 0, 4, 8, 12 of each half), P47 their
      // high halves (codes 4-7); code tt goes in at mantissa bit 4
      uint32_t P03[4], P47[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        P03[v] = __builtin_amdgcn_perm(R.vw[2 * v + 1], R.vw[2 * v], 0x05040100u);
        P47[v] = __builtin_amdgcn_perm(R.vw[2 * v + 1], R.vw[2 * v], 0x07060302u);
      }
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        v4u av;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint32_t y = tt < 4 ? P03[v] : P47[v];
          const int q = tt & 3;
          const uint32_t x = q == 0 ? y << 4 : q == 1 ? y : q == 2 ? y >> 4 : y >> 8;
          av[v] = x & 0x00F000F0u;
        }
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, av), bw, acc[tt], 0, 0, 0);
      }
    } else {
      // the 24-bit groups of the token pair (4rg + v, 16 + 4rg + v); P03
      // holds bits 0-15 of each in its two halves (codes 0-4), P47 bits
      // 8-23 (codes 4-7 at bits 4, 7, 10, 13); code tt goes in at mantissa
      // bit code_bit3(tt): 0 and 1 from P03 << 4, 2 from P03, 3 from
      // P03 >> 2, 4 and 5 from P47, 6 and 7 from P47 >> 6
      uint32_t P03[4], P47[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint32_t ga = __builtin_amdgcn_alignbit(R3.vw[4 * v + 1], R3.vw[4 * v], gsh);
        const uint32_t gb = __builtin_amdgcn_alignbit(R3.vw[4 * v + 3], R3.vw[4 * v + 2], gsh);
        P03[v] = __builtin_amdgcn_perm(gb, ga, 0x05040100u);
        P47[v] = __builtin_amdgcn_perm(gb, ga, 0x06050201u);
      }
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const uint32_t msk = 0x00070007u << code_bit3(tt);
        v4u av;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint32_t x = tt < 2    ? P03[v] << 4
                             : tt == 2 ? P03[v]
                             : tt == 3 ? P03[v] >> 2
                             : tt < 6  ? P47[v]
                                       : P47[v] >> 6;
          av[v] = x & msk;
        }
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, av), bw, acc[tt], 0, 0, 0);
      }
    }
  };
  for (int i = 0; i < nmine; i += kRing) {
    progress_priority(nmine - i, nmine);
    ring_round<kRing>(body, i, nmine);
  }
  __builtin_amdgcn_s_setprio(0);
  // the ring is reused below: no load of this wave may still be landing, and
  // every wave must be done with its stages
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // wave totals: l and the scalar term per head (row sums), P.V per column
  // (column n < G: head n's hi part, G + h: its lo part); maxima stay in
  // log2 units until the partial is written
#pragma unroll
  for (int q = 0; q < NS; ++q) {
    lsum[q] = row16_sum(lsum[q]);
    t1[q] = row16_sum(t1[q]);
  }
  if (t == 0) {
#pragma unroll
    for (int q = 0; q < NS; ++q)
      if (4 * q + hl < G) {
        s.mw[wid][4 * q + hl] = m[q] == kFloor ? -INFINITY : m[q];   // -inf: no token took part
        s.lw[wid][4 * q + hl] = lsum[q];
      }
  }
  float t1n = 0.f;                                // the scalar term goes with the hi column
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float th = lane_value(t1[h / 4], 16 * (h % 4));   // every lane active (see the rescale above)
    t1n = n == h ? th : t1n;
  }
  const int se = sexp == 127 ? 0 : sexp;
  if (n < 2 * G) {
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const float f = __builtin_ldexpf(1.0f, 24 - code_bit_of<BB>(tt) - se);
#pragma unroll
      for (int j = 0; j < 4; ++j) s.u.accw[wid][n][32 * rg + 8 * j + tt] = fmaf(acc[tt][j], f, t1n);
    }
  }
  __syncthreads();
  // the work-group's partial: the waves' (m, l, acc) merged, hi + lo columns
  float* part = p.part + ((int64_t)kvh * (p.n_sel_blk + p.n_split) + p.n_sel_blk + split) * G * kPartStride;
  for (int i = tid; i < G * kHeadDim; i += 64 * NW) {
    const int h = i / kHeadDim, d = i % kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s.mw[w][h]);
    float A = 0.f, L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float e = __builtin_amdgcn_exp2f(s.mw[w][h] - M);   // 0 for a wave without tokens
        A += e * (s.u.accw[w][h][d] + s.u.accw[w][G + h][d]);
        L += e * s.lw[w][h];
      }
    }
    part[h * kPartStride + d] = A;
    if (d == 0) {
      part[h * kPartStride + kHeadDim] = M * 0.6931471805599453f;   // natural-log units
      part[h * kPartStride + kHeadDim + 1] = L;
    }
  }
}

template <int G, int NW, bool Batched, int BB = 2>
__global__ void __launch_bounds__(64 * NW) attend_mfma(DecodeParams p) {
  __shared__ __align__(16) uint8_t smem[cmax(sizeof(SelLds<BB, G, NW, 16>), sizeof(MfmaLds<G, NW, BB>))];
  if ((int)blockIdx.x < p.n_sel_blk)
    selected_block_any<BB, G, NW, true, Batched>(p, blockIdx.x, blockIdx.y, smem);
  else
    base_split_mfma<G, NW, Batched, BB>(p, blockIdx.x - p.n_sel_blk, blockIdx.y, smem);
}

template <bool Batched, int BB>
static bool launch_score_mfma_b(const DecodeParams& p, dim3 grid, hipStream_t st, KernelEvents ev) {
  switch (p.grp) {
    case 1: sf_launch(score_mfma<1, kScoreWaves, Batched, BB>, grid, dim3(64 * kScoreWaves), st, ev, p); return true;
    case 2: sf_launch(score_mfma<2, kScoreWaves, Batched, BB>, grid, dim3(64 * kScoreWaves), st, ev, p); return true;
    case 4: sf_launch(score_mfma<4, kScoreWaves, Batched, BB>, grid, dim3(64 * kScoreWaves), st, ev, p); return true;
    case 8: sf_launch(score_mfma<8, kScoreWaves, Batched, BB>, grid, dim3(64 * kScoreWaves), st, ev, p); return true;
  }
  return false;
}

template <bool Batched, int BB>
static bool launch_attend_mfma_b(const DecodeParams& p, dim3 grid, hipStream_t st, KernelEvents ev) {
  switch (p.grp) {
    case 1: sf_launch(attend_mfma<1, kAttendWaves, Batched, BB>, grid, dim3(64 * kAttendWaves), st, ev, p); return true;
    case 2: sf_launch(attend_mfma<2, kAttendWaves, Batched, BB>, grid, dim3(64 * kAttendWaves), st, ev, p); return true;
    case 4: sf_launch(attend_mfma<4, kAttendWaves, Batched, BB>, grid, dim3(64 * kAttendWaves), st, ev, p); return true;
    case 8: sf_launch(attend_mfma<8, kAttendWaves, Batched, BB>, grid, dim3(64 * kAttendWaves), st, ev, p); return true;
  }
  return false;
}

// Single-sequence steps take the instantiations without the batched
// sequence search, so that their kernels' start stays as short as it can be.
bool launch_score(const DecodeParams& p, dim3 grid, hipStream_t st, KernelEvents ev) {
  if (p.b == 2)
    return p.batch > 1 ? launch_score_mfma_b<true, 2>(p, grid, st, ev) : launch_score_mfma_b<false, 2>(p, grid, st, ev);
  if (p.b == 3)
    return p.batch > 1 ? launch_score_mfma_b<true, 3>(p, grid, st, ev) : launch_score_mfma_b<false, 3>(p, grid, st, ev);
  if (p.b == 4)
    return p.batch > 1 ? launch_score_mfma_b<true, 4>(p, grid, st, ev) : launch_score_mfma_b<false, 4>(p, grid, st, ev);
  return false;
}

bool launch_attend(const DecodeParams& p, dim3 grid, hipStream_t st, KernelEvents ev) {
  if (p.b == 2)
    return p.batch > 1 ? launch_attend_mfma_b<true, 2>(p, grid, st, ev) : launch_attend_mfma_b<false, 2>(p, grid, st, ev);
  if (p.b == 3)
    return p.batch > 1 ? launch_attend_mfma_b<true, 3>(p, grid, st, ev) : launch_attend_mfma_b<false, 3>(p, grid, st, ev);
  if (p.b == 4)
    return p.batch > 1 ? launch_attend_mfma_b<true, 4>(p, grid, st, ev) : launch_attend_mfma_b<false, 4>(p, grid, st, ev);
  return false;
}

}  // namespace sfk

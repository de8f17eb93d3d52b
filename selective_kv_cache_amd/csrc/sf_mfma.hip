// Matrix-core (CDNA4 MFMA) forms of the score pass and of the base attention
// pass, for 2-bit base codes and GQA groups of up to 4 query heads.
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
// subnormals taken straight from the packed bits (a code c at mantissa bit
// 2t reads as c * 2^(2t-24), exactly; the power of two is undone per tile).
// The codes of 8 tokens at one element are gathered with one v_perm_b32 per
// token pair, so the packed rows are read as they are stored.
#include <math.h>
#include <stddef.h>

#include "sf_attend_common.h"

namespace sfk {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr float kInv254 = 1.0f / 254.0f;

// 2-bit codes to the int8 B operands of the two logit MFMAs: byte b of
// dword v of operand i carries element 16i + v + 4b of the lane group's 32
// ((dword >> 2v) & 0x03030303 spreads four codes into four bytes).
__device__ inline void decode_b2(uint32_t w0, uint32_t w1, v4i& b0, v4i& b1) {
  b0 = v4i{(int)(w0 & 0x03030303u), (int)((w0 >> 2) & 0x03030303u), (int)((w0 >> 4) & 0x03030303u),
           (int)((w0 >> 6) & 0x03030303u)};
  b1 = v4i{(int)(w1 & 0x03030303u), (int)((w1 >> 2) & 0x03030303u), (int)((w1 >> 4) & 0x03030303u),
           (int)((w1 >> 6) & 0x03030303u)};
}

// Query digits and per-head constants of the score pass.  The digits are
// stored in A-operand order: op[h][k][g] holds the 32 bytes lane group g of
// row (h, k) feeds its two MFMAs (operand i, dword v, byte b = element
// 32g + 16i + v + 4b, matching decode_b2's element order).
struct QPrep {
  alignas(16) int8_t op[4][4][4][32];   // [head][digit][lane group][byte]
  float scale[4];                        // s_h
  float sumq[4];                         // sum(q_h)
};

// The query elements wave h < G turns into digits: elements 2*lane, 2*lane+1
// of head h.  Loaded before anything else of the work-group so that their
// latency overlaps the stream's first loads.
template <int G>
__device__ inline float2 load_query(const float* q) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (wid < G) return *reinterpret_cast<const float2*>(q + wid * kHeadDim + 2 * lane);
  return make_float2(0.f, 0.f);
}

// Work-group prologue: wave h < G turns query head h into 4 base-254 int8
// digits, q = s * (d0 + d1/254 + d2/254^2 + d3/254^3), s = max|q|/127.  Then
// each lane reads its two A operands (row = 4*head + digit, 16 bytes each of
// lane group l/16) with two 16-byte LDS reads.
template <int G>
__device__ inline void prep_query(float2 x, QPrep& qp, v4i& a0, v4i& a1) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (wid < 4) {
    const float amax = wave_max(fmaxf(fabsf(x.x), fabsf(x.y)));
    const float sum = wave_sum(x.x + x.y);
    const float sc = amax > 0.f ? amax / 127.0f : 1.0f;
    const float xs[2] = {x.x / sc, x.y / sc};
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int d = 2 * lane + e, g = d >> 5, r = d & 31;
      const int pos = 16 * (r >> 4) + 4 * (r & 3) + ((r & 15) >> 2);
      float rr = xs[e];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float dg = fminf(fmaxf(rintf(rr), -127.f), 127.f);
        qp.op[wid][k][g][pos] = wid < G ? (int8_t)dg : (int8_t)0;
        rr = (rr - dg) * 254.0f;
      }
    }
    if (lane == 0) {
      qp.scale[wid] = wid < G ? sc : 1.0f;
      qp.sumq[wid] = wid < G ? sum : 0.f;
    }
  }
  __syncthreads();
  const int m = lane & 15, g = lane >> 4;
  const v4i* src = reinterpret_cast<const v4i*>(&qp.op[m >> 2][m & 3][g][0]);
  a0 = src[0];
  a1 = src[1];
}

// Logit of (head l/16, token l%16) from the digit sums; -inf for heads >= G.
template <int G>
__device__ inline float logit_from(const v4i& D, float2 ksc, float scale, float sumq, int hl) {
  const float S = (float)D[0] + ((float)D[1] + ((float)D[2] + (float)D[3] * kInv254) * kInv254) * kInv254;
  const float lg = (fmaf(0.5f, ksc.y, ksc.x) * sumq + ksc.y * (S * scale)) * kRsqrtD;
  return hl < G ? lg : -INFINITY;
}

// The same logit with the 1/sqrt(D) (and any other constant factor) folded
// into scale and sumq.
__device__ inline float logit_scaled(const v4i& D, float2 ksc, float scale, float sumq) {
  const float S = (float)D[0] + ((float)D[1] + ((float)D[2] + (float)D[3] * kInv254) * kInv254) * kInv254;
  return fmaf(ksc.y, S * scale, fmaf(0.5f, ksc.y, ksc.x) * sumq);
}

// ---------------------------------------------------------------------------
// Direct global->LDS loads and asm LDS access, shared by both streaming
// kernels.  global_load_lds puts lane i's 16 (or 4) bytes at offset 16*i (4*i)
// of the destination, so loads in flight hold no registers.  LDS reads of
// such buffers are written in asm: a read the compiler sees makes it wait for
// every direct load in flight (it cannot tell ring stages apart), which would
// serialise the stream.  Each asm read waits for itself before it ends.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void* lds_void_t;

__device__ inline void dma16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t)l, 16, 0, 0);
}
__device__ inline void dma4(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t)l, 4, 0, 0);
}

// Sum over the 16 lanes of a row (DPP row rotations).
__device__ inline float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false));
  return x;
}

// Maximum over the 16 lanes of a row (DPP row rotations, no LDS traffic).
__device__ inline float row16_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false)));
  return x;
}

__device__ inline float lane_value(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

__device__ inline uint32_t lds_addr(const void* l) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)l;
}

// Wait until at most `ahead` stages of PER direct loads each are still in
// flight (a wave's vector loads complete in order).  `ahead` is wave-uniform
// and at most 3.
template <int PER>
__device__ inline void wait_stages(int ahead) {
  if (ahead >= 3)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * PER) : "memory");
  else if (ahead == 2)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PER) : "memory");
  else if (ahead == 1)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__device__ inline void lds_add_u32(uint32_t a, uint32_t v) {
  asm volatile("ds_add_u32 %0, %1" ::"v"(a), "v"(v) : "memory");
}

__device__ inline void lds_write_u32(uint32_t a, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(a), "v"(v) : "memory");
}

__device__ inline v8h lds_read_v8h(uint32_t a) {
  v4u v;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(a) : "memory");
  return __builtin_bit_cast(v8h, v);
}

// Two 16-byte reads 1 KiB apart.
__device__ inline void lds_read_2v8h(uint32_t a, v8h& x, v8h& y) {
  v4u u, v;
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:1024\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(u), "=&v"(v)
               : "v"(a)
               : "memory");
  x = __builtin_bit_cast(v8h, u);
  y = __builtin_bit_cast(v8h, v);
}

// ---------------------------------------------------------------------------
// Score pass: grid (n_score_split, hkv), 4 wavefronts.  Each wave streams
// 32-token chunks (two logit tiles) of its split through an LDS ring; the
// per-head logits go to the logits buffer for the attention pass, their
// maximum over the group to the scores and the level-1 histogram.
// ---------------------------------------------------------------------------
constexpr int kSRing = 4;                      // stages per wavefront
constexpr int kSRingLoads = 2;                 // direct loads per stage

struct SStage {
  uint8_t k[32 * 32];
  float2 ks[32];
};

template <int G>
__global__ void __launch_bounds__(256) score_mfma(DecodeParams p) {
  __shared__ QPrep qp;
  __shared__ uint32_t lhist[kHistBins];
  __shared__ SStage ring[4][kSRing];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int kvh = blockIdx.y;
  int64_t lo, hi;
  int first;
  const int seq = locate_unit(p.seq_off, p.batch, p.score_split, blockIdx.x, false, 0, lo, hi, first);
  const float2 qx = load_query<G>(p.q + ((int64_t)seq * p.hq + kvh * G) * kHeadDim);
  const int64_t a = p.seq_off[seq];
  const int64_t t0 = (int64_t)kvh * p.cap + a + lo;            // first token row of the split
  const uint8_t* kbase = p.kc + t0 * 32;
  const float* kscg = p.ks + t0 * 2;
  const int nsp = (int)(hi - lo);
  const int nchunks = (nsp + 31) / 32;
  const int nmine = nchunks > wid ? (nchunks - wid + 3) / 4 : 0;
  // stage i <- chunk wid + 4i of the wave's own chunks (tokens past the
  // split read its last token)
  auto issue = [&](int i) {
    const int c = wid + 4 * i;
    int rel = 32 * c + (lane >> 1);
    rel = rel < nsp ? rel : nsp - 1;
    SStage& st = ring[wid][i % kSRing];
    dma16(kbase + (uint32_t)rel * 32u + 16u * (uint32_t)(lane & 1), st.k);
    dma4(kscg + (uint32_t)rel * 2u + (uint32_t)(lane & 1), st.ks);
  };
  const bool hist = p.top_t > 0;   // no selection, no histogram
  for (int i = tid; i < kHistBins; i += 256) lhist[i] = 0u;
#pragma unroll
  for (int i = 0; i < kSRing - 1; ++i)
    if (i < nmine) issue(i);
  v4i a0, a1;
  prep_query<G>(qx, qp, a0, a1);
  const int t = lane & 15, hl = lane >> 4;
  const float scale = qp.scale[hl < G ? hl : 0], sumq = qp.sumq[hl < G ? hl : 0];
  float* scores = p.scores + (int64_t)kvh * p.ntot + (a - p.off0) + lo;
  float* lgo = p.logits + ((int64_t)kvh * p.ntot + (a - p.off0) + lo) * G;
  const uint32_t ring0 = lds_addr(&ring[wid][0]);
  const uint32_t offK = (uint32_t)(t * 32 + 8 * hl);
  const uint32_t offS = (uint32_t)(offsetof(SStage, ks) + 8 * t);
  const int hx = hl >> 1;                         // after the reduction: tile of this lane
  const uint32_t hist0 = lds_addr(&lhist[0]);
  for (int i = 0; i < nmine; ++i) {
    if (i + kSRing - 1 < nmine) issue(i + kSRing - 1);
    wait_stages<kSRingLoads>(min(kSRing - 1, nmine - 1 - i));
    const int c = wid + 4 * i;
    const uint32_t sb = ring0 + (uint32_t)(i % kSRing) * (uint32_t)sizeof(SStage);
    uint64_t kw[2], ks[2];
    asm volatile(
        "ds_read_b64 %0, %4\n\t"
        "ds_read_b64 %1, %4 offset:512\n\t"
        "ds_read_b64 %2, %5\n\t"
        "ds_read_b64 %3, %5 offset:128\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(kw[0]), "=&v"(kw[1]), "=&v"(ks[0]), "=&v"(ks[1])
        : "v"(sb + offK), "v"(sb + offS)
        : "memory");
    float lg[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint2 w = __builtin_bit_cast(uint2, kw[k]);
      v4i b0, b1;
      decode_b2(w.x, w.y, b0, b1);
      v4i D = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, v4i{0, 0, 0, 0}, 0, 0, 0);
      D = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, D, 0, 0, 0);
      lg[k] = logit_from<G>(D, __builtin_bit_cast(float2, ks[k]), scale, sumq, hl);
      const int rel = 32 * c + 16 * k + t;
      if (hl < G && rel < nsp) lgo[rel * G + hl] = lg[k];   // kept for the attention pass
    }
    // maximum over the heads, two tiles at once: after the first exchange a
    // lane keeps tile hl/2 over heads {hl, hl^2}, after the second over all
    const float r = __shfl_xor(hx ? lg[0] : lg[1], 32);
    float y = fmaxf(hx ? lg[1] : lg[0], r);
    y = fmaxf(y, __shfl_xor(y, 16));
    const int rel = 32 * c + 16 * hx + t;
    if ((hl & 1) == 0 && rel < nsp) {
      scores[rel] = y;
      if (hist) lds_add_u32(hist0 + 4u * (score_key(y) >> (32 - kHistBits)), 1u);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (!hist) return;
  __syncthreads();
  uint32_t* gh = p.hist + ((int64_t)seq * p.hkv + kvh) * kHistBins;   // level-1 histogram
  for (int i = tid; i < kHistBins; i += 256) {
    const uint32_t c = lhist[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

// The base pass streams its split through a per-wavefront ring of LDS stages
// filled by direct global->LDS loads (global_load_lds: lane i's 16 or 4 bytes
// land at stage offset 16*i or 4*i), so the loads in flight hold no
// registers.  One stage is one 32-token chunk: the per-head logits the score
// pass left, V codes (1 KiB, as stored) and V scales (256 B).  K is not read
// again.
constexpr int kRing = 4;                       // stages per wavefront; kRing - 1 chunks in flight
constexpr int kRingLoads = 3;                  // direct loads per stage

template <int G>
struct Stage {
  float lg[32 * G];
  uint8_t v[32 * 32];
  float2 vs[32];
};

template <int G>
struct MfmaLds {
  alignas(16) _Float16 wt[4][2][16][32];   // per wave: P.V weights, hi and lo parts [column][kappa]
  float mw[4][G], lw[4][G];
  union {
    Stage<G> ring[4][kRing];
    float accw[4][G + 1][kHeadDim];        // after the stream: per-wave P.V totals (row G: unused lanes)
  } u;
};

// One lane's operands of a stage.  The LDS reads are written in asm: a read
// the compiler sees makes it wait for every direct load in flight (it cannot
// tell the ring stages apart), which would serialise the stream.  The block
// waits for its own reads before it ends, so every output is complete.
struct StageRegs {
  float lg[2];             // logits of tokens t, 16 + t for head hl
  uint64_t vsc[2];         // (lo, delta) of tokens t, 16 + t
  uint32_t vw[8];          // V dword vdw of tokens 4rg+v (vw[2v]) and 16+4rg+v (vw[2v+1])
};

template <int G>
__device__ inline void read_stage(uint32_t aL, uint32_t aS, const uint32_t (&aV)[4], StageRegs& r) {
  asm volatile(
      "ds_read_b32 %0, %12\n\t"
      "ds_read_b32 %1, %12 offset:%18\n\t"
      "ds_read_b64 %2, %13\n\t"
      "ds_read_b64 %3, %13 offset:128\n\t"
      "ds_read_b32 %4, %14\n\t"
      "ds_read_b32 %5, %14 offset:512\n\t"
      "ds_read_b32 %6, %15\n\t"
      "ds_read_b32 %7, %15 offset:512\n\t"
      "ds_read_b32 %8, %16\n\t"
      "ds_read_b32 %9, %16 offset:512\n\t"
      "ds_read_b32 %10, %17\n\t"
      "ds_read_b32 %11, %17 offset:512\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r.lg[0]), "=&v"(r.lg[1]), "=&v"(r.vsc[0]), "=&v"(r.vsc[1]), "=&v"(r.vw[0]), "=&v"(r.vw[1]),
        "=&v"(r.vw[2]), "=&v"(r.vw[3]), "=&v"(r.vw[4]), "=&v"(r.vw[5]), "=&v"(r.vw[6]), "=&v"(r.vw[7])
      : "v"(aL), "v"(aS), "v"(aV[0]), "v"(aV[1]), "v"(aV[2]), "v"(aV[3]), "n"(16 * G * 4)
      : "memory");
}

template <int G>
__device__ inline void base_split_mfma(const DecodeParams& p, int split, int kvh, uint8_t* smem) {
  using Lds = MfmaLds<G>;
  using St = Stage<G>;
  Lds& s = *reinterpret_cast<Lds*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int64_t lo, hi;
  int first;
  const int seq = locate_unit(p.seq_off, p.batch, p.split, split, false, 0, lo, hi, first);
  const int64_t a = p.seq_off[seq];
  const int64_t sk = (int64_t)seq * p.hkv + kvh;
  const bool masked = p.use_refine != 0;
  const int64_t t0 = (int64_t)kvh * p.cap + a + lo;            // first token row of the split
  const uint8_t* vbase = p.vc + t0 * 32;
  const float* vscg = p.vs + t0 * 2;
  const uint8_t* lbase = reinterpret_cast<const uint8_t*>(p.logits + ((int64_t)kvh * p.ntot + (a - p.off0) + lo) * G);
  const int nsp = (int)(hi - lo);                               // tokens of the split (<= 4096)
  const int nchunks = (nsp + 31) / 32;
  const int nmine = nchunks > wid ? (nchunks - wid + 3) / 4 : 0;   // chunks wid, wid+4, ...

  // Stage i of this wave <- chunk wid + 4*i.  Lane L loads the scale word L
  // of the chunk (token L/2), lanes L < 8G the logits' bytes [16L, 16L+16),
  // and half L&1 of V row (L/2) ^ ((L/8) & 3): row r of the chunk sits at
  // stage row r ^ ((r/4) & 3), so that the four rows one P.V read takes
  // (4rg + v, rg = 0..3) fall in different LDS banks.  Only the wave's own
  // chunks are issued; tokens past the split's end read its last token's V
  // row (logits: the buffer has a chunk of slack), so every load is in
  // bounds.
  const int vrow = (lane >> 1) ^ ((lane >> 3) & 3);
  auto issue = [&](int i) {
    const int c = wid + 4 * i;
    int rel = 32 * c + (lane >> 1);
    rel = rel < nsp ? rel : nsp - 1;
    int relv = 32 * c + vrow;
    relv = relv < nsp ? relv : nsp - 1;
    St& st = s.u.ring[wid][i % kRing];
    if (lane < 8 * G) dma16(lbase + (uint32_t)c * (32u * G * 4u) + 16u * (uint32_t)lane, st.lg);
    dma16(vbase + (uint32_t)relv * 32u + 16u * (uint32_t)(lane & 1), st.v);
    dma4(vscg + (uint32_t)rel * 2u + (uint32_t)(lane & 1), st.vs);
  };
#pragma unroll
  for (int i = 0; i < kRing - 1; ++i)
    if (i < nmine) issue(i);

  for (int i = lane; i < 2 * 16 * 32; i += 64) (&s.wt[wid][0][0][0])[i] = (_Float16)0.f;
  // selection words of the split (one per chunk) in two registers: lane L
  // holds those of chunks L and 64 + L; splits start on a word boundary
  constexpr int kMaxSplitWords = 4096 / 32;
  static_assert(kMaxSplitWords <= 128, "two words per lane");
  static_assert(kRing <= 4, "wait_stages covers up to 3 stages ahead");
  const uint32_t* bmw = p.bitmap + sk * p.bm_words + (lo >> 5);
  const uint32_t sw0 = masked && lane < nchunks ? bmw[lane] : 0u;
  const uint32_t sw1 = masked && 64 + lane < nchunks ? bmw[64 + lane] : 0u;
  __syncthreads();
  const int t = lane & 15, hl = lane >> 4;        // logit layout: token t (and 16 + t), head hl
  const int n = lane & 15, rg = lane >> 4;        // P.V layout: column n, k-group rg
  const int hlc = hl < G ? hl : 0;
  constexpr float kLog2e = 1.4426950408889634f;   // softmax in log2 units
  // v_perm_b32 selector: half (n & 1) of each of two dwords
  const uint32_t hsel = 2u * (uint32_t)(n & 1);
  const uint32_t psel = hsel | ((hsel + 1u) << 8) | ((hsel + 4u) << 16) | ((hsel + 5u) << 24);
  const int vdw = n >> 1;                         // dword of the V row holding elements 8n..8n+7

  // LDS addresses of this lane's stage operands.  P.V k index kappa = 2u + j
  // stands for token 16j + u, so lane (n, rg) takes tokens 4rg..4rg+3 and
  // 16+4rg..16+4rg+3, and a logit lane's two weights are adjacent.
  const uint32_t ring0 = lds_addr(&s.u.ring[wid][0]);
  const uint32_t wt0 = lds_addr(&s.wt[wid][0][n][8 * rg]);
  const uint32_t wts = lds_addr(&s.wt[wid][0][hlc][2 * t]);
  static_assert(sizeof(s.wt[0][0]) == 1024, "lo part 1 KiB after the hi part");
  const uint32_t offL = (uint32_t)(offsetof(St, lg) + 4 * (t * G + hlc));
  const uint32_t offS = (uint32_t)(offsetof(St, vs) + 8 * t);
  uint32_t offV[4];                               // token 4rg + v at stage row 4rg + (v ^ rg)
#pragma unroll
  for (int v = 0; v < 4; ++v) offV[v] = (uint32_t)(offsetof(St, v) + (4 * rg + (v ^ rg)) * 32 + 4 * vdw);

  float m = -INFINITY, lsum = 0.f, t1 = 0.f;
  int sexp = 127;                                 // weight scale 2^sexp; 127 = not set yet
  float wsc = 1.0f;                               // 2^sexp once set
  v4f acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < nmine; ++i) {
    if (i + kRing - 1 < nmine) issue(i + kRing - 1);
    // this wave's loads complete in order: stage i is in once no more than
    // the stages issued after it are outstanding
    wait_stages<kRingLoads>(min(kRing - 1, nmine - 1 - i));
    const int c = wid + 4 * i;
    const uint32_t sb = ring0 + (uint32_t)(i % kRing) * (uint32_t)sizeof(St);
    const int rem = nsp - 32 * c;                 // tokens of this chunk inside the split
    const uint32_t selw = (uint32_t)__builtin_amdgcn_readlane((int)(c < 64 ? sw0 : sw1), c & 63);
    StageRegs R;
    const uint32_t aV[4] = {sb + offV[0], sb + offV[1], sb + offV[2], sb + offV[3]};
    read_stage<G>(sb + offL, sb + offS, aV, R);
    float lg[2];
    float2 vsc[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const bool ok = hl < G && 16 * k + t < rem && !((selw >> (16 * k + t)) & 1u);
      lg[k] = ok ? R.lg[k] * kLog2e : -INFINITY;
      vsc[k] = ok ? __builtin_bit_cast(float2, R.vsc[k]) : make_float2(0.f, 0.f);
    }
    // online softmax: maximum over the row of 16 lanes (one head)
    const float mnew = fmaxf(m, row16_max(fmaxf(lg[0], lg[1])));
    // weight scale: keep delta * 2^sexp below 2^14 over the chunk; the
    // chunk's largest delta is needed only when one reaches 2^(14 - sexp)
    float dmax = fmaxf(vsc[0].y, vsc[1].y);
    int need = sexp;
    if (__ballot(dmax > 0.f && (sexp == 127 || dmax >= __builtin_ldexpf(1.0f, 14 - sexp))) != 0ull) {
      dmax = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_max(dmax))));
      int e2;
      frexpf(dmax, &e2);
      need = 14 - e2;       // wave-uniform, and so is sexp
    }
    const bool grow = __ballot(mnew > m) != 0ull;
    if (grow || need < sexp) {
      const float alpha = mnew > m ? (m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mnew)) : 1.f;
      lsum *= alpha;
      t1 *= alpha;
      const int hc = n < 2 * G ? n % G : 0;
      float f = lane_value(alpha, 0);
#pragma unroll
      for (int h = 1; h < G; ++h) f = hc == h ? lane_value(alpha, 16 * h) : f;
      if (need < sexp) {
        if (sexp != 127) f = __builtin_ldexpf(f, need - sexp);
        sexp = need;
        wsc = __builtin_ldexpf(1.0f, sexp);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] *= f;
      m = mnew;
    }
    float wv[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float pk = lg[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(lg[k] - m);
      lsum += pk;
      t1 = fmaf(pk, fmaf(0.5f, vsc[k].y, vsc[k].x), t1);
      wv[k] = pk * (vsc[k].y * wsc);
    }
    // weights as fp16 hi + lo (truncated hi, exact remainder): 22 bits
    const auto whi = __builtin_amdgcn_cvt_pkrtz(wv[0], wv[1]);
    const auto wlo = __builtin_amdgcn_cvt_pkrtz(wv[0] - (float)whi[0], wv[1] - (float)whi[1]);
    if (hl < G) {
      lds_write_u32(wts, __builtin_bit_cast(uint32_t, whi));
      lds_write_u32(wts + 1024u, __builtin_bit_cast(uint32_t, wlo));
    }
    v8h bhi, blo;
    lds_read_2v8h(wt0, bhi, blo);
    const uint32_t* vw = R.vw;
    uint32_t P[4], Q[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      P[v] = __builtin_amdgcn_perm(vw[2 * v + 1], vw[2 * v], psel);
      Q[v] = P[v] >> 10;
    }
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const uint32_t mk = 0x00030003u << (2 * (tt <= 4 ? tt : tt - 5));
      v4u av;
#pragma unroll
      for (int v = 0; v < 4; ++v) av[v] = (tt <= 4 ? P[v] : Q[v]) & mk;
      acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, av), bhi, acc[tt], 0, 0, 0);
      acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, av), blo, acc[tt], 0, 0, 0);
    }
  }
  // the ring is reused below: no load of this wave may still be landing, and
  // every wave must be done with its stages
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // wave totals: l and the scalar term per head (row sums), P.V per head
  // (column n = head n); the maximum goes back to natural-log units
  lsum = row16_sum(lsum);
  t1 = row16_sum(t1);
  if (hl < G && t == 0) {
    s.mw[wid][hl] = m * 0.6931471805599453f;
    s.lw[wid][hl] = lsum;
  }
  float t1n = lane_value(t1, 0);
#pragma unroll
  for (int h = 1; h < G; ++h) t1n = n == h ? lane_value(t1, 16 * h) : t1n;
  const int se = sexp == 127 ? 0 : sexp;
  const int nrow = n < G ? n : G;
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) {
    const float f = __builtin_ldexpf(1.0f, 24 - 2 * (tt <= 4 ? tt : tt - 5) - se);
#pragma unroll
    for (int j = 0; j < 4; ++j) s.u.accw[wid][nrow][32 * rg + 8 * j + tt] = fmaf(acc[tt][j], f, t1n);
  }
  __syncthreads();
  float* part = p.part + ((int64_t)kvh * (p.n_sel_blk + p.n_split) + p.n_sel_blk + split) * G * kPartStride;
  write_partial<G, G + 1>(part, s.mw, s.lw, s.u.accw);
}

template <int G>
__global__ void __launch_bounds__(256) attend_mfma(DecodeParams p) {
  __shared__ __align__(16) uint8_t smem[cmax(sizeof(SelLds<2, G>), sizeof(MfmaLds<G>))];
  if ((int)blockIdx.x < p.n_sel_blk)
    selected_block<2, G>(p, blockIdx.x, blockIdx.y, smem);
  else
    base_split_mfma<G>(p, blockIdx.x - p.n_sel_blk, blockIdx.y, smem);
}

bool launch_score_mfma(const DecodeParams& p, dim3 grid, hipStream_t st, KernelEvents ev) {
  if (p.b != 2) return false;
  switch (p.grp) {
    case 1: sf_launch(score_mfma<1>, grid, dim3(256), st, ev, p); return true;
    case 2: sf_launch(score_mfma<2>, grid, dim3(256), st, ev, p); return true;
    case 4: sf_launch(score_mfma<4>, grid, dim3(256), st, ev, p); return true;
  }
  return false;
}

bool launch_attend_mfma(const DecodeParams& p, dim3 grid, hipStream_t st, KernelEvents ev) {
  if (p.b != 2) return false;
  switch (p.grp) {
    case 1: sf_launch(attend_mfma<1>, grid, dim3(256), st, ev, p); return true;
    case 2: sf_launch(attend_mfma<2>, grid, dim3(256), st, ev, p); return true;
    case 4: sf_launch(attend_mfma<4>, grid, dim3(256), st, ev, p); return true;
  }
  return false;
}

}  // namespace sfk

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
// subnormals taken from the packed bits with a shift and a mask (a code c at
// mantissa bit k reads as c * 2^(k-24), exactly; the power of two is undone
// per tile).  Every code is placed at bit k >= 4: measured on gfx950, the
// product's sums lose precision on the smallest subnormals (codes at bit 0
// gave errors near 1e-4 of the result, bit 2 near 2e-5, bits 4-8 the fp32
// level, 1e-6).  The codes of 8 tokens at one element are gathered with one
// v_perm_b32 per token pair, so the packed rows are read as they are stored.
#include <math.h>
#include <stddef.h>

#include <type_traits>

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
// flight (a wave's vector loads complete in order).  `ahead` is wave-uniform;
// A is its largest value.
template <int PER, int A>
__device__ inline void wait_stages(int ahead) {
  static_assert(A * PER < 64, "vmcnt holds 6 bits");
  if constexpr (A == 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    if (ahead >= A)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(A * PER) : "memory");
    else
      wait_stages<PER, A - 1>(ahead);
  }
}

// One round of a ring loop: f(stage K, chunk i + K) for the stages K < R
// whose chunk exists, with K a compile-time constant (the stage's LDS offset
// becomes an immediate of its reads).
template <int R, int K = 0, typename F>
__device__ inline void ring_round(F& f, int i, int n) {
  if constexpr (K < R) {
    if (i + K < n) {
      f(std::integral_constant<int, K>{}, i + K);
      ring_round<R, K + 1>(f, i, n);
    }
  }
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

// Buffer loads straight to LDS: a raw buffer resource (base, byte range) in
// SGPRs, a per-lane byte offset that stays fixed and a wave-uniform one that
// walks the chunks, so issuing a stage costs no vector instructions.  Reads
// past the range return zeros (the hardware's range check), which is how the
// split's last chunk stays inside the split.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ inline void bdma16(rsrc_t r, uint32_t voff, uint32_t soff, void* l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t)l, 16, voff, soff, 0, 0);
}
__device__ inline void bdma4(rsrc_t r, uint32_t voff, uint32_t soff, void* l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t)l, 4, voff, soff, 0, 0);
}

// Issue priority by progress: a wavefront with more of its stream left gets
// a higher priority (s_setprio 0-3), so that the work-groups sharing a CU
// finish together instead of in dispatch order (the arbiter otherwise
// favours the oldest wavefronts).  `left` and `total` are wave-uniform.
__device__ inline void progress_priority(int left, int total) {
  const int q = (4 * left) / total;
  if (q >= 3)
    __builtin_amdgcn_s_setprio(3);
  else if (q == 2)
    __builtin_amdgcn_s_setprio(2);
  else if (q == 1)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

// A store written through the L2 (device scope): the score pass's logits and
// scores then leave no dirty lines for the end of the kernel to write back,
// which on a short pass (32K tokens per head) was a large share of its time;
// they still reach the memory-side cache, where the next passes read them.
__device__ inline void store_through(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// v_cndmask with a wave-uniform 64-bit lane mask (SGPR pair): lane l takes
// yes where bit l of mask is set, else no.
__device__ inline float lane_select(uint64_t mask, float yes, float no) {
  float r;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(no), "v"(yes), "s"(mask));
  return r;
}

// ---------------------------------------------------------------------------
// Score pass: grid (n_score_split, hkv), NW wavefronts.  Each wave streams
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

// Maximum over the four rows of two tiles at once: x0, x1 are a lane's
// values of tiles 0 and 1; the result holds tile 0's maximum over lanes
// l, l ^ 16, l ^ 32, l ^ 48 in rows 0 and 1 and tile 1's in rows 2 and 3.
// permlane32_swap(x0, x1) returns (rows 0-1 of x0 | rows 0-1 of x1) and
// (rows 2-3 of x0 | rows 2-3 of x1), so their maximum pairs each lane's tile
// with the other half's; permlane16_swap does the same across rows 0-1 and
// 2-3.  One v_max each (the values are never signalling NaNs).
__device__ inline float max_two_tiles(float x0, float x1) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x0), __float_as_uint(x1), false, false);
  float y;
  asm("v_max_f32 %0, %1, %2" : "=v"(y) : "v"(__uint_as_float(r[0])), "v"(__uint_as_float(r[1])));
  auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  asm("v_max_f32 %0, %1, %2" : "=v"(y) : "v"(__uint_as_float(q[0])), "v"(__uint_as_float(q[1])));
  return y;
}

template <int G, int NW, bool Batched>
__global__ void __launch_bounds__(64 * NW) score_mfma(DecodeParams p) {
  static_assert(NW >= 4, "waves 0-3 prepare the query digits");
  __shared__ QPrep qp;
  __shared__ uint32_t lhist[kHistBins];
  __shared__ SStage ring[NW][kSRing];
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
  // stage i <- chunk wid + NW i of the wave's own chunks: lane L loads half
  // L&1 of K row L/2 and scale word L; the resources end at the split's end
  // (tokens past it read as zeros)
  const rsrc_t rK = make_rsrc(p.kc + t0 * 32, (uint32_t)nsp * 32u);
  const rsrc_t rS = make_rsrc(p.ks + t0 * 2, (uint32_t)nsp * 8u);
  const uint32_t oK = 16u * (uint32_t)lane, oS = 4u * (uint32_t)lane;
  auto issue = [&](int i, SStage& st) {
    const uint32_t c = (uint32_t)(wid + NW * i);
    bdma16(rK, oK, c * 1024u, st.k);
    bdma4(rS, oS, c * 256u, st.ks);
  };
  const bool hist = p.top_t > 0;   // no selection, no histogram
  for (int i = tid; i < kHistBins; i += 64 * NW) lhist[i] = 0u;
#pragma unroll
  for (int k = 0; k < kSRing - 1; ++k)
    if (k < nmine) issue(k, ring[wid][k]);
  v4i a0, a1;
  prep_query<G>(qx, qp, a0, a1);
  // logits in log2 units (1/sqrt(D) and log2(e) folded into the per-head
  // constants): the attention pass's softmax takes them as they are
  constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
  const int t = lane & 15, hl = lane >> 4;
  const float scale = qp.scale[hl < G ? hl : 0] * (kRsqrtD * kLog2e);
  const float sumq = qp.sumq[hl < G ? hl : 0] * (kRsqrtD * kLog2e);
  float* scores = p.scores + (int64_t)kvh * p.ntot + (a - p.off0) + lo;
  float* lgo = p.logits + ((int64_t)kvh * p.ntot + (a - p.off0) + lo) * G;
  const uint32_t ring0 = lds_addr(&ring[wid][0]);
  const uint32_t aK = ring0 + (uint32_t)(t * 32 + 8 * hl);
  const uint32_t aS = ring0 + (uint32_t)(offsetof(SStage, ks) + 8 * t);
  const int hx = hl >> 1;                         // the tile a lane writes the score of
  const uint32_t hist0 = lds_addr(&lhist[0]);
  auto body = [&](auto kc, int i) {
    constexpr int k = decltype(kc)::value;        // stage of chunk i
    constexpr int OFF = k * (int)sizeof(SStage);
    if (i + kSRing - 1 < nmine) issue(i + kSRing - 1, ring[wid][(k + kSRing - 1) % kSRing]);
    // this wave's loads complete in order: stage i is in once no more than
    // the stages issued after it are outstanding (stores only add to the count)
    wait_stages<kSRingLoads, kSRing - 1>(min(kSRing - 1, nmine - 1 - i));
    const int c = wid + NW * i;
    uint64_t kw[2], ks[2];
    asm volatile(
        "ds_read_b64 %0, %4 offset:%6\n\t"
        "ds_read_b64 %1, %4 offset:%7\n\t"
        "ds_read_b64 %2, %5 offset:%6\n\t"
        "ds_read_b64 %3, %5 offset:%8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(kw[0]), "=&v"(kw[1]), "=&v"(ks[0]), "=&v"(ks[1])
        : "v"(aK), "v"(aS), "n"(OFF), "n"(OFF + 512), "n"(OFF + 128)
        : "memory");
    const bool full = 32 * c + 32 <= nsp;         // every token of the chunk inside the split
    float lg[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint2 w = __builtin_bit_cast(uint2, kw[j]);
      v4i b0, b1;
      decode_b2(w.x, w.y, b0, b1);
      v4i D = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, v4i{0, 0, 0, 0}, 0, 0, 0);
      D = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, D, 0, 0, 0);
      const float x = logit_scaled(D, __builtin_bit_cast(float2, ks[j]), scale, sumq);
      lg[j] = hl < G ? x : -INFINITY;
      const int rel = 32 * c + 16 * j + t;
      if (hl < G && (full || rel < nsp)) store_through(&lgo[rel * G + hl], x);   // kept for the attention pass
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
  for (int i = 0; i < nmine; i += kSRing) {
    progress_priority(nmine - i, nmine);
    ring_round<kSRing>(body, i, nmine);
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

template <int G, int NW>
struct MfmaLds {
  alignas(16) _Float16 wt[NW][2 * G][32];   // per wave: P.V weights [column][kappa]: hi parts, then lo parts
  alignas(16) _Float16 wzero[8];            // weight columns >= 2G read zeros
  float mw[NW][G], lw[NW][G];
  union {
    Stage<G> ring[NW][kRing];
    float accw[NW][2 * G][kHeadDim + 1];    // after the stream: per-wave P.V, hi and lo columns
                                            // (rows padded by a word: the 16 columns one write spans hit different banks)
  } u;
};

// Maximum over the 16 lanes of a row: four DPP row rotations, each folded
// into its v_max (s_nop 1 covers the VALU-write to DPP-read hazard).
__device__ inline float row16_max_dpp(float x) {
  float y;
  asm volatile(
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %1, %1 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 row_ror:2 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 row_ror:1 row_mask:0xf bank_mask:0xf"
      : "=&v"(y)
      : "v"(x));
  return y;
}

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

// Mantissa bit at which the P.V product takes code tt (0-7) of a token's
// 8-element group.
constexpr int code_bit(int tt) { return tt < 2 ? 2 * tt + 4 : tt < 5 ? 2 * tt : 2 * tt - 6; }

template <int G, int NW, bool Batched>
__device__ inline void base_split_mfma(const DecodeParams& p, int split, int kvh, uint8_t* smem) {
  using Lds = MfmaLds<G, NW>;
  using St = Stage<G>;
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
  // and half L&1 of V row (L/2) ^ ((L/8) & 3): row r of the chunk sits at
  // stage row r ^ ((r/4) & 3), so that the four rows one P.V read takes
  // (4rg + v, rg = 0..3) fall in different LDS banks.  The resources end at
  // the split's end: tokens past it read as zeros.
  const rsrc_t rV = make_rsrc(p.vc + t0 * 32, (uint32_t)nsp * 32u);
  const rsrc_t rS = make_rsrc(p.vs + t0 * 2, (uint32_t)nsp * 8u);
  const rsrc_t rL = make_rsrc(p.logits + ((int64_t)kvh * p.ntot + (a - p.off0) + lo) * G, (uint32_t)nsp * G * 4u);
  const uint32_t oV = (uint32_t)(((lane >> 1) ^ ((lane >> 3) & 3)) * 32 + 16 * (lane & 1));
  const uint32_t oS = 4u * (uint32_t)lane, oL = 16u * (uint32_t)lane;
  auto issue = [&](int i, St& st) {
    const uint32_t c = (uint32_t)(wid + NW * i);
    if (lane < 8 * G) bdma16(rL, oL, c * (32u * G * 4u), st.lg);
    bdma16(rV, oV, c * 1024u, st.v);
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
  const uint32_t wtHi = lds_addr(&s.wt[wid][hlc][2 * t]), wtLo = lds_addr(&s.wt[wid][G + hlc][2 * t]);
  const uint32_t aL = ring0 + (uint32_t)(offsetof(St, lg) + 4 * (t * G + hlc));
  const uint32_t aS = ring0 + (uint32_t)(offsetof(St, vs) + 8 * t);
  uint32_t aV[4];                                 // token 4rg + v at stage row 4rg + (v ^ rg)
#pragma unroll
  for (int v = 0; v < 4; ++v) aV[v] = ring0 + (uint32_t)(offsetof(St, v) + (4 * rg + (v ^ rg)) * 32 + 4 * vdw);
  // rows hl < G hold heads; the others take no part
  const uint64_t rows = G >= 4 ? ~0ull : (1ull << (16 * (G & 3))) - 1ull;
  const float ninf = -INFINITY;

  // running maximum: a finite floor below every logit until a token takes
  // part, so exp2(logit - m) is 0 (not NaN) for the -inf of tokens left out
  constexpr float kFloor = -1e30f;
  constexpr int kSlack = 6;                       // weights up to 2^kSlack (log2 units of the reference)
  float m = kFloor, lsum = 0.f, t1 = 0.f;
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
    read_stage<G, k * (int)sizeof(St)>(aL, aS, aV, R);
    // logits (log2 units, as the score pass kept them); -inf where the token
    // takes no part
    float lg[2];
    float2 vsc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      lg[j] = lane_select(mk[j], R.lg[j], ninf);
      vsc[j] = __builtin_bit_cast(float2, R.vsc[j]);
    }
    // online softmax with a lazy reference: m moves (and the sums are
    // rescaled) only when a logit exceeds it by more than kSlack, so the
    // weights stay below 2^kSlack and most chunks need no row maximum
    const float xm = fmaxf(lg[0], lg[1]);
    const bool grow = __ballot(xm > m + kSlack) != 0ull;
    const float mnew = grow ? fmaxf(m, row16_max_dpp(xm)) : m;
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
      const float alpha = mnew > m ? __builtin_amdgcn_exp2f(m - mnew) : 1.f;   // 0 from the floor
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
    for (int j = 0; j < 2; ++j) {
      const float pk = __builtin_amdgcn_exp2f(lg[j] - m);   // exp2(-inf) = 0: tokens left out
      lsum += pk;
      t1 = fmaf(pk, fmaf(0.5f, vsc[j].y, vsc[j].x), t1);
      wv[j] = pk * (vsc[j].y * wsc);
    }
    // weights as fp16 hi + lo (truncated hi, exact remainder): 22 bits, the
    // two parts in separate columns of one product
    const auto whi = __builtin_amdgcn_cvt_pkrtz(wv[0], wv[1]);
    const auto wlo = __builtin_amdgcn_cvt_pkrtz(wv[0] - (float)whi[0], wv[1] - (float)whi[1]);
    if (hl < G) {
      lds_write_u32(wtHi, __builtin_bit_cast(uint32_t, whi));
      lds_write_u32(wtLo, __builtin_bit_cast(uint32_t, wlo));
    }
    const v8h bw = lds_read_v8h(wtR);
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
  lsum = row16_sum(lsum);
  t1 = row16_sum(t1);
  if (hl < G && t == 0) {
    s.mw[wid][hl] = m == kFloor ? -INFINITY : m;   // -inf: no token took part
    s.lw[wid][hl] = lsum;
  }
  float t1n = 0.f;                                // the scalar term goes with the hi column
#pragma unroll
  for (int h = 0; h < G; ++h) t1n = n == h ? lane_value(t1, 16 * h) : t1n;
  const int se = sexp == 127 ? 0 : sexp;
  if (n < 2 * G) {
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const float f = __builtin_ldexpf(1.0f, 24 - code_bit(tt) - se);
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

template <int G, int NW, bool Batched>
__global__ void __launch_bounds__(64 * NW) attend_mfma(DecodeParams p) {
  __shared__ __align__(16) uint8_t smem[cmax(sizeof(SelLds<2, G, NW, 16>), sizeof(MfmaLds<G, NW>))];
  if ((int)blockIdx.x < p.n_sel_blk)
    selected_block_any<2, G, NW, true, Batched>(p, blockIdx.x, blockIdx.y, smem);
  else
    base_split_mfma<G, NW, Batched>(p, blockIdx.x - p.n_sel_blk, blockIdx.y, smem);
}

template <bool Batched>
static bool launch_score_mfma_b(const DecodeParams& p, dim3 grid, hipStream_t st, KernelEvents ev) {
  switch (p.grp) {
    case 1: sf_launch(score_mfma<1, kScoreWaves, Batched>, grid, dim3(64 * kScoreWaves), st, ev, p); return true;
    case 2: sf_launch(score_mfma<2, kScoreWaves, Batched>, grid, dim3(64 * kScoreWaves), st, ev, p); return true;
    case 4: sf_launch(score_mfma<4, kScoreWaves, Batched>, grid, dim3(64 * kScoreWaves), st, ev, p); return true;
  }
  return false;
}

template <bool Batched>
static bool launch_attend_mfma_b(const DecodeParams& p, dim3 grid, hipStream_t st, KernelEvents ev) {
  switch (p.grp) {
    case 1: sf_launch(attend_mfma<1, kAttendWaves, Batched>, grid, dim3(64 * kAttendWaves), st, ev, p); return true;
    case 2: sf_launch(attend_mfma<2, kAttendWaves, Batched>, grid, dim3(64 * kAttendWaves), st, ev, p); return true;
    case 4: sf_launch(attend_mfma<4, kAttendWaves, Batched>, grid, dim3(64 * kAttendWaves), st, ev, p); return true;
  }
  return false;
}

// Single-sequence steps take the instantiations without the batched
// sequence search, so that their kernels' start stays as short as it can be.
bool launch_score_mfma(const DecodeParams& p, dim3 grid, hipStream_t st, KernelEvents ev) {
  if (p.b != 2) return false;
  return p.batch > 1 ? launch_score_mfma_b<true>(p, grid, st, ev) : launch_score_mfma_b<false>(p, grid, st, ev);
}

bool launch_attend_mfma(const DecodeParams& p, dim3 grid, hipStream_t st, KernelEvents ev) {
  if (p.b != 2) return false;
  return p.batch > 1 ? launch_attend_mfma_b<true>(p, grid, st, ev) : launch_attend_mfma_b<false>(p, grid, st, ev);
}

}  // namespace sfk

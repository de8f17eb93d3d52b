// Matrix-core (CDNA4 MFMA) building blocks shared by the streaming kernels:
// the int8-digit query operands of the logit products, direct global->LDS
// loads into per-wavefront rings, LDS access in asm (so that it does not wait
// on the ring's loads in flight), DPP row reductions and lane selects.
// sf_mfma.hip states the arithmetic of the logit and P.V products.
#pragma once

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

// Four 3-bit codes (bits 3j, j = 0..3, of w; higher bits ignored) spread to
// the four bytes of a dword: the pair (c0, c1) stays at bits 0-5 and (c2, c3)
// moves to bits 16-21 (one bit-field insert), then c1 and c3 move up by 5 to
// bits 8 and 24 while c0 and c2 stay at 0 and 16.
__device__ inline uint32_t spread3x4(uint32_t w) {
  const uint32_t t = (w & 0x3Fu) | ((w << 10) & ~0x3Fu);
  return ((t << 5) & 0x07000700u) | (t & 0x00070007u);
}

// 3-bit codes to the int8 B operands of the two logit MFMAs.  A lane's 32
// codes are 96 consecutive bits of the packed row (w0, w1, w2): four groups
// of 8 codes (24 bits each), each group's halves spread by spread3x4, so
// byte b of dword v of operand i carries element 16i + 4v + b of the lane
// group's 32 (the codes in their own order).
__device__ inline void decode_b3(uint32_t w0, uint32_t w1, uint32_t w2, v4i& b0, v4i& b1) {
  const uint32_t g0 = w0, g1 = __builtin_amdgcn_alignbit(w1, w0, 24), g2 = __builtin_amdgcn_alignbit(w2, w1, 16),
                 g3 = w2 >> 8;
  b0 = v4i{(int)spread3x4(g0), (int)spread3x4(g0 >> 12), (int)spread3x4(g1), (int)spread3x4(g1 >> 12)};
  b1 = v4i{(int)spread3x4(g2), (int)spread3x4(g2 >> 12), (int)spread3x4(g3), (int)spread3x4(g3 >> 12)};
}

// 4-bit codes to the int8 B operands: operand i takes the lane's dwords
// w[2i], w[2i + 1] (codes 16i .. 16i + 15); (w >> 4s) & 0x0F0F0F0F keeps
// the even (s = 0) or odd (s = 1) nibbles, so byte b of dword v of operand i
// carries element 16i + 8 (v >> 1) + 2b + (v & 1) of the lane group's 32.
__device__ inline void decode_b4(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, v4i& b0, v4i& b1) {
  b0 = v4i{(int)(w0 & 0x0F0F0F0Fu), (int)((w0 >> 4) & 0x0F0F0F0Fu), (int)(w1 & 0x0F0F0F0Fu),
           (int)((w1 >> 4) & 0x0F0F0F0Fu)};
  b1 = v4i{(int)(w2 & 0x0F0F0F0Fu), (int)((w2 >> 4) & 0x0F0F0F0Fu), (int)(w3 & 0x0F0F0F0Fu),
           (int)((w3 >> 4) & 0x0F0F0F0Fu)};
}

// Query digits and per-head constants of the score pass.  The digits are
// stored in A-operand order: op[h][k][g] holds the 32 bytes lane group g of
// row (h, k) feeds its two MFMAs (operand i, dword v, byte b = element
// 32g + 16i + v + 4b for 2-bit codes, matching decode_b2's element order,
// 32g + 16i + 4v + b for 3-bit codes, decode_b3's, and
// 32g + 16i + 8 (v >> 1) + 2b + (v & 1) for 4-bit codes, decode_b4's).
template <int NH>
struct QPrepN {
  alignas(16) int8_t op[NH][4][4][32];  // [head][digit][lane group][byte]
  float scale[NH];                       // s_h
  float sumq[NH];                        // sum(q_h)
};
using QPrep = QPrepN<4>;

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
// digits, q = s * (d0 + d1/254 + d2/254^2 + d3/254^3), s = max|q|/127 (waves
// G .. NH - 1 write zero digits).  Then each lane reads its A operands (row
// = 4*head + digit of a tile of 4 heads, 16 bytes each of lane group l/16)
// with 16-byte LDS reads: two per tile.
template <int G, int BB, int NH>
__device__ inline void prep_digits(float2 x, QPrepN<NH>& qp) {
  static_assert(BB >= 2 && BB <= 4, "2-, 3- or 4-bit codes");
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (wid < NH) {
    const float amax = wave_max(fmaxf(fabsf(x.x), fabsf(x.y)));
    const float sum = wave_sum(x.x + x.y);
    const float sc = amax > 0.f ? amax / 127.0f : 1.0f;
    const float xs[2] = {x.x / sc, x.y / sc};
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int d = 2 * lane + e, g = d >> 5, r = d & 31;
      const int r16 = r & 15;
      const int pos = BB == 3   ? r
                      : BB == 4 ? 16 * (r >> 4) + 4 * (((r16 >> 3) << 1) | (r16 & 1)) + ((r16 & 7) >> 1)
                                : 16 * (r >> 4) + 4 * (r & 3) + (r16 >> 2);
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
}

// Groups of up to 4 query heads: one tile of 4 heads x 4 digits.
template <int G, int BB = 2>
__device__ inline void prep_query(float2 x, QPrep& qp, v4i& a0, v4i& a1) {
  static_assert(G <= 4, "one tile of heads");
  prep_digits<G, BB, 4>(x, qp);
  const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
  const v4i* src = reinterpret_cast<const v4i*>(&qp.op[m >> 2][m & 3][g][0]);
  a0 = src[0];
  a1 = src[1];
}

// Groups of 8 query heads: tile 0 holds heads 0-3 (a[0], a[1]), tile 1 heads
// 4-7 (a[2], a[3]).
template <int BB = 2>
__device__ inline void prep_query8(float2 x, QPrepN<8>& qp, v4i (&a)[4]) {
  prep_digits<8, BB, 8>(x, qp);
  const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
#pragma unroll
  for (int tl = 0; tl < 2; ++tl) {
    const v4i* src = reinterpret_cast<const v4i*>(&qp.op[4 * tl + (m >> 2)][m & 3][g][0]);
    a[2 * tl] = src[0];
    a[2 * tl + 1] = src[1];
  }
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
// yes where bit l of mask is set, else no.  The mask's halves go through
// readfirstlane, which costs nothing for a value already in SGPRs and keeps
// the operand scalar when the compiler cannot prove the value uniform.
__device__ inline float lane_select(uint64_t mask, float yes, float no) {
  const uint64_t m = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(mask >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)mask);
  float r;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(no), "v"(yes), "s"(m));
  return r;
}

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

// Mantissa bit at which the P.V product takes code tt (0-7) of a token's
// 8-element group: 2-bit codes at bits 4, 6, 4, 6, 8, 4, 6, 8; 3-bit codes at
// bits 4, 7, 6, 7, 4, 7, 4, 7; 4-bit codes at bit 4 (every code inside the 10
// mantissa bits, its lowest bit at 4 or above).
constexpr int code_bit(int tt) { return tt < 2 ? 2 * tt + 4 : tt < 5 ? 2 * tt : 2 * tt - 6; }
constexpr int code_bit3(int tt) { return tt == 0 || tt == 4 || tt == 6 ? 4 : tt == 2 ? 6 : 7; }
template <int BB>
constexpr int code_bit_of(int tt) { return BB == 2 ? code_bit(tt) : BB == 3 ? code_bit3(tt) : 4; }

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

}  // namespace sfk

// Nested quantization of K/V rows into the resident cache (sf_kv_quantize).
//
// Method: page "StrataFlux -- Selective precision streaming -- What does it
// mean?", paragraph "What travels over the link": the base code names one of
// 2^b equal bins of the row's range and r refinement bits split that bin into
// 2^r equal sub-bins.  One fine (b+r)-bit code per element carries both: its
// top b bits are the resident base code, its low r bits the refinement.
//
// One wavefront quantizes one row of D = 128 values (two per lane): min/max by
// butterfly shuffles, then per element one fp32 subtraction and one correctly
// rounded fp32 division, then the codes are OR-ed into the row's LSB-first
// bitstream in LDS and written out as 32-bit words.
#include <stdio.h>
#include <string.h>

#include "sf_internal.h"

namespace sfk {

static thread_local char g_err[256];

void set_hip_error(hipError_t e, const char* where) {
  snprintf(g_err, sizeof(g_err), "%s: %s", where, hipGetErrorString(e));
}
void clear_error() { g_err[0] = 0; }
void set_error_text(const char* what) { snprintf(g_err, sizeof(g_err), "%s", what); }

__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// OR `nbits` (<= 16) bits of `val` into a bitstream at bit `pos`.
__device__ inline void or_bits(uint32_t* words, int pos, uint32_t val, int nbits) {
  const int w = pos >> 5, sh = pos & 31;
  atomicOr(&words[w], val << sh);
  if (sh + nbits > 32) atomicOr(&words[w + 1], val >> (32 - sh));
}

constexpr int kRowsPerBlock = 4;

// The largest fp16 value <= x and the smallest >= x (x finite, within the
// fp16 range), as fp32: the nearest fp16, moved one step when it lies on the
// wrong side (one step down from +0 is the negative smallest subnormal).
__device__ inline float fp16_down(float x) {
  const _Float16 h = (_Float16)x;
  if ((float)h <= x) return (float)h;
  uint16_t u = __builtin_bit_cast(uint16_t, h);
  u = (u & 0x8000u) ? (uint16_t)(u + 1u) : (u == 0u ? (uint16_t)0x8001u : (uint16_t)(u - 1u));
  return (float)__builtin_bit_cast(_Float16, u);
}
__device__ inline float fp16_up(float x) {
  const _Float16 h = (_Float16)x;
  if ((float)h >= x) return (float)h;
  uint16_t u = __builtin_bit_cast(uint16_t, h);
  u = (u & 0x8000u) ? (u == 0x8000u ? (uint16_t)1u : (uint16_t)(u - 1u)) : (uint16_t)(u + 1u);
  return (float)__builtin_bit_cast(_Float16, u);
}

__global__ void __launch_bounds__(256)
quantize_rows_kernel(const float* __restrict__ x, int64_t n_rows, int hkv, int64_t n_tok,
                     int64_t tok_begin, int64_t cap, int b, int r, uint8_t* __restrict__ codes,
                     float* __restrict__ scales, uint8_t* __restrict__ refine_rows, int fp16_scales) {
  __shared__ uint32_t words[kRowsPerBlock][16 + 33];   // 4b <= 16 base words, 4r <= 32 refine words
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + wid;  // row = token * hkv + head
  if (row >= n_rows) return;                                      // wave-uniform
  const int64_t t = row / hkv;
  const int h = (int)(row - t * hkv);

  const float2 v = reinterpret_cast<const float2*>(x + row * kHeadDim)[lane];
  float mn = fminf(v.x, v.y), mx = fmaxf(v.x, v.y);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o));
    mx = fmaxf(mx, __shfl_xor(mx, o));
  }
  const int f = b + r;
  // fp16 scales: lo rounded down, delta from the stored lo rounded up (the
  // stored range reaches the maximum); else the fp32 row minimum and range
  const float lo = fp16_scales ? fp16_down(mn) : mn;
  const float range = __fsub_rn(mx, lo);
  const float delta = fp16_scales ? fp16_up(__fmul_rn(range, __builtin_ldexpf(1.0f, -b)))
                                  : __fmul_rn(range, __builtin_ldexpf(1.0f, -b));   // exact power-of-two scaling
  const float delta_f = fp16_scales ? __fmul_rn(delta, __builtin_ldexpf(1.0f, -r))
                                    : __fmul_rn(range, __builtin_ldexpf(1.0f, -f));
  const uint32_t qmax = (1u << f) - 1u;
  uint32_t q0 = 0, q1 = 0;
  if (delta_f != 0.0f) {
    const float u0 = __fdiv_rn(__fsub_rn(v.x, lo), delta_f);   // >= 0: lo <= every element
    const float u1 = __fdiv_rn(__fsub_rn(v.y, lo), delta_f);
    q0 = min((uint32_t)floorf(u0), qmax);
    q1 = min((uint32_t)floorf(u1), qmax);
  }
  const uint32_t rmask = (1u << r) - 1u;
  const uint32_t cb = (q0 >> r) | ((q1 >> r) << b);
  const uint32_t cr = (q0 & rmask) | ((q1 & rmask) << r);

  uint32_t* wb = words[wid];
  uint32_t* wr = words[wid] + 16;
  if (lane < 16 + 33) wb[lane] = 0u;
  wave_sync();
  or_bits(wb, 2 * b * lane, cb, 2 * b);
  if (r) or_bits(wr, 2 * r * lane, cr, 2 * r);
  wave_sync();

  const int nwb = 4 * b;  // 128*b bits = 4b words
  uint32_t* dst = reinterpret_cast<uint32_t*>(codes + ((int64_t)h * cap + tok_begin + t) * (16 * b));
  if (lane < nwb) dst[lane] = wb[lane];
  if (r) {
    uint32_t* dr = reinterpret_cast<uint32_t*>(refine_rows + ((int64_t)h * n_tok + t) * (16 * r));
    if (lane < 4 * r) dr[lane] = wr[lane];
  }
  if (lane == 0) {
    float2* s = reinterpret_cast<float2*>(scales) + ((int64_t)h * cap + tok_begin + t);
    *s = make_float2(lo, delta);
  }
}

}  // namespace sfk

using namespace sfk;

extern "C" const char* sf_status_string(sf_status s) {
  switch (s) {
    case SF_OK: return "SF_OK";
    case SF_ERR_INVALID_ARG: return "SF_ERR_INVALID_ARG: invalid argument";
    case SF_ERR_UNSUPPORTED: return "SF_ERR_UNSUPPORTED: configuration not supported";
    case SF_ERR_HIP: return "SF_ERR_HIP: a HIP call failed";
    case SF_ERR_OOM: return "SF_ERR_OOM: allocation failed";
    case SF_ERR_TIMEOUT: return "SF_ERR_TIMEOUT: a bounded wait on the device expired";
    case SF_ERR_STATE: return "SF_ERR_STATE: store consistency check failed";
  }
  return "unknown sf_status";
}

extern "C" const char* sf_last_error_string(void) { return g_err; }

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shared geometry check (also used by the decode path).
sf_status sf_check_geom(const sf_geom* g) {
  if (!g) return SF_ERR_INVALID_ARG;
  if (g->head_dim <= 0 || g->n_q_heads <= 0 || g->n_kv_heads <= 0) return SF_ERR_INVALID_ARG;
  if (g->n_q_heads % g->n_kv_heads) return SF_ERR_INVALID_ARG;
  if (g->base_bits < 1 || g->refine_bits < 0 || g->base_bits + g->refine_bits > 16) return SF_ERR_INVALID_ARG;
  if (g->head_dim != kHeadDim) return SF_ERR_UNSUPPORTED;
  if (g->base_bits < 2 || g->base_bits > 4 || g->refine_bits > 8) return SF_ERR_UNSUPPORTED;
  const int grp = g->n_q_heads / g->n_kv_heads;
  if (grp != 1 && grp != 2 && grp != 4 && grp != 8) return SF_ERR_UNSUPPORTED;
  return SF_OK;
}

extern "C" sf_status sf_kv_quantize_ex(const sf_geom* geom, const float* x, int64_t n_tok, int64_t tok_begin,
                                       int64_t cap, uint8_t* codes, float* scales, uint8_t* refine_rows,
                                       int32_t flags, void* stream) {
  clear_error();
  if (flags & ~SF_QUANT_FP16_SCALES) return SF_ERR_INVALID_ARG;
  sf_status st = sf_check_geom(geom);
  if (st != SF_OK) return st;
  if (n_tok < 0 || tok_begin < 0 || cap <= 0 || tok_begin + n_tok > cap) return SF_ERR_INVALID_ARG;
  if (n_tok == 0) return SF_OK;
  if (!x || !codes || !scales) return SF_ERR_INVALID_ARG;
  if ((geom->refine_bits > 0) != (refine_rows != nullptr)) return SF_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) ||
      (refine_rows && !aligned16(refine_rows)))
    return SF_ERR_INVALID_ARG;
  const int64_t n_rows = n_tok * geom->n_kv_heads;
  const int64_t blocks = (n_rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (blocks > 0x7fffffffLL) return SF_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     x, n_rows, geom->n_kv_heads, n_tok, tok_begin, cap, geom->base_bits,
                     geom->refine_bits, codes, scales, refine_rows, (flags & SF_QUANT_FP16_SCALES) ? 1 : 0);
  SF_LAUNCH_CHECK("quantize_rows_kernel");
  return SF_OK;
}

extern "C" sf_status sf_kv_quantize(const sf_geom* geom, const float* x, int64_t n_tok,
                                    int64_t tok_begin, int64_t cap, uint8_t* codes, float* scales,
                                    uint8_t* refine_rows, void* stream) {
  return sf_kv_quantize_ex(geom, x, n_tok, tok_begin, cap, codes, scales, refine_rows, 0, stream);
}

// Device-side parameter block and helpers of the decode step.
#pragma once

#include "sf_internal.h"

namespace sfk {

struct DecodeParams {
  int32_t batch, hq, hkv, grp, b, r, top_t;
  int32_t split, sel_chunk, corr_chunk;
  int32_t n_split, n_corr, bm_words;
  int64_t cap, ntot, off0, max_seq;
  const int64_t* seq_off;
  const float* q;
  const uint8_t* kc;
  const float* ks;
  const uint8_t* vc;
  const float* vs;
  float* scores;       // [hkv][ntot]
  uint32_t* hist;      // [batch][hkv][kHistBins]
  uint32_t* counters;  // [batch][hkv][4]: 0 candidates, 1 selection ticket
  uint2* cand;         // [batch][hkv][max_seq] (score key, token)
  uint32_t* bitmap;    // [batch][hkv][bm_words]
  int32_t* sel;        // [batch][hkv][top_t]
  int32_t* sel_out;    // optional copy of sel
  float* part;         // [hkv][n_split][grp][kPartStride]
  float* corr;         // [hkv][n_corr][grp][kPartStride]
  // refinement rows: device tier store, or host-tier device cache
  const uint8_t* ref_rows;    // [2][hkv][cap][rb] or NULL
  const uint8_t* cache_data;  // [max_seqs][hkv][slots][2][rb] or NULL
  const int32_t* tok_slot;    // [hkv][cap]
  int32_t slots, rb;
  float* out;          // [batch][hq][D]
};

__device__ inline void wave_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <typename T>
__device__ inline T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Unit x of a flat enumeration where sequence s contributes ceil(len_s / unit)
// units, len_s = n_s (tokens) or min(T, n_s) (selected tokens) when `sel_len`.
// Returns the sequence and the unit's [lo, hi) range in sequence-local terms;
// `first` receives the flat index of the sequence's first unit.
__device__ inline int locate_unit(const int64_t* off, int batch, int64_t unit, int x, bool sel_len,
                                  int64_t top_t, int64_t& lo, int64_t& hi, int& first) {
  int base = 0;
  for (int s = 0; s < batch; ++s) {
    int64_t len = off[s + 1] - off[s];
    if (sel_len) len = len < top_t ? len : top_t;
    const int n = (int)((len + unit - 1) / unit);
    if (x < base + n) {
      lo = (int64_t)(x - base) * unit;
      hi = lo + unit < len ? lo + unit : len;
      first = base;
      return s;
    }
    base += n;
  }
  lo = hi = 0;
  first = base;
  return -1;
}

// Code d of a row held as 32-bit words (w-bit codes, LSB-first bitstream).
template <int W>
__device__ inline uint32_t code_at(const uint32_t* words, int d) {
  const int pos = d * W, wi = pos >> 5, sh = pos & 31;
  uint32_t v = words[wi] >> sh;
  if (sh + W > 32) v |= words[wi + 1] << (32 - sh);
  return v & ((1u << W) - 1u);
}

}  // namespace sfk

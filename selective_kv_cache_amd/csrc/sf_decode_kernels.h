// Device-side parameter block and helpers of the decode step.
#pragma once

#include <hip/hip_ext.h>

#include "sf_internal.h"

namespace sfk {

struct DecodeParams {
  int32_t batch, hq, hkv, grp, b, r, top_t;
  int32_t score_split, split, sel_chunk;   // tokens per score / attention / selection work-group
  int32_t n_score_split, n_split, bm_words;
  int32_t use_refine;                      // selected rows take their refinement codes
  int32_t n_sel_blk;                       // work-groups of selected tokens (sel_blk_tok each)
  int32_t sel_blk_tok;                     // selected tokens per attention work-group: 16 per wavefront
  int32_t cnt_stride;                      // selection chunks per sequence (max) + 2
  int64_t cap, ntot, off0, max_seq;
  const int64_t* seq_off;
  const float* q;
  const uint8_t* kc;
  const float* ks;
  const uint8_t* vc;
  const float* vs;
  float* scores;       // [hkv][ntot]
  float* logits;       // [hkv][ntot][grp] per-head logits (matrix-core path)
  uint32_t* hist;      // [batch][hkv][kHistBins]: histogram of the scores' top key bits
  uint32_t* counters;  // [batch][hkv][cnt_stride]: candidates of each selection chunk,
                       // then the level-1 boundary bin and the count still needed there
  uint2* cand;         // [batch][hkv][max_seq] (score key, token); chunk c's at c*sel_chunk
  uint32_t* bitmap;    // [batch][hkv][bm_words]
  int32_t* sel;        // [batch][hkv][top_t]
  int32_t* sel_out;    // optional copy of sel
  float* part;         // [hkv][n_sel_blk + n_split][grp][kPartStride]: selected-token
                       // partials first, then the base partials of the splits
  // refinement rows: device tier store, or host-tier device cache
  const uint8_t* ref_rows;    // [2][hkv][cap][rb] or NULL
  const uint8_t* cache_data;  // [max_seqs][hkv][slots][2][rb] or NULL
  const int32_t* tok_slot;    // [hkv][cap] global slot id (seq * hkv + kvh) * slots + slot, -1 if none
  int32_t* store_err;         // host tier: the store's error word (inconsistent cache tables)
  int32_t slots, rb;
  float* out;          // [batch][hq][D]
  // comparison variants (five-kernel form only)
  int32_t drop;               // the unselected tokens take no part (no base splits)
  int32_t score_mode;         // 0: maximum logit over the group; 1: summed softmax probability
  const _Float16* rows16;     // [2][hkv][cap][D] fp16 K and V rows of the selected tokens, or NULL
  float2* sstat;              // [hkv][n_score_split][grp] (maximum, sum) of 2^logit per score unit
  // single-launch (fused) path
  int32_t fr;          // tokens per work-group
  int32_t fscores;     // write the scores to `scores` (the caller asked for them)
  int32_t fsel;        // write the selection to sel_out
  int32_t ftie_stride; // work-groups per (sequence, KV head) at most
  uint32_t* fz;        // [batch][hkv][kFZWords]: histograms and counters, zero between steps
  uint32_t* ftie;      // [batch][hkv][ftie_stride]: tie counts of the work-groups
  uint32_t* fstatus;   // the workspace's status word (bit 0: a bounded wait expired)
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

// Cross-lane steps through DPP (data-parallel primitives: a VALU operand taken
// from another lane of the same 16-lane row) and lane reads into scalar
// registers, instead of LDS permutes.  All 64 lanes must be active.
template <int CTRL>
__device__ inline uint32_t dpp_u32(uint32_t fill, uint32_t x) {
  // lanes whose source lies outside their row keep `fill`
  return (uint32_t)__builtin_amdgcn_update_dpp((int)fill, (int)x, CTRL, 0xF, 0xF, false);
}

// Inclusive prefix sum over the wavefront (lane 0 first): row_shr 1, 2, 4, 8
// inside each row, then the rows' totals.
__device__ inline uint32_t wave_inclusive_scan(uint32_t x) {
  x += dpp_u32<0x111>(0u, x);
  x += dpp_u32<0x112>(0u, x);
  x += dpp_u32<0x114>(0u, x);
  x += dpp_u32<0x118>(0u, x);
  const uint32_t r0 = __builtin_amdgcn_readlane(x, 15);
  const uint32_t r1 = r0 + __builtin_amdgcn_readlane(x, 31);
  const uint32_t r2 = r1 + __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row == 0 ? 0u : row == 1 ? r0 : row == 2 ? r1 : r2);
}

// Maximum and sum over the wavefront, the same value in every lane: quad
// permutes and row mirrors reduce each row, then the four row results.
__device__ inline float row_fold_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
}
__device__ inline float wave_max_dpp(float v) {
  v = row_fold_max(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ inline float wave_sum_dpp(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Offset of sequence s (0 <= s <= batch).  A single sequence's offsets are
// in the parameter block (off0, off0 + ntot), so that a kernel's first memory
// accesses need not wait for a load of the offsets.
__device__ inline int64_t seq_at(const DecodeParams& p, int s) {
  if (p.batch == 1) return s == 0 ? p.off0 : p.off0 + p.ntot;
  return p.seq_off[s];
}

// Unit x of a flat enumeration where sequence s contributes ceil(len_s / unit)
// units, len_s = n_s (tokens) or min(T, n_s) (selected tokens) when `sel_len`.
// Returns the sequence and the unit's [lo, hi) range in sequence-local terms;
// `first` receives the flat index of the sequence's first unit.
//
// Called by whole wavefronts (every lane active).  The Batched form (the
// kernels' instantiation for steps of several sequences) searches a batch of
// 2 to 63 sequences in one memory round trip: lane i reads offsets i and
// i + 1, a wave prefix sum of the unit counts and a ballot name the sequence.
// Otherwise the offsets are walked one sequence at a time (a single
// sequence's come from the parameter block, no load).
template <bool Batched = false>
__device__ inline int locate_unit(const DecodeParams& p, int64_t unit, int x, bool sel_len, int64_t& lo,
                                  int64_t& hi, int& first) {
  if constexpr (Batched) {
    if (p.batch < 64) {
      const int lane = threadIdx.x & 63;
      const bool in = lane < p.batch;
      int64_t len = in ? p.seq_off[lane + 1] - p.seq_off[lane] : 0;
      if (sel_len) len = len < p.top_t ? len : (int64_t)p.top_t;
      const uint32_t n = in ? (uint32_t)((len + unit - 1) / unit) : 0u;
      const uint32_t incl = wave_inclusive_scan(n);
      const uint64_t m = __ballot(in && (uint32_t)x < incl);
      if (m == 0ull) {
        lo = hi = 0;
        first = (int)__builtin_amdgcn_readlane(incl, 63);
        return -1;
      }
      const int s = __ffsll((unsigned long long)m) - 1;
      const int base = (int)__builtin_amdgcn_readlane(incl - n, s);
      const int64_t ls = (int64_t)(((uint64_t)__builtin_amdgcn_readlane((uint32_t)((uint64_t)len >> 32), s) << 32) |
                                   (uint64_t)__builtin_amdgcn_readlane((uint32_t)len, s));
      lo = (int64_t)(x - base) * unit;
      hi = lo + unit < ls ? lo + unit : ls;
      first = base;
      return s;
    }
  }
  int base = 0;
  int64_t o0 = seq_at(p, 0);
  for (int s = 0; s < p.batch; ++s) {
    const int64_t o1 = seq_at(p, s + 1);
    int64_t len = o1 - o0;
    o0 = o1;
    if (sel_len) len = len < p.top_t ? len : (int64_t)p.top_t;
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

// Block-wide exclusive prefix sum of one value per thread (NT threads);
// `lds` holds NT/64 words.  Every thread receives the block total too.
template <int NT>
__device__ inline uint32_t block_exclusive_scan(uint32_t v, uint32_t* lds, uint32_t& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t x = wave_inclusive_scan(v);
  if (lane == 63) lds[wid] = x;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t t = lds[w];
    base += (w < wid) ? t : 0u;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return base + x - v;
}

// Find, in a histogram of NB bins counted from the top bin down, the bin b
// with count(bins > b) < need <= count(bins >= b); writes b and the number
// still needed inside b (need - count(bins > b)).  NT threads, NB % NT == 0;
// needs 1 <= need <= total count.
template <int NT, int NB>
__device__ inline void find_threshold(const uint32_t* hist, uint32_t need, uint32_t* scan_lds, int* out_bin,
                                      uint32_t* out_need) {
  constexpr int PER = NB / NT;
  const int top = NB - PER * (int)threadIdx.x;   // this thread: bins [top - PER, top)
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) s += hist[top - 1 - i];
  uint32_t tot;
  const uint32_t above = block_exclusive_scan<NT>(s, scan_lds, tot);
  if (above < need && need <= above + s) {
    uint32_t cum = above;
    for (int i = 0; i < PER; ++i) {
      const int b = top - 1 - i;
      if (cum + hist[b] >= need) {
        *out_bin = b;
        *out_need = need - cum;
        break;
      }
      cum += hist[b];
    }
  }
  __syncthreads();
}

// find_threshold computed by wavefront 0 alone, without block-wide scans
// (the other wavefronts wait at the closing barrier).  `hist` is 16-byte
// aligned LDS, 256 <= NB <= 4096.  Lane l first sums bins
// [NB - PER (l + 1), NB - PER l), PER = NB / 64; the lane whose range holds
// the boundary is found from the prefix over lanes, then its PER bins are
// taken one per lane.
template <int NB>
__device__ inline void find_threshold_wave(const uint32_t* hist, uint32_t need, int* out_bin, uint32_t* out_need) {
  static_assert(NB % 256 == 0 && NB <= 4096, "one bin per lane in the second step");
  constexpr int PER = NB / 64, Q = PER / 4;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const uint4* h4 = reinterpret_cast<const uint4*>(hist) + (NB / 4 - Q * (lane + 1));
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < Q; ++i) {
      // rotated start: neighbouring lanes read different LDS banks
      const uint4 x = h4[(i + lane) % Q];
      s += x.x + x.y + x.z + x.w;
    }
    const uint32_t inc = wave_inclusive_scan(s);
    const uint64_t hit = __ballot(inc - s < need && need <= inc);
    if (hit) {
      const int L = __ffsll((unsigned long long)hit) - 1;
      const uint32_t above = __builtin_amdgcn_readlane(inc - s, L);
      const int top = NB - PER * L;
      const uint32_t c = lane < PER ? hist[top - 1 - lane] : 0u;
      const uint32_t cum = wave_inclusive_scan(c);
      const uint64_t hit2 = __ballot(above + cum >= need);
      const int j = __ffsll((unsigned long long)hit2) - 1;
      if (lane == j) {
        *out_bin = top - 1 - j;
        *out_need = need - (above + cum - c);
      }
    }
  }
  __syncthreads();
}

// Optional events attached to a kernel's dispatch: `stop` completes with the
// kernel itself (no marker packet after it); `start` is recorded just before
// it.
struct KernelEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

template <typename K>
inline void sf_launch(K kernel, dim3 grid, dim3 block, hipStream_t st, KernelEvents ev, const DecodeParams& p) {
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, ev.start, ev.stop, 0, p);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, st, p);
}

// Launchers (one per stage source file).
bool launch_score(const DecodeParams& p, dim3 grid, hipStream_t st, KernelEvents ev = {});
void launch_select(const DecodeParams& p, dim3 grid, hipStream_t st, KernelEvents scan_ev = {},
                   KernelEvents resolve_ev = {});
bool launch_attend(const DecodeParams& p, dim3 grid, hipStream_t st, KernelEvents ev = {});
void launch_combine(const DecodeParams& p, hipStream_t st, KernelEvents ev = {});

constexpr int kScoreWaves = 16;         // wavefronts per score work-group (matrix-core path)
constexpr int kSelThreads = 512;
constexpr int32_t kSelChunk = 4096;
constexpr int32_t kMaxSelChunks = 512;   // longest sequence: kMaxSelChunks * kSelChunk tokens
constexpr int32_t kSelBlkTok = 64;     // selected tokens per attention work-group: 4 wavefronts x 16 tokens,
constexpr int32_t kSelBlkTokMin = 16;  // or 4 wavefronts x 4 tokens when those work-groups still fit
constexpr int kAttendWaves = 4;         // wavefronts per attention work-group (matrix-core path)
constexpr int kCombineMax = 2048;      // partials per (sequence, query head)

// Single-launch path: per (sequence, KV head) region of the level-1,
// level-2 and level-3 histograms and the counters (barrier arrivals, done),
// zero between steps, then the level-1 candidates' list (a slot of keys and
// one of token indices per work-group, and each work-group's count; not
// cleared).
constexpr int kFListMax = 4096;         // list entries of a head (slots of kFListMax / ranges each)
constexpr int kFListRanges = 64;        // work-groups per head the list serves at most
constexpr int kFZH1 = 0, kFZH2 = kHistBins, kFZH3 = 2 * kHistBins, kFZC = 2 * kHistBins + 256;
constexpr int kFZL = kFZC + 16;         // keys; tokens at kFZL + kFListMax; counts at kFZL + 2 kFListMax
constexpr int kFZWords = kFZL + 2 * kFListMax + kFListRanges;
constexpr int kFusedRmax = 4096;        // tokens per work-group at most
constexpr int kFusedMinR = 256;         // and at least (a multiple of it)
constexpr int kFusedMaxRanges = 512;    // work-groups per (sequence, KV head) at most
bool launch_fused(const DecodeParams& p, dim3 grid, hipStream_t st, KernelEvents ev);
bool launch_softmax_scores(const DecodeParams& p, dim3 grid, hipStream_t st);   // the score variant's two kernels
int fused_capacity(int grp, bool batched);   // co-resident work-groups on the device

}  // namespace sfk

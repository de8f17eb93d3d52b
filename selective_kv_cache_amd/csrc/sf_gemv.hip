// Weight-side refinement GEMV: y = W x with the nested-quantized W of
// sf_w_quantize, the top-k input channels of largest |x| per chunk refined.
//
// Page "StrataFlux -- Selective precision streaming -- What does it mean?":
// paragraph "Which tiles count ..." (chunks of 1,024 input channels, the k
// channels of largest activation magnitude refined at this step), paragraph
// "What travels over the link ..." (refinement bits subdivide the bin of the
// resident code), and the worked example (k = 32 of 1,024, 4-bit refinement
// values on 3-bit weights).
//
// Layout: codes [m][k/128][16 b] bytes (per row and 128-channel group an
// LSB-first bitstream of b-bit codes), scales [m][k/128] {lo, delta},
// refinement codes column-major [k][m r / 8] (a channel's codes for every
// row, LSB-first over rows).
//
// One launch, two kinds of work-group:
// * the first work-groups select, one chunk per wavefront (the top-k of the
//   chunk's |x|, ties to the lower index; see select_chunk_wave), and write
//   the chosen channels in ascending order, each tagged with the call's
//   epoch (device-scope stores; the epoch comes from counters in the
//   workspace that every wavefront advances when it starts);
// * the others compute 8 P output rows over all of k.  The input channels
//   are cut into slices of 2,048 (64 lanes x 32 channels); wavefront (slice
//   s, row group g) reads its 32 channels of x from LDS and, for each of its
//   8 rows, decodes the lane's 32 base codes: with c the codes, the
//   segment's sum of (lo + (c + 1/2) delta) x is lo S0 + delta (sum c x +
//   S0 / 2), S0 the segment's sum of x.  The 8 row sums are reduced across
//   the lanes at once (halving exchanges), the slices summed in LDS in a
//   fixed order.  The selection, loaded early, is taken once every entry
//   carries the call's epoch (the selecting work-groups come first in the
//   dispatch order and wait for nothing; a bounded wait otherwise), and per
//   (row, selected channel) delta ((s + 1/2) 2^-r - 1/2) x_c is added, s the
//   channel's refinement code for the row.
// Every result is summed in a fixed order: the call is deterministic.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>

#include "sf_decode_kernels.h"
#include "sf_internal.h"

namespace sfk {

constexpr int kWGroup = 128;          // channels per quantization group
constexpr int kWSeg = 32;             // channels per lane segment
constexpr int kWSlice = 64 * kWSeg;   // channels per wavefront slice
constexpr int kWMaxChunk = 4096;
constexpr int kWMaxK = 15360;         // at most 8 slices: 8 wavefronts per work-group
constexpr int kWMaxThreads = 512;
constexpr int kWSpinLimit = 1 << 18;  // bounded wait: about 0.2 s
constexpr int kWTile = 1024;          // selected channels staged in LDS at a time
constexpr int kWCalls = 16;           // counters of started wavefronts (the call's epoch)
constexpr int kWCallStride = 32;      // words between them (separate cache lines)

__device__ inline uint32_t wld(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline int32_t wld(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void wst(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void wst(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline uint64_t wld64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void wst64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

typedef __amdgpu_buffer_rsrc_t wrsrc_t;
// Raw buffer resource over [base, base + bytes): loads past the range return zeros.
__device__ inline wrsrc_t wrsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// The B words of one lane segment in one load.
template <int B>
__device__ inline void load_seg(wrsrc_t r, uint32_t off, uint32_t (&w)[4]) {
  if constexpr (B == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
    w[0] = v[0], w[1] = v[1], w[2] = 0u, w[3] = 0u;
  } else if constexpr (B == 3) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, (int)off, 0, 0);
    w[0] = v[0], w[1] = v[1], w[2] = v[2], w[3] = 0u;
  } else {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    w[0] = v[0], w[1] = v[1], w[2] = v[2], w[3] = v[3];
  }
}
// Position of float4 unit u of x in LDS: the 8 units of a lane segment are
// rotated by the segment's index, so that 8 neighbouring lanes reading their
// i-th units hit distinct banks.
__device__ inline int xswz(int u) { return (u & ~7) | ((u & 7) ^ ((u >> 3) & 7)); }

struct WLds {
  uint32_t hist[kWMaxThreads / 64][256];   // per-wavefront radix histograms (selection)
  float red[kWMaxThreads / 64][8];     // per-wavefront row sums
  float cred[kWMaxThreads];            // per-thread correction sums
  int32_t tile[kWTile];                // selected channels being added
};

// Inclusive prefix sum over the 64 lanes: shifts within rows of 16, then
// the rows' totals broadcast to the rows above.
__device__ inline uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// Order of one wavefront's LDS operations across its lanes: the LDS unit
// serves a wavefront's instructions in issue order; this keeps the compiler
// from moving them.
__device__ inline void wave_lds_order() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

struct WArgs {
  const uint8_t* codes;
  const float2* scales;
  const uint8_t* refine_cols;
  const float* x;
  float* y;
  int32_t* sel;
  uint64_t* tags;       // [nchunks kout] selected channels tagged with the call's epoch
  uint32_t* calls;      // [kWCalls] 64-bit counters of started wavefronts, kWCallStride words apart
  uint32_t* status;     // set nonzero when a wait expired
  int32_t m, k, r, top_k, chunk, kout, nchunks, nsel_wg, ns, p;
  int32_t merged;       // the selecting work-groups go on to their own rows
};

// The call's epoch, without host state (so that a captured graph replays
// correctly): every wavefront of the launch adds 1 to counter gw mod kWCalls
// (gw its index in the launch; counters on separate cache lines) when it
// starts.  With a fixed launch shape counter j gains the same n_j every
// call, so v / n_j (v the value it returned) is the number of earlier calls,
// the same for every wavefront of the call.  The counter's value is read
// where the epoch is needed, late, so the atomic's latency is hidden.
__device__ inline uint64_t start_count(const WArgs& a) {
  const uint32_t gw = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  unsigned long long v = 0ull;
  if ((threadIdx.x & 63) == 0)
    v = atomicAdd(reinterpret_cast<unsigned long long*>(a.calls + (gw % kWCalls) * kWCallStride), 1ull);
  return v;
}

// The call's epoch from a wavefront's start count v (see start_count): the
// number of earlier calls plus 1.
__device__ inline uint32_t epoch_of(uint64_t v) {
  const uint32_t wpg = blockDim.x >> 6;
  const uint32_t gw = blockIdx.x * wpg + (threadIdx.x >> 6);
  const uint32_t total = gridDim.x * wpg, j = gw % kWCalls;
  const uint32_t n_j = (total - j + kWCalls - 1) / kWCalls;
  const uint64_t v0 = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 0) << 32) |
                      (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 0);
  return (uint32_t)(v0 / n_j) + 1u;
}

// The need-th largest (1 <= need <= count) of the lanes' 31-bit values v
// where `active`, by bisection from the top bit: the largest T with at
// least `need` active values >= T.  Ballots and scalar counts only.
__device__ inline uint32_t wave_kth_largest(uint32_t v, bool active, uint32_t need) {
  uint32_t t = 0u;
#pragma unroll
  for (int b = 30; b >= 0; --b) {
    const uint32_t c = t | (1u << b);
    if ((uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(active && v >= c)) >= need) t = c;
  }
  return t;
}

// Number of lanes below this one whose bit is set in `mask`.
__device__ inline uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Inlined, so that its histogram accesses are LDS instructions (a generic
// pointer would make them flat accesses).
// One wavefront: the top-k channels of x[c0, c0 + n) by |x|, ties to the
// lower index.  The chunk's |x| bits are staged in LDS (xl, element e of the
// chunk at xl[e]) and read in blocks of 16 rounds of 64 (element 64 r +
// lane), all of a block's reads in flight at once.
// * A lower bound of the kk-th largest magnitude (kk = min(k, n)): when kk
//   <= 64, the kk-th largest of the 64 lanes' maxima (kk lanes hold an
//   element at least that large); else 0.  Only the candidates at or above
//   it can be chosen.  For chunks of at most 1,024 (lane l holding 16
//   consecutive elements) with at most 64 candidates, they are listed in
//   index order one per lane (a prefix sum of the lanes' counts), the kk-th
//   largest of them found by bisection, and those above it and the first of
//   those equal to it written in list order: done.
// * Else a radix select over the candidates' 31 bits of |x| (digits of 8,
//   8, 8 and 7 bits, a 256-bin histogram in `hist`) finds the kk-th largest.
// * Round by round, the channels above it and the first of those equal to
//   it are ranked with ballots (the lanes below in the round plus the
//   earlier rounds) and written ascending to out[0, kk) and to tags[] with
//   the epoch in the upper half (device-scope stores); out[kk, kout) = -1.
__device__ __attribute__((always_inline)) inline void select_chunk_wave(const WArgs& a, uint32_t* hist, uint32_t* xl,
                                                                       const float* __restrict__ x, int c0, int n,
                                                                       int k, int kout, int32_t* __restrict__ out,
                                                                       uint64_t* __restrict__ tags, uint64_t& started) {
  const int lane = threadIdx.x & 63;
  const int kk = min(k, n);
  const int rounds = (n + 63) / 64;
  constexpr int kR = 16;                     // rounds per block
  {
    const uint32_t* xg = reinterpret_cast<const uint32_t*>(x + c0);
    for (int r0 = 0; r0 < rounds; r0 += kR) {
      uint32_t v[kR];
#pragma unroll
      for (int j = 0; j < kR; ++j) v[j] = xg[min((r0 + j) * 64 + lane, n - 1)];
#pragma unroll
      for (int j = 0; j < kR; ++j) {
        const int e = (r0 + j) * 64 + lane;
        if (e < n) xl[e] = v[j] & 0x7FFFFFFFu;
      }
    }
    wave_lds_order();
  }
  // counted after the staging loads, so that waiting for them does not wait
  // for the atomic
  started = start_count(a);
  // the block's values: u[j] of element (r0 + j) 64 + lane, 0 past the chunk
  auto load_block = [&](int r0, uint32_t (&u)[kR]) {
#pragma unroll
    for (int j = 0; j < kR; ++j) {
      const int e = (r0 + j) * 64 + lane;
      const uint32_t t = xl[min(e, n - 1)];
      u[j] = e < n ? t : 0u;
    }
  };
  uint32_t floor_u = 0u;
  if (kk < n && kk <= 64 && n <= 64 * kR) {
    // lane l holds elements l E .. l E + E - 1 (E = rounds <= kR), so that
    // lane order then element order is index order
    const int E = rounds;
    uint32_t u[kR];
    uint32_t valid = 0u, lm = 0u;
#pragma unroll
    for (int j = 0; j < kR; ++j) {
      const int e = lane * E + j;
      const bool ok = j < E && e < n;
      u[j] = ok ? xl[min(e, n - 1)] : 0u;
      valid |= ok ? 1u << j : 0u;
      lm = max(lm, u[j]);
    }
    // the kk-th largest of the lanes' maxima bounds the kk-th largest below
    floor_u = wave_kth_largest(lm, true, (uint32_t)kk);
    uint32_t cm = 0u;
#pragma unroll
    for (int j = 0; j < kR; ++j) cm |= ((valid >> j) & 1u) && u[j] >= floor_u ? 1u << j : 0u;
    const uint32_t c = (uint32_t)__builtin_popcount(cm);
    const uint32_t inc = wave_incl_scan(c);
    const uint32_t cnt = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
    if (cnt <= 64u) {
      // the candidates in index order, one per lane, through LDS
      uint32_t* cu = hist;          // magnitudes
      uint32_t* ce = hist + 64;     // element indices
      uint32_t pos = inc - c;
#pragma unroll
      for (int j = 0; j < kR; ++j)
        if ((cm >> j) & 1u) {
          cu[pos] = u[j];
          ce[pos] = (uint32_t)(lane * E + j);
          ++pos;
        }
      wave_lds_order();
      // the kk-th largest magnitude among them; those above it, and the
      // first of those equal to it, are chosen
      const bool mine = (uint32_t)lane < cnt;
      const uint32_t mu = mine ? cu[lane] : 0u, me = mine ? ce[lane] : 0u;
      const uint32_t thr = wave_kth_largest(mu, mine, (uint32_t)kk);
      const uint32_t n_above = (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(mine && mu > thr));
      const uint64_t beq = __builtin_amdgcn_ballot_w64(mine && mu == thr);
      const bool chosen = mine && (mu > thr || (mu == thr && lanes_below(beq) < (uint32_t)kk - n_above));
      const uint32_t p = lanes_below(__builtin_amdgcn_ballot_w64(chosen));
      const uint64_t tag = (uint64_t)epoch_of(started) << 32;
      if (chosen && p < (uint32_t)kout) {
        out[p] = c0 + (int)me;
        wst64(tags + p, tag | (uint32_t)(c0 + (int)me));
      }
      for (int t = kk + lane; t < kout; t += 64) {
        out[t] = -1;
        wst64(tags + t, tag | 0xFFFFFFFFull);
      }
      return;
    }
    wave_lds_order();
  } else if (kk < n && kk <= 64) {
    // longer chunks: the same bound, the candidates left to the radix select
    uint32_t lm = 0u;
    for (int r0 = 0; r0 < rounds; r0 += kR) {
      uint32_t u[kR];
      load_block(r0, u);
#pragma unroll
      for (int j = 0; j < kR; ++j) lm = max(lm, u[j]);
    }
    floor_u = wave_kth_largest(lm, true, (uint32_t)kk);
  }
  // the general case: a radix select over the candidates
  uint32_t prefix = 0u, pmask = 0u, need = (uint32_t)kk;
  if (kk < n) {
    constexpr int kShift[4] = {23, 15, 7, 0};
    constexpr int kBits[4] = {8, 8, 8, 7};
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = kShift[pass], nb = 1 << kBits[pass], bpl = nb / 64;
#pragma unroll
      for (int j = 0; j < 4; ++j) hist[lane + 64 * j] = 0u;
      wave_lds_order();
      for (int r0 = 0; r0 < rounds; r0 += kR) {
        uint32_t u[kR];
        load_block(r0, u);
#pragma unroll
        for (int j = 0; j < kR; ++j) {
          const bool match = (r0 + j) * 64 + lane < n && u[j] >= floor_u && (u[j] & pmask) == prefix;
          if (match) atomicAdd(&hist[(u[j] >> shift) & (uint32_t)(nb - 1)], 1u);
        }
      }
      wave_lds_order();
      // lane l: bins nb - 1 - (bpl l + j), from the top down
      uint32_t hb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) hb[j] = j < bpl ? hist[nb - 1 - (bpl * lane + j)] : 0u;
      const uint32_t ls = hb[0] + hb[1] + hb[2] + hb[3];
      const uint32_t inc = wave_incl_scan(ls);
      uint32_t run = inc - ls;
      const uint64_t hit = __builtin_amdgcn_ballot_w64(run < need && inc >= need);
      const int L = hit ? (int)__builtin_ctzll(hit) : 0;
      // in lane L: the boundary bin among its bpl bins
      uint32_t digit = 0u, above = run;
      bool found = false;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool here = !found && j < bpl && run + hb[j] >= need;
        digit = here ? (uint32_t)(nb - 1 - (bpl * lane + j)) : digit;
        above = here ? run : above;
        found = found || here;
        run += found ? 0u : hb[j];
      }
      digit = (uint32_t)__builtin_amdgcn_readlane((int)digit, L);
      above = (uint32_t)__builtin_amdgcn_readlane((int)above, L);
      prefix |= digit << shift;
      pmask |= (uint32_t)(nb - 1) << shift;
      need -= above;
      wave_lds_order();
    }
  } else {
    prefix = 0u;     // every channel is chosen: all are above or equal to 0
    need = (uint32_t)n;
  }
  const uint64_t tag = (uint64_t)epoch_of(started) << 32;
  uint32_t eq_seen = 0u, pos = 0u;
  for (int r0 = 0; r0 < rounds; r0 += kR) {
    uint32_t u[kR];
    load_block(r0, u);
#pragma unroll
    for (int j = 0; j < kR; ++j) {
      const int e = (r0 + j) * 64 + lane;
      const bool valid = e < n;
      const bool eq = valid && u[j] == prefix;
      const uint64_t beq = __builtin_amdgcn_ballot_w64(eq);
      const bool chosen = valid && (u[j] > prefix || (eq && eq_seen + lanes_below(beq) < need));
      const uint64_t bch = __builtin_amdgcn_ballot_w64(chosen);
      const uint32_t p = pos + lanes_below(bch);
      if (chosen && p < (uint32_t)kout) {
        out[p] = c0 + e;
        wst64(tags + p, tag | (uint32_t)(c0 + e));
      }
      eq_seen += (uint32_t)__builtin_popcountll(beq);
      pos += (uint32_t)__builtin_popcountll(bch);
    }
  }
  for (int t = kk + lane; t < kout; t += 64) {
    out[t] = -1;
    wst64(tags + t, tag | 0xFFFFFFFFull);
  }
}

// The 32 codes of one segment (b words from `w`, b <= 4) as integers.
template <int B>
__device__ inline void seg_codes(const uint32_t (&w)[4], float (&c)[kWSeg]) {
#pragma unroll
  for (int j = 0; j < kWSeg; ++j) {
    const int pos = j * B, wi = pos >> 5, sh = pos & 31;
    uint32_t v = w[wi] >> sh;
    if (sh + B > 32) v |= w[wi + 1] << (32 - sh);
    c[j] = (float)(v & ((1u << B) - 1u));
  }
}

// Sum of p[i] over the 64 lanes for 8 values at once: after the exchanges
// lane l holds row ((l >> 5) & 1) 4 + ((l >> 4) & 1) 2 + ((l >> 3) & 1).
__device__ inline float reduce8_rows(const float (&p)[8]) {
  const int lane = threadIdx.x & 63;
  float q[4], r[2];
  const bool h1 = lane & 32, h2 = lane & 16, h3 = lane & 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = (h1 ? p[i + 4] : p[i]) + __shfl_xor(h1 ? p[i] : p[i + 4], 32);
#pragma unroll
  for (int i = 0; i < 2; ++i) r[i] = (h2 ? q[i + 2] : q[i]) + __shfl_xor(h2 ? q[i] : q[i + 2], 16);
  float v = (h3 ? r[1] : r[0]) + __shfl_xor(h3 ? r[0] : r[1], 8);
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 1);
  return v;
}



template <int B>
__global__ void __launch_bounds__(kWMaxThreads) w_gemv(WArgs a) {
  __shared__ WLds s;
  extern __shared__ float4 xs4[];                      // x, k / 4 units, rotated (xswz)
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint64_t started = 0ull;                             // the call's epoch: epoch_of(started)
  const bool selecting = (int)blockIdx.x < a.nsel_wg;
  if (selecting) {
    // the selection is a chain of dependent steps that the row work-groups
    // wait for at their end: it takes the issue slots first
    __builtin_amdgcn_s_setprio(3);
    // wavefront wv of selecting work-group b: chunk b (blockDim / 64) + wv
    const int q = blockIdx.x * (int)(blockDim.x >> 6) + wv;
    if (q < a.nchunks) {
      const int c0 = q * a.chunk;
      // the chunks of one work-group are disjoint ranges of k: each
      // wavefront stages its chunk at the chunk's own place in the x area
      select_chunk_wave(a, s.hist[wv], reinterpret_cast<uint32_t*>(xs4) + c0, a.x, c0, min(a.chunk, a.k - c0),
                        a.top_k, a.kout, a.sel + (int64_t)q * a.kout, a.tags + (int64_t)q * a.kout, started);
    } else {
      started = start_count(a);                        // every wavefront counts itself, once
    }
    if (!a.merged) return;
    // merged: this work-group goes on to its own rows once every wavefront
    // is done with the selection's staging area
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
  }
  const int rb = 8 * a.p;                              // rows of the work-group
  // XCD-aware rows: work-groups are dealt to the 8 XCDs in turn, so base
  // work-group b runs on XCD (b + nsel_wg) mod 8; the blocks that share an
  // XCD take contiguous rows, and a selected channel's refinement line
  // (whose rows span several blocks) is fetched into that XCD's L2 once
  // instead of by every XCD
  int row0;
  {
    const int nb = a.m / rb, b = a.merged ? (int)blockIdx.x : (int)blockIdx.x - a.nsel_wg;
    const int q8 = nb >> 3, r8 = nb & 7, x8 = b & 7;
    row0 = (x8 * q8 + min(x8, r8) + (b >> 3)) * rb;
  }
  const int ngrp = a.k / kWGroup, nseg = a.k / kWSeg;
  const uint32_t row_bytes = (uint32_t)a.k * B / 8;
  const int n_sel = a.kout > 0 ? a.nchunks * a.kout : 0;
  // x into LDS
  {
    const float4* xg = reinterpret_cast<const float4*>(a.x);
    for (int u = tid; u < a.k / 4; u += blockDim.x) xs4[xswz(u)] = xg[u];
  }
  // wavefront wv: slice wv / p, rows row0 + 8 (wv % p) + [0, 8)
  const int slice = wv / a.p, grp = wv % a.p;
  const int sg = slice * 64 + lane;
  const bool live = sg < nseg;
  const int rr0 = row0 + 8 * grp;
  uint32_t w[8][4];
  float2 sc[8];
  {
    const wrsrc_t rc = wrsrc(a.codes + (uint64_t)rr0 * row_bytes, 8u * row_bytes);
    const wrsrc_t rs = wrsrc(a.scales + (int64_t)rr0 * ngrp, 8u * (uint32_t)ngrp * 8u);
    const uint32_t coff = live ? (uint32_t)sg * B * 4u : 0x80000000u;   // past the range: zeros
    const uint32_t soff = live ? (uint32_t)(sg / (kWGroup / kWSeg)) * 8u : 0x80000000u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      load_seg<B>(rc, coff + (uint32_t)i * row_bytes, w[i]);
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)(soff + (uint32_t)i * (uint32_t)ngrp * 8u), 0, 0);
      sc[i] = make_float2(__uint_as_float(v[0]), __uint_as_float(v[1]));
    }
  }
  // counted after the code loads (waiting for them then does not wait for
  // the atomic); a wavefront that selected has counted already
  if (!selecting) started = start_count(a);
  // the first tile of the selection, speculatively: an entry is valid once
  // it carries this call's epoch
  constexpr int kSpec = kWTile / 256;
  uint64_t spec[kSpec];
#pragma unroll
  for (int u = 0; u < kSpec; ++u) {
    const int j = tid + u * (int)blockDim.x;
    spec[u] = j < min(n_sel, kWTile) ? wld64(a.tags + j) : 0ull;
  }
  __syncthreads();                                     // x staged
  float xv[kWSeg];
  float s0 = 0.f;
#pragma unroll
  for (int i = 0; i < kWSeg / 4; ++i) {
    const float4 t = live ? xs4[xswz(sg * 8 + i)] : make_float4(0.f, 0.f, 0.f, 0.f);
    xv[4 * i] = t.x, xv[4 * i + 1] = t.y, xv[4 * i + 2] = t.z, xv[4 * i + 3] = t.w;
  }
#pragma unroll
  for (int j = 0; j < kWSeg; ++j) s0 += xv[j];
  float part[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float c[kWSeg];
    seg_codes<B>(w[i], c);
    float d = 0.f;
#pragma unroll
    for (int j = 0; j < kWSeg; ++j) d = fmaf(c[j], xv[j], d);
    part[i] = fmaf(sc[i].x, s0, sc[i].y * (d + 0.5f * s0));
  }
  const float v = reduce8_rows(part);
  if ((lane & 7) == 0) s.red[wv][((lane >> 5) & 1) * 4 + ((lane >> 4) & 1) * 2 + ((lane >> 3) & 1)] = v;
  // corrections: the selection in tiles of kWTile entries staged in LDS;
  // thread (row i, slot j0) over the tile's entries j0, j0 + tpr, ...
  const int i = tid % rb, j0 = tid / rb, tpr = blockDim.x / rb;
  const int row = row0 + i;
  const float sub = __builtin_ldexpf(1.0f, -a.r);
  const int64_t col_bytes = (int64_t)a.m * a.r / 8;
  const int64_t bit = (int64_t)row * a.r;
  const uint32_t mask = (1u << a.r) - 1u;
  const float2* srow = a.scales + (int64_t)row * ngrp;
  float corr = 0.f;
  bool ok = true;
  const uint32_t epoch = n_sel > 0 ? epoch_of(started) : 0u;
  for (int t0 = 0; t0 < n_sel && ok; t0 += kWTile) {
    const int nt = min(kWTile, n_sel - t0);
    bool mine = true;                                  // this thread's entries of the tile are valid
    if (t0 == 0) {
#pragma unroll
      for (int u = 0; u < kSpec; ++u) {
        const int j = tid + u * (int)blockDim.x;
        if (j < nt) {
          mine = mine && (uint32_t)(spec[u] >> 32) == epoch;
          s.tile[j] = (int32_t)(uint32_t)spec[u];
        }
      }
    } else {
      mine = false;
    }
    int spins = 0;
    while (!__syncthreads_and(mine)) {
      if (!mine) __builtin_amdgcn_s_sleep(1);
      mine = true;
      for (int j = tid; j < nt; j += blockDim.x) {
        const uint64_t e = wld64(a.tags + t0 + j);
        mine = mine && (uint32_t)(e >> 32) == epoch;
        s.tile[j] = (int32_t)(uint32_t)e;
      }
      if (++spins > kWSpinLimit) {
        ok = false;
        break;
      }
    }
    if (!ok) break;
    constexpr int kU = 8;                            // entries a thread loads at once
    for (int j = j0; j < nt; j += kU * tpr) {
      int c[kU];
      uint32_t lo8[kU], hi8[kU];
      float dl[kU], xc[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) c[u] = j + u * tpr < nt ? s.tile[j + u * tpr] : -1;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int cc = c[u] < 0 ? 0 : c[u];
        const uint8_t* col = a.refine_cols + (int64_t)cc * col_bytes + (bit >> 3);
        lo8[u] = col[0];
        hi8[u] = ((bit & 7) + a.r > 8) ? col[1] : 0u;
        dl[u] = srow[cc / kWGroup].y;
        const float4 xq = xs4[xswz(cc >> 2)];
        xc[u] = (cc & 2) ? ((cc & 1) ? xq.w : xq.z) : ((cc & 1) ? xq.y : xq.x);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const uint32_t code = ((lo8[u] | (hi8[u] << 8)) >> (bit & 7)) & mask;
        const float t = dl[u] * fmaf((float)code + 0.5f, sub, -0.5f) * xc[u];
        corr += c[u] < 0 ? 0.f : t;
      }
    }
    __syncthreads();
  }
  if (!ok && tid == 0) atomicOr(a.status, 1u);
  s.cred[tid] = corr;
  __syncthreads();
  if (tid < rb) {
    const int g8 = tid >> 3, ri = tid & 7;
    float y = 0.f;
    for (int sl = 0; sl < a.ns; ++sl) y += s.red[sl * a.p + g8][ri];
    for (int jj = 0; jj < tpr; ++jj) y += s.cred[jj * rb + tid];
    a.y[row0 + tid] = ok ? y : __builtin_nanf("");
  }
}

// Column-major refinement codes from the row-major ones of the quantizer:
// thread (channel c, 32-row block) gathers 32 r-bit codes into r words.
__global__ void __launch_bounds__(256) w_refine_columns(const uint8_t* __restrict__ rows, uint8_t* __restrict__ cols,
                                                        int32_t m, int32_t k, int32_t r) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nblk = m / 32;
  if (t >= (int64_t)k * nblk) return;
  const int c = (int)(t / nblk), blk = (int)(t % nblk);
  const int g = c / kWGroup, e = c % kWGroup;
  const int64_t grp_bytes = 16 * r;       // 128 r bits per (row, group)
  uint32_t out[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  for (int i = 0; i < 32; ++i) {
    const int row = blk * 32 + i;
    const uint8_t* src = rows + ((int64_t)row * (k / kWGroup) + g) * grp_bytes;
    const int bit = e * r;
    const uint32_t lo8 = src[bit >> 3];
    const uint32_t hi8 = ((bit & 7) + r > 8) ? src[(bit >> 3) + 1] : 0u;
    const uint32_t s = ((lo8 | (hi8 << 8)) >> (bit & 7)) & ((1u << r) - 1u);
    const int ob = i * r;
    out[ob >> 5] |= s << (ob & 31);
    if ((ob & 31) + r > 32) out[(ob >> 5) + 1] |= s >> (32 - (ob & 31));
  }
  uint32_t* dst = reinterpret_cast<uint32_t*>(cols + (int64_t)c * m * r / 8 + (int64_t)blk * 4 * r);
  for (int i = 0; i < r; ++i) dst[i] = out[i];
}

}  // namespace sfk

using namespace sfk;

static sf_status check_wgeom(const sf_wgeom* g) {
  if (!g || g->m <= 0 || g->k <= 0 || g->m % 32 || g->k % kWGroup || g->base_bits < 2 || g->base_bits > 4 ||
      g->refine_bits < 1 || g->refine_bits > 8 || g->top_k < 0 || g->chunk <= 0 || g->chunk > kWMaxChunk ||
      g->top_k > g->chunk)
    return SF_ERR_INVALID_ARG;
  if (g->k > kWMaxK) return SF_ERR_UNSUPPORTED;
  return SF_OK;
}

extern "C" sf_status sf_w_quantize(const sf_wgeom* g, const float* w, uint8_t* codes, float* scales,
                                   uint8_t* refine_cols, uint8_t* scratch, void* stream) {
  clear_error();
  sf_status s = check_wgeom(g);
  if (s != SF_OK) return s;
  if (!w || !codes || !scales || !refine_cols || !scratch) return SF_ERR_INVALID_ARG;
  // every (row, group of 128 channels) is one row of the nested quantizer
  const sf_geom qg{kWGroup, 1, 1, g->base_bits, g->refine_bits};
  const int64_t n_rows = (int64_t)g->m * (g->k / kWGroup);
  s = sf_kv_quantize(&qg, w, n_rows, 0, n_rows, codes, scales, scratch, stream);
  if (s != SF_OK) return s;
  const int64_t threads = (int64_t)g->k * (g->m / 32);
  hipLaunchKernelGGL(w_refine_columns, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                     scratch, refine_cols, g->m, g->k, g->refine_bits);
  SF_LAUNCH_CHECK("w_refine_columns");
  return SF_OK;
}

// Work-groups of w_gemv<b> (threads, dynamic LDS) resident at once on the
// current device; cached per shape.
static int resident_wgs(int b, int threads, size_t lds) {
  static std::mutex mu;
  static std::map<std::tuple<int, int, int, size_t>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1 << 30;
  const auto key = std::make_tuple(dev, b, threads, lds);
  {
    std::lock_guard<std::mutex> lk(mu);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  int per_cu = 0, cus = 0;
  hipError_t e = b == 2   ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, w_gemv<2>, threads, lds)
                 : b == 3 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, w_gemv<3>, threads, lds)
                          : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, w_gemv<4>, threads, lds);
  if (e != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 1 << 30;      // unknown: the extra selecting work-groups
  }
  const int n = per_cu * cus;
  std::lock_guard<std::mutex> lk(mu);
  cache[key] = n;
  return n;
}

extern "C" sf_status sf_w_gemv_workspace_words(const sf_wgeom* g, int32_t* words) {
  clear_error();
  sf_status s = check_wgeom(g);
  if (s != SF_OK) return s;
  if (!words) return SF_ERR_INVALID_ARG;
  const int32_t nchunks = (g->k + g->chunk - 1) / g->chunk;
  *words = kWCallStride * kWCalls + 2 * nchunks * std::min(g->top_k, g->chunk) + 2;
  return SF_OK;
}

extern "C" sf_status sf_w_gemv(const sf_wgeom* g, const uint8_t* codes, const float* scales,
                               const uint8_t* refine_cols, const float* x, float* y, int32_t* sel,
                               uint32_t* workspace, void* stream) {
  clear_error();
  sf_status s = check_wgeom(g);
  if (s != SF_OK) return s;
  if (!codes || !scales || !refine_cols || !x || !y || !sel || !workspace) return SF_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(scales) | reinterpret_cast<uintptr_t>(codes) |
       reinterpret_cast<uintptr_t>(workspace)) & 15)
    return SF_ERR_INVALID_ARG;
  WArgs a{};
  a.codes = codes;
  a.scales = reinterpret_cast<const float2*>(scales);
  a.refine_cols = refine_cols;
  a.x = x;
  a.y = y;
  a.sel = sel;
  a.m = g->m;
  a.k = g->k;
  a.r = g->refine_bits;
  a.top_k = g->top_k;
  a.chunk = g->chunk;
  a.kout = std::min(g->top_k, g->chunk);
  a.nchunks = (g->k + g->chunk - 1) / g->chunk;
  a.ns = (g->k + kWSlice - 1) / kWSlice;
  a.p = a.ns == 1 ? 4 : (a.ns <= 3 ? 2 : 1);        // at least 4 wavefronts; 8 P rows per work-group
  const int threads = 64 * a.ns * a.p;
  a.nsel_wg = a.kout > 0 ? (a.nchunks + threads / 64 - 1) / (threads / 64) : 0;   // one chunk per wavefront
  // workspace: counters, then the tagged selection, then the status word
  a.calls = workspace;
  a.tags = reinterpret_cast<uint64_t*>(workspace + kWCallStride * kWCalls);
  a.status = workspace + kWCallStride * kWCalls + 2 * (int64_t)a.nchunks * a.kout + 1;   // the last word
  // the selecting work-groups are extra ones, dispatched first, while the
  // whole launch fits the device's resident work-groups; when it would not,
  // the first row work-groups select before taking their rows (one resident
  // wave: no work-group waits for another to leave)
  const int nb = g->m / (8 * a.p);
  const size_t lds = (size_t)g->k * sizeof(float);
  a.merged = (a.nsel_wg > 0 && a.nsel_wg <= nb && a.nsel_wg + nb > resident_wgs(g->base_bits, threads, lds)) ? 1 : 0;
  const dim3 grid((unsigned)(a.merged ? nb : a.nsel_wg + nb));
  hipStream_t st = (hipStream_t)stream;
  switch (g->base_bits) {
    case 2: hipLaunchKernelGGL(w_gemv<2>, grid, dim3(threads), lds, st, a); break;
    case 3: hipLaunchKernelGGL(w_gemv<3>, grid, dim3(threads), lds, st, a); break;
    default: hipLaunchKernelGGL(w_gemv<4>, grid, dim3(threads), lds, st, a); break;
  }
  SF_LAUNCH_CHECK("w_gemv");
  return SF_OK;
}

// The decode step of one layer in a single launch (2-bit base codes, GQA
// groups of 1, 2 or 4 query heads).
//
// Method: page "StrataFlux -- Selective precision streaming -- What does it
// mean?".  Paragraph "Which tiles count ...": every cached token is scored
// from the resident low-bit keys, the highest-scoring tokens of each KV head
// are refined, everything else takes part at low precision.  Paragraph "What
// travels over the link ...": r refinement bits subdivide the bin the base
// code names.  Paragraph "Where it earns its keep ...": which tokens to refine
// depends on the scores themselves, so the refinement cannot be overlapped
// with the attention around it.
//
// The launch is one wave of work-groups that are all resident at once (the
// host checks the device's capacity).  Work-group (range j, KV head k) of
// sequence s owns tokens [j R, j R + R) of that head, R <= 4096:
//   A  stream the range's K codes once (LDS ring of direct loads), compute
//      the G per-head logits on the matrix cores and keep them in LDS
//      (16 KiB per 1,024 tokens at G = 4), histogram the score keys' top 12
//      bits, add the histogram into the head's global one;
//   B  wait for the head's other work-groups (a counter in device memory),
//      find the boundary bin of the exact top-T from the global histogram:
//      tokens above it are selected, tokens below it are not, tokens in it
//      are candidates (all selected when the bin is taken whole);
//   B' candidates: every work-group writes their keys and token indices to
//      its slot of the head's list in device memory; after one more wait
//      each reads the whole list and takes the exact boundary key by a radix
//      select in LDS, ties to the lower token index (when a range overflows
//      its slot, the next 12 and the last 8 key bits settle them through
//      histograms in device memory, one wait per level);
//   C  11 wavefronts stream the range's V codes once: every token that is
//      not selected enters the online softmax at base precision (logits
//      from LDS, P.V on the matrix cores as in the two-pass form); beside
//      them 5 wavefronts take the selected tokens in batches of 16 (refined
//      logit and value from their refinement rows, on the vector units);
//   D  the wavefronts' partials merge into the range's partial (m, l,
//      acc[D]) per query head, written to device memory;
//   E  the last work-group of the head to finish merges the partials into
//      the output, lists the selection when asked, and clears the head's
//      histograms and counters for the next step.
// Every term of the softmax is positive: each token enters exactly once,
// with its final logit and value.  K and V are read once; the logits never
// leave the compute unit.
//
// Coherence between work-groups without cache write-backs: everything one
// work-group hands to another is written with device-scope stores or
// atomics (they bypass the non-coherent L2), each wavefront waits for its
// stores before the work-group arrives at a counter, and readers use
// device-scope loads (which miss the L2) once the counter is complete.
// Waits are bounded: a wait that expires (the work-groups were not all
// resident) sets the status word (sf_decode_check reports it) and ends the
// work-group.
#include "sf_mfma_common.h"

namespace sfk {

constexpr int kFW = 16;          // wavefronts per work-group
constexpr int kFVW = 11;         // of them streaming V in phase C,
constexpr int kFSW = kFW - kFVW; // and refining the selected tokens beside them (5 x 16 tokens
                                 // a round: a 4,096-token range's share of a 2,048-token
                                 // selection of 128K, 64 +- 8, in one round)
constexpr int kFRing = 3;        // phase A: ring stages per wavefront (2 chunks in flight)
constexpr int kFRingV = kFW * kFRing / kFVW;   // phase C: 4 stages per streaming wavefront (44 of the 48)
constexpr int kFTPW = 16;        // selected tokens per batch of a refining wavefront (4 lanes each)
static_assert(kFRingV * kFVW <= kFW * kFRing, "phase C's ring lies in phase A's");
constexpr int kFSpinLimit = 1 << 18;   // bounded waits: about 0.2 s
static_assert(2 * kFusedMaxRanges + kHeadDim <= kFW * kHeadDim, "merge arrays fit in the wave partials");

struct FStage {
  uint8_t c[32 * 32];            // codes of one 32-token chunk, as stored
  float2 s[32];                  // its (lo, delta)
};

template <int G>
struct FSpec {                   // the refining wavefronts' staging (in the histogram's place)
  uint32_t vt[kFSW][kFTPW][9];   // V base codes (2 bits: 8 words + a zero word)
  uint32_t vr[kFSW][kFTPW][33];  // V refinement rows (r <= 8: 32 words + a zero word)
  float2 vsc[kFSW][kFTPW];       // V (lo, delta)
  float wt[kFSW][G][kFTPW];
};

template <int G>
struct FusedLds {
  float lg[kFusedRmax * G];                  // per-head logits, log2 units, [token][head]
  union {
    struct {
      FStage ring[kFW * kFRing];             // A: [wave][kFRing]; C: [streaming wave][kFRingV]
      union {
        uint32_t hist[kHistBins];            // level 1 of the selection
        FSpec<G> sp;                         // C: the selected tokens' staging
      } h;
    } st;
    float acc[kFW][G][kHeadDim];             // per-wave partials (after C)
  } u;
  float qs[G][kHeadDim];                     // the query (C)
  QPrep qp;
  alignas(16) _Float16 wt[kFW][2 * G][32];   // P.V weights of the stream: hi parts, then lo parts
  alignas(16) _Float16 wzero[8];
  uint32_t sel[kFusedRmax / 32];             // selected (at level 1, then settled by the later levels)
  uint32_t cand[kFusedRmax / 32];            // in the level-1 boundary bin, left to the later levels
  uint32_t csel[kFusedRmax / 32];            // candidates the histogram levels selected
  uint16_t pre1[kFusedRmax / 32 + 1];        // selected tokens before each word
  uint32_t lcnt[kFListRanges];               // candidates of each range of the head
  float mw[kFW][G], lw[kFW][G];              // per-wave partials: maxima (log2 units), sums
  float mstar[G];                            // E: each head's denominator
  uint32_t scan[kFW];
  int sh_bin;
  uint32_t sh_need, sh_flag;
  uint32_t shist[256];                       // radix histogram of the candidates' keys
  uint32_t sh_cnt, n1;                       // boundary key's count; selected tokens of the range
  uint32_t used3;                            // level 3 taken
};

__device__ inline uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float ld_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Device-scope (sc1) loads through a buffer resource: coherent across the
// XCDs' caches like the atomic loads above, but plain loads to the compiler,
// so that many can be in flight at once.
__device__ inline uint4 ld_dev4(rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 16));
}
__device__ inline float ld_devf(rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_off, 0, 16));
}
// Copy n words (n a multiple of 4, 4 n <= 16 * blockDim) of device memory into LDS.
__device__ inline void copy_dev_words(uint32_t* lds, const uint32_t* g, int n) {
  const rsrc_t r = make_rsrc(g, (uint32_t)n * 4u);
  if ((int)threadIdx.x < n / 4) reinterpret_cast<uint4*>(lds)[threadIdx.x] = ld_dev4(r, 16u * threadIdx.x);
}

__device__ inline void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Arrive at `ctr` and wait until `expected` work-groups have.  Every wave has
// its device-scope stores and atomics complete before the work-group arrives.
// Returns false (status word set) when the wait expired.
template <int G>
__device__ inline bool group_wait(FusedLds<G>& s, uint32_t* ctr, uint32_t expected, uint32_t* status) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    atomicAdd(ctr, 1u);
    uint32_t ok = 1u;
    int spins = 0;
    while (ld_dev(ctr) < expected) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kFSpinLimit) {
        atomicOr(status, 1u);
        ok = 0u;
        break;
      }
    }
    s.sh_flag = ok;
  }
  __syncthreads();
  return s.sh_flag != 0u;
}

// Key of a token's score from its logits in LDS: the same fp32 operations as
// the score computation of phase A (maximum over the group, times ln 2).
template <int G>
__device__ inline uint32_t token_key(const float* lg, int t) {
  float y = lg[t * G];
#pragma unroll
  for (int h = 1; h < G; ++h) y = fmaxf(y, lg[t * G + h]);
  return score_key(y * 0.6931471805599453f);
}

// Reads of one V stage: the two tokens' logits (dynamic LDS addresses), the
// scales and the V dwords at the stage's offset OFF (immediates).
template <int OFF>
__device__ inline void read_vstage(uint32_t aL0, uint32_t aL1, uint32_t aS, const uint32_t (&aV)[4], float (&lgv)[2],
                                   uint64_t (&vsc)[2], uint32_t (&vw)[8]) {
  asm volatile(
      "ds_read_b32 %0, %12\n\t"
      "ds_read_b32 %1, %13\n\t"
      "ds_read_b64 %2, %14 offset:%19\n\t"
      "ds_read_b64 %3, %14 offset:%20\n\t"
      "ds_read_b32 %4, %15 offset:%19\n\t"
      "ds_read_b32 %5, %15 offset:%21\n\t"
      "ds_read_b32 %6, %16 offset:%19\n\t"
      "ds_read_b32 %7, %16 offset:%21\n\t"
      "ds_read_b32 %8, %17 offset:%19\n\t"
      "ds_read_b32 %9, %17 offset:%21\n\t"
      "ds_read_b32 %10, %18 offset:%19\n\t"
      "ds_read_b32 %11, %18 offset:%21\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(lgv[0]), "=&v"(lgv[1]), "=&v"(vsc[0]), "=&v"(vsc[1]), "=&v"(vw[0]), "=&v"(vw[1]), "=&v"(vw[2]),
        "=&v"(vw[3]), "=&v"(vw[4]), "=&v"(vw[5]), "=&v"(vw[6]), "=&v"(vw[7])
      : "v"(aL0), "v"(aL1), "v"(aS), "v"(aV[0]), "v"(aV[1]), "v"(aV[2]), "v"(aV[3]), "n"(OFF), "n"(OFF + 128),
        "n"(OFF + 512)
      : "memory");
}

// Arrive at `ctr` and wait until `expected` work-groups have, for one
// wavefront alone (wavefront 0 in the histogram levels, the others wait at
// the work-group's barrier): its device-scope stores and atomics complete
// first.  Returns false (status word set) when the wait
// expired.
__device__ inline bool wave_group_wait(uint32_t* ctr, uint32_t expected, uint32_t* status) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  uint32_t ok = 1u;
  if ((threadIdx.x & 63) == 0) {
    atomicAdd(ctr, 1u);
    int spins = 0;
    while (ld_dev(ctr) < expected) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kFSpinLimit) {
        atomicOr(status, 1u);
        ok = 0u;
        break;
      }
    }
  }
  return __builtin_amdgcn_readfirstlane(ok) != 0u;
}

// The boundary bin of a histogram of NB bins in device memory, counted from
// the top bin down, by one wavefront: bin b with count(bins > b) < need <=
// count(bins >= b), the number still needed inside b, and b's count (every
// lane receives them).  Lane l first sums bins [NB - PER (l + 1), NB - PER l)
// (device-scope loads); the lane whose range holds the boundary is found
// from the prefix over lanes, then its PER bins are loaded one per lane.
// Needs 1 <= need <= the histogram's total.
template <int NB>
__device__ inline void find_threshold_dev(const uint32_t* hist, uint32_t need, int& bin, uint32_t& need_out,
                                          uint32_t& count) {
  static_assert(NB % 256 == 0 && NB <= 4096, "PER = NB / 64 bins per lane, a multiple of 4");
  constexpr int PER = NB / 64, Q = PER / 4;
  const int lane = threadIdx.x & 63;
  const rsrc_t r = make_rsrc(hist, NB * 4u);
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < Q; ++i) {
    const uint4 x = ld_dev4(r, 4u * (uint32_t)(NB - PER * (lane + 1)) + 16u * i);
    sum += x.x + x.y + x.z + x.w;
  }
  const uint32_t inc = wave_inclusive_scan(sum);
  const uint64_t hit = __ballot(inc - sum < need && need <= inc);
  const int L = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)hit) - 1);
  const uint32_t above = __builtin_amdgcn_readlane(inc - sum, L);
  // lane j takes bin NB - PER L - 1 - j
  const uint32_t c = lane < PER ? __builtin_bit_cast(uint32_t, ld_devf(r, 4u * (uint32_t)(NB - PER * L - 1 - lane))) : 0u;
  const uint32_t cum = wave_inclusive_scan(c);
  const uint64_t hit2 = __ballot(lane < PER && above + cum >= need);
  const int j = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)hit2) - 1);
  bin = NB - PER * L - 1 - j;
  count = __builtin_amdgcn_readlane(c, j);
  need_out = need - above - __builtin_amdgcn_readlane(cum - c, j);
}

// Boundary bin of an LDS histogram of NB bins (16 or 256) by one
// wavefront, from the top bin down: the bin d with count(bins > d) < need <=
// count(bins >= d), count(bins > d) and d's count (uniform).
template <int NB>
__device__ inline void wave_boundary(const uint32_t* h, uint32_t need, int& d, uint32_t& above, uint32_t& cnt) {
  constexpr int PER = NB >= 64 ? NB / 64 : 1, LANES = NB / PER;
  const int lane = threadIdx.x & 63;
  uint32_t v[PER], sum = 0u;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    v[i] = lane < LANES ? h[NB - PER * (lane + 1) + i] : 0u;
    sum += v[i];
  }
  const uint32_t inc = wave_inclusive_scan(sum);
  const uint64_t hit = __ballot(inc - sum < need && need <= inc);
  const int L = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)hit) - 1);
  uint32_t cum = __builtin_amdgcn_readlane(inc - sum, L);
  d = -1;
  above = cnt = 0u;
#pragma unroll
  for (int i = PER - 1; i >= 0; --i) {
    const uint32_t b = __builtin_amdgcn_readlane(v[i], L);
    if (d < 0 && cum + b >= need) {
      d = NB - PER * (L + 1) + i;
      above = cum;
      cnt = b;
    }
    cum += b;
  }
}

// Levels 2 and 3 of the selection and the index ties through the head's
// histograms in device memory, by wavefront 0: the fallback when a range
// has more level-1 candidates than its slot of the list.  The level-2
// histogram is complete (every work-group added its candidates before the
// wait at Z[kFZC + 1]).
template <int G>
__device__ inline void select_by_histograms(const DecodeParams& p, FusedLds<G>& s, uint32_t* Z, const uint32_t (&cw)[2],
                                            uint32_t (&selw)[2], uint32_t nwg, uint32_t need1, int64_t sk, int wi) {
  const int lane = threadIdx.x & 63;
  uint32_t next[2] = {0u, 0u};
  int b2;
  uint32_t need2, cnt2;
  find_threshold_dev<kHistBins>(&Z[kFZH2], need1, b2, need2, cnt2);
  const bool lvl3 = cnt2 != need2;
#pragma unroll
  for (int k = 0; k < 2; ++k)
    for (uint32_t bits = cw[k]; bits; bits &= bits - 1u) {
      const int bit = __ffs(bits) - 1;
      const uint32_t key = token_key<G>(s.lg, 32 * (64 * k + lane) + bit);
      const int mid = (int)((key >> 8) & 0xFFFu);
      if (mid > b2 || (mid == b2 && !lvl3)) {
        selw[k] |= 1u << bit;
      } else if (mid == b2) {
        next[k] |= 1u << bit;
        atomicAdd(&Z[kFZH3 + (key & 0xFFu)], 1u);
      }
    }
  if (!lvl3) return;
  if (lane == 0) s.used3 = 1u;
  if (!wave_group_wait(&Z[kFZC + 2], nwg, p.fstatus)) return;
  int b3;
  uint32_t need3, cnt3;
  find_threshold_dev<256>(&Z[kFZH3], need2, b3, need3, cnt3);
  const bool lvl4 = cnt3 != need3;
  uint32_t ties[2] = {0u, 0u};
#pragma unroll
  for (int k = 0; k < 2; ++k)
    for (uint32_t bits = next[k]; bits; bits &= bits - 1u) {
      const int bit = __ffs(bits) - 1;
      const int low = (int)(token_key<G>(s.lg, 32 * (64 * k + lane) + bit) & 0xFFu);
      if (low > b3 || (low == b3 && !lvl4))
        selw[k] |= 1u << bit;
      else if (low == b3)
        ties[k] |= 1u << bit;
    }
  if (!lvl4) return;
  // rank of each tie in the range (words in token order: lane, then 64 +
  // lane), the range's count to the head, then the ties of the head's
  // ranges before this one
  const uint32_t c0 = (uint32_t)__popc(ties[0]), c1 = (uint32_t)__popc(ties[1]);
  const uint32_t i0 = wave_inclusive_scan(c0), i1 = wave_inclusive_scan(c1);
  const uint32_t t0 = __builtin_amdgcn_readlane(i0, 63);
  const uint32_t mine = t0 + __builtin_amdgcn_readlane(i1, 63);
  uint32_t rank[2] = {i0 - c0, t0 + i1 - c1};
  if (lane == 0) st_dev(&p.ftie[sk * p.ftie_stride + wi], mine);
  if (!wave_group_wait(&Z[kFZC + 3], nwg, p.fstatus)) return;
  uint32_t before = 0u;
  for (int w = lane; w < wi; w += 64) before += ld_dev(&p.ftie[sk * p.ftie_stride + w]);
  before = __builtin_amdgcn_readlane(wave_inclusive_scan(before), 63);
  const uint32_t take = need3 > before ? need3 - before : 0u;   // ties of this range still taken
#pragma unroll
  for (int k = 0; k < 2; ++k)
    for (uint32_t bits = ties[k]; bits; bits &= bits - 1u, ++rank[k])
      if (rank[k] < take) selw[k] |= 1u << (__ffs(bits) - 1);
}

// q . s over quarter qd of head_dim for each of the G heads, from the lane's
// R-bit refinement codes in registers: four codes at a time, each taken by
// every head (few registers live).
template <int R, int G, int N>
__device__ inline void quarter_qs(const uint32_t (&kr)[N], const float* qs, int qd, float (&ds)[G]) {
  static_assert(R <= N, "the codes fit the words");
#pragma unroll
  for (int h = 0; h < G; ++h) ds[h] = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float c0 = (float)code_at<R>(kr, 4 * i), c1 = (float)code_at<R>(kr, 4 * i + 1);
    const float c2 = (float)code_at<R>(kr, 4 * i + 2), c3 = (float)code_at<R>(kr, 4 * i + 3);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float4 v = reinterpret_cast<const float4*>(qs + h * kHeadDim + 32 * qd)[i];
      ds[h] = fmaf(v.x, c0, ds[h]);
      ds[h] = fmaf(v.y, c1, ds[h]);
      ds[h] = fmaf(v.z, c2, ds[h]);
      ds[h] = fmaf(v.w, c3, ds[h]);
    }
  }
}

// Rows of a batch of selected tokens held in registers between their fetch
// and their use: lane (tl, qd) holds quarter qd (elements 32 qd .. 32 qd +
// 31) of token tl.
template <int NWD = 8>
struct SelRows {
  uint32_t vb[2], kr[NWD], vr[NWD];   // V base codes, K and V refinement codes (r <= NWD words each)
  float2 vsc;                     // V (lo, delta)
  float kd;                       // K delta
  int off;                        // the token within the range
};

// Fetch the rows of the range's selected tokens j0 .. j0 + cnt - 1 (cnt <=
// kFTPW, in token order).
template <int G, int NWD>
__device__ inline void sel_fetch(const DecodeParams& p, const FusedLds<G>& s, uint32_t j0, int cnt, int kvh,
                                 int64_t row0, int nw, SelRows<NWD>& rw) {
  const int lane = threadIdx.x & 63, tl = lane >> 2, qd = lane & 3;
  const int r = p.r;
  rw.vb[0] = rw.vb[1] = 0u;
#pragma unroll
  for (int i = 0; i < NWD; ++i) rw.kr[i] = rw.vr[i] = 0u;
  rw.vsc = make_float2(0.f, 0.f);
  rw.kd = 0.f;
  rw.off = 0;
  if (tl >= cnt) return;
  // the word holding the j-th selected token (the first w with pre1[w + 1] >
  // j; pre1[nw] is the count), then its bit
  const uint32_t j = j0 + (uint32_t)tl;
  int lo_w = 0, hi_w = nw - 1;
  while (lo_w < hi_w) {
    const int mid = (lo_w + hi_w) >> 1;
    if (s.pre1[mid + 1] > j) hi_w = mid; else lo_w = mid + 1;
  }
  uint32_t bits = s.sel[lo_w];
  for (uint32_t k = s.pre1[lo_w]; k < j; ++k) bits &= bits - 1u;
  rw.off = 32 * lo_w + __ffs(bits) - 1;
  const int64_t row = row0 + rw.off;                     // kvh * cap + token
  const int64_t tok = row - (int64_t)kvh * p.cap;
  const uint32_t* srcv = reinterpret_cast<const uint32_t*>(p.vc + row * 32) + qd * 2;
  rw.vb[0] = srcv[0];
  rw.vb[1] = srcv[1];
  rw.vsc = reinterpret_cast<const float2*>(p.vs)[row];
  const uint32_t* rk = reinterpret_cast<const uint32_t*>(p.ref_rows + ((int64_t)kvh * p.cap + tok) * p.rb) + qd * r;
  const uint32_t* rv =
      reinterpret_cast<const uint32_t*>(p.ref_rows + (((int64_t)p.hkv + kvh) * p.cap + tok) * p.rb) + qd * r;
#pragma unroll
  for (int i = 0; i < NWD; ++i) {
    rw.kr[i] = i < r ? rk[i] : 0u;
    rw.vr[i] = i < r ? rv[i] : 0u;
  }
  rw.kd = reinterpret_cast<const float2*>(p.ks)[row].y;
}

// A fetched batch of cnt selected tokens enters refining wavefront w's online softmax
// (natural units) with refined keys and values: the refined logit from the
// base logit in LDS plus the refinement's change, the quarter dots summed
// over the token's four lanes; the V rows through the wave's staging to the
// P.V, where the lane holds output elements 2 lane and 2 lane + 1.
template <int G, int NWD>
__device__ inline void sel_compute(const DecodeParams& p, FusedLds<G>& s, int w, const SelRows<NWD>& rw, int cnt,
                                   const float (&qsum)[G], float (&m_run)[G], float (&l_run)[G],
                                   float (&acc)[G][2]) {
  static_assert(kFTPW * 4 == 64, "four lanes a token");
  FSpec<G>& sp = s.u.st.h.sp;
  const int lane = threadIdx.x & 63, tl = lane >> 2, qd = lane & 3;
  const int r = p.r;
  const float sub = __builtin_ldexpf(1.0f, -r);
  const bool valid = tl < cnt;
  // the V rows into the wave's staging first (zeros for a token past cnt)
  sp.vt[w][tl][2 * qd] = rw.vb[0];
  sp.vt[w][tl][2 * qd + 1] = rw.vb[1];
#pragma unroll
  for (int i = 0; i < NWD; ++i)
    if (i < r) sp.vr[w][tl][qd * r + i] = rw.vr[i];
  const bool lead = qd == 0;
  if (lead) {
    sp.vt[w][tl][8] = 0u;
    for (int i = 4 * r; i < 33; ++i) sp.vr[w][tl][i] = 0u;
    sp.vsc[w][tl] = rw.vsc;
  }
  float lgt[G];
#pragma unroll
  for (int h = 0; h < G; ++h) lgt[h] = valid ? s.lg[rw.off * G + h] : 0.f;
  float ds[G];
  switch (r) {
    case 1: quarter_qs<1, G>(rw.kr, &s.qs[0][0], qd, ds); break;
    case 2: quarter_qs<2, G>(rw.kr, &s.qs[0][0], qd, ds); break;
    case 3: quarter_qs<3, G>(rw.kr, &s.qs[0][0], qd, ds); break;
    case 4: quarter_qs<4, G>(rw.kr, &s.qs[0][0], qd, ds); break;
    default:
      if constexpr (NWD == 8) {
        switch (r) {
          case 5: quarter_qs<5, G>(rw.kr, &s.qs[0][0], qd, ds); break;
          case 6: quarter_qs<6, G>(rw.kr, &s.qs[0][0], qd, ds); break;
          case 7: quarter_qs<7, G>(rw.kr, &s.qs[0][0], qd, ds); break;
          default: quarter_qs<8, G>(rw.kr, &s.qs[0][0], qd, ds); break;
        }
      }
      break;
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    // refined - base = delta / sqrt(D) (2^-r q.s + (2^-r - 1) sum(q) / 2)
    const float lr =
        fmaf(lgt[h], 0.6931471805599453f, rw.kd * kRsqrtD * fmaf(sub, quad_sum(ds[h]), 0.5f * (sub - 1.0f) * qsum[h]));
    const float mwv = wave_max_dpp(valid ? lr : -INFINITY);
    const float mnew = fmaxf(m_run[h], mwv);
    const float alpha = __expf(m_run[h] - mnew);
    const float ew = valid ? __expf(lr - mnew) : 0.f;
    if (lead) sp.wt[w][h][tl] = ew;
    l_run[h] = fmaf(l_run[h], alpha, wave_sum_dpp(lead ? ew : 0.f));
    acc[h][0] *= alpha;
    acc[h][1] *= alpha;
    m_run[h] = mnew;
  }
  wave_barrier();
  // P.V: the reads of four tokens, then their products; value = lo + delta
  // (c + (s + 1/2) 2^-r)
  const int cpos = 4 * lane, cwi = cpos >> 5, csh = cpos & 31;
  const int rpos = 2 * lane * r, rwi = rpos >> 5, rsh = rpos & 31;
  const uint32_t rmask = (1u << r) - 1u;
  const float hsub = 0.5f * sub;
  constexpr int kPart = 4;
#pragma unroll 1
  for (int j1 = 0; j1 < kFTPW; j1 += kPart) {
    uint32_t cwd[kPart], rw0[kPart], rw1[kPart];
    float2 scv[kPart];
    float wv[kPart][G];
#pragma unroll
    for (int jj = 0; jj < kPart; ++jj) {
      cwd[jj] = sp.vt[w][j1 + jj][cwi];
      rw0[jj] = sp.vr[w][j1 + jj][rwi];
      rw1[jj] = sp.vr[w][j1 + jj][rwi + 1];
      scv[jj] = sp.vsc[w][j1 + jj];
#pragma unroll
      for (int h = 0; h < G; ++h) wv[jj][h] = sp.wt[w][h][j1 + jj];
    }
#pragma unroll
    for (int jj = 0; jj < kPart; ++jj) {
      const uint32_t cc = cwd[jj] >> csh;
      const uint32_t rr = (uint32_t)((((uint64_t)rw1[jj] << 32) | rw0[jj]) >> rsh);
      const float c0 = (float)(cc & 3u), c1 = (float)((cc >> 2) & 3u);
      const float s0 = (float)(rr & rmask), s1 = (float)((rr >> r) & rmask);
      const float2 sc = scv[jj];
      const float v0 = fmaf(fmaf(s0, sub, hsub), sc.y, fmaf(c0, sc.y, sc.x));
      const float v1 = fmaf(fmaf(s1, sub, hsub), sc.y, fmaf(c1, sc.y, sc.x));
#pragma unroll
      for (int h = 0; h < G; ++h) {
        acc[h][0] = fmaf(wv[jj][h], v0, acc[h][0]);
        acc[h][1] = fmaf(wv[jj][h], v1, acc[h][1]);
      }
    }
  }
  wave_barrier();
}

template <int G, bool Batched>
__global__ void __launch_bounds__(64 * kFW) fused_decode(DecodeParams p) {
  __shared__ __align__(16) uint8_t fsmem[sizeof(FusedLds<G>)];
  FusedLds<G>& s = *reinterpret_cast<FusedLds<G>*>(fsmem);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kvh = blockIdx.y;
  int64_t lo, hi;
  int first;
  const int seq = locate_unit<Batched>(p, p.fr, blockIdx.x, false, lo, hi, first);
  const float2 qx = load_query<G>(p.q + ((int64_t)seq * p.hq + kvh * G) * kHeadDim);
  const int64_t a = seq_at(p, seq);
  const int64_t n_s = seq_at(p, seq + 1) - a;
  const int wi = blockIdx.x - first;                          // this work-group's place in the head
  const uint32_t nwg = (uint32_t)((n_s + p.fr - 1) / p.fr);  // work-groups of the head
  const int64_t sk = (int64_t)seq * p.hkv + kvh;
  uint32_t* Z = p.fz + sk * kFZWords;
  const int64_t t0 = (int64_t)kvh * p.cap + a + lo;           // first row of the range
  const int nsp = (int)(hi - lo);
  const int nchunks = (nsp + 31) / 32;
  const int nw = nchunks;                                     // selection words of the range
  const int nmine = nchunks > wid ? (nchunks - wid + kFW - 1) / kFW : 0;
  const int64_t tn = n_s < p.top_t ? n_s : (int64_t)p.top_t;
  const bool select = p.top_t > 0;
  const bool all = select && tn == n_s;                       // every token is selected
  const bool use_hist = select && !all;
  constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;

  // ---- A: K once; logits into LDS; histogram of the score keys -------------
  const rsrc_t rK = make_rsrc(p.kc + t0 * 32, (uint32_t)nsp * 32u);
  const rsrc_t rKS = make_rsrc(p.ks + t0 * 2, (uint32_t)nsp * 8u);
  const uint32_t oK = 16u * (uint32_t)lane, oS = 4u * (uint32_t)lane;
  auto issueK = [&](int i, FStage& st) {
    const uint32_t c = (uint32_t)(wid + kFW * i);
    bdma16(rK, oK, c * 1024u, st.c);
    bdma4(rKS, oS, c * 256u, st.s);
  };
  for (int i = tid; i < kHistBins; i += 64 * kFW) s.u.st.h.hist[i] = 0u;
#pragma unroll
  for (int k = 0; k < kFRing - 1; ++k)
    if (k < nmine) issueK(k, s.u.st.ring[wid * kFRing + k]);
  v4i a0, a1;
  prep_query<G>(qx, s.qp, a0, a1);
  // the query in fp32 for the refining wavefronts of C (wave h < G holds
  // head h's elements 2 lane, 2 lane + 1), staged now rather than loaded
  // again between the selection and the V stream
  if (wid < G) *reinterpret_cast<float2*>(&s.qs[wid][2 * lane]) = qx;
  {
    const int t = lane & 15, hl = lane >> 4;
    const float scale = s.qp.scale[hl < G ? hl : 0] * (kRsqrtD * kLog2e);
    const float sumq = s.qp.sumq[hl < G ? hl : 0] * (kRsqrtD * kLog2e);
    float* scores = p.scores + (int64_t)kvh * p.ntot + (a - p.off0) + lo;
    const uint32_t ring0 = lds_addr(&s.u.st.ring[wid * kFRing]);
    const uint32_t aK = ring0 + (uint32_t)(t * 32 + 8 * hl);
    const uint32_t aS = ring0 + (uint32_t)(offsetof(FStage, s) + 8 * t);
    const int hx = hl >> 1;
    const uint32_t hist0 = lds_addr(&s.u.st.h.hist[0]);
    const uint32_t lg0 = lds_addr(&s.lg[0]);
    auto body = [&](auto kc, int i) {
      constexpr int k = decltype(kc)::value;
      constexpr int OFF = k * (int)sizeof(FStage);
      if (i + kFRing - 1 < nmine) issueK(i + kFRing - 1, s.u.st.ring[wid * kFRing + (k + kFRing - 1) % kFRing]);
      wait_stages<2, kFRing - 1>(min(kFRing - 1, nmine - 1 - i));
      const int c = wid + kFW * i;
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
      const bool full = 32 * c + 32 <= nsp;
      float lgv[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint2 w = __builtin_bit_cast(uint2, kw[j]);
        v4i b0, b1;
        decode_b2(w.x, w.y, b0, b1);
        v4i D = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, v4i{0, 0, 0, 0}, 0, 0, 0);
        D = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, D, 0, 0, 0);
        const float x = logit_scaled(D, __builtin_bit_cast(float2, ks[j]), scale, sumq);
        lgv[j] = hl < G ? x : -INFINITY;
        const int rel = 32 * c + 16 * j + t;
        if (hl < G && (full || rel < nsp)) lds_write_u32(lg0 + 4u * (uint32_t)(rel * G + hl), __float_as_uint(x));
      }
      const float y = max_two_tiles(lgv[0], lgv[1]);
      const int rel = 32 * c + 16 * hx + t;
      if ((hl & 1) == 0 && (full || rel < nsp)) {
        const float sc = y * kLn2;
        if (p.fscores) store_through(&scores[rel], sc);
        if (use_hist) lds_add_u32(hist0 + 4u * (score_key(sc) >> (32 - kHistBits)), 1u);
      }
    };
    for (int i = 0; i < nmine; i += kFRing) {
      progress_priority(nmine - i, nmine);
      ring_round<kFRing>(body, i, nmine);
    }
    __builtin_amdgcn_s_setprio(0);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  }
  __syncthreads();

  // ---- B: level 1 of the exact top-T of the head ---------------------------
  uint32_t* hist = s.u.st.h.hist;
  bool lvl2 = false;   // the level-1 boundary bin is split (the later levels run)
  uint32_t b1 = 0u, need1 = 0u;   // the boundary bin and the count still needed there
  for (int w = tid; w < kFusedRmax / 32; w += 64 * kFW) s.sel[w] = s.cand[w] = s.csel[w] = 0u;
  __syncthreads();
  if (all) {
    for (int w = tid; w < nw; w += 64 * kFW) {
      const int rem = nsp - 32 * w;
      s.sel[w] = rem >= 32 ? ~0u : (1u << rem) - 1u;
    }
  } else if (use_hist) {
    for (int i = tid; i < kHistBins; i += 64 * kFW) {
      const uint32_t c = hist[i];
      if (c) atomicAdd(&Z[kFZH1 + i], c);
    }
    if (!group_wait(s, &Z[kFZC + 0], nwg, p.fstatus)) return;
    copy_dev_words(hist, &Z[kFZH1], kHistBins);
    __syncthreads();
    find_threshold_wave<kHistBins>(hist, (uint32_t)tn, &s.sh_bin, &s.sh_need);
    b1 = (uint32_t)s.sh_bin;
    need1 = s.sh_need;
    lvl2 = hist[b1] != need1;
    // above b1 selected, in b1 candidates (all selected when b1 is taken
    // whole), below b1 not selected
    for (int base = 0; base < nsp; base += 64 * kFW) {
      const int t = base + tid;
      bool above = false, in = false;
      if (t < nsp) {
        const uint32_t bin = token_key<G>(s.lg, t) >> (32 - kHistBits);
        above = bin > b1;
        in = bin == b1;
      }
      const uint64_t bs = __ballot(above || (in && !lvl2)), bc = __ballot(in && lvl2);
      if (lane == 0) {
        const int w = (base + 64 * wid) >> 5;
        if (w < kFusedRmax / 32) {
          s.sel[w] = (uint32_t)bs;
          s.cand[w] = (uint32_t)bc;
          s.sel[w + 1] = (uint32_t)(bs >> 32);
          s.cand[w + 1] = (uint32_t)(bc >> 32);
        }
      }
    }
  }
  __syncthreads();

  // ---- B': the later levels, when level 1 leaves its boundary bin split ---
  // Every work-group adds its candidates to the head's level-2 histogram (the
  // next 12 key bits) and writes their keys and token indices to its slot of
  // the head's list, with its count.  After one wait, when every range
  // fitted its slot (the head has at most kFListRanges ranges), each
  // work-group reads the whole list (4 entries a thread, into registers) and
  // takes the exact need1-th largest key by a radix select (digits of 8, 8
  // and 4 bits below the level-1 bin's 12, counted in LDS): keys above it
  // are selected, and of the keys equal to it the lowest token indices fill
  // what is still needed.  Otherwise the histograms settle it, one more wait
  // per level (select_by_histograms, by wavefront 0).
  if (tid == 0) s.used3 = 0u;
  if (lvl2) {
    const bool listed = nwg <= (uint32_t)kFListRanges;
    const uint32_t slot = listed ? (uint32_t)(kFListMax / nwg) & ~63u : 0u;   // a multiple of 64
    uint32_t* keys = Z + kFZL;
    uint32_t* toks = keys + kFListMax;
    uint32_t* counts = toks + kFListMax;
    {
      const uint32_t cw = tid < nw ? s.cand[tid] : 0u;
      uint32_t total;
      uint32_t pos = block_exclusive_scan<64 * kFW>((uint32_t)__popc(cw), s.scan, total);
      for (uint32_t bits = cw; bits; bits &= bits - 1u, ++pos) {
        const int t = 32 * tid + __ffs(bits) - 1;
        const uint32_t key = token_key<G>(s.lg, t);
        atomicAdd(&Z[kFZH2 + ((key >> 8) & 0xFFFu)], 1u);
        if (pos < slot) {
          st_dev(&keys[(uint32_t)wi * slot + pos], key);
          st_dev(&toks[(uint32_t)wi * slot + pos], (uint32_t)(lo + t));
        }
      }
      if (listed && tid == 0) st_dev(&counts[wi], total);
    }
    if (!group_wait(s, &Z[kFZC + 1], nwg, p.fstatus)) return;
    // the counts and the list's keys in one round of loads; entry e = tid +
    // 1024 i is position e % slot of range e / slot
    constexpr int KPT = kFListMax / (64 * kFW);
    uint32_t kk[KPT];
    if (listed) {
      const rsrc_t rk = make_rsrc(keys, (uint32_t)kFListMax * 4u);
#pragma unroll
      for (int i = 0; i < KPT; ++i) kk[i] = __builtin_bit_cast(uint32_t, ld_devf(rk, 4u * (uint32_t)(tid + 64 * kFW * i)));
      if (tid < (int)nwg) s.lcnt[tid] = ld_dev(&counts[tid]);
    }
    if (tid == 0) s.sh_flag = listed ? 1u : 0u;
    __syncthreads();
    if (tid < (int)nwg && listed && s.lcnt[tid] > slot) s.sh_flag = 0u;
    __syncthreads();
    if (s.sh_flag) {
      // key 0 marks an empty entry: no candidate has it (the level-1 bin's
      // 12 bits are those of a real score)
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const uint32_t e = (uint32_t)(tid + 64 * kFW * i), rg2 = e / slot;
        if (rg2 >= nwg || e % slot >= s.lcnt[rg2]) kk[i] = 0u;
      }
      // after each digit: keys above the boundary digit are selected; when
      // its bin is taken whole the keys from hval up are (no ties), else
      // the next digit splits it
      uint32_t hval = b1 << (32 - kHistBits), hmask = ~0u << (32 - kHistBits), need = need1, cnt = 0u;
      bool whole = false;
#pragma unroll
      for (int pass = 0; pass < 3; ++pass) {
        if (whole) break;
        const int shift = pass == 0 ? 12 : pass == 1 ? 4 : 0;
        const uint32_t dmask = pass == 2 ? 0xFu : 0xFFu;
        if (tid < 256) s.shist[tid] = 0u;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < KPT; ++i)
          if (kk[i] != 0u && (kk[i] & hmask) == hval) atomicAdd(&s.shist[(kk[i] >> shift) & dmask], 1u);
        __syncthreads();
        if (wid == 0) {
          int d;
          uint32_t above, c;
          if (pass == 2)
            wave_boundary<16>(s.shist, need, d, above, c);
          else
            wave_boundary<256>(s.shist, need, d, above, c);
          if (lane == 0) {
            s.sh_bin = d;
            s.sh_need = need - above;
            s.sh_cnt = c;
          }
        }
        __syncthreads();
        need = s.sh_need;
        cnt = s.sh_cnt;
        hval |= (uint32_t)s.sh_bin << shift;
        hmask |= dmask << shift;
        whole = need == cnt;
      }
      // whole: every key >= hval selected (hval's lower bits are zero); else
      // keys above hval selected, `need` of the `cnt` keys equal to it taken
      const uint32_t thr = hval, take = need;
      uint32_t selw = 0u, tw = 0u;
      if (tid < nw)
        for (uint32_t bits = s.cand[tid]; bits; bits &= bits - 1u) {
          const int bit = __ffs(bits) - 1;
          const uint32_t key = token_key<G>(s.lg, 32 * tid + bit);
          if (whole ? key >= thr : key > thr)
            selw |= 1u << bit;
          else if (key == thr)
            tw |= 1u << bit;
        }
      if (!whole) {
        // equal keys: the head's tied tokens before this range, then this
        // range's ties in token order
        const rsrc_t rt = make_rsrc(toks, (uint32_t)kFListMax * 4u);
        uint32_t bf = 0u;
#pragma unroll
        for (int i = 0; i < KPT; ++i)
          if (kk[i] == thr)
            bf += __builtin_bit_cast(uint32_t, ld_devf(rt, 4u * (uint32_t)(tid + 64 * kFW * i))) < (uint32_t)lo ? 1u : 0u;
        uint32_t before, ntie;
        (void)block_exclusive_scan<64 * kFW>(bf, s.scan, before);
        uint32_t rank = block_exclusive_scan<64 * kFW>((uint32_t)__popc(tw), s.scan, ntie) + before;
        for (uint32_t bits = tw; bits; bits &= bits - 1u, ++rank)
          if (rank < take) selw |= 1u << (__ffs(bits) - 1);
      }
      if (tid < nw) s.sel[tid] |= selw;
    } else {
      if (wid == 0) {
        uint32_t cw[2], selw[2] = {0u, 0u};
#pragma unroll
        for (int k = 0; k < 2; ++k) cw[k] = 64 * k + lane < nw ? s.cand[64 * k + lane] : 0u;
        select_by_histograms<G>(p, s, Z, cw, selw, nwg, need1, sk, wi);
#pragma unroll
        for (int k = 0; k < 2; ++k)
          if (64 * k + lane < nw) s.csel[64 * k + lane] = selw[k];
      }
      __syncthreads();
      if (tid < nw) s.sel[tid] |= s.csel[tid];
    }
    __syncthreads();
  }
  if (select && p.fsel && tid < nw) st_dev(&p.bitmap[sk * p.bm_words + (lo >> 5) + tid], s.sel[tid]);

  // ---- C: V once (kFVW wavefronts), the selected tokens beside it (kFSW) ----
  // the streaming wavefronts take every token that is not selected; the
  // selected tokens go to the refining wavefronts in batches of kFTPW,
  // round-robin (fixed, so that the sums do not depend on timing), each
  // fetching its first batch's rows before the stream starts (they lead the
  // memory queue), at top issue priority (they are few and latency-bound)
  const bool masked = select && p.use_refine != 0;
  if (masked) {
    uint32_t total;
    const uint32_t pos = block_exclusive_scan<64 * kFW>(tid < nw ? (uint32_t)__popc(s.sel[tid]) : 0u, s.scan, total);
    if (tid < nw) s.pre1[tid] = (uint16_t)pos;
    if (tid == 0) {
      s.pre1[nw] = (uint16_t)total;
      s.n1 = total;
    }
  } else if (tid == 0) {
    s.n1 = 0u;
  }
  if (wid < kFVW)
    for (int i = lane; i < 2 * G * 32; i += 64) (&s.wt[wid][0][0])[i] = (_Float16)0.f;
  if (tid < 8) s.wzero[tid] = (_Float16)0.f;
  __syncthreads();
  const int t = lane & 15, hl = lane >> 4;        // logit layout: token t (and 16 + t), head hl
  const int n = lane & 15, rg = lane >> 4;        // P.V layout: column n, k-group rg
  // each wave's partial, kept in registers until the ring is free: a
  // streaming wave's P.V (lanes n in [G, 2G)), maximum and sum; a refining
  // wave's running softmax
  float out[8][4];
  float mx = -INFINITY, ls = 0.f;
  float msn[G], lsn[G], accs[G][2];
  if (wid < kFVW) {
    const rsrc_t rV = make_rsrc(p.vc + t0 * 32, (uint32_t)nsp * 32u);
    const rsrc_t rVS = make_rsrc(p.vs + t0 * 2, (uint32_t)nsp * 8u);
    const int nv = nchunks > wid ? (nchunks - wid + kFVW - 1) / kFVW : 0;   // chunks wid, wid + kFVW, ...
    // half L&1 of V row (L/2) ^ ((L/8) & 3): the four rows one P.V read
    // takes fall in different LDS banks
    const uint32_t oV = (uint32_t)(((lane >> 1) ^ ((lane >> 3) & 3)) * 32 + 16 * (lane & 1));
    FStage* ring = &s.u.st.ring[wid * kFRingV];
    auto issueV = [&](int i, FStage& st) {
      const uint32_t c = (uint32_t)(wid + kFVW * i);
      bdma16(rV, oV, c * 1024u, st.c);
      bdma4(rVS, oS, c * 256u, st.s);
    };
  #pragma unroll
    for (int k = 0; k < kFRingV - 1; ++k)
      if (k < nv) issueV(k, ring[k]);
    // the tokens the special wavefronts take: lane L holds words L and 64 + L
    const uint32_t sw0 = masked && lane < nw ? s.sel[lane] : 0u;
    const uint32_t sw1 = masked && 64 + lane < nw ? s.sel[64 + lane] : 0u;
    const int hlc = hl < G ? hl : 0;
    const uint32_t hsel = 2u * (uint32_t)(n & 1);
    const uint32_t psel = hsel | ((hsel + 1u) << 8) | ((hsel + 4u) << 16) | ((hsel + 5u) << 24);
    const int vdw = n >> 1;
    const uint32_t ring0 = lds_addr(ring);
    const uint32_t wtR = n < 2 * G ? lds_addr(&s.wt[wid][n][8 * rg]) : lds_addr(&s.wzero[0]);
    const uint32_t wtHi = lds_addr(&s.wt[wid][hlc][2 * t]), wtLo = lds_addr(&s.wt[wid][G + hlc][2 * t]);
    const uint32_t lgA = lds_addr(&s.lg[0]) + 4u * (uint32_t)(t * G + hlc);
    const uint32_t aS = ring0 + (uint32_t)(offsetof(FStage, s) + 8 * t);
    uint32_t aV[4];
  #pragma unroll
    for (int v = 0; v < 4; ++v) aV[v] = ring0 + (uint32_t)(offsetof(FStage, c) + (4 * rg + (v ^ rg)) * 32 + 4 * vdw);
    const uint64_t rows = G >= 4 ? ~0ull : (1ull << (16 * (G & 3))) - 1ull;
    const float ninf = -INFINITY;
    constexpr float kFloor = -1e30f;
    constexpr int kSlack = 6;
    float m = kFloor, lsum = 0.f, t1 = 0.f;
    int sexp = 127;
    float wsc = 1.0f;
    v4f acc[8];
  #pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
    auto body = [&](auto kc, int i) {
      constexpr int k = decltype(kc)::value;
      if (i + kFRingV - 1 < nv) issueV(i + kFRingV - 1, ring[(k + kFRingV - 1) % kFRingV]);
      wait_stages<2, kFRingV - 1>(min(kFRingV - 1, nv - 1 - i));
      const int c = wid + kFVW * i;
      const int rem = nsp - 32 * c;
      uint32_t vm = ~(uint32_t)__builtin_amdgcn_readlane((int)(c < 64 ? sw0 : sw1), c & 63);
      if (rem < 32) vm &= (1u << rem) - 1u;
      const uint32_t y0 = (vm & 0xFFFFu) | (vm << 16), y1 = (vm >> 16) | (vm & 0xFFFF0000u);
      const uint64_t mk[2] = {((uint64_t)y0 | ((uint64_t)y0 << 32)) & rows,
                              ((uint64_t)y1 | ((uint64_t)y1 << 32)) & rows};
      float lgr[2];
      uint64_t vsr[2];
      uint32_t vw[8];
      const uint32_t aL0 = lgA + 4u * (uint32_t)(32 * c * G), aL1 = aL0 + 4u * (uint32_t)(16 * G);
      read_vstage<k * (int)sizeof(FStage)>(aL0, aL1, aS, aV, lgr, vsr, vw);
      float lgx[2];
      float2 vsc[2];
  #pragma unroll
      for (int j = 0; j < 2; ++j) {
        lgx[j] = lane_select(mk[j], lgr[j], ninf);
        vsc[j] = __builtin_bit_cast(float2, vsr[j]);
      }
      // online softmax with a lazy reference: m moves (and the sums are
      // rescaled) only when a logit exceeds it by more than kSlack
      const float xm = fmaxf(lgx[0], lgx[1]);
      const bool grow = __ballot(xm > m + kSlack) != 0ull;
      const float mnew = grow ? fmaxf(m, row16_max_dpp(xm)) : m;
      float dmax = fmaxf(lane_select(mk[0], vsc[0].y, 0.f), lane_select(mk[1], vsc[1].y, 0.f));
      int need = sexp;
      if (__ballot(dmax > 0.f && (sexp == 127 || dmax >= __builtin_ldexpf(1.0f, 14 - kSlack - sexp))) != 0ull) {
        dmax = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_max(dmax))));
        int e2;
        frexpf(dmax, &e2);
        need = 14 - kSlack - e2;
      }
      if (grow || need < sexp) {
        const float alpha = mnew > m ? __builtin_amdgcn_exp2f(m - mnew) : 1.f;
        lsum *= alpha;
        t1 *= alpha;
        const int hc = n < 2 * G ? n % G : 0;
        float f = lane_value(alpha, 0);
  #pragma unroll
        for (int h = 1; h < G; ++h) {
          // read with every lane active (a lane read inside the selection
          // could run where lane 16 h is off)
          const float ah = lane_value(alpha, 16 * h);
          f = hc == h ? ah : f;
        }
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
        const float pk = __builtin_amdgcn_exp2f(lgx[j] - m);
        lsum += pk;
        t1 = fmaf(pk, fmaf(0.5f, vsc[j].y, vsc[j].x), t1);
        wv[j] = pk * (vsc[j].y * wsc);
      }
      const auto whi = __builtin_amdgcn_cvt_pkrtz(wv[0], wv[1]);
      const auto wlo = __builtin_amdgcn_cvt_pkrtz(wv[0] - (float)whi[0], wv[1] - (float)whi[1]);
      if (hl < G) {
        lds_write_u32(wtHi, __builtin_bit_cast(uint32_t, whi));
        lds_write_u32(wtLo, __builtin_bit_cast(uint32_t, wlo));
      }
      const v8h bw = lds_read_v8h(wtR);
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
    for (int i = 0; i < nv; i += kFRingV) {
      progress_priority(nv - i, nv);
      ring_round<kFRingV>(body, i, nv);
    }
    __builtin_amdgcn_s_setprio(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // the wave's row sums (l and the scalar term per head); lane n in
    // [G, 2G) holds head n - G's lo column, row_shr:G brings it the hi
    // column of lane n - G, and the scalar term goes with it
    lsum = row16_sum(lsum);
    t1 = row16_sum(t1);
    float t1h = 0.f;
  #pragma unroll
    for (int h = 0; h < G; ++h) {
      const float th = lane_value(t1, 16 * h);   // every lane active (see the rescale above)
      t1h = n - G == h ? th : t1h;
    }
    const int se = sexp == 127 ? 0 : sexp;
  #pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const float f = __builtin_ldexpf(1.0f, 24 - code_bit(tt) - se);
  #pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = acc[tt][j] * f;
        const float hi_part =
            __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + G, 0xF, 0xF, false));
        out[tt][j] = x + hi_part + t1h;
      }
    }
    mx = m == kFloor ? -INFINITY : m;
    ls = lsum;
  } else {
    const int sw = wid - kFVW;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      msn[h] = -1e30f;
      lsn[h] = 0.f;
      accs[h][0] = accs[h][1] = 0.f;
    }
    const uint32_t nsel = s.n1;
    if ((uint32_t)(kFTPW * sw) < nsel) {
      __builtin_amdgcn_s_setprio(3);
      constexpr uint32_t st = (uint32_t)(kFTPW * kFSW);
      auto cnt = [&](uint32_t j0) { return (int)min((uint32_t)kFTPW, nsel - j0); };
      float qsum[G];
#pragma unroll
      for (int h = 0; h < G; ++h) qsum[h] = wave_sum_dpp(s.qs[h][lane] + s.qs[h][64 + lane]);
      uint32_t j = (uint32_t)(kFTPW * sw);
      if (p.r <= 4) {
        // the wave's batches j, j + st, ... in turn, the rows of the next
        // batch fetched before the current one is computed (two sets of rows
        // in registers, r <= 4 words each), so that a wave with two batches
        // waits for one round of memory latency, not two
        SelRows<4> ra, rb;
        sel_fetch<G>(p, s, j, cnt(j), kvh, t0, nw, ra);
        if (j + st < nsel) sel_fetch<G>(p, s, j + st, cnt(j + st), kvh, t0, nw, rb);
        for (;;) {
          sel_compute<G>(p, s, sw, ra, cnt(j), qsum, msn, lsn, accs);
          if (j + 2 * st < nsel) sel_fetch<G>(p, s, j + 2 * st, cnt(j + 2 * st), kvh, t0, nw, ra);
          j += st;
          if (j >= nsel) break;
          sel_compute<G>(p, s, sw, rb, cnt(j), qsum, msn, lsn, accs);
          if (j + 2 * st < nsel) sel_fetch<G>(p, s, j + 2 * st, cnt(j + 2 * st), kvh, t0, nw, rb);
          j += st;
          if (j >= nsel) break;
        }
      } else {
        SelRows<8> rw;
        for (; j < nsel; j += st) {
          sel_fetch<G>(p, s, j, cnt(j), kvh, t0, nw, rw);
          sel_compute<G>(p, s, sw, rw, cnt(j), qsum, msn, lsn, accs);
        }
      }
      __builtin_amdgcn_s_setprio(0);
    }
  }
  __syncthreads();   // every wave is done with the ring and the staging
  if (wid < kFVW) {
    if (hl < G && t == 0) {
      s.mw[wid][hl] = mx;
      s.lw[wid][hl] = ls;
    }
    if (n >= G && n < 2 * G) {
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j) s.u.acc[wid][n - G][32 * rg + 8 * j + tt] = out[tt][j];
    }
  } else {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s.u.acc[wid][h][2 * lane] = accs[h][0];
      s.u.acc[wid][h][2 * lane + 1] = accs[h][1];
      if (lane == 0) {
        s.mw[wid][h] = lsn[h] > 0.f ? msn[h] * kLog2e : -INFINITY;   // log2 units, as the stream's
        s.lw[wid][h] = lsn[h];
      }
    }
  }
  __syncthreads();

  // ---- D: the range's partial: the waves' partials merged -------------------
  float* part = p.part + ((int64_t)kvh * gridDim.x + blockIdx.x) * G * kPartStride;
  for (int i = tid; i < G * kHeadDim; i += 64 * kFW) {
    const int h = i / kHeadDim, d = i % kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kFW; ++w) M = fmaxf(M, s.mw[w][h]);
    float A = 0.f, L = 0.f;
    if (M != -INFINITY) {
#pragma unroll 4
      for (int w = 0; w < kFW; ++w) {
        const float e = __builtin_amdgcn_exp2f(s.mw[w][h] - M);   // 0 for a wave without tokens
        A = fmaf(e, s.u.acc[w][h][d], A);
        L = fmaf(e, s.lw[w][h], L);
      }
    }
    st_dev(&part[h * kPartStride + d], A);
    if (d == 0) {
      st_dev(&part[h * kPartStride + kHeadDim], M);
      st_dev(&part[h * kPartStride + kHeadDim + 1], L);
    }
  }

  // ---- E: the head's last work-group merges -------------------------------
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) s.sh_flag = atomicAdd(&Z[kFZC + 4], 1u) == nwg - 1u ? 1u : 0u;
  __syncthreads();
  if (!s.sh_flag) return;
  // the head's partials in one round of loads: (m, l) of every range and
  // head into LDS by the first G nwg threads (the host keeps nwg <=
  // kFusedMaxRanges, which fits these arrays), and at the same time each
  // output element's accumulators by two threads, half the ranges each
  const float* part0 = p.part + ((int64_t)kvh * gridDim.x + first) * G * kPartStride;
  const rsrc_t rP = make_rsrc(part0, nwg * (uint32_t)(G * kPartStride * 4));
  float* mwg = reinterpret_cast<float*>(&s.u.acc[0][0][0]);   // [G][nwg] maxima, then weights
  float* lwg = mwg + G * nwg;                                   // [G][nwg] sums
  float* half = lwg + G * nwg;                                  // [G][kHeadDim] second halves
  for (int i = tid; i < G * (int)nwg; i += 64 * kFW) {
    const int h = i / nwg, w = i % nwg;
    const uint32_t o = (uint32_t)((w * G + h) * kPartStride + kHeadDim) * 4u;
    mwg[i] = ld_devf(rP, o);
    lwg[i] = ld_devf(rP, o + 4u);
  }
  const int io = tid % (G * kHeadDim), hlf = tid / (G * kHeadDim);   // G * kHeadDim <= 512 outputs
  const int ho = io / kHeadDim, dout = io % kHeadDim;
  const uint32_t w0 = hlf ? nwg / 2 : 0u, w1 = hlf ? nwg : nwg / 2;
  constexpr int kMaxHalf = kFusedMaxRanges / 2;
  float xa[kMaxHalf < 32 ? kMaxHalf : 32];
  const bool summer = tid < 2 * G * kHeadDim;
  // the first 32 ranges of the thread's half are loaded before the barrier
#pragma unroll
  for (int j = 0; j < 32; ++j)
    xa[j] = summer && w0 + j < w1 ? ld_devf(rP, (uint32_t)(((w0 + j) * G + ho) * kPartStride + dout) * 4u) : 0.f;
  __syncthreads();
  // wavefront h < G: head h's maximum over the ranges, each range's weight
  // 2^(m_w - m*) (in place of its maximum) and the denominator
  // sum_w weight_w l_w, as wavefront reductions
  if (wid < G) {
    float* mh = mwg + wid * nwg;
    const float* lh = lwg + wid * nwg;
    float M = -INFINITY;
    for (uint32_t w = (uint32_t)lane; w < nwg; w += 64) M = fmaxf(M, mh[w]);
    M = wave_max_dpp(M);
    float den = 0.f;
    for (uint32_t w = (uint32_t)lane; w < nwg; w += 64) {
      const float mv = mh[w];
      const float e = mv == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mv - M);
      mh[w] = e;
      den = fmaf(e, lh[w], den);
    }
    den = wave_sum_dpp(den);
    if (lane == 0) s.mstar[wid] = den;
  }
  __syncthreads();
  float num = 0.f;
  if (summer) {
#pragma unroll
    for (int j = 0; j < 32; ++j)
      if (w0 + j < w1) num = fmaf(mwg[ho * nwg + w0 + j], xa[j], num);
    for (uint32_t w = w0 + 32; w < w1; ++w)
      num = fmaf(mwg[ho * nwg + w], ld_devf(rP, (uint32_t)((w * G + ho) * kPartStride + dout) * 4u), num);
    if (hlf) half[io] = num;
  }
  __syncthreads();
  if (tid < G * kHeadDim) p.out[((int64_t)seq * p.hq + kvh * G + ho) * kHeadDim + dout] = (num + half[io]) / s.mstar[ho];
  if (select && p.fsel) {
    // the selection, ascending, from the ranges' words
    const uint32_t* bm = p.bitmap + sk * p.bm_words;
    const int64_t nwh = (n_s + 31) >> 5;
    const int64_t per = (nwh + 64 * kFW - 1) / (64 * kFW);
    const int64_t ww0 = tid * per < nwh ? tid * per : nwh, ww1 = ww0 + per < nwh ? ww0 + per : nwh;
    uint32_t cnt = 0;
    for (int64_t w = ww0; w < ww1; ++w) cnt += __popc(ld_dev(&bm[w]));
    uint32_t tot;
    uint32_t pos = block_exclusive_scan<64 * kFW>(cnt, s.scan, tot);
    int32_t* selo = p.sel_out + sk * p.top_t;
    for (int64_t w = ww0; w < ww1; ++w)
      for (uint32_t bits = ld_dev(&bm[w]); bits; bits &= bits - 1u, ++pos)
        if (pos < (uint32_t)p.top_t) selo[pos] = (int32_t)((w << 5) + __ffs(bits) - 1);
    for (int64_t j = tn + tid; j < p.top_t; j += 64 * kFW) selo[j] = -1;
  }
  // the head's histograms and counters, zero for the next step (the levels
  // taken: every work-group of the head took the same)
  for (int i = tid; i < kHistBins; i += 64 * kFW) {
    if (use_hist) st_dev(&Z[kFZH1 + i], 0u);
    if (lvl2) st_dev(&Z[kFZH2 + i], 0u);
  }
  if (s.used3 && tid < 256) st_dev(&Z[kFZH3 + tid], 0u);
  if (tid < 16) st_dev(&Z[kFZC + tid], 0u);
}

template <int G, bool Batched>
static int fused_capacity_g() {
  static const int cap = [] {
    int per_cu = 0, dev = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fused_decode<G, Batched>, 64 * kFW, 0) != hipSuccess ||
        hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    return per_cu * cus;
  }();
  return cap;
}

int fused_capacity(int grp, bool batched) {
  switch (grp) {
    case 1: return batched ? fused_capacity_g<1, true>() : fused_capacity_g<1, false>();
    case 2: return batched ? fused_capacity_g<2, true>() : fused_capacity_g<2, false>();
    case 4: return batched ? fused_capacity_g<4, true>() : fused_capacity_g<4, false>();
  }
  return 0;
}

template <int G, bool Batched>
static void launch_fused_g(const DecodeParams& p, dim3 grid, hipStream_t st, KernelEvents ev) {
  auto kern = fused_decode<G, Batched>;
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kern, grid, dim3(64 * kFW), 0, st, ev.start, ev.stop, 0, p);
  else
    hipLaunchKernelGGL(kern, grid, dim3(64 * kFW), 0, st, p);
}

bool launch_fused(const DecodeParams& p, dim3 grid, hipStream_t st, KernelEvents ev) {
  const bool b = p.batch > 1;
  switch (p.grp) {
    case 1: b ? launch_fused_g<1, true>(p, grid, st, ev) : launch_fused_g<1, false>(p, grid, st, ev); return true;
    case 2: b ? launch_fused_g<2, true>(p, grid, st, ev) : launch_fused_g<2, false>(p, grid, st, ev); return true;
    case 4: b ? launch_fused_g<4, true>(p, grid, st, ev) : launch_fused_g<4, false>(p, grid, st, ev); return true;
  }
  return false;
}

}  // namespace sfk

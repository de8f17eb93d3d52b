// Internal declarations of the HIP library behind include/sf_kv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sf_kv.h"

namespace sfk {

constexpr int kHeadDim = 128;            // the kernels are specialised for D = 128
constexpr int kHistBits = 12;            // first-level score histogram: top 12 key bits
constexpr int kHistBins = 1 << kHistBits;
constexpr int kPartStride = kHeadDim + 2;  // one partial: acc[D], m, l

void set_hip_error(hipError_t e, const char* where);
void clear_error();
void set_error_text(const char* what);

// Order-preserving map of an fp32 score to uint32 (larger score -> larger
// key); -0 and +0 map to the same key.
__host__ __device__ inline uint32_t score_key(float s) {
  uint32_t u = __builtin_bit_cast(uint32_t, s);
  if ((u << 1) == 0) return 0x80000000u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Workspace carve-out (byte offsets from the workspace base).
struct Carve {
  size_t status, hist, zero_end, ftie, scores, logits, counters, cand, bitmap, sel, part, sstat, total;
};

int32_t choose_split(int64_t total_tokens, int32_t n_kv_heads, int32_t groups);
int32_t choose_score_split(int64_t total_tokens, int32_t n_kv_heads, int32_t groups);
Carve carve(const sf_geom& g, int32_t batch, int64_t total_tokens, int64_t max_seq_tokens,
            int32_t top_t, int32_t n_split_bound);

}  // namespace sfk

// Geometry check shared by every entry point.
sf_status sf_check_geom(const sf_geom* g);

// Store internals, shared by the decode path.
struct sf_store_s {
  sf_geom g;
  int64_t cap;
  int32_t max_seqs;
  int32_t tier;
  int32_t slots;
  int32_t row_bytes;       // refinement row: D * r / 8
  int device;
  // refinement rows [2][Hkv][cap][row_bytes]: device tier in HBM, host tier pinned
  uint8_t* dev_rows;
  uint8_t* host_rows;
  // host tier: device refinement cache per (sequence slot, KV head)
  uint8_t* cache_data;     // [max_seqs][Hkv][slots][2][row_bytes]
  int32_t* tok_slot;       // [Hkv][cap] global slot id caching the token, -1 if none
                           // (id (seq * Hkv + kvh) * slots + slot)
  int32_t* err;            // device error word: 1 = a refinement row was missing from the cache,
                           // 2 = the check found the slot <-> token tables inconsistent
  int32_t* slot_tok;       // [max_seqs][Hkv][slots] token in the slot, -1 if free
  int32_t* stamp;          // [max_seqs][Hkv][slots] last step the token was selected
  int32_t* dstep;          // device word: lookups so far (this step's LRU stamp); the fetch kernel
                           // advances it, so a step's launches can be captured in a graph and replayed
  // staging for fetched rows and the miss lists
  uint8_t* host_rows_dev;   // host_rows as the device addresses it
  int32_t* h_miss;         // pinned: the miss lists, copied back only for statistics
  int32_t* miss;           // [max_seqs][Hkv][2 (slots + 1)]: the last lookup's miss lists
  // skip-on-miss steps fetch on a side stream (default priority); the next
  // call on the store waits for `fetched` when `fetch_pending`
  hipStream_t side;
  hipEvent_t looked_up, fetched;
  int32_t fetch_pending;
};

#define SF_HIP_CHECK(call)                                   \
  do {                                                       \
    hipError_t e_ = (call);                                  \
    if (e_ != hipSuccess) {                                  \
      sfk::set_hip_error(e_, #call);                         \
      return SF_ERR_HIP;                                     \
    }                                                        \
  } while (0)

#define SF_LAUNCH_CHECK(what)                                \
  do {                                                       \
    hipError_t e_ = hipGetLastError();                       \
    if (e_ != hipSuccess) {                                  \
      sfk::set_hip_error(e_, what);                          \
      return SF_ERR_HIP;                                     \
    }                                                        \
  } while (0)

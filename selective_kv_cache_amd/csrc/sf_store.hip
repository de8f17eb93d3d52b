// Refinement store, device refinement cache and the host-tier fetch.
//
// Method: page "StrataFlux -- Selective precision streaming -- What does it
// mean?": refinement bits sit off the GPU, in host RAM on a machine with a
// dedicated GPU (paragraph "Think about how a map app ..."); only the bits of
// the selected tokens cross the link (comparison table, row "StrataFlux");
// fetched bits are kept and reused across steps because selections repeat
// (paragraph "The map app also loads tiles ...").
//
// Host tier, per decode step (after the selection is known):
//   cache_lookup  (device, one work-group per (sequence, KV head)): a
//                 selected token already cached is a hit and is stamped with
//                 the step; misses, in ascending token order, take free slots
//                 first, then the slots of residents not selected now, oldest
//                 stamp first (lower token index first); the miss list
//                 (token, slot) goes to the workspace
//   cache_fetch   (device, many work-groups per (sequence, KV head)): the K
//                 and V refinement rows of every miss are read over the link
//                 straight from the pinned store (mapped into the device's
//                 address space), 16 bytes per lane with several reads in
//                 flight, into the miss's slot
// No host step and no synchronization, unless the caller asks for the step's
// statistics.  Policy on a miss (same page, paragraph "The map app also loads
// tiles ..."): "wait", the fetch runs before the attention and the step uses
// every selected refinement; or "skip", the lookup marks the misses in the
// selection list, the attention takes them at base precision, and the fetch
// runs on the store's side stream for later steps.
// Appends (sf_refine_store) write the new rows into the pinned store with a
// kernel, through the store's mapped address, and drop cached copies.
#include <string.h>

#include <algorithm>

#include "sf_decode_kernels.h"

namespace sfk {

__global__ void fill_i32(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// Put refinement rows [Hkv][n_tok][rb] of tokens [t0, t0 + n_tok) into the
// pinned store through its mapped address (16-byte stores over the link, rb
// is a multiple of 16), and forget cached rows of those tokens (their
// refinement was rewritten).
__global__ void store_put(const uint8_t* rows, int64_t n_tok, int64_t t0, int32_t hkv, int64_t cap, int32_t rb,
                          int32_t which, uint8_t* host_rows, int32_t* slot_tok, int32_t* tok_slot,
                          int64_t n_slots_total, int32_t slots) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t pieces = rb / 16, per_head = n_tok * pieces;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < hkv * per_head; i += stride) {
    const int64_t h = i / per_head, rest = i - h * per_head;
    const int64_t t = rest / pieces, pc = rest - t * pieces;
    const uint4 v = reinterpret_cast<const uint4*>(rows + (h * n_tok + t) * rb)[pc];
    reinterpret_cast<uint4*>(host_rows + (((int64_t)which * hkv + h) * cap + t0 + t) * rb)[pc] = v;
  }
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_slots_total; i += stride) {
    const int32_t tok = slot_tok[i];
    if (tok >= t0 && tok < t0 + n_tok) {
      const int64_t kvh = (i / slots) % hkv;
      atomicCAS(&tok_slot[kvh * cap + tok], (int32_t)i, -1);   // i is the slot's global id
      slot_tok[i] = -1;
    }
  }
}

// Consistency of the cache tables (debug check): every token entry names a
// slot of its KV head that holds the token, and every occupied slot holds a
// token inside the capacity.  (A slot may still hold a token whose entry names
// another batch position's slot, after the batch was reordered: that copy is
// never read.)  A violation sets bit 2 of the error word.
__global__ void check_tables(const int32_t* slot_tok, const int32_t* tok_slot, int64_t n_slots_total, int32_t slots,
                             int32_t hkv, int64_t cap, int32_t* err) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_slots_total; i += stride) {
    const int32_t tok = slot_tok[i];
    if (tok >= cap) atomicOr(err, 2);
  }
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < hkv * cap; i += stride) {
    const int32_t g = tok_slot[i];
    if (g >= 0) {
      const int64_t kvh = i / cap, tok = i - kvh * cap;
      if (g >= n_slots_total || (g / slots) % hkv != kvh || slot_tok[g] != (int32_t)tok) atomicOr(err, 2);
    }
  }
}

constexpr int kLookupThreads = 1024;
constexpr int kMaxSlots = 4096;   // keeps the lookup's keys and lists in LDS (<= 96 KiB)

// One work-group per (sequence, KV head).  Dynamic LDS: the slots' victim
// keys (uint64) and selected-resident flags, the misses' ranks and the victim
// list (top_t each).
__global__ void __launch_bounds__(kLookupThreads)
cache_lookup(DecodeParams p, int32_t* slot_tok, int32_t* stamp, int32_t* tok_slot, const int32_t* dstep,
             int32_t* miss, int32_t mark_misses) {
  const int32_t step = *dstep;                                    // this step's stamp
  extern __shared__ uint64_t keys[];                              // [slots]: victim keys
  uint32_t* flag = reinterpret_cast<uint32_t*>(keys + p.slots);   // [slots]: 1 = selected resident
  int32_t* mrank = reinterpret_cast<int32_t*>(flag + p.slots);    // [top_t]: rank among misses, -1 = hit
  int32_t* vlist = mrank + p.top_t;                               // [top_t]: victim slots in slot order
  __shared__ uint32_t cnt[kLookupThreads / 64];
  __shared__ uint32_t rh[256];
  __shared__ uint64_t sh_prefix, sh_mask;
  __shared__ uint32_t sh_left, sh_whole;

  const int tid = threadIdx.x;
  const int64_t sk = blockIdx.x;
  const int seq = (int)(sk / p.hkv), kvh = (int)(sk % p.hkv);
  const int64_t a = seq_at(p, seq);
  const int64_t n = seq_at(p, seq + 1) - a;
  const int32_t tn = (int32_t)(n < p.top_t ? n : p.top_t);
  const int32_t* sel = p.sel + sk * p.top_t;
  int32_t* st_tok = slot_tok + sk * p.slots;
  int32_t* st_stamp = stamp + sk * p.slots;
  int32_t* ts = tok_slot + (int64_t)kvh * p.cap;
  const int32_t gbase = (int32_t)(sk * p.slots);   // this cache's first global slot id

  for (int i = tid; i < p.slots; i += kLookupThreads) flag[i] = 0u;
  __syncthreads();
  // hits are stamped; misses flagged (the loads of a thread's tokens are
  // issued together: top_t <= slots <= kMaxSlots).  tok_slot holds global slot
  // ids; a token counts as a hit only when its id lies in this (sequence,
  // KV head)'s cache and that slot holds the token.
  static_assert(kMaxSlots <= 4 * kLookupThreads, "four selected tokens per thread at most");
  int32_t slot4[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int j = tid + u * kLookupThreads;
    const int32_t gs = j < tn ? ts[a + sel[j]] : -1;
    slot4[u] = (gs >= gbase && gs < gbase + p.slots) ? gs - gbase : -1;
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int j = tid + u * kLookupThreads;
    if (j < tn && slot4[u] >= 0 && st_tok[slot4[u]] != (int32_t)(a + sel[j])) slot4[u] = -1;
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int j = tid + u * kLookupThreads;
    if (j < tn) {
      const int32_t slot = slot4[u];
      if (slot >= 0) {
        st_stamp[slot] = step;
        flag[slot] = 1u;
        mrank[j] = -1;
      } else {
        mrank[j] = 0;
      }
    }
  }
  __syncthreads();
  // rank the misses in ascending token order (the selection is ascending)
  const int per = (tn + kLookupThreads - 1) / kLookupThreads;
  const int j0 = tid * per, j1 = std::min(j0 + per, (int)tn);
  uint32_t c = 0;
  for (int j = j0; j < j1; ++j) c += (mrank[j] == 0);
  uint32_t nmiss;
  uint32_t rk = block_exclusive_scan<kLookupThreads>(c, cnt, nmiss);
  if (tid == 0) miss[sk * 2 * (int64_t)(p.top_t + 1)] = (int32_t)nmiss;
  for (int j = j0; j < j1; ++j)
    if (mrank[j] == 0) mrank[j] = (int32_t)(rk++);
  // Victims: free slots first, then the residents not selected now, oldest
  // stamp first (lower token first): the nmiss smallest of the keys
  //   free slot i: i;   resident: (stamp + 1) << tb | token,
  // tb the token index's width, at least 12 bits (so that every resident's
  // key lies above every free slot's: slots <= 4096); hits and selected
  // slots take no part (~0).  Every key differs, so the nmiss-th smallest,
  // found by an 8-bit radix select, splits them exactly; the victims are
  // then listed in slot order (which miss takes which victim does not change
  // what stays cached).  A resident's stamp is at most this step, so no key
  // has a bit above hb = tb + bitlen(step + 1) - 1 and the select starts at
  // the byte holding hb.
  const int tb = max(12, p.cap > 1 ? 64 - __clzll((unsigned long long)(p.cap - 1)) : 0);
  const uint64_t tmask = (1ull << tb) - 1ull;
  for (int i = tid; i < p.slots; i += kLookupThreads) {
    uint64_t k = ~0ull;
    const int32_t tok = st_tok[i];
    if (tok < 0)
      k = (uint64_t)i;
    else if (!flag[i])
      k = ((uint64_t)(uint32_t)(st_stamp[i] + 1) << tb) | (uint64_t)(uint32_t)tok;
    keys[i] = k;
  }
  const int hb = tb + (32 - __clz((uint32_t)step + 1u)) - 1;
  const int start = (hb >> 3) << 3;
  if (tid == 0) {
    sh_prefix = 0ull;
    sh_mask = start + 8 < 64 ? ~0ull << (start + 8) : 0ull;
    sh_left = nmiss;
    sh_whole = nmiss == 0 ? 1u : 0u;
  }
  __syncthreads();
  for (int shift = start; shift >= 0 && !sh_whole; shift -= 8) {
    for (int i = tid; i < 256; i += kLookupThreads) rh[i] = 0u;
    __syncthreads();
    const uint64_t pre = sh_prefix, msk = sh_mask;
    for (int i = tid; i < p.slots; i += kLookupThreads) {
      const uint64_t k = keys[i];
      if (k != ~0ull && (k & msk) == pre) atomicAdd(&rh[(k >> shift) & 0xFFu], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // bucket holding the sh_left-th smallest: inclusive prefix over the
      // 256 buckets, 4 per lane in ascending order
      uint32_t c4[4], sum = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        c4[u] = rh[4 * tid + u];
        sum += c4[u];
      }
      const uint32_t inc = wave_inclusive_scan(sum), left = sh_left;
      uint32_t below = inc - sum;
      const uint64_t hit = __ballot(below < left && left <= inc);
      if (hit && tid == __ffsll((unsigned long long)hit) - 1) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (below < left && left <= below + c4[u]) {
            sh_prefix = pre | ((uint64_t)(4 * tid + u) << shift);
            sh_mask = msk | (0xFFull << shift);
            sh_left = left - below;
            sh_whole = (c4[u] == left - below) ? 1u : 0u;
            break;
          }
          below += c4[u];
        }
      }
    }
    __syncthreads();
  }
  // the victims in slot order
  const uint64_t vpre = sh_prefix, vmsk = sh_mask;
  const int sper = (p.slots + kLookupThreads - 1) / kLookupThreads;
  const int s0 = tid * sper, s1 = std::min(s0 + sper, p.slots);
  uint32_t nv = 0;
  for (int i = s0; i < s1; ++i) {
    const uint64_t k = keys[i];
    nv += (nmiss > 0 && k != ~0ull && (k & vmsk) <= vpre) ? 1u : 0u;
  }
  uint32_t vtot;
  uint32_t vpos = block_exclusive_scan<kLookupThreads>(nv, cnt, vtot);
  for (int i = s0; i < s1; ++i) {
    const uint64_t k = keys[i];
    if (nmiss > 0 && k != ~0ull && (k & vmsk) <= vpre) {
      if (vpos < (uint32_t)p.top_t) vlist[vpos] = i;
      ++vpos;
    }
  }
  __syncthreads();
  // install the mapping of each miss into its victim slot
  int32_t* ml = miss + sk * 2 * (int64_t)(p.top_t + 1) + 2;
  for (int j = tid; j < tn; j += kLookupThreads) {
    const int32_t k = mrank[j];
    if (k < 0 || k >= (int32_t)vtot) continue;   // fewer victims than misses: cannot happen with slots >= T
    const int32_t slot = vlist[k];
    const uint64_t key = keys[slot];
    if (key > tmask)   // the resident leaves (its token's entry, if it still names this slot)
      atomicCAS(&ts[(int32_t)(key & tmask)], gbase + slot, -1);
    const int32_t g = (int32_t)(a + sel[j]);
    st_tok[slot] = g;
    st_stamp[slot] = step;
    ts[g] = gbase + slot;
    ml[2 * k] = g;
    ml[2 * k + 1] = slot;
    // skip on a miss: the attention takes this token at base precision (its
    // rows arrive for later steps); the entry is marked as ~token
    if (mark_misses) const_cast<int32_t*>(sel)[j] = ~sel[j];
  }
}

// Read the missed rows from the pinned store into their cache slots: grid
// (sequence x KV head, kFetchWGs); 16-byte pieces (a row is D r / 8 bytes, a
// multiple of 16), kFetchUnroll reads in flight per lane.
constexpr int kFetchWGs = 16;
constexpr int kFetchUnroll = 4;
__global__ void __launch_bounds__(256)
cache_fetch(const int32_t* miss, int32_t top_t, int32_t hkv, int64_t cap, int32_t slots, int32_t rb,
            const uint8_t* host_rows, uint8_t* cache_data, int32_t* dstep) {
  // the step's lookup is done (stream order): the next step stamps with the next value
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *dstep += 1;
  const int64_t sk = blockIdx.x;
  const int kvh = (int)(sk % hkv);
  const int32_t* m = miss + sk * 2 * (int64_t)(top_t + 1);
  const int64_t pieces = rb / 16;                  // per row
  const int64_t items = (int64_t)m[0] * 2 * pieces;
  const int64_t step = (int64_t)gridDim.y * blockDim.x;
  for (int64_t i0 = (int64_t)blockIdx.y * blockDim.x + threadIdx.x; i0 < items; i0 += kFetchUnroll * step) {
    uint4 v[kFetchUnroll];
    int64_t dst[kFetchUnroll];
#pragma unroll
    for (int u = 0; u < kFetchUnroll; ++u) {
      const int64_t i = i0 + u * step;
      dst[u] = -1;
      if (i < items) {
        const int64_t k = i / (2 * pieces), rest = i - k * 2 * pieces;
        const int which = (int)(rest / pieces), piece = (int)(rest - which * pieces);
        const int64_t tok = m[2 + 2 * k], slot = m[2 + 2 * k + 1];
        v[u] = reinterpret_cast<const uint4*>(host_rows + (((int64_t)which * hkv + kvh) * cap + tok) * rb)[piece];
        dst[u] = (((sk * slots + slot) * 2 + which) * rb) / 16 + piece;
      }
    }
#pragma unroll
    for (int u = 0; u < kFetchUnroll; ++u)
      if (dst[u] >= 0) reinterpret_cast<uint4*>(cache_data)[dst[u]] = v[u];
  }
}

}  // namespace sfk

using namespace sfk;

static void free_store(sf_store_s* s) {
  if (!s) return;
  if (s->dev_rows) (void)hipFree(s->dev_rows);
  if (s->host_rows) (void)hipHostFree(s->host_rows);
  if (s->cache_data) (void)hipFree(s->cache_data);
  if (s->tok_slot) (void)hipFree(s->tok_slot);
  if (s->slot_tok) (void)hipFree(s->slot_tok);
  if (s->stamp) (void)hipFree(s->stamp);
  if (s->h_miss) (void)hipHostFree(s->h_miss);
  if (s->err) (void)hipFree(s->err);
  if (s->miss) (void)hipFree(s->miss);
  if (s->dstep) (void)hipFree(s->dstep);
  if (s->looked_up) (void)hipEventDestroy(s->looked_up);
  if (s->fetched) (void)hipEventDestroy(s->fetched);
  if (s->side) (void)hipStreamDestroy(s->side);
  delete s;
}

extern "C" sf_status sf_store_create(const sf_geom* geom, int64_t cap_tokens, int32_t max_seqs, int32_t tier,
                                     int32_t cache_slots, sf_store* out) {
  clear_error();
  sf_status st = sf_check_geom(geom);
  if (st != SF_OK) return st;
  if (!out || cap_tokens <= 0 || max_seqs <= 0 || cap_tokens > 0x7fffffffLL) return SF_ERR_INVALID_ARG;
  if (tier != SF_TIER_DEVICE && tier != SF_TIER_HOST_PINNED) return SF_ERR_INVALID_ARG;
  if (geom->refine_bits == 0) return SF_ERR_INVALID_ARG;
  if (tier == SF_TIER_HOST_PINNED && (cache_slots <= 0 || cache_slots > kMaxSlots)) return SF_ERR_INVALID_ARG;
  // global slot ids are int32
  if (tier == SF_TIER_HOST_PINNED && (int64_t)max_seqs * geom->n_kv_heads * cache_slots > 0x7fffffffLL)
    return SF_ERR_INVALID_ARG;
  *out = nullptr;
  sf_store_s* s = new sf_store_s();
  memset(s, 0, sizeof(*s));
  s->g = *geom;
  s->cap = cap_tokens;
  s->max_seqs = max_seqs;
  s->tier = tier;
  s->slots = tier == SF_TIER_HOST_PINNED ? cache_slots : 0;
  s->row_bytes = geom->head_dim * geom->refine_bits / 8;
  const int64_t hkv = geom->n_kv_heads;
  const size_t rows_bytes = (size_t)2 * hkv * cap_tokens * s->row_bytes;
  if (hipGetDevice(&s->device) != hipSuccess) {
    delete s;
    return SF_ERR_HIP;
  }
#define SF_ALLOC(call)          \
  if ((call) != hipSuccess) {   \
    (void)hipGetLastError();    \
    free_store(s);              \
    return SF_ERR_OOM;          \
  }
  if (tier == SF_TIER_DEVICE) {
    SF_ALLOC(hipMalloc((void**)&s->dev_rows, rows_bytes));
    SF_ALLOC(hipMemset(s->dev_rows, 0, rows_bytes));
  } else {
    const int64_t nslots = (int64_t)max_seqs * hkv * s->slots;
    SF_ALLOC(hipHostMalloc((void**)&s->host_rows, rows_bytes, hipHostMallocDefault));
    memset(s->host_rows, 0, rows_bytes);
    SF_ALLOC(hipHostGetDevicePointer((void**)&s->host_rows_dev, s->host_rows, 0));
    SF_ALLOC(hipMalloc((void**)&s->cache_data, (size_t)nslots * 2 * s->row_bytes));
    SF_ALLOC(hipMalloc((void**)&s->tok_slot, (size_t)hkv * cap_tokens * 4));
    SF_ALLOC(hipMalloc((void**)&s->slot_tok, (size_t)nslots * 4));
    SF_ALLOC(hipMalloc((void**)&s->stamp, (size_t)nslots * 4));
    SF_ALLOC(hipMemset(s->tok_slot, 0xFF, (size_t)hkv * cap_tokens * 4));
    SF_ALLOC(hipMemset(s->slot_tok, 0xFF, (size_t)nslots * 4));
    SF_ALLOC(hipMemset(s->stamp, 0xFF, (size_t)nslots * 4));
    SF_ALLOC(hipHostMalloc((void**)&s->h_miss, (size_t)max_seqs * hkv * (2 * (s->slots + 1) + 1) * 4,
                           hipHostMallocDefault));
    SF_ALLOC(hipMalloc((void**)&s->miss, (size_t)max_seqs * hkv * (2 * (s->slots + 1) + 1) * 4));
    SF_ALLOC(hipMalloc((void**)&s->dstep, 4));
    SF_ALLOC(hipMemset(s->dstep, 0, 4));
    SF_ALLOC(hipStreamCreateWithFlags(&s->side, hipStreamNonBlocking));
    SF_ALLOC(hipEventCreateWithFlags(&s->looked_up, hipEventDisableTiming));
    SF_ALLOC(hipEventCreateWithFlags(&s->fetched, hipEventDisableTiming));
  }
  SF_ALLOC(hipMalloc((void**)&s->err, 4));
  SF_ALLOC(hipMemset(s->err, 0, 4));
#undef SF_ALLOC
  *out = s;
  return SF_OK;
}

extern "C" sf_status sf_store_destroy(sf_store store) {
  clear_error();
  if (!store) return SF_ERR_INVALID_ARG;
  (void)hipDeviceSynchronize();
  free_store(store);
  return SF_OK;
}

// A skip-step fetch still in flight on the side stream: `st` waits for it.
static sf_status wait_side_fetch(sf_store_s* s, hipStream_t st) {
  if (s->fetch_pending) {
    SF_HIP_CHECK(hipStreamWaitEvent(st, s->fetched, 0));
    s->fetch_pending = 0;
  }
  return SF_OK;
}

extern "C" sf_status sf_refine_store(sf_store s, int32_t which, const uint8_t* refine_rows, int64_t tok_begin,
                                     int64_t n_tok, void* stream) {
  clear_error();
  if (!s || (which != SF_K && which != SF_V) || tok_begin < 0 || n_tok < 0 || tok_begin + n_tok > s->cap)
    return SF_ERR_INVALID_ARG;
  if (n_tok == 0) return SF_OK;
  if (!refine_rows) return SF_ERR_INVALID_ARG;
  hipStream_t hs = (hipStream_t)stream;
  const int64_t hkv = s->g.n_kv_heads;
  const size_t rb = s->row_bytes;
  const size_t width = (size_t)n_tok * rb;
  if (s->tier == SF_TIER_DEVICE) {
    uint8_t* dst = s->dev_rows + ((size_t)which * hkv * s->cap + tok_begin) * rb;
    SF_HIP_CHECK(hipMemcpy2DAsync(dst, (size_t)s->cap * rb, refine_rows, width, width, hkv,
                                  hipMemcpyDeviceToDevice, hs));
    return SF_OK;
  }
  const sf_status ws = wait_side_fetch(s, hs);
  if (ws != SF_OK) return ws;
  const int64_t nslots = (int64_t)s->max_seqs * hkv * s->slots;
  const int64_t work = std::max<int64_t>(hkv * n_tok * (int64_t)(rb / 16), nslots);
  hipLaunchKernelGGL(store_put, dim3((unsigned)std::min<int64_t>((work + 255) / 256, 1024)), dim3(256), 0, hs,
                     refine_rows, n_tok, tok_begin, (int32_t)hkv, s->cap, (int32_t)rb, which, s->host_rows_dev,
                     s->slot_tok, s->tok_slot, nslots, s->slots);
  SF_LAUNCH_CHECK("store_put");
  return SF_OK;
}

extern "C" sf_status sf_store_clear_cache(sf_store s, void* stream) {
  clear_error();
  if (!s) return SF_ERR_INVALID_ARG;
  if (s->tier != SF_TIER_HOST_PINNED) return SF_OK;
  hipStream_t hs = (hipStream_t)stream;
  const sf_status ws = wait_side_fetch(s, hs);
  if (ws != SF_OK) return ws;
  const int64_t hkv = s->g.n_kv_heads;
  const int64_t nslots = (int64_t)s->max_seqs * hkv * s->slots;
  hipLaunchKernelGGL(fill_i32, dim3(1024), dim3(256), 0, hs, s->tok_slot, hkv * s->cap, -1);
  hipLaunchKernelGGL(fill_i32, dim3(256), dim3(256), 0, hs, s->slot_tok, nslots, -1);
  hipLaunchKernelGGL(fill_i32, dim3(256), dim3(256), 0, hs, s->stamp, nslots, -1);
  SF_LAUNCH_CHECK("fill_i32");
  return SF_OK;
}

extern "C" sf_status sf_store_check(sf_store s, void* stream) {
  clear_error();
  if (!s) return SF_ERR_INVALID_ARG;
  hipStream_t hs = (hipStream_t)stream;
  const sf_status ws = wait_side_fetch(s, hs);
  if (ws != SF_OK) return ws;
  if (s->tier == SF_TIER_HOST_PINNED) {
    const int64_t nslots = (int64_t)s->max_seqs * s->g.n_kv_heads * s->slots;
    hipLaunchKernelGGL(check_tables, dim3(256), dim3(256), 0, hs, s->slot_tok, s->tok_slot, nslots, s->slots,
                       (int32_t)s->g.n_kv_heads, s->cap, s->err);
    SF_LAUNCH_CHECK("check_tables");
  }
  int32_t e = 0;
  SF_HIP_CHECK(hipMemcpyAsync(&e, s->err, 4, hipMemcpyDeviceToHost, hs));
  SF_HIP_CHECK(hipStreamSynchronize(hs));
  if (e == 0) return SF_OK;
  SF_HIP_CHECK(hipMemsetAsync(s->err, 0, 4, hs));
  SF_HIP_CHECK(hipStreamSynchronize(hs));
  return SF_ERR_STATE;
}

// Host tier: look up the selection in the device cache, install the misses
// and fetch their rows over the link.  Policy "wait": the fetch runs on `st`
// before the attention.  Policy "skip": the lookup marks the misses in the
// selection list (the attention takes them at base precision) and the fetch
// runs on the store's side stream, overlapping the rest of the step; the
// store's next call waits for it.  Nothing waits on the host unless `stats`.
sf_status sf_store_fetch(sf_store s, const DecodeParams& p, hipStream_t st, bool skip, sf_step_stats* stats) {
  const int32_t B = p.batch, hkv = p.hkv;
  const int64_t groups = (int64_t)B * hkv;
  const size_t lds = (size_t)s->slots * 12 + (size_t)p.top_t * 8;
  int32_t* miss_dev = s->miss;
  // the previous skip step's fetch reads the miss lists and fills slots
  const sf_status ws = wait_side_fetch(s, st);
  if (ws != SF_OK) return ws;
  hipLaunchKernelGGL(cache_lookup, dim3((unsigned)groups), dim3(kLookupThreads), lds, st, p, s->slot_tok,
                     s->stamp, s->tok_slot, s->dstep, miss_dev, skip ? 1 : 0);
  SF_LAUNCH_CHECK("cache_lookup");
  hipStream_t fs = st;
  if (skip) {
    SF_HIP_CHECK(hipEventRecord(s->looked_up, st));
    SF_HIP_CHECK(hipStreamWaitEvent(s->side, s->looked_up, 0));
    fs = s->side;
  }
  hipLaunchKernelGGL(cache_fetch, dim3((unsigned)groups, kFetchWGs), dim3(256), 0, fs, miss_dev, p.top_t, hkv,
                     s->cap, s->slots, (int32_t)s->row_bytes, s->host_rows_dev, s->cache_data, s->dstep);
  SF_LAUNCH_CHECK("cache_fetch");
  if (skip) {
    SF_HIP_CHECK(hipEventRecord(s->fetched, s->side));
    s->fetch_pending = 1;
  }
  if (stats) {
    // the miss counts, for the caller's statistics (this synchronizes)
    const size_t stride = 2 * (size_t)(p.top_t + 1);
    SF_HIP_CHECK(hipMemcpyAsync(s->h_miss, miss_dev, groups * stride * 4, hipMemcpyDeviceToHost, st));
    SF_HIP_CHECK(hipStreamSynchronize(st));
    int64_t total = 0;
    for (int64_t g = 0; g < groups; ++g) total += s->h_miss[g * stride];
    stats->misses = total;
    stats->h2d_bytes = total * 2 * s->row_bytes;
  }
  return SF_OK;
}

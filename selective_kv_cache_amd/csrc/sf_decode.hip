// The decode step (sf_decode_step): score, select, refine, attend.
//
// Method: page "StrataFlux -- Selective precision streaming -- What does it
// mean?", paragraph "Which tiles count ...": every cached token is scored by
// the attention it receives, computed from the resident low-bit keys; the
// highest-scoring tokens of each KV head (the set its GQA group of query heads
// shares) are refined; everything not selected still takes part at low
// precision.  Paragraph "What travels over the link ...": refinement bits
// subdivide the bin the base code names.
//
// Kernel sequence on the caller's stream (one layer):
//   zero_words     clear the score-key histogram (unless the caller vouches
//                  that the last step left it zero)
//   score          read the base K codes of every token: token score (max over
//                  the GQA group of the scaled logit) and a histogram of the
//                  scores' order-preserving keys
//   select_scan,   per (sequence, KV head): the exact top-T (score desc,
//   select_resolve token asc) as a bitmap and an ascending list
//   [host-pinned store only: cache lookup, fetch of the misses, install]
//   attend         read the per-head logits the score pass kept and the V
//                  codes, and run split-K online-softmax attention with every
//                  selected row refined
//   combine        merge the split partials of each query head
//
// Refinement depends on the selection, and the selection on all scores (the
// same page, paragraph "Where it earns its keep", notes that the refinement
// step cannot be overlapped with the attention around it), so attention runs
// after the selection; each token then enters the softmax once, with its
// final logit and value.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "sf_decode_kernels.h"

namespace sfk {


__global__ void zero_words(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Tokens per attention work-group of base tokens: about `groups` of them
// over the chip (a few wavefronts per SIMD), few enough partials to keep the
// combine small.  At most 4096 (the base passes' selection-word layout).
int32_t choose_split(int64_t total_tokens, int32_t n_kv_heads, int32_t groups) {
  const int64_t work = total_tokens * n_kv_heads;
  int32_t s = 256;
  while (s < 4096 && work / s > groups) s *= 2;
  return s;
}

// The attention pass's shape: the matrix-core form (2-, 3- or 4-bit base
// codes, GQA groups of 1, 2, 4 or 8) runs kAttendWaves wavefronts per work-group, the
// VALU form 4; about 2048 wavefronts of base tokens either way.
struct AttendShape {
  int32_t split;
};
static AttendShape attend_shape(const sf_geom& g, int64_t total_tokens) {
  const int32_t grp = g.n_q_heads / g.n_kv_heads;
  const bool mfma = g.base_bits >= 2 && g.base_bits <= 4 && (grp == 1 || grp == 2 || grp == 4 || grp == 8);
  const int waves = mfma ? kAttendWaves : 4;
  return AttendShape{choose_split(total_tokens, g.n_kv_heads, 2048 / waves)};
}

// Tokens per score work-group: about `groups` work-groups.
int32_t choose_score_split(int64_t total_tokens, int32_t n_kv_heads, int32_t groups) {
  const int64_t work = total_tokens * n_kv_heads;
  int32_t s = 256;
  while (s < 16384 && work / s > groups) s *= 2;
  return s;
}

Carve carve(const sf_geom& g, int32_t batch, int64_t total_tokens, int64_t max_seq_tokens,
            int32_t top_t, int32_t n_part_bound) {
  const int grp = g.n_q_heads / g.n_kv_heads;
  const int64_t hkv = g.n_kv_heads;
  const int64_t bm_words = ((max_seq_tokens + kSelThreads - 1) / kSelThreads) * (kSelThreads / 32);
  const int64_t t = top_t > 0 ? top_t : 1;
  Carve c{};
  size_t at = 0;
  // what must be zero between steps comes first (its place depends on
  // (batch, hkv) only, so a workspace that a step left clean can be reused as
  // such): the status word, then per (sequence, KV head) the selection
  // histograms and counters (the single-launch path's blocks of kFZWords
  // words; the multi-pass path's level-1 histograms are the first
  // batch * hkv * kHistBins words of the same region)
  c.status = at; at += 256;
  c.hist = at; at += align256((size_t)batch * hkv * kFZWords * 4);
  c.zero_end = at;
  c.ftie = at; at += align256((size_t)batch * hkv * ((max_seq_tokens + kFusedMinR - 1) / kFusedMinR) * 4);
  c.scores = at; at += align256((size_t)hkv * total_tokens * 4);
  // per-head logits; one chunk of slack for the attention pass's last loads
  c.logits = at; at += align256((size_t)hkv * total_tokens * grp * 4 + 32 * 8 * 4);
  c.counters = at; at += align256((size_t)batch * hkv * ((max_seq_tokens + kSelChunk - 1) / kSelChunk + 2) * 4);
  c.cand = at; at += align256((size_t)batch * hkv * max_seq_tokens * 8);
  c.bitmap = at; at += align256((size_t)batch * hkv * bm_words * 4);
  c.sel = at; at += align256((size_t)batch * hkv * t * 4);
  c.part = at; at += align256((size_t)hkv * n_part_bound * grp * kPartStride * 4);
  // the summed-probability score's (maximum, sum) per score unit (units of
  // at least 256 tokens)
  c.sstat = at; at += align256((size_t)hkv * (total_tokens / 256 + batch) * grp * 8);
  c.total = at;
  return c;
}

// Upper bound of the partials of a step: splits of every sequence plus the
// selected-token work-groups.
static int32_t part_bound(int64_t total, int32_t batch, int32_t split, int32_t top_t) {
  const int64_t multi = total / split + batch + (int64_t)batch * ((top_t + kSelBlkTokMin - 1) / kSelBlkTokMin);
  const int64_t fused = total / kFusedMinR + batch;   // single-launch ranges
  return (int32_t)(multi > fused ? multi : fused);
}

// Compute units of the current device (the selected blocks' size depends on
// how many work-groups fit at once).
static int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

}  // namespace sfk

using namespace sfk;

// The single-launch path: 2-bit base codes, groups of 1, 2 or 4, the
// refinement rows in HBM (or none), policy "wait", and every work-group of
// the launch resident at once: the smallest range R (a multiple of
// kFusedMinR) whose work-groups fit the device.  Returns R (0: the five
// kernels) and the work-groups per KV head in `n_units`.
static int32_t fused_plan(const sf_geom& g, const sf_decode_args& a, bool refine, int32_t* n_units) {
  const int32_t grp = g.n_q_heads / g.n_kv_heads;
  *n_units = 0;
  if ((a.flags & (SF_DECODE_MULTI_PASS | SF_DECODE_SKIP_MISSES | SF_DECODE_DROP_UNSELECTED | SF_DECODE_ROWS16 |
                  SF_DECODE_SCORE_SOFTMAX)) || g.base_bits != 2 ||
      !(grp == 1 || grp == 2 || grp == 4) || (refine && a.store->tier == SF_TIER_HOST_PINNED))
    return 0;
  const int cap = fused_capacity(grp, a.batch > 1);
  const int64_t* off = a.seq_off_host;
  for (int32_t R = kFusedMinR; R <= kFusedRmax; R += kFusedMinR) {
    int64_t u = 0, umax = 0;
    for (int i = 0; i < a.batch; ++i) {
      const int64_t ui = (off[i + 1] - off[i] + R - 1) / R;
      u += ui;
      umax = ui > umax ? ui : umax;
    }
    if (u * g.n_kv_heads <= cap && umax <= kFusedMaxRanges) {
      *n_units = (int32_t)u;
      return R;
    }
  }
  return 0;
}

extern "C" sf_status sf_decode_form(const sf_geom* geom, const sf_decode_args* a, int32_t* kernels) {
  clear_error();
  sf_status s = sf_check_geom(geom);
  if (s != SF_OK) return s;
  if (!a || !kernels || a->batch <= 0 || !a->seq_off_host || a->top_t < 0) return SF_ERR_INVALID_ARG;
  for (int i = 0; i < a->batch; ++i)
    if (a->seq_off_host[i + 1] - a->seq_off_host[i] <= 0) return SF_ERR_INVALID_ARG;
  const bool refine = a->top_t > 0 && geom->refine_bits > 0;
  if (refine && !a->store) return SF_ERR_INVALID_ARG;
  int32_t n_units = 0;
  *kernels = fused_plan(*geom, *a, refine, &n_units) ? 1 : 5;
  return SF_OK;
}

// Host-tier fetch (sf_store.hip): lookup, copy of the misses, install.
sf_status sf_store_fetch(sf_store store, const DecodeParams& p, hipStream_t st, bool skip, sf_step_stats* stats);

extern "C" sf_status sf_decode_workspace_size(const sf_geom* geom, int32_t batch, int64_t total_tokens,
                                              int64_t max_seq_tokens, int32_t top_t, size_t* bytes) {
  clear_error();
  sf_status s = sf_check_geom(geom);
  if (s != SF_OK) return s;
  if (!bytes || batch <= 0 || total_tokens <= 0 || max_seq_tokens <= 0 || top_t < 0 ||
      max_seq_tokens > total_tokens)
    return SF_ERR_INVALID_ARG;
  if (max_seq_tokens > (int64_t)kMaxSelChunks * kSelChunk) return SF_ERR_UNSUPPORTED;
  // the bound of the form with the most partials: smallest splits, 4 waves
  const int32_t split = choose_split(total_tokens, geom->n_kv_heads, 512);
  *bytes = carve(*geom, batch, total_tokens, max_seq_tokens, top_t, part_bound(total_tokens, batch, split, top_t)).total;
  return SF_OK;
}

// The decode step on a given workspace (the caller's, or the library's static
// scratch for sf_decode_step_noalloc).
sf_status sf_decode_step_ws(const sf_geom* geom, const sf_decode_args* a, void* workspace, size_t workspace_bytes,
                            void* stream) {
  clear_error();
  sf_status s = sf_check_geom(geom);
  if (s != SF_OK) return s;
  if (!a || a->batch <= 0 || !a->seq_off_host || !a->seq_off_dev || !a->q || !a->k_codes ||
      !a->k_scales || !a->v_codes || !a->v_scales || !a->out || !workspace || a->cap <= 0 ||
      a->top_t < 0 ||
      (a->flags & ~(SF_DECODE_HIST_CLEAN | SF_DECODE_SKIP_MISSES | SF_DECODE_MULTI_PASS | SF_DECODE_DROP_UNSELECTED |
                    SF_DECODE_ROWS16 | SF_DECODE_SCORE_SOFTMAX)) != 0)
    return SF_ERR_INVALID_ARG;
  const bool rows16 = (a->flags & SF_DECODE_ROWS16) != 0;
  const bool drop = (a->flags & SF_DECODE_DROP_UNSELECTED) != 0;
  const bool smax = (a->flags & SF_DECODE_SCORE_SOFTMAX) != 0;
  if (rows16 != (a->rows16 != nullptr) || (rows16 && a->top_t <= 0)) return SF_ERR_INVALID_ARG;
  const int32_t B = a->batch;
  const int64_t* off = a->seq_off_host;
  if (off[0] < 0) return SF_ERR_INVALID_ARG;
  int64_t max_seq = 0;
  for (int i = 0; i < B; ++i) {
    const int64_t n = off[i + 1] - off[i];
    if (n <= 0) return SF_ERR_INVALID_ARG;   // softmax over an empty set is undefined
    max_seq = std::max(max_seq, n);
  }
  if (off[B] > a->cap) return SF_ERR_INVALID_ARG;
  if (max_seq > (int64_t)kMaxSelChunks * kSelChunk) return SF_ERR_UNSUPPORTED;
  const int64_t total = off[B] - off[0];
  // refinement codes read for the selection (not with 16-bit rows); the
  // selected tokens' work-groups run with either
  const bool refine = a->top_t > 0 && geom->refine_bits > 0 && !rows16;
  const bool sel_work = refine || rows16;
  if (drop && !sel_work) return SF_ERR_INVALID_ARG;   // the selection must take part
  if (refine) {
    if (!a->store) return SF_ERR_INVALID_ARG;
    const sf_store_s* st = a->store;
    // the kernels index the store's rows and tables with the caches' pitch
    if (st->g.head_dim != geom->head_dim || st->g.n_kv_heads != geom->n_kv_heads ||
        st->g.refine_bits != geom->refine_bits || st->cap != a->cap)
      return SF_ERR_INVALID_ARG;
    if (st->tier == SF_TIER_HOST_PINNED && (B > st->max_seqs || a->top_t > st->slots))
      return SF_ERR_INVALID_ARG;
  }
  const AttendShape ash = attend_shape(*geom, total);
  const int32_t split = ash.split;
  // the matrix-core score pass runs kScoreWaves wavefronts per work-group,
  // the other 4: about 4096 wavefronts either way
  const int32_t grp = geom->n_q_heads / geom->n_kv_heads;
  const bool score_mfma = geom->base_bits >= 2 && geom->base_bits <= 4 && (grp == 1 || grp == 2 || grp == 4 || grp == 8);
  // the summed-probability score needs the score pass's per-head logits (its
  // kernels take groups of up to 4)
  if (smax && (!score_mfma || grp > 4)) return SF_ERR_UNSUPPORTED;
  const int32_t score_split = choose_score_split(total, geom->n_kv_heads, score_mfma ? 4096 / kScoreWaves : 1024);
  const Carve c = carve(*geom, B, total, max_seq, a->top_t, part_bound(total, B, split, a->top_t));
  if (workspace_bytes < c.total) return SF_ERR_INVALID_ARG;
  int32_t n_units = 0;
  const int32_t fr = fused_plan(*geom, *a, refine, &n_units);
  int32_t n_split = 0, n_score = 0, n_sel = 0, n_small = 0;
  for (int i = 0; i < B; ++i) {
    const int64_t n = off[i + 1] - off[i];
    n_split += (int32_t)((n + split - 1) / split);
    n_score += (int32_t)((n + score_split - 1) / score_split);
    n_sel += (int32_t)((n + kSelChunk - 1) / kSelChunk);
    if (sel_work) n_small += (int32_t)((std::min<int64_t>(n, a->top_t) + kSelBlkTokMin - 1) / kSelBlkTokMin);
  }
  static_assert(kAttendWaves == 4 && kSelBlkTokMin == 4 * 4 && kSelBlkTok == 4 * 16,
                "selected blocks: 4 wavefronts of 4 or 16 tokens");
  // selected blocks of 16 tokens (shorter per-lane chains) when the attention
  // launch still fits three work-groups per CU with them, else of 64
  static const int cus = device_cus();
  const int32_t sel_blk_tok =
      (int64_t)(n_small + n_split) * geom->n_kv_heads <= 3 * (int64_t)cus ? kSelBlkTokMin : kSelBlkTok;
  int32_t n_sel_blk = 0;
  for (int i = 0; i < B && sel_work; ++i)
    n_sel_blk += (int32_t)((std::min<int64_t>(off[i + 1] - off[i], a->top_t) + sel_blk_tok - 1) / sel_blk_tok);
  if (max_seq / split + 1 + (a->top_t + sel_blk_tok - 1) / sel_blk_tok > kCombineMax) return SF_ERR_UNSUPPORTED;

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  DecodeParams p{};
  p.batch = B;
  p.hq = geom->n_q_heads;
  p.hkv = geom->n_kv_heads;
  p.grp = geom->n_q_heads / geom->n_kv_heads;
  p.b = geom->base_bits;
  p.r = geom->refine_bits;
  p.top_t = a->top_t;
  p.score_split = score_split;
  p.split = split;
  p.sel_chunk = kSelChunk;
  p.n_score_split = n_score;
  p.n_split = n_split;
  p.bm_words = (int32_t)(((max_seq + kSelThreads - 1) / kSelThreads) * (kSelThreads / 32));
  p.use_refine = sel_work ? 1 : 0;
  p.drop = drop ? 1 : 0;
  p.score_mode = smax ? 1 : 0;
  p.rows16 = static_cast<const _Float16*>(a->rows16);
  p.sstat = reinterpret_cast<float2*>(ws + c.sstat);
  p.n_sel_blk = n_sel_blk;
  p.sel_blk_tok = sel_blk_tok;
  p.cnt_stride = (int32_t)((max_seq + kSelChunk - 1) / kSelChunk) + 2;   // + level-1 boundary
  p.cap = a->cap;
  p.ntot = total;
  p.off0 = off[0];
  p.max_seq = max_seq;
  p.seq_off = a->seq_off_dev;
  p.q = a->q;
  p.kc = a->k_codes;
  p.ks = a->k_scales;
  p.vc = a->v_codes;
  p.vs = a->v_scales;
  p.scores = a->scores_out ? a->scores_out : reinterpret_cast<float*>(ws + c.scores);
  p.logits = reinterpret_cast<float*>(ws + c.logits);
  p.hist = reinterpret_cast<uint32_t*>(ws + c.hist);
  p.counters = reinterpret_cast<uint32_t*>(ws + c.counters);
  p.cand = reinterpret_cast<uint2*>(ws + c.cand);
  p.bitmap = reinterpret_cast<uint32_t*>(ws + c.bitmap);
  p.sel = reinterpret_cast<int32_t*>(ws + c.sel);
  p.sel_out = a->sel_out;
  p.part = reinterpret_cast<float*>(ws + c.part);
  p.out = a->out;
  p.fr = fr;
  p.fscores = a->scores_out ? 1 : 0;
  p.fsel = a->sel_out ? 1 : 0;
  p.ftie_stride = (int32_t)((max_seq + kFusedMinR - 1) / kFusedMinR);
  p.fz = reinterpret_cast<uint32_t*>(ws + c.hist);
  p.ftie = reinterpret_cast<uint32_t*>(ws + c.ftie);
  p.fstatus = reinterpret_cast<uint32_t*>(ws + c.status);
  if (refine) {
    sf_store_s* st = a->store;
    p.rb = st->row_bytes;
    p.slots = st->slots;
    if (st->tier == SF_TIER_DEVICE) {
      p.ref_rows = st->dev_rows;
    } else {
      p.cache_data = st->cache_data;
      p.tok_slot = st->tok_slot;
      p.store_err = st->err;
    }
  }

  hipStream_t hs = (hipStream_t)stream;
  if (!(a->flags & SF_DECODE_HIST_CLEAN)) {
    // every successful step leaves this region zero again: select_resolve
    // clears its histograms once read, the single-launch path's last
    // work-group of each head its histograms and counters
    const int64_t nzero = (int64_t)(c.zero_end / 4);
    hipLaunchKernelGGL(zero_words, dim3((unsigned)std::min<int64_t>((nzero + 255) / 256, 1024)), dim3(256), 0, hs,
                       reinterpret_cast<uint32_t*>(ws), nzero);
    SF_LAUNCH_CHECK("zero_words");
  }
  const auto stop = [&](int i) { return KernelEvents{(hipEvent_t)a->start_events[i], (hipEvent_t)a->events[i]}; };
  if (fr) {
    if (a->stats) {
      memset(a->stats, 0, sizeof(*a->stats));
      int64_t sel = 0;
      for (int i = 0; i < B; ++i) sel += std::min<int64_t>(off[i + 1] - off[i], a->top_t);
      a->stats->selected = sel * p.hkv;
    }
    if (!launch_fused(p, dim3(n_units, p.hkv), hs, stop(0))) return SF_ERR_UNSUPPORTED;
    SF_LAUNCH_CHECK("fused_decode");
    return SF_OK;
  }
  if (!launch_score(p, dim3(n_score, p.hkv), hs, stop(0)))
    return SF_ERR_UNSUPPORTED;
  SF_LAUNCH_CHECK("score");
  if (smax) {
    if (!launch_softmax_scores(p, dim3(n_score, p.hkv), hs)) return SF_ERR_UNSUPPORTED;
    SF_LAUNCH_CHECK("softmax_scores");
  }
  if (a->top_t > 0) {
    launch_select(p, dim3(n_sel, p.hkv), hs, stop(1), stop(2));
    SF_LAUNCH_CHECK("select_top_t");
  }
  if (a->stats) {
    memset(a->stats, 0, sizeof(*a->stats));
    int64_t sel = 0;
    for (int i = 0; i < B; ++i) sel += std::min<int64_t>(off[i + 1] - off[i], a->top_t);
    a->stats->selected = sel * p.hkv;
  }
  if (refine && a->store->tier == SF_TIER_HOST_PINNED) {
    s = sf_store_fetch(a->store, p, hs, (a->flags & SF_DECODE_SKIP_MISSES) != 0, a->stats);
    if (s != SF_OK) return s;
    if (a->stats) a->stats->hits = a->stats->selected - a->stats->misses;
  }
  if (!launch_attend(p, dim3(n_sel_blk + (drop ? 0 : n_split), p.hkv), hs, stop(3)))
    return SF_ERR_UNSUPPORTED;
  SF_LAUNCH_CHECK("attend");
  launch_combine(p, hs, stop(4));
  SF_LAUNCH_CHECK("combine");
  return SF_OK;
}

extern "C" sf_status sf_decode_step(const sf_geom* geom, const sf_decode_args* a, void* stream) {
  if (!a) return SF_ERR_INVALID_ARG;
  return sf_decode_step_ws(geom, a, a->workspace, a->workspace_bytes, stream);
}

// The workspace's status word (the library's scratch when `workspace` is NULL).
sf_status sf_noalloc_scratch(void** out);

extern "C" sf_status sf_decode_check(void* workspace, void* stream) {
  clear_error();
  void* ws = workspace;
  if (!ws) {
    const sf_status s = sf_noalloc_scratch(&ws);
    if (s != SF_OK) return s;
  }
  hipStream_t hs = (hipStream_t)stream;
  uint32_t st = 0;
  SF_HIP_CHECK(hipMemcpyAsync(&st, ws, 4, hipMemcpyDeviceToHost, hs));
  SF_HIP_CHECK(hipStreamSynchronize(hs));
  if (st == 0) return SF_OK;
  const uint32_t zero = 0;
  SF_HIP_CHECK(hipMemcpyAsync(ws, &zero, 4, hipMemcpyHostToDevice, hs));
  SF_HIP_CHECK(hipStreamSynchronize(hs));
  return SF_ERR_TIMEOUT;
}

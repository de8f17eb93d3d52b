/*
 * sf_kv.h -- C ABI of the MI355X (gfx950) KV-cache refinement decode step.
 *
 * The method (StrataFlux selective precision streaming, as described on the
 * page "StrataFlux -- Selective precision streaming -- What does it mean?"):
 *   - the GPU keeps a resident low-bit KV cache: b-bit codes per element plus
 *     a per-row scale (paragraph "Think about how a map app ...");
 *   - each decode step scores every cached token against the current query
 *     from the resident low-bit keys and picks the highest-scoring tokens per
 *     KV head, a set shared by that head's GQA group of query heads
 *     (paragraph "Which tiles count ...");
 *   - the selected tokens' keys and values are refined with r extra bits that
 *     subdivide the bin the base code already names (nested quantization,
 *     paragraph "What travels over the link ...");
 *   - attention runs over all tokens; unselected ones keep their low-bit value
 *     (same paragraph; comparison table, row "StrataFlux");
 *   - fetched refinement bits are kept and reused across steps (paragraph
 *     "The map app also loads tiles ...").
 *
 * Conventions for every call:
 *   - Pointers marked "device" are HIP device memory (hipMalloc or torch CUDA
 *     tensors); "host" pointers are ordinary host memory.  The caller owns
 *     every buffer it passes; the library never frees caller memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously on it unless stated otherwise.
 *   - Every call returns an sf_status and never throws.  Arguments are checked
 *     before anything is enqueued: SF_ERR_INVALID_ARG / SF_ERR_UNSUPPORTED
 *     mean nothing was written.  SF_ERR_HIP reports a HIP launch or copy
 *     failure (sf_last_error_string() gives HIP's message).
 *   - Inputs must be finite, with a finite max - min per row.
 *
 * Layouts (D = head_dim, Hkv = n_kv_heads, b = base_bits, r = refine_bits):
 *   - a "row" is one token of one KV head: D values of K or of V;
 *   - packed codes: each row is one little-endian bitstream, element d at bits
 *     [w*d, w*d + w) (w = b for base codes, w = r for refinement codes), so a
 *     row takes D*w/8 bytes;
 *   - caches are head-major: codes [Hkv][cap][D*b/8] uint8, scales
 *     [Hkv][cap][2] float = {lo, delta} with lo the row minimum and delta the
 *     base bin width (max - min) / 2^b;
 *   - a batch of sequences is packed along the token axis: sequence s owns
 *     tokens [seq_off[s], seq_off[s+1]) of every head.
 */
#ifndef SF_KV_H
#define SF_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sf_status {
  SF_OK = 0,
  SF_ERR_INVALID_ARG = -1, /* bad pointer, size or combination; nothing written */
  SF_ERR_UNSUPPORTED = -2, /* valid but not built for (e.g. head_dim != 128)  */
  SF_ERR_HIP = -3,         /* a HIP call failed                                */
  SF_ERR_OOM = -4,         /* device or pinned host allocation failed          */
  SF_ERR_TIMEOUT = -5,     /* a bounded wait on the device expired             */
  SF_ERR_STATE = -6        /* a consistency check of the store failed          */
} sf_status;

/* Attention geometry and code widths.  Supported: head_dim == 128;
 * n_q_heads % n_kv_heads == 0 with group G = n_q_heads / n_kv_heads <= 8;
 * base_bits in {2, 3, 4}; refine_bits in [0, 8]. */
typedef struct sf_geom {
  int32_t head_dim;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t base_bits;
  int32_t refine_bits;
} sf_geom;

/* Human-readable name of a status. */
const char* sf_status_string(sf_status s);
/* HIP's message for the last SF_ERR_HIP on this thread ("" if none). */
const char* sf_last_error_string(void);

/*
 * sf_kv_quantize -- quantize and place rows of K or V (nested quantization,
 * paragraph "What travels over the link ...").  Call once for K, once for V.
 *
 * Per row x[0..D): lo = min x, hi = max x, R = hi - lo (fp32),
 * delta = R * 2^-b, delta_f = R * 2^-(b+r); fine code
 * q_d = min(floor((x_d - lo) / delta_f), 2^(b+r) - 1) with one fp32
 * subtraction and one correctly rounded fp32 division (q_d = 0 when
 * delta_f == 0); base code c_d = q_d >> r, refinement code s_d = q_d & (2^r-1).
 *
 *   x            device, [n_tok][Hkv][D] fp32, token-major
 *   n_tok        rows per head to quantize (>= 0; 0 is a no-op)
 *   tok_begin    first token slot written in the cache, tok_begin + n_tok <= cap
 *   cap          token capacity (row pitch) of codes/scales
 *   codes        device, [Hkv][cap][D*b/8]; rows tok_begin.. are written
 *   scales       device, [Hkv][cap][2]; {lo, delta} written for the same rows
 *   refine_rows  device, [Hkv][n_tok][D*r/8] refinement codes; NULL iff r == 0
 */
sf_status sf_kv_quantize(const sf_geom* geom, const float* x, int64_t n_tok,
                         int64_t tok_begin, int64_t cap, uint8_t* codes,
                         float* scales, uint8_t* refine_rows, void* stream);

/* sf_kv_quantize_ex flags: fp16 scale storage (the pages fix no scale
 * format; 4 bytes per row instead of 8).  lo is the row minimum rounded down
 * to IEEE fp16 and delta = (max - lo) * 2^-b rounded up to fp16, so that lo +
 * 2^b delta still reaches the maximum; the codes are measured against those
 * values (one fp32 subtraction, one fp32 division by delta * 2^-r, clamped
 * to the top code).  The scales land in the same [Hkv][cap][2] fp32 slots,
 * holding fp16 values, so the decode step reads them unchanged.  Rows must
 * lie within the fp16 range. */
#define SF_QUANT_FP16_SCALES 1

/* sf_kv_quantize with flags (0 or SF_QUANT_FP16_SCALES); same arguments and
 * errors otherwise. */
sf_status sf_kv_quantize_ex(const sf_geom* geom, const float* x, int64_t n_tok, int64_t tok_begin, int64_t cap,
                            uint8_t* codes, float* scales, uint8_t* refine_rows, int32_t flags, void* stream);

/* ---------------------------------------------------------------------------
 * Weight-side refinement GEMV (page "StrataFlux -- Selective precision
 * streaming -- What does it mean?", paragraph "Which tiles count ...": the
 * input channels of a projection are split into chunks of 1,024 and the k
 * channels with the largest activation magnitude in each chunk are refined at
 * this step; paragraph "What travels over the link ...": the refinement bits
 * subdivide the bin of the resident code; the worked example: k = 32, 4-bit
 * refinements of 3-bit weights).
 *
 * y = W x with W [m][k]: along each output row, groups of 128 input channels
 * are quantized with the nested quantizer of sf_kv_quantize (b-bit base code,
 * r refinement bits, fp32 (lo, delta) per group).  The step selects, per chunk
 * of `chunk` input channels, the top_k channels of largest |x| (ties to the
 * lower index) and uses their refined weights; the other channels use the
 * base weights (bin centres).
 * ------------------------------------------------------------------------- */
typedef struct sf_wgeom {
  int32_t m;            /* output rows, a multiple of 32                         */
  int32_t k;            /* input channels, a multiple of 128, at most 15,360
                           (x is staged in LDS; SF_ERR_UNSUPPORTED above)        */
  int32_t base_bits;    /* b: 2, 3 or 4                                          */
  int32_t refine_bits;  /* r: 1 .. 8                                             */
  int32_t top_k;        /* channels refined per chunk, 0 <= top_k <= chunk       */
  int32_t chunk;        /* input channels per selection chunk, 1 .. 4096 (1,024
                           on the page); the last chunk may be shorter           */
} sf_wgeom;

/* Quantize W (device [m][k] fp32, row-major) into
 *   codes        device [m][k*b/8]: per row, per group of 128 channels an
 *                LSB-first bitstream of the b-bit base codes
 *   scales       device [m][k/128][2] fp32 {lo, delta}
 *   refine_cols  device [k][m*r/8]: per input channel, the r-bit refinement
 *                codes of every output row (LSB-first bitstream over rows):
 *                a selected channel's column is what crosses the link
 *   scratch      device, m*k*r/8 bytes (the codes row-major before the
 *                transpose)
 * All pointers 16-byte aligned.  SF_ERR_INVALID_ARG for a bad shape. */
sf_status sf_w_quantize(const sf_wgeom* g, const float* w, uint8_t* codes, float* scales, uint8_t* refine_cols,
                        uint8_t* scratch, void* stream);

/* Words of the workspace sf_w_gemv takes: 514 + 2 ceil(k / chunk)
 * min(top_k, chunk). */
sf_status sf_w_gemv_workspace_words(const sf_wgeom* g, int32_t* words);

/* y = W x as above: x device [k] fp32, y device [m] fp32, sel device int32
 * [ceil(k/chunk) * min(top_k, chunk)]: the selected channels, ascending within
 * each chunk (written by the call; a shorter last chunk pads with -1).
 * workspace: device uint32 [sf_w_gemv_workspace_words], zero-filled before
 * its first use and then left to the calls: counters that every call's
 * wavefronts advance (they give the call its epoch on the device, so that
 * captured graphs replay correctly), the selection tagged with the epoch,
 * and a status word.  A workspace serves one geometry: calls with another
 * geometry need a workspace of their own (zero-filled).  One kernel on
 * `stream`: its first work-groups select the channels, the others compute
 * the rows and take the selection once it carries the call's epoch (a
 * bounded wait, about 0.2 s) to add the refined channels.  A wait that
 * expires sets the status word (the last workspace word) nonzero and leaves
 * NaN in the rows concerned.  Calls that share a workspace must not overlap.
 * x, scales, codes and workspace 16-byte aligned, else SF_ERR_INVALID_ARG. */
sf_status sf_w_gemv(const sf_wgeom* g, const uint8_t* codes, const float* scales, const uint8_t* refine_cols,
                    const float* x, float* y, int32_t* sel, uint32_t* workspace, void* stream);

/* ---------------------------------------------------------------------------
 * Refinement store and device refinement cache.
 *
 * The store holds the refinement codes of every cached row (paragraph "Think
 * about how a map app ...": the refinement bits live off the GPU, in host RAM
 * on a machine with a dedicated GPU).  SF_TIER_DEVICE keeps them in HBM (no
 * link, no cache); SF_TIER_HOST_PINNED keeps them in pinned host memory and
 * gives each (sequence slot, KV head) a device cache of `cache_slots` rows
 * that reuses fetched bits across steps (paragraph "The map app also loads
 * tiles ..."): a selected resident is a hit; each miss is read over the link
 * by a kernel, straight from the pinned store, into a free slot, else in
 * place of the resident not selected now that was selected longest ago
 * (lower token index first).  Misses are waited for (policy "wait"); the
 * step involves no host work and no synchronization.
 * All memory is allocated by sf_store_create and freed by sf_store_destroy.
 * A store must not be used from two streams at once.
 * ------------------------------------------------------------------------- */
typedef struct sf_store_s* sf_store;

enum { SF_TIER_DEVICE = 0, SF_TIER_HOST_PINNED = 1 };
enum { SF_K = 0, SF_V = 1 };

/* cap_tokens: token capacity, the row pitch of the caches the store is used
 * with (sf_decode_args.cap must equal it); max_seqs: batch slots with a cache
 * of their own; cache_slots: rows per (seq, KV head) cache, 1 <= cache_slots
 * <= 4096 and >= every top_t used with the store (so a host-tier store serves
 * T <= 4096; with the usual 2T slots, T <= 2048).  cache_slots is ignored for
 * SF_TIER_DEVICE.  Returns SF_ERR_OOM, with nothing left allocated, when a
 * device or pinned host allocation is refused.
 *
 * Batch positions (host tier): the cache of batch position s serves the tokens
 * [seq_off[s], seq_off[s+1]) of the steps that use it.  A position must keep
 * its token range from step to step (a sequence may grow at its end); after
 * the batch is reordered or sequences are dropped, call sf_store_clear_cache.
 * A token whose cached rows belong to another position's cache is a miss. */
sf_status sf_store_create(const sf_geom* geom, int64_t cap_tokens, int32_t max_seqs,
                          int32_t tier, int32_t cache_slots, sf_store* out);
sf_status sf_store_destroy(sf_store store);

/*
 * sf_refine_store -- put refinement rows produced by sf_kv_quantize into the
 * store at tokens [tok_begin, tok_begin + n_tok) of every head.
 *   which        SF_K or SF_V
 *   refine_rows  device, [Hkv][n_tok][D*r/8]
 * Rows already cached on the device for those tokens are invalidated.
 * Stream-ordered for both tiers, nothing waits on the host: refine_rows must
 * stay valid until `stream` has run the copy.  For SF_TIER_HOST_PINNED a
 * kernel writes the rows into the pinned store through its mapped device
 * address (and invalidates in the same launch).
 */
sf_status sf_refine_store(sf_store store, int32_t which, const uint8_t* refine_rows,
                          int64_t tok_begin, int64_t n_tok, void* stream);

/* Drop every cached refinement row (next step misses on every selection). */
sf_status sf_store_clear_cache(sf_store store, void* stream);

/* Debug check of the store (synchronizes `stream`): for a host-pinned store,
 * every token -> slot entry of the device cache must name a slot of its KV
 * head that holds that token, and no decode step since the last check may
 * have found a selected token without its cached rows.  Returns SF_OK, or
 * SF_ERR_STATE (and clears the recorded error).  A device-tier store always
 * passes. */
sf_status sf_store_check(sf_store store, void* stream);

/* ---------------------------------------------------------------------------
 * Decode step.
 * ------------------------------------------------------------------------- */
typedef struct sf_step_stats {
  int64_t selected;   /* selected (token, KV head) pairs in the step        */
  int64_t hits;       /* of those, found in the device refinement cache    */
  int64_t misses;     /* fetched over the link                             */
  int64_t h2d_bytes;  /* refinement bytes copied host -> device            */
} sf_step_stats;

/* sf_decode_args.flags: the score-key histogram at the start of the workspace
 * is already zero, so the step skips clearing it.  Every successful step
 * leaves it zero; it holds for a workspace that the previous successful step
 * used with the same batch size and KV-head count, or that the caller
 * zero-filled.  Do not pass it after a failed step. */
#define SF_DECODE_HIST_CLEAN 1

/* sf_decode_args.flags: policy "skip" on a refinement-cache miss (page
 * "StrataFlux -- Selective precision streaming -- What does it mean?",
 * paragraph "The map app also loads tiles ...": on a miss the runtime may
 * use the low-bit value now while the bits are loaded for later steps).
 * With a host-pinned store, a selected token whose refinement rows are not
 * cached takes part in this step at base precision; its rows are read over
 * the link on the store's own side stream, beside the attention, and
 * installed for later steps (the store's next call waits for that read).
 * Hits, misses and bytes are counted as under the default policy, "wait",
 * where every miss is fetched before the attention.  No effect with a
 * device-tier store (nothing misses).  A step with this flag must not be
 * captured into a graph (it forks onto the side stream). */
#define SF_DECODE_SKIP_MISSES 2

/* sf_decode_args.flags: run the step as its five kernels (score, selection
 * scan, selection resolve, attention, combine) even where the single-launch
 * form applies.  The single-launch form is taken for 2-bit base codes, GQA
 * groups of 1, 2 or 4, a device-tier store (or none), policy "wait", and
 * steps whose work-groups (ranges of at most 4,096 tokens of one KV head) are
 * all resident on the device at once; it reads the K and V codes once and
 * gives the same selection and outputs within the tolerances of the
 * multi-pass form (different summation order). */
#define SF_DECODE_MULTI_PASS 4

/* sf_decode_args.flags, the comparison variants of page "StrataFlux --
 * Selective precision streaming -- What does it mean?" (paragraph "What
 * travels over the link ..." and the comparison table); each runs the step
 * as its five kernels.
 *
 * SF_DECODE_DROP_UNSELECTED: the unselected tokens are left out of the
 * attention (table row "Sparse attention"): the softmax runs over the
 * selected tokens alone.  Needs top_t > 0 and refinement (r > 0 and a
 * store) or SF_DECODE_ROWS16.
 *
 * SF_DECODE_ROWS16: the selected tokens take their complete 16-bit K and V
 * rows (table row "SpeCache (16-bit fetching)"): args.rows16 holds, in
 * device memory, [2][Hkv][cap][D] IEEE fp16 rows, K then V; the store and
 * the refinement codes are not read.  Needs top_t > 0.
 *
 * SF_DECODE_SCORE_SOFTMAX: a token's score is the attention it receives
 * (paragraph "Which tiles count ..."): the sum over its KV head's group of
 * the softmax probability, over the sequence's tokens, of q_h . Khat_i /
 * sqrt(D) (the logits from the base keys), instead of the maximum logit.
 * Supported for groups of 1, 2 or 4 query heads (a group of 8:
 * SF_ERR_UNSUPPORTED). */
#define SF_DECODE_DROP_UNSELECTED 8
#define SF_DECODE_ROWS16 16
#define SF_DECODE_SCORE_SOFTMAX 32

typedef struct sf_decode_args {
  int32_t batch;                 /* B >= 1 sequences                                    */
  const int64_t* seq_off_host;   /* host [B+1], nondecreasing, every sequence non-empty,
                                    seq_off[B] <= cap                                   */
  const int64_t* seq_off_dev;    /* device copy of the same [B+1] offsets               */
  const float* q;                /* device [B][Hq][D] fp32 current queries              */
  const uint8_t* k_codes;        /* device [Hkv][cap][D*b/8] base key codes             */
  const float* k_scales;         /* device [Hkv][cap][2]                                */
  const uint8_t* v_codes;        /* device [Hkv][cap][D*b/8] base value codes           */
  const float* v_scales;         /* device [Hkv][cap][2]                                */
  int64_t cap;                   /* token capacity of the caches                        */
  sf_store store;                /* refinement store; may be NULL iff top_t == 0 or r == 0 */
  int32_t top_t;                 /* T >= 0 tokens refined per (sequence, KV head);
                                    all tokens when the sequence has <= T               */
  float* out;                    /* device [B][Hq][D] fp32 attention output             */
  int32_t* sel_out;              /* optional device [B][Hkv][T]: selected token indices
                                    (relative to the sequence start), ascending, -1 pad */
  float* scores_out;             /* optional device [Hkv][seq_off[B]-seq_off[0]] fp32:
                                    the token scores the selection used                 */
  sf_step_stats* stats;          /* optional host; filled when the call returns (for the
                                    host tier the call then waits for the step's miss
                                    lists: pass NULL to keep the step asynchronous)     */
  void* workspace;               /* device scratch of sf_decode_workspace_size() bytes  */
  size_t workspace_bytes;
  int32_t flags;                 /* 0 or SF_DECODE_HIST_CLEAN | SF_DECODE_SKIP_MISSES |
                                    SF_DECODE_MULTI_PASS | SF_DECODE_DROP_UNSELECTED |
                                    SF_DECODE_ROWS16 | SF_DECODE_SCORE_SOFTMAX          */
  void* start_events[5];         /* optional hipEvent_t pairs (NULL = none) that time the */
  void* events[5];               /* step's kernels: start_events[k] is recorded just
                                    before kernel k is dispatched, events[k] completes
                                    with it: [0] score, [1] selection scan, [2] selection
                                    resolve, [3] attention, [4] combine.  The selection
                                    pair is not recorded when T == 0.  A single-launch
                                    step records pair [0] only, around its one kernel.
                                    elapsed(start, stop) is the kernel's time (create
                                    both without the system-scope fence).               */
  const void* rows16;            /* device [2][Hkv][cap][D] fp16 K and V rows for
                                    SF_DECODE_ROWS16, else NULL                         */
} sf_decode_args;

/* Scratch needed by sf_decode_step for this batch shape.
 *   total_tokens   seq_off[B] - seq_off[0]
 *   max_seq_tokens the longest sequence */
sf_status sf_decode_workspace_size(const sf_geom* geom, int32_t batch, int64_t total_tokens,
                                   int64_t max_seq_tokens, int32_t top_t, size_t* bytes);

/*
 * sf_decode_step -- one decode step of one layer for a packed batch.
 *
 * For each sequence s and KV head k (query head h belongs to KV head
 * floor(h / G)):
 *   1. score every token i of s from the resident base keys:
 *      s_i = max over h in k's group of q_h . Khat_i / sqrt(D), where
 *      Khat = lo + (c + 1/2) * delta (centre of the bin the code names);
 *   2. select the T highest scores (ties to the lower token index);
 *   3. refine the selected K and V rows with the stored r-bit codes:
 *      Ktilde = lo + c * delta + (s + 1/2) * delta / 2^r;
 *   4. out_h = softmax over all tokens of q_h . K* / sqrt(D), applied to V*,
 *      with K*, V* refined for selected tokens and base-precision otherwise.
 * Kernels: score (reads the K codes), select, attention (reads the V codes
 * and, for 2-bit base codes with G <= 4, the per-head logits the score pass
 * left, else the K codes again; and the refinement rows of the selection),
 * combine; a host-pinned
 * store adds, after the selection, the cache lookup and a kernel that reads
 * the missed rows over the link.  No call waits on the host unless `stats`
 * is given with a host-pinned store.
 * The workspace need not be initialised (unless SF_DECODE_HIST_CLEAN is
 * passed); apart from the histogram it leaves zero, its contents are
 * undefined after the call.
 */
sf_status sf_decode_step(const sf_geom* geom, const sf_decode_args* args, void* stream);

/* The form sf_decode_step would take for these arguments, without running
 * it: *kernels = 1 (the single launch) or 5 (score, selection scan and
 * resolve, attention, combine).  Only geometry, batch, offsets, top_t, store
 * and flags are read. */
sf_status sf_decode_form(const sf_geom* geom, const sf_decode_args* args, int32_t* kernels);

/*
 * sf_decode_check -- status of the steps run on a workspace (NULL: the
 * scratch of sf_decode_step_noalloc on the current device).  Synchronizes
 * `stream`.  The single-launch form waits inside its kernel for the other
 * work-groups of a KV head; those waits are bounded (about 0.2 s), and
 * one that expires (its work-groups were not all resident, e.g. beside other
 * work on the device) leaves that step's outputs undefined and is recorded in
 * the workspace.  Returns SF_ERR_TIMEOUT if any step since the workspace was
 * last cleared (a step without SF_DECODE_HIST_CLEAN clears it) recorded one,
 * and clears the record; else SF_OK.
 */
sf_status sf_decode_check(void* workspace, void* stream);

/*
 * sf_decode_step_noalloc -- sf_decode_step for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same step, with the scratch it needs taken from a buffer
 * the library holds in device memory instead of args->workspace
 * (args->workspace and args->workspace_bytes are ignored, and so is
 * SF_DECODE_HIST_CLEAN: the buffer's histograms are cleared by every call).
 * The call allocates nothing: no hipMalloc, hipFree or allocating library
 * routine.  The buffer, sf_decode_noalloc_max_bytes() bytes per GPU, is held
 * from the library's first use on a GPU until the process ends; a step whose
 * sf_decode_workspace_size() exceeds it is refused with SF_ERR_UNSUPPORTED
 * before anything is enqueued (use sf_decode_step with a workspace of its
 * own).  All calls on one GPU share that GPU's buffer: calls that overlap on
 * one GPU (several streams or threads) race on it and must be serialized by
 * the caller.  Everything else is as sf_decode_step.
 */
sf_status sf_decode_step_noalloc(const sf_geom* geom, const sf_decode_args* args, void* stream);

/* Size of the device buffer of sf_decode_step_noalloc (96 MiB). */
size_t sf_decode_noalloc_max_bytes(void);


/*
 * sf_stream_read -- measurement utility: read `bytes` of device memory at
 * `buf` once (16-byte pieces, `blocks` work-groups of 256 threads in a
 * grid-stride loop), the reference for the bandwidth a streaming kernel can
 * reach on the device.  `sink` (device, `blocks` words) is written only where
 * a work-group's fold of the data equals `never` (pass a value the data rules
 * out).  buf 16-byte aligned, bytes a multiple of 16.  Asynchronous on
 * `stream`.
 */
sf_status sf_stream_read(const void* buf, size_t bytes, uint32_t never, uint32_t* sink, int32_t blocks,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SF_KV_H */

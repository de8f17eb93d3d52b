// sf_decode_step_noalloc: the decode step on a scratch buffer that the
// library holds in device memory, for callers that cannot allocate (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The scratch is one file-scope device array of kScratchBytes per GPU.  Its
// device address is looked up once per device (hipGetSymbolAddress, with that
// device current, on the entry point's first call there) and kept; host code
// passes only that address to the kernels, never the array's name.  Every
// call on a GPU shares the array and finds the previous call's contents, so
// each call clears the part that must start at zero (the selection
// histograms); calls that overlap on one GPU race on the scratch.
#include <stdio.h>

#include <mutex>

#include "sf_internal.h"

namespace sfk {

constexpr size_t kScratchBytes = (size_t)96 << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

static void* g_scratch[kMaxDevices];
static std::mutex g_scratch_mu;

// The scratch's device address on the current device (looked up once).
static sf_status scratch_ptr(void** out) {
  int dev = 0;
  SF_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return SF_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    SF_HIP_CHECK(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (!ptr) return SF_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return SF_OK;
}

}  // namespace sfk

sf_status sf_noalloc_scratch(void** out) { return sfk::scratch_ptr(out); }

sf_status sf_decode_step_ws(const sf_geom* geom, const sf_decode_args* a, void* workspace, size_t workspace_bytes,
                            void* stream);

extern "C" size_t sf_decode_noalloc_max_bytes(void) { return sfk::kScratchBytes; }

extern "C" sf_status sf_decode_step_noalloc(const sf_geom* geom, const sf_decode_args* a, void* stream) {
  sfk::clear_error();
  sf_status s = sf_check_geom(geom);
  if (s != SF_OK) return s;
  if (!a || a->batch <= 0 || !a->seq_off_host || a->top_t < 0) return SF_ERR_INVALID_ARG;
  int64_t total = 0, max_seq = 0;
  for (int i = 0; i < a->batch; ++i) {
    const int64_t n = a->seq_off_host[i + 1] - a->seq_off_host[i];
    if (n <= 0) return SF_ERR_INVALID_ARG;
    total += n;
    max_seq = n > max_seq ? n : max_seq;
  }
  size_t need = 0;
  s = sf_decode_workspace_size(geom, a->batch, total, max_seq, a->top_t, &need);
  if (s != SF_OK) return s;
  if (need > sfk::kScratchBytes) {   // beyond the scratch: use sf_decode_step
    char msg[160];
    snprintf(msg, sizeof(msg), "sf_decode_step_noalloc: the step needs %zu bytes of scratch, more than the %zu held",
             need, sfk::kScratchBytes);
    sfk::set_error_text(msg);
    return SF_ERR_UNSUPPORTED;
  }
  void* ws = nullptr;
  s = sfk::scratch_ptr(&ws);
  if (s != SF_OK) return s;
  sf_decode_args b = *a;
  b.flags &= ~SF_DECODE_HIST_CLEAN;   // the scratch's histograms are cleared by every call
  return sf_decode_step_ws(geom, &b, ws, sfk::kScratchBytes, stream);
}

// sf_stream_read: a plain streaming read of a device buffer, the reference
// for the bandwidth the decode kernels can reach on this device (their bound
// is HBM bandwidth: they stream packed codes and scales once per step).
//
// Each thread reads 16-byte pieces in a grid-stride loop, four loads in
// flight, and folds them into one word; a work-group writes its fold only if
// it equals a value the caller rules out, so the reads cannot be dropped and
// nothing is written in practice.
#include "sf_internal.h"

namespace sfk {

constexpr int kProbeThreads = 256;

__global__ void __launch_bounds__(kProbeThreads) stream_read(const uint4* __restrict__ p, uint64_t n16,
                                                             uint32_t never, uint32_t* sink) {
  const uint64_t stride = (uint64_t)gridDim.x * kProbeThreads;
  uint64_t i = (uint64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = p[i];
    const uint4 b = p[i + stride];
    const uint4 c = p[i + 2 * stride];
    const uint4 d = p[i + 3 * stride];
    acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n16; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == never) sink[blockIdx.x] = acc;
}

}  // namespace sfk

extern "C" sf_status sf_stream_read(const void* buf, size_t bytes, uint32_t never, uint32_t* sink, int32_t blocks,
                                    void* stream) {
  sfk::clear_error();
  if (!buf || !sink || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(buf) & 15) != 0 || blocks <= 0)
    return SF_ERR_INVALID_ARG;
  hipLaunchKernelGGL(sfk::stream_read, dim3((unsigned)blocks), dim3(sfk::kProbeThreads), 0, (hipStream_t)stream,
                     static_cast<const uint4*>(buf), (uint64_t)(bytes / 16), never, sink);
  SF_LAUNCH_CHECK("stream_read");
  return SF_OK;
}

// Measurement utility: the HBM streaming-read rate this GPU reaches with
// plain or non-temporal 16-byte loads, the ceiling the attention kernels'
// achieved bandwidth is compared with.  Not part of the decode step.
#include "kvev_internal.h"

namespace kvev {
namespace {

typedef unsigned int u32x4c __attribute__((ext_vector_type(4)));
constexpr int kCalNT = 256, kCalUnroll = 8;

// Grid-stride over n 16-byte elements, kCalUnroll independent loads per
// thread and iteration, folded by XOR so that no load is dead; one word per
// block is written.
template <bool NT>
__global__ __launch_bounds__(kCalNT) void stream_read_kernel(const u32x4c* __restrict__ buf, int64_t n,
                                                            uint32_t* __restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kCalNT;
  u32x4c acc = {0u, 0u, 0u, 0u};
  int64_t i = static_cast<int64_t>(blockIdx.x) * kCalNT + threadIdx.x;
  for (; i + (kCalUnroll - 1) * stride < n; i += kCalUnroll * stride) {
    u32x4c v[kCalUnroll];
#pragma unroll
    for (int u = 0; u < kCalUnroll; ++u) v[u] = NT ? __builtin_nontemporal_load(buf + i + u * stride) : buf[i + u * stride];
#pragma unroll
    for (int u = 0; u < kCalUnroll; ++u) acc ^= v[u];
  }
  for (; i < n; i += stride) acc ^= NT ? __builtin_nontemporal_load(buf + i) : buf[i];
  __shared__ uint32_t red[kCalNT / kWave];
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, kWave);
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
#pragma unroll
    for (int w = 0; w < kCalNT / kWave; ++w) y ^= red[w];
    sink[blockIdx.x] = y;
  }
}

}  // namespace
}  // namespace kvev

extern "C" kvev_status kvev_calibrate_read(const void* buf, int64_t bytes, int32_t nontemporal, int32_t blocks,
                                           uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes <= 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0 || blocks <= 0)
    return KVEV_EINVAL;
  const auto* b = static_cast<const kvev::u32x4c*>(buf);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (nontemporal)
    kvev::stream_read_kernel<true><<<blocks, kvev::kCalNT, 0, s>>>(b, bytes / 16, sink);
  else
    kvev::stream_read_kernel<false><<<blocks, kvev::kCalNT, 0, s>>>(b, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? KVEV_OK : KVEV_EHIP;
}

// Measurement only: a plain streaming read of device memory, the floor the decode's
// split pass is measured against.  It is not part of the attention computation.
//
// One 64-lane wave per workgroup; wave w reads the contiguous span
// [w*span, (w+1)*span) of 16-byte elements (span = ceil(n / waves)) with non-temporal
// 16-byte loads, eight per lane in flight, as the decode's split waves read their
// chunks.  The loaded words are folded into one checksum per lane, which is stored only
// if it equals a sentinel, so the loads cannot be dropped and nothing is written.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

__global__ __launch_bounds__(64) void measure_read_kernel(const u32x4* __restrict__ p, size_t n16, size_t span,
                                                          uint32_t* sink) {
  constexpr int U = 8;
  const size_t s0 = (size_t)group_x() * span;
  const size_t s1 = s0 + span < n16 ? s0 + span : n16;
  uint32_t acc = 0;
  for (size_t i = s0 + thread_x(); i < s1; i += 64 * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = (i + u * 64 < s1) ? __builtin_nontemporal_load(p + i + u * 64) : (u32x4){0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == 0x9e3779b9u) sink[(size_t)group_x() * 64 + thread_x()] = acc;
}

hipError_t launch_measure_read(const void* buf, size_t bytes, int waves, uint32_t* sink, hipStream_t st) {
  const size_t n16 = bytes / 16;
  const size_t span = (n16 + waves - 1) / waves;
  hipLaunchKernelGGL(measure_read_kernel, dim3(waves), dim3(64), 0, st, (const u32x4*)buf, n16, span, sink);
  return hipGetLastError();
}

}  // namespace attn

// Plain streaming read of one or two device buffers (declared in
// include/bnbx_probe.h): the achievable read rate for a given size, the
// ceiling the decode GEMV's HBM fraction is read against.
//
// Every thread loads 16-byte units t, t + T, t + 2T, ... (T threads in the
// grid; kRUnroll loads in flight at a time, indices past the end load unit 0
// and are discarded), folds them into an XOR, and the workgroup's XOR goes
// to sink[workgroup].  Non-temporal loads, as the GEMV streams its weights.
// Of the shapes timed on MI355X back to back in a graph (128-1024 threads
// per workgroup, 1-4 loads in flight per thread, up to 8192 workgroups),
// 512-thread workgroups, one load per thread per round and at most 1024
// workgroups were fastest at both decode sizes (8.65 MB: 3.5 us, 23.2 MB:
// 5.6 us per launch).
#include "../../include/bnbx_probe.h"
#include "bnbx_device.hpp"
#include "bnbx_internal.hpp"

namespace bnbx {
namespace {

constexpr int kRThreads = 512;
constexpr int kRUnroll = 1;

__global__ __launch_bounds__(kRThreads) void stream_read_kernel(
    const uint4* __restrict__ a, uint64_t na, const uint4* __restrict__ b, uint64_t nb,
    uint32_t* __restrict__ sink) {
  __shared__ uint32_t red[kRThreads / 64];
  const uint64_t total = na + nb;
  const uint64_t T = (uint64_t)gridDim.x * kRThreads;
  uint32_t acc = 0;
  for (uint64_t i = (uint64_t)blockIdx.x * kRThreads + threadIdx.x; i < total; i += kRUnroll * T) {
    uint4 v[kRUnroll];
#pragma unroll
    for (int u = 0; u < kRUnroll; ++u) {
      uint64_t k = i + (uint64_t)u * T;
      k = k < total ? k : 0;
      const uint4* p = k < na ? a + k : b + (k - na);
      v[u] = load_nt16(p);
    }
#pragma unroll
    for (int u = 0; u < kRUnroll; ++u)
      if (i + (uint64_t)u * T < total) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // XOR over the wave, then over the workgroup's waves.
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
#pragma unroll
    for (int w = 0; w < kRThreads / 64; ++w) r ^= red[w];
    sink[blockIdx.x] = r;
  }
}

}  // namespace
}  // namespace bnbx

extern "C" int bnbx_probe_stream_read(const void* a, size_t a_bytes, const void* b,
                                      size_t b_bytes, uint32_t* sink, void* stream) {
  if ((a == nullptr && a_bytes > 0) || (b == nullptr && b_bytes > 0) || sink == nullptr ||
      a_bytes + b_bytes == 0 || a_bytes % 16 != 0 || b_bytes % 16 != 0)
    return BNBX_E_INVAL;
  if (((uintptr_t)a % 16) != 0 || ((uintptr_t)b % 16) != 0 || ((uintptr_t)sink % 4) != 0)
    return BNBX_E_ALIGN;
  const uint64_t na = a_bytes / 16, nb = b_bytes / 16;
  const uint64_t per_wg = (uint64_t)bnbx::kRThreads * bnbx::kRUnroll;
  uint64_t grid = (na + nb + per_wg - 1) / per_wg;
  if (grid > BNBX_PROBE_SINK_WORDS) grid = BNBX_PROBE_SINK_WORDS;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(bnbx::stream_read_kernel, dim3((unsigned)grid), dim3(bnbx::kRThreads), 0,
                     (hipStream_t)stream, (const uint4*)a, na, (const uint4*)b, nb, sink);
  return hipGetLastError() == hipSuccess ? BNBX_OK : BNBX_E_HIP;
}

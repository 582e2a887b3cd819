// Dequantize NF4 to bfloat16 for gfx950 (mlqm.cn bitsandbytes article, sec.
// 3.4: weights stored in 4 bits are turned back into BF16 for the multiply).
//
// Each lane reads 16 packed bytes (32 weights, half a block), looks up the
// level pair of each byte in an LDS table, multiplies by the block scale in
// binary32 and rounds the pair to bf16 with one v_cvt_pk_bf16_f32, writing
// 64 bytes.  The block scale follows the stored format exactly:
// a_b, or fl32(fl32(q_b * fl32(s_g / 127)) + mean) with double quantization.
#include "bnbx_device.hpp"
#include "bnbx_internal.hpp"

namespace bnbx {
namespace {

constexpr int kDThreads = 256;

__device__ __forceinline__ float level_of(const LevelTable& lv, uint32_t c) {
  float v = lv.level[0];
#pragma unroll
  for (uint32_t i = 1; i < 16; ++i) v = (c == i) ? lv.level[i] : v;
  return v;
}

__device__ __forceinline__ float exact_block_scale(int64_t blk, const void* absmax,
                                                   const float* absmax2, float mu, int dq) {
  if (!dq) return ((const float*)absmax)[blk];
  const float q = (float)((const int8_t*)absmax)[blk];
  const float step = absmax2[blk / kGroup] / 127.0f;   // correctly rounded
  const float prod = q * step;                        // rounded on its own ...
  return prod + mu;                                   // ... then the add (no FMA)
}

__global__ __launch_bounds__(kDThreads) void dequant_kernel(
    const uint8_t* __restrict__ packed, int64_t n, const void* __restrict__ absmax,
    const float* __restrict__ absmax2, const float* __restrict__ mean, int dq,
    uint16_t* __restrict__ out, LevelTable lv) {
  __shared__ float2 tab[256];   // byte -> (L[high nibble], L[low nibble])
  for (int e = threadIdx.x; e < 256; e += kDThreads)
    tab[e] = make_float2(level_of(lv, (uint32_t)e >> 4), level_of(lv, (uint32_t)e & 15u));
  __syncthreads();
  const float mu = dq ? *mean : 0.0f;
  const int64_t nbytes = n >> 1;
  const int64_t nchunks = (nbytes + 15) >> 4;
  for (int64_t c = (int64_t)blockIdx.x * kDThreads + threadIdx.x; c < nchunks;
       c += (int64_t)gridDim.x * kDThreads) {
    const int64_t byte0 = c << 4;
    const float sc = exact_block_scale((byte0 << 1) / kBlock, absmax, absmax2, mu, dq);
    if (byte0 + 16 <= nbytes) {
      const uint4 p = load_nt16(packed + byte0);
      const uint32_t d[4] = {p.x, p.y, p.z, p.w};
      uint32_t o[16];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float2 L = tab[(d[k] >> (8 * i)) & 0xffu];
          o[4 * k + i] = pack_bf16x2(L.x * sc, L.y * sc);
        }
      }
      uint4* dst = (uint4*)(out + (byte0 << 1));
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint4 v;
        v.x = o[4 * k];
        v.y = o[4 * k + 1];
        v.z = o[4 * k + 2];
        v.w = o[4 * k + 3];
        store_nt16(dst + k, v);
      }
    } else {
      for (int64_t b = byte0; b < nbytes; ++b) {
        const float2 L = tab[packed[b]];
        const uint32_t pr = pack_bf16x2(L.x * sc, L.y * sc);
        out[2 * b] = (uint16_t)(pr & 0xffffu);
        out[2 * b + 1] = (uint16_t)(pr >> 16);
      }
    }
  }
}

}  // namespace

hipError_t launch_dequantize(const uint8_t* packed, int64_t n, const void* absmax,
                             const float* absmax2, const float* mean, int double_quant,
                             uint16_t* out, hipStream_t stream) {
  const int64_t nchunks = ((n >> 1) + 15) >> 4;
  int64_t grid = (nchunks + kDThreads - 1) / kDThreads;
  if (grid > 4096) grid = 4096;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)grid), dim3(kDThreads), 0, stream, packed, n,
                     absmax, absmax2, mean, double_quant, out, level_table());
  return hipGetLastError();
}

}  // namespace bnbx

// Dequantize 4-bit codes (NF4 or FP4 levels) to bfloat16 or FP16 for gfx950
// (mlqm.cn bitsandbytes article, sec. 3.4: weights stored in 4 bits are
// turned back into BF16 or FP16 for the multiply; sec. 4: the compute dtype).
//
// Each lane reads 16 packed bytes (32 weights, half a block), looks up the
// level pair of each byte in an LDS table, multiplies by the block scale in
// binary32 and rounds the pair to the compute type (one v_cvt_pk_bf16_f32,
// or two v_cvt_f16_f32), writing 64 bytes.  The block scale follows the stored format exactly:
// a_b, or with double quantization fl32(fl32(q_b * fl32(s_g / 127)) + mean)
// (linear map) or fl32(fl32(map[q_b] * s_g) + mean) (dynamic map, read from
// a copy in LDS).
#include "bnbx_device.hpp"
#include "bnbx_internal.hpp"

namespace bnbx {
namespace {

constexpr int kDThreads = 1024;  // 1024 threads, one chunk per wave per round: measured fastest
constexpr int kDWaves = kDThreads / 64;
constexpr int kChunk = 1024;    // packed bytes per wave per chunk (2048 weights, 32 blocks)
constexpr int kDUnroll = 1;     // chunks per wave per round
// LDS table copies (lane & 3).  At 2 KB apart they share banks, so they do
// not spread conflicts; interleaving them per entry measured the same time
// (8.2 / 21.2 us per call at 4096^2 / 11008x4096): the kernel is bound by
// its HBM writes, not by these reads.
constexpr int kCopies = 4;

template <int DQ>
__device__ __forceinline__ float exact_block_scale(int64_t blk, const void* absmax,
                                                   const float* absmax2, float mu,
                                                   const float* dmap) {
  if (DQ == kDqNone) return ((const float*)absmax)[blk];
  if (DQ == kDqDynamic) {
    const float v = dmap[((const uint8_t*)absmax)[blk]];
    const float prod = v * absmax2[blk / kGroup];
    return prod + mu;
  }
  const float q = (float)((const int8_t*)absmax)[blk];
  const float step = absmax2[blk / kGroup] / 127.0f;   // correctly rounded
  const float prod = q * step;                        // rounded on its own ...
  return prod + mu;                                   // ... then the add (no FMA)
}

// 8 weights (one packed dword) -> 16 bytes of the compute type.
template <bool F16>
__device__ __forceinline__ uint4 expand8(uint32_t d, float sc, const float2* tab) {
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float2 lp = tab[(d >> (8 * i)) & 0xffu];
    o[i] = pack16x2<F16>(lp.x * sc, lp.y * sc);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Wave-level layout: in a 1 KB chunk of packed bytes, lane l handles packed
// dwords l, 64+l, 128+l and 192+l, so every load instruction reads 256
// contiguous bytes and every store instruction writes 1 KB contiguous.
template <int DQ, bool F16>
__global__ __launch_bounds__(kDThreads) void dequant_kernel(
    const uint8_t* __restrict__ packed, int64_t n, const void* __restrict__ absmax,
    const float* __restrict__ absmax2, const float* __restrict__ mean,
    uint16_t* __restrict__ out, LevelTable lv) {
  __shared__ float2 tabs[kCopies][256];   // byte -> (L[high nibble], L[low nibble])
  __shared__ float dmap[DQ == kDqDynamic ? 256 : 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t nbytes = n >> 1;
  const int64_t full = nbytes / kChunk;
  const int64_t gw = (int64_t)blockIdx.x * kDWaves + (tid >> 6);
  const int64_t nw = (int64_t)gridDim.x * kDWaves;

  const int lvl = level_lanes(lv);
  for (int e = tid; e < kCopies * 256; e += kDThreads) {
    const uint32_t b = (uint32_t)e & 255u;
    tabs[e >> 8][b] = make_float2(level_lookup(lvl, b >> 4), level_lookup(lvl, b & 15u));
  }
  if (DQ == kDqDynamic && tid < 256) dmap[tid] = kDynMapDev.v[tid];
  __syncthreads();
  const float2* tab = tabs[lane & (kCopies - 1)];
  const float mu = DQ != kDqNone ? *mean : 0.0f;

  for (int64_t c0 = gw; c0 < full; c0 += nw * kDUnroll) {
    uint32_t d[kDUnroll][4];
    float scl[kDUnroll];
#pragma unroll
    for (int u = 0; u < kDUnroll; ++u) {
      const int64_t c = c0 + u * nw < full ? c0 + u * nw : full - 1;   // clamped, uniform
      const uint32_t* src = (const uint32_t*)(packed + c * kChunk);
#pragma unroll
      for (int k = 0; k < 4; ++k) d[u][k] = __builtin_nontemporal_load(src + k * 64 + lane);
    }
#pragma unroll
    for (int u = 0; u < kDUnroll; ++u) {
      const int64_t c = c0 + u * nw < full ? c0 + u * nw : full - 1;
      // lanes 0..31 each form one of the chunk's 32 block scales
      scl[u] = exact_block_scale<DQ>(c * 32 + (lane & 31), absmax, absmax2, mu, dmap);
    }
#pragma unroll
    for (int u = 0; u < kDUnroll; ++u) {
      const int64_t c = c0 + u * nw;
      if (c < full) {   // wave-uniform
        uint4* dst = (uint4*)(out + c * (2 * kChunk));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          // dword k*64 + lane covers weights 8*(k*64+lane) .. +7: block 8k + lane/8
          const float sc = __int_as_float(
              __builtin_amdgcn_ds_bpermute((8 * k + (lane >> 3)) << 2, __float_as_int(scl[u])));
          store_nt16(dst + k * 64 + lane, expand8<F16>(d[u][k], sc, tab));
        }
      }
    }
  }

  // ragged tail (fewer than 1 KB of packed bytes) on the last wave, bytewise
  if (full * kChunk < nbytes && gw == nw - 1) {
    for (int64_t b = full * kChunk + lane; b < nbytes; b += 64) {
      const float sc = exact_block_scale<DQ>((b << 1) / kBlock, absmax, absmax2, mu, dmap);
      const float2 lp = tab[packed[b]];
      const uint32_t pr = pack16x2<F16>(lp.x * sc, lp.y * sc);
      out[2 * b] = (uint16_t)(pr & 0xffffu);
      out[2 * b + 1] = (uint16_t)(pr >> 16);
    }
  }
}

}  // namespace

hipError_t launch_dequantize(const uint8_t* packed, int64_t n, const void* absmax,
                             const float* absmax2, const float* mean, int double_quant,
                             int quant_type, bool f16, uint16_t* out, hipStream_t stream) {
  const int64_t chunks = (n >> 1) / kChunk;
  int64_t grid = (chunks + kDWaves * kDUnroll - 1) / (kDWaves * kDUnroll);
  if (grid > 2048) grid = 2048;
  if (grid < 1) grid = 1;
  const LevelTable& lv = level_table(quant_type);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kDThreads), 0, stream, packed, n, absmax,
                       absmax2, mean, out, lv);
  };
  if (double_quant == kDqDynamic) {
    if (f16) go(dequant_kernel<kDqDynamic, true>);
    else go(dequant_kernel<kDqDynamic, false>);
  } else if (double_quant) {
    if (f16) go(dequant_kernel<kDqLinear, true>);
    else go(dequant_kernel<kDqLinear, false>);
  } else {
    if (f16) go(dequant_kernel<kDqNone, true>);
    else go(dequant_kernel<kDqNone, false>);
  }
  return hipGetLastError();
}

}  // namespace bnbx

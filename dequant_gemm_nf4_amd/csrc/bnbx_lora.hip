// LoRA down-projection for gfx950: XA[M, r] = rnd(fl32(s * (X[M, K] . A[r, K]^T)))
// with fp32 accumulation (the pomoai.com overview, QLoRA: trainable low-rank
// adapters beside the frozen 4-bit base layer; A is the adapter's
// nn.Linear(K, r) weight, s its scale).  XA then feeds the fused low-rank
// term of the 4-bit GEMM (bnbx_gemm_nf4_lora), which adds XA . B^T.
//
// One workgroup of W waves (16 for r <= 128, else 8) takes 16 rows of X and
// all r columns; wave w takes the w-th of W parts of K (in steps of 32, four
// steps' loads in flight) and runs v_mfma_f32_16x16x32 with X
// as the A operand (lane l: row l % 16, k 8 (l / 16) .. +8 of the step) and
// rows of the adapter weight as the B operand in the same lane layout, one
// accumulator per 16 columns.  The waves' partial sums are added in LDS in
// wave order (a fixed order: the result does not depend on timing), scaled
// once and rounded once to the compute type.  Rows of X past M and rows of A
// past r read zero through the buffer range check.
#include "bnbx_device.hpp"
#include "bnbx_internal.hpp"

namespace bnbx {
namespace {

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// RT column tiles of 16 (r <= 16 RT); kq: K per wave, a multiple of 32.
template <bool F16, int RT, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void lora_down_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* __restrict__ a, int64_t lda,
    int M, int K, int r, float scale, uint16_t* __restrict__ xa, int64_t ldxa, int kq) {
  constexpr int kLWaves = WAVES;
  constexpr int kLThreads = WAVES * 64;
  __shared__ f32x4_t red[kLWaves][RT][64];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int i = lane & 15, g = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * 16;
  const int rows = M - m0 < 16 ? (int)(M - m0) : 16;
  const rsrc_t rx = make_rsrc(x + m0 * ldx, (uint32_t)(((int64_t)(rows - 1) * ldx + K) * 2));
  const rsrc_t ra = make_rsrc(a, (uint32_t)(((int64_t)(r - 1) * lda + K) * 2));
  const uint32_t xo = (uint32_t)(((int64_t)i * ldx + 8 * g) * 2);
  uint32_t ao[RT];
#pragma unroll
  for (int c = 0; c < RT; ++c) ao[c] = (uint32_t)(((int64_t)(16 * c + i) * lda + 8 * g) * 2);

  f32x4_t acc[RT];
#pragma unroll
  for (int c = 0; c < RT; ++c) acc[c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int k0 = wave * kq;
  const int k1 = k0 + kq < K ? k0 + kq : K;
#pragma unroll 4
  for (int k = k0; k < k1; k += 32) {
    const uint32_t kb = (uint32_t)k * 2u;
    const u32x4_t xv = __builtin_amdgcn_raw_buffer_load_b128(rx, xo, kb, 0);
    u32x4_t av[RT];
#pragma unroll
    for (int c = 0; c < RT; ++c) av[c] = __builtin_amdgcn_raw_buffer_load_b128(ra, ao[c], kb, 0);
#pragma unroll
    for (int c = 0; c < RT; ++c) acc[c] = mfma_16x16x32<F16>(xv, av[c], acc[c]);
  }

#pragma unroll
  for (int c = 0; c < RT; ++c) red[wave][c][lane] = acc[c];
  __syncthreads();
  // Output e: tile c = e / 256, lane l = (e / 4) % 64, value v = e % 4, i.e.
  // XA[m0 + 4 (l / 16) + v][16 c + l % 16] (the 16x16 MFMA's D layout).
  for (int e = t; e < RT * 256; e += kLThreads) {
    const int c = e >> 8, l = (e >> 2) & 63, v = e & 3;
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < kLWaves; ++w) s += red[w][c][l][v];
    const int row = 4 * (l >> 4) + v, col = 16 * c + (l & 15);
    if (row < rows && col < r) {
      const float o = scale * s;
      xa[(m0 + row) * ldxa + col] = f32_to_16<F16>(o);
    }
  }
}

template <bool F16>
hipError_t launch_rt(int rt, const uint16_t* x, int64_t ldx, const uint16_t* a, int64_t lda,
                     int M, int K, int r, float scale, uint16_t* xa, int64_t ldxa,
                     hipStream_t stream) {
  const int64_t grid = ((int64_t)M + 15) / 16;
#define BNBX_LORA_RT(RT)                                                                       \
  if (rt == RT) {                                                                              \
    constexpr int W = RT <= 8 ? 16 : 8;   /* LDS: W x RT KB of partial sums */                  \
    const int kq = ((K + W - 1) / W + 31) / 32 * 32;                                           \
    hipLaunchKernelGGL((lora_down_kernel<F16, RT, W>), dim3((unsigned)grid), dim3(W * 64), 0,  \
                       stream, x, ldx, a, lda, M, K, r, scale, xa, ldxa, kq);                  \
    return hipGetLastError();                                                                  \
  }
  BNBX_LORA_RT(1)
  BNBX_LORA_RT(2)
  BNBX_LORA_RT(4)
  BNBX_LORA_RT(8)
  BNBX_LORA_RT(16)
#undef BNBX_LORA_RT
  return hipErrorNotSupported;
}

}  // namespace

hipError_t launch_lora_down(const uint16_t* x, int64_t ldx, const uint16_t* a, int64_t lda,
                            int M, int K, int r, float scale, bool f16, uint16_t* xa,
                            int64_t ldxa, hipStream_t stream) {
  // 32-bit buffer offsets: 16 rows of X and all r rows of A must fit.
  if (16 * ldx * 2 >= ((int64_t)1 << 31) || ((int64_t)r * lda) * 2 >= ((int64_t)1 << 31))
    return hipErrorNotSupported;
  int rt = 1;
  while (16 * rt < r) rt *= 2;   // column tiles, rounded up to a power of two
  if (rt > 16) return hipErrorNotSupported;
  return f16 ? launch_rt<true>(rt, x, ldx, a, lda, M, K, r, scale, xa, ldxa, stream)
             : launch_rt<false>(rt, x, ldx, a, lda, M, K, r, scale, xa, ldxa, stream);
}

}  // namespace bnbx

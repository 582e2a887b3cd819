// Prefill GEMM with NF4 weights for gfx950: Y[M, N] = X[M, K] . W_hat[N, K]^T
// (mlqm.cn bitsandbytes article, sec. 3.4: 4-bit storage, dequantize to BF16,
// multiply in 16-bit with fp32 accumulation).
//
// Each workgroup owns a BM x BN tile of Y and walks K in steps of BK = 64, one
// NF4 block per weight row per step.  Per step it stages the X tile in LDS,
// dequantizes the packed weight tile once (LDS level-pair table, binary32
// multiply by the block scale, v_cvt_pk_bf16_f32) into LDS, and the four
// waves run v_mfma_f32_32x32x16_bf16 on both operands from LDS.
#include "bnbx_device.hpp"
#include "bnbx_internal.hpp"

namespace bnbx {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_ROW = BK + 8;   // bf16 per LDS row (8 of padding against bank conflicts)
constexpr int kThreads = 256;

__device__ __forceinline__ float gemm_block_scale(int64_t blk, const void* absmax,
                                                  const float* absmax2, float mu, int dq) {
  if (!dq) return ((const float*)absmax)[blk];
  const float q = (float)((const int8_t*)absmax)[blk];
  return __builtin_fmaf(q, absmax2[blk / kGroup] * (1.0f / 127.0f), mu);
}

__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ packed,
    const void* __restrict__ absmax, const float* __restrict__ absmax2,
    const float* __restrict__ mean, int dq, int M, int N, int K, uint16_t* __restrict__ y,
    int64_t ldy, LevelTable lv) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDS_ROW];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDS_ROW];
  __shared__ float2 tab[256];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t n0 = (int64_t)blockIdx.x * BN;
  const int lvl = level_lanes(lv);
  for (int e = tid; e < 256; e += kThreads)
    tab[e] = make_float2(level_lookup(lvl, (uint32_t)e >> 4), level_lookup(lvl, (uint32_t)e & 15u));
  const float mu = dq ? *mean : 0.0f;
  const int64_t rowK2 = (int64_t)(K >> 1);
  const int64_t nkb = K >> 6;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // B tile: thread -> (row, half of the 32 packed bytes)
  const int brow = tid >> 1, bhalf = tid & 1;
  const int64_t gn = n0 + brow;
  const bool bok = gn < N;
  __syncthreads();

  for (int64_t kb = 0; kb < nkb; ++kb) {
    const int64_t k0 = kb * BK;
    // X tile -> LDS (rows past M are zero)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + i * kThreads;
      const int r = idx >> 3, c8 = (idx & 7) * 8;
      const int64_t gm = m0 + r;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (gm < M) v = *(const uint4*)(x + gm * ldx + k0 + c8);
      *(uint4*)(As + r * LDS_ROW + c8) = v;
    }
    // weight tile: 16 packed bytes -> 32 bf16 in LDS
    {
      uint4 p = make_uint4(0, 0, 0, 0);
      float sc = 0.0f;
      if (bok) {
        p = *(const uint4*)(packed + gn * rowK2 + (k0 >> 1) + bhalf * 16);
        sc = gemm_block_scale(gn * nkb + kb, absmax, absmax2, mu, dq);
      }
      const uint32_t d[4] = {p.x, p.y, p.z, p.w};
      uint32_t o[16];
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float2 lp = tab[(d[k] >> (8 * i)) & 0xffu];
          o[4 * k + i] = pack_bf16x2(lp.x * sc, lp.y * sc);
        }
      uint4* dst = (uint4*)(Bs + brow * LDS_ROW + bhalf * 32);
#pragma unroll
      for (int k = 0; k < 4; ++k) dst[k] = make_uint4(o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8_t a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *(const bf16x8_t*)(As + (wm * 64 + i * 32 + (lane & 31)) * LDS_ROW + ks * 16 + (lane >> 5) * 8);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *(const bf16x8_t*)(Bs + (wn * 64 + j * 32 + (lane & 31)) * LDS_ROW + ks * 16 + (lane >> 5) * 8);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  // D layout of a 32x32 MFMA tile: lane l, value v -> column l%32,
  // row 8*(v/4) + 4*(l/32) + v%4.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
        if (row < M && col < N) y[row * ldy + col] = f32_to_bf16(acc[i][j][v]);
      }
}

}  // namespace

hipError_t launch_gemm(const uint16_t* x, int64_t ldx, const uint8_t* packed, const void* absmax,
                       const float* absmax2, const float* mean, int double_quant, int M, int N,
                       int K, uint16_t* y, int64_t ldy, hipStream_t stream) {
  const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  if (grid.y > 65535u) return hipErrorNotSupported;
  hipLaunchKernelGGL(gemm_kernel, grid, dim3(kThreads), 0, stream, x, ldx, packed, absmax,
                     absmax2, mean, double_quant, M, N, K, y, ldy, level_table());
  return hipGetLastError();
}

}  // namespace bnbx

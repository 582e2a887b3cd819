// Prefill GEMM with NF4 weights for gfx950: Y[M, N] = X[M, K] . W_hat[N, K]^T
// (mlqm.cn bitsandbytes article, sec. 3.4: 4-bit storage, dequantize to BF16,
// multiply in 16-bit with fp32 accumulation).
//
// Tiling.  A workgroup (4 waves) owns a 256 x 256 tile of Y; each wave a
// 128 x 128 quarter, i.e. 4 x 4 tiles of v_mfma_f32_32x32x16_bf16.  K is
// walked in steps of 64 = one NF4 block per weight row, so a whole weight-tile
// row shares one block scale.
//
// Pipeline.  LDS holds two buffers of the X tile and of the dequantized
// weight tile (rows padded to 144 B so that 16 lanes reading 16 B from 16
// consecutive rows hit 64 distinct banks).  In step t the waves run the 64
// MFMAs of buffer t%2 while the loads of step t+1 (X: 128 B per thread,
// packed weight: 32 B per thread, plus the block scale) are in flight; then
// each thread dequantizes its weight row for step t+1 (LDS level-pair table,
// binary32 multiply, v_cvt_pk_bf16_f32) and writes it with X into buffer
// (t+1)%2.  One barrier per step.
//
// Tile order is XCD-aware: workgroup b runs on XCD b % 8, so consecutive
// tile ids (which share the same 256 rows of X) are given to the same XCD
// and meet in its L2.
#include "bnbx_device.hpp"
#include "bnbx_internal.hpp"

namespace bnbx {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int LDS_ROW = BK + 8;             // bf16 per LDS row (144 B)
constexpr int kThreads = 256;
constexpr int kTabCopies = 4;
constexpr int kXcds = 8;
constexpr int kABuf = BM * LDS_ROW;         // bf16 elements per X buffer
constexpr int kBBuf = BN * LDS_ROW;         // bf16 elements per weight buffer

template <bool DQ>
__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ packed,
    const void* __restrict__ absmax, const float* __restrict__ absmax2,
    const float* __restrict__ mean, int M, int N, int K, uint16_t* __restrict__ y, int64_t ldy,
    int tiles_m, int tiles_n, LevelTable lv) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* As = (uint16_t*)smem;                       // [2][BM][LDS_ROW]
  uint16_t* Bs = As + 2 * kABuf;                        // [2][BN][LDS_ROW]
  float2* tabs = (float2*)(Bs + 2 * kBBuf);             // [kTabCopies][256]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // XCD-aware tile id: workgroups b, b+8, b+16, ... share an XCD.
  const int ntiles = tiles_m * tiles_n;
  const int per_xcd = (ntiles + kXcds - 1) / kXcds;
  const int b = blockIdx.x;
  const int tile = (b % kXcds) * per_xcd + b / kXcds;
  if (tile >= ntiles) return;
  const int64_t m0 = (int64_t)(tile / tiles_n) * BM;
  const int64_t n0 = (int64_t)(tile % tiles_n) * BN;

  const int lvl = level_lanes(lv);
  for (int e = tid; e < kTabCopies * 256; e += kThreads) {
    const uint32_t v = (uint32_t)e & 255u;
    tabs[e] = make_float2(level_lookup(lvl, v >> 4), level_lookup(lvl, v & 15u));
  }
  const float2* tab = tabs + (lane & (kTabCopies - 1)) * 256;
  const float mu = DQ ? *mean : 0.0f;
  const int64_t rowK2 = (int64_t)(K >> 1);
  const int64_t nkb = K >> 6;

  // Global -> register staging for one K step.
  //   X: thread t loads rows i*32 + t/8 (i = 0..7), 16-byte chunk t%8.
  //   W: thread t loads weight row t (32 packed bytes) and its scale.
  const int arow = tid >> 3, achunk = tid & 7;
  const int64_t gnr = n0 + tid;
  const bool bok = gnr < N;
  const int64_t gn = bok ? gnr : N - 1;
  uint4 ar[8];
  uint4 br[2];
  int qraw = 0;
  float sraw = 0.0f;

  auto load_step = [&](int64_t kb) {
    const int64_t k0 = kb * BK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t gm = m0 + i * 32 + arow;
      const int64_t gmc = gm < M ? gm : M - 1;
      ar[i] = *(const uint4*)(x + gmc * ldx + k0 + achunk * 8);
      if (gm >= M) ar[i] = make_uint4(0, 0, 0, 0);
    }
    const uint4* src = (const uint4*)(packed + gn * rowK2 + (k0 >> 1));
    br[0] = src[0];
    br[1] = src[1];
    const int64_t blk = gn * nkb + kb;
    if (DQ) {
      qraw = ((const int8_t*)absmax)[blk];
      sraw = absmax2[blk >> 8];
    } else {
      sraw = ((const float*)absmax)[blk];
    }
  };
  auto store_step = [&](int buf) {
    uint16_t* a = As + buf * kABuf;
#pragma unroll
    for (int i = 0; i < 8; ++i) *(uint4*)(a + (i * 32 + arow) * LDS_ROW + achunk * 8) = ar[i];
    float sc = DQ ? __builtin_fmaf((float)qraw, sraw * (1.0f / 127.0f), mu) : sraw;
    sc = bok ? sc : 0.0f;
    uint16_t* bw = Bs + buf * kBBuf + tid * LDS_ROW;
    const uint32_t d[8] = {br[0].x, br[0].y, br[0].z, br[0].w, br[1].x, br[1].y, br[1].z, br[1].w};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float2 lp = tab[(d[q] >> (8 * i)) & 0xffu];
        o[i] = pack_bf16x2(lp.x * sc, lp.y * sc);
      }
      *(uint4*)(bw + q * 8) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  __syncthreads();   // table ready
  load_step(0);
  store_step(0);
  __syncthreads();

  const int arow_op = wm * 128 + (lane & 31);
  const int brow_op = wn * 128 + (lane & 31);
  const int kcol = (lane >> 5) * 8;
  for (int64_t kb = 0; kb < nkb; ++kb) {
    const int buf = (int)(kb & 1);
    const bool more = kb + 1 < nkb;
    if (more) load_step(kb + 1);
    const uint16_t* a = As + buf * kABuf;
    const uint16_t* bb = Bs + buf * kBBuf;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8_t av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        av[i] = *(const bf16x8_t*)(a + (arow_op + i * 32) * LDS_ROW + ks * 16 + kcol);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bv[j] = *(const bf16x8_t*)(bb + (brow_op + j * 32) * LDS_ROW + ks * 16 + kcol);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (more) store_step(buf ^ 1);
    __syncthreads();
  }

  // D layout of a 32x32 MFMA tile: lane l, value v -> column l%32,
  // row 8*(v/4) + 4*(l/32) + v%4.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * 128 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int64_t col = n0 + wn * 128 + j * 32 + (lane & 31);
        if (row < M && col < N) y[row * ldy + col] = f32_to_bf16(acc[i][j][v]);
      }
}

constexpr size_t kSmemBytes =
    (size_t)(2 * kABuf + 2 * kBBuf) * sizeof(uint16_t) + kTabCopies * 256 * sizeof(float2);

}  // namespace

hipError_t launch_gemm(const uint16_t* x, int64_t ldx, const uint8_t* packed, const void* absmax,
                       const float* absmax2, const float* mean, int double_quant, int M, int N,
                       int K, uint16_t* y, int64_t ldy, hipStream_t stream) {
  const int64_t tm = ((int64_t)M + BM - 1) / BM, tn = ((int64_t)N + BN - 1) / BN;
  const int64_t ntiles = tm * tn;
  if (ntiles > (int64_t)1 << 30) return hipErrorNotSupported;
  const int64_t per_xcd = (ntiles + kXcds - 1) / kXcds;
  const unsigned grid = (unsigned)(per_xcd * kXcds);
  const void* fn = double_quant ? (const void*)gemm_kernel<true> : (const void*)gemm_kernel<false>;
  // Dynamic LDS above 64 KB must be enabled per kernel (idempotent call).
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)kSmemBytes);
  if (e != hipSuccess) return e;
  if (double_quant)
    hipLaunchKernelGGL(gemm_kernel<true>, dim3(grid), dim3(kThreads), kSmemBytes, stream, x, ldx,
                       packed, absmax, absmax2, mean, M, N, K, y, ldy, (int)tm, (int)tn,
                       level_table());
  else
    hipLaunchKernelGGL(gemm_kernel<false>, dim3(grid), dim3(kThreads), kSmemBytes, stream, x, ldx,
                       packed, absmax, absmax2, mean, M, N, K, y, ldy, (int)tm, (int)tn,
                       level_table());
  return hipGetLastError();
}

}  // namespace bnbx

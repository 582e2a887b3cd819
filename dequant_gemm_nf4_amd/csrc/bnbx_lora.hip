// LoRA down-projection for gfx950: XA[M, r] = rnd(fl32(s * (X[M, K] . A[r, K]^T)))
// with fp32 accumulation (the pomoai.com overview, QLoRA: trainable low-rank
// adapters beside the frozen 4-bit base layer; A is the adapter's
// nn.Linear(K, r) weight, s its scale).  XA then feeds the fused low-rank
// term of the 4-bit GEMM (bnbx_gemm_nf4_lora), which adds XA . B^T.
//
// One workgroup of W waves (16 for r <= 128, else 8) takes R rows of X (16,
// or 8 when 16-row workgroups would leave CUs idle) and all r columns; wave w
// takes the w-th of W parts of K in steps of 32 and runs v_mfma_f32_16x16x32
// with X as the A operand (lane l: row l % 16, k 8 (l / 16) .. +8 of the
// step; rows past R are zero) and rows of the adapter weight as the B
// operand in the same lane layout, one accumulator per 16 columns.
//
// Loads are quad-coalesced: lane x reads 16 bytes of row x / 4 at piece
// x % 4, so that one instruction covers 16 rows x 64 contiguous bytes (the
// MFMA layout, where neighbouring lanes read different rows, made every lane
// its own memory request).  A 1 KB LDS stage per wave turns each loaded
// value into the MFMA layout: lane x writes slot 16 p + ((r + 4 p) mod 16)
// and lane (q, r) reads slot 16 q + ((r + 4 q) mod 16), both free of bank
// conflicts.  The waves' partial sums are added in LDS in wave order (a fixed
// order: the result does not depend on timing), scaled once and rounded once
// to the compute type.  Rows of X past M and rows of A past r read zero
// through the buffer range check.
#include "bnbx_device.hpp"
#include "bnbx_internal.hpp"

namespace bnbx {
namespace {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kFar = 0x80000000u;   // an offset past every buffer resource

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// RT column tiles of 16 (r <= 16 RT); R rows of X per workgroup (16 or 8);
// kq: K per wave, a multiple of 32.
template <bool F16, int RT, int WAVES, int R>
__global__ __launch_bounds__(WAVES * 64) void lora_down_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* __restrict__ a, int64_t lda,
    int M, int K, int r, float scale, uint16_t* __restrict__ xa, int64_t ldxa, int kq) {
  constexpr int kLWaves = WAVES;
  constexpr int kLThreads = WAVES * 64;
  __shared__ f32x4_t red[kLWaves][RT][64];
  __shared__ __attribute__((aligned(16))) unsigned char stages[kLWaves][1024];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  unsigned char* const stage = stages[wave];
  const int lr = lane >> 2, lp = lane & 3;        // load layout: row, piece
  const int i = lane & 15, g = lane >> 4;         // MFMA layout
  const uint32_t wslot = 16u * (uint32_t)(16 * lp + ((lr + 4 * lp) & 15));
  const uint32_t rslot = 16u * (uint32_t)(16 * g + ((i + 4 * g) & 15));
  const int64_t m0 = (int64_t)blockIdx.x * R;
  const int rows = M - m0 < R ? (int)(M - m0) : R;
  const rsrc_t rx = make_rsrc(x + m0 * ldx, (uint32_t)(((int64_t)(rows - 1) * ldx + K) * 2));
  const rsrc_t ra = make_rsrc(a, (uint32_t)(((int64_t)(r - 1) * lda + K) * 2));
  const uint32_t xo = lr < R ? (uint32_t)(((int64_t)lr * ldx + 8 * lp) * 2) : kFar;
  uint32_t ao[RT];
#pragma unroll
  for (int c = 0; c < RT; ++c) ao[c] = (uint32_t)(((int64_t)(16 * c + lr) * lda + 8 * lp) * 2);
  // load layout -> MFMA layout through the wave's stage
  auto relayout = [&](u32x4_t v) {
    *(u32x4_t*)(stage + wslot) = v;
    return *(const u32x4_t*)(stage + rslot);
  };

  f32x4_t acc[RT];
#pragma unroll
  for (int c = 0; c < RT; ++c) acc[c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int k0 = wave * kq;
  const int k1 = k0 + kq < K ? k0 + kq : K;
  // Groups of U steps; the next group's loads go out before the current
  // group is multiplied (two register sets; with 8 or more column tiles one
  // step's loads are many already, and a second set would spill).  Steps
  // past the wave's part of K load from an offset outside both buffers and
  // read zero.
  constexpr int U = RT == 1 ? 4 : RT == 2 ? 2 : 1;
  constexpr bool kRoll = RT <= 4;
  struct Grp {
    u32x4_t x[U];
    u32x4_t a[U][RT];
  };
  auto load_grp = [&](Grp& gr, int k) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = k + 32 * u < k1;
      const uint32_t kb = (uint32_t)(k + 32 * u) * 2u;
      gr.x[u] = __builtin_amdgcn_raw_buffer_load_b128(rx, in ? xo : kFar, kb, 0);
#pragma unroll
      for (int c = 0; c < RT; ++c)
        gr.a[u][c] = __builtin_amdgcn_raw_buffer_load_b128(ra, in ? ao[c] : kFar, kb, 0);
    }
  };
  auto mul_grp = [&](const Grp& gr) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const u32x4_t xv = relayout(gr.x[u]);
#pragma unroll
      for (int c = 0; c < RT; ++c) acc[c] = mfma_16x16x32<F16>(xv, relayout(gr.a[u][c]), acc[c]);
    }
  };
  if constexpr (kRoll) {
    Grp g0, g1;
    load_grp(g0, k0);
    for (int k = k0; k < k1; k += 64 * U) {
      if (k + 32 * U < k1) load_grp(g1, k + 32 * U);
      mul_grp(g0);
      if (k + 32 * U >= k1) break;
      if (k + 64 * U < k1) load_grp(g0, k + 64 * U);
      mul_grp(g1);
    }
  } else {
    for (int k = k0; k < k1; k += 32) {
      Grp g0;
      load_grp(g0, k);
      mul_grp(g0);
    }
  }

#pragma unroll
  for (int c = 0; c < RT; ++c) red[wave][c][lane] = acc[c];
  __syncthreads();
  // Output e: tile c = e / 256, lane l = (e / 4) % 64, value v = e % 4, i.e.
  // XA[m0 + 4 (l / 16) + v][16 c + l % 16] (the 16x16 MFMA's D layout).
  for (int e = t; e < RT * 256; e += kLThreads) {
    const int c = e >> 8, l = (e >> 2) & 63, v = e & 3;
    const int row = 4 * (l >> 4) + v, col = 16 * c + (l & 15);
    if (row < rows && col < r) {
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < kLWaves; ++w) s += red[w][c][l][v];
      const float o = scale * s;
      xa[(m0 + row) * ldxa + col] = f32_to_16<F16>(o);
    }
  }
}

template <bool F16, int R>
hipError_t launch_rt(int rt, const uint16_t* x, int64_t ldx, const uint16_t* a, int64_t lda,
                     int M, int K, int r, float scale, uint16_t* xa, int64_t ldxa,
                     hipStream_t stream) {
  const int64_t grid = ((int64_t)M + R - 1) / R;
#define BNBX_LORA_RT(RT)                                                                        \
  if (rt == RT) {                                                                               \
    constexpr int W = RT <= 8 ? 16 : 8;   /* LDS: W x RT KB of partial sums */                   \
    const int kq = ((K + W - 1) / W + 31) / 32 * 32;                                            \
    hipLaunchKernelGGL((lora_down_kernel<F16, RT, W, R>), dim3((unsigned)grid), dim3(W * 64),   \
                       0, stream, x, ldx, a, lda, M, K, r, scale, xa, ldxa, kq);                \
    return hipGetLastError();                                                                   \
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
  // 16-row workgroups while they fill the GPU, else 8 rows (the MFMA's
  // other 8 rows are zero): the down-projection is bound by reading X.
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, v = 0;
    cus = hipGetDevice(&dev) == hipSuccess &&
                  hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) ==
                      hipSuccess &&
                  v > 0
              ? v
              : 256;
  }
  const bool r16 = ((int64_t)M + 15) / 16 >= cus;
  if (f16)
    return r16 ? launch_rt<true, 16>(rt, x, ldx, a, lda, M, K, r, scale, xa, ldxa, stream)
               : launch_rt<true, 8>(rt, x, ldx, a, lda, M, K, r, scale, xa, ldxa, stream);
  return r16 ? launch_rt<false, 16>(rt, x, ldx, a, lda, M, K, r, scale, xa, ldxa, stream)
             : launch_rt<false, 8>(rt, x, ldx, a, lda, M, K, r, scale, xa, ldxa, stream);
}

}  // namespace bnbx

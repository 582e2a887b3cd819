// Decode GEMV with NF4 weights for gfx950: Y[M, N] = X[M, K] . W_hat[N, K]^T,
// M <= 16 (mlqm.cn bitsandbytes article, sec. 3.4 "4-bit storage, 16-bit
// compute", and the sec. 7 pitfall that 4-bit only pays off when the layer is
// bound by weight traffic: so the packed weight is streamed exactly once).
//
// Layout of the work.  A row of W is C = K/32 chunks of 16 packed bytes
// (32 weights, half a 64-block).  A workgroup is R "teams" of S threads
// (S a multiple of 64, S >= C/P); slot s of a team owns chunks s, s+S, ... of
// whatever row the team is on, so its slice of X stays in registers for the
// whole kernel while the team walks G rows.  Every thread issues all of its
// 16-byte weight loads before it builds the lookup table, so the HBM latency
// overlaps the table build.
//
// Dequant in registers.  An LDS table maps each packed byte to the bf16 pair
// (L[high nibble], L[low nibble]); it is replicated 64 times with a 256-byte
// stride so that lane l always reads bank l (no conflicts), and the byte
// address (byte << 8 | lane << 2) is formed by one v_perm_b32.  The pair feeds
// v_dot2_f32_bf16 against the matching X pair; the 32-weight partial sum is
// scaled once by the block scale (fp32), so dequant costs about one VALU
// instruction per weight.
#include "bnbx_device.hpp"
#include "bnbx_internal.hpp"

namespace bnbx {
namespace {

// Tunables (compile-time; the defaults are the measured best on MI355X).
#ifndef BNBX_GEMV_MAX_THREADS
#define BNBX_GEMV_MAX_THREADS 512     // threads per workgroup
#endif
#ifndef BNBX_GEMV_TAB_COPIES
#define BNBX_GEMV_TAB_COPIES 32       // lane copies of the byte table (32 or 64)
#endif
#ifndef BNBX_GEMV_MIN_WAVES
#define BNBX_GEMV_MIN_WAVES 1         // launch-bounds occupancy hint (waves per SIMD)
#endif
#ifndef BNBX_GEMV_WG_TARGET
#define BNBX_GEMV_WG_TARGET 512       // workgroups the rows are spread over
#endif
#ifndef BNBX_GEMV_W_FIRST
#define BNBX_GEMV_W_FIRST 0           // 1: issue weight loads before the X loads
#endif
constexpr int kMaxThreads = BNBX_GEMV_MAX_THREADS;
constexpr int kGMax = 8;
constexpr int kCopies = BNBX_GEMV_TAB_COPIES;
constexpr int kTabDwords = 256 * 64;   // 256 B per byte value; kCopies dwords used

template <int MM, int P, bool DQ, int G>
__global__ __launch_bounds__(kMaxThreads, BNBX_GEMV_MIN_WAVES) void gemv_valu_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ packed,
    const void* __restrict__ absmax, const float* __restrict__ absmax2,
    const float* __restrict__ mean, int N, int K, uint16_t* __restrict__ y, int64_t ldy, int S,
    int R, LevelTable lv) {
  __shared__ __attribute__((aligned(16))) uint32_t tab[kTabDwords];
  __shared__ float red[kGMax * MM * (kMaxThreads / 64)];

  const int t = threadIdx.x;
  const int T = blockDim.x;
  const int team = t / S, s = t - team * S;
  const int C = K >> 5;
  const int64_t rowK2 = (int64_t)(K >> 1);
  const int64_t nkb = K >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * R * G + team;
  static_assert(G * P <= kGMax, "at most 8 chunks per thread");
  constexpr int GM = G;
  const int lvl = level_lanes(lv);

  // X slice of this thread: 32 bf16 (16 pairs) per chunk per row of X
  uint32_t xr[MM][P][16];
  auto load_x = [&]() {
#pragma unroll
    for (int m = 0; m < MM; ++m) {
#pragma unroll
      for (int j = 0; j < P; ++j) {
        const int c = s + j * S;
        const int cc = c < C ? c : C - 1;
        const uint4* src = (const uint4*)(x + (int64_t)m * ldx + (int64_t)cc * 32);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 v = src[q];
          xr[m][j][4 * q] = v.x;
          xr[m][j][4 * q + 1] = v.y;
          xr[m][j][4 * q + 2] = v.z;
          xr[m][j][4 * q + 3] = v.w;
        }
      }
    }
  };
  // 1. X (small, cache-resident) and every weight load, each followed by its
  //    raw block-scale loads, all in flight before anything waits (addresses
  //    clamped instead of branched; out-of-range rows/chunks are zeroed
  //    through their scale).  Scales are converted only after the barrier,
  //    so using row g waits only for the loads issued up to row g.
  if (!BNBX_GEMV_W_FIRST) load_x();
  uint4 wv[GM][P];
  int qraw[GM][P];
  float sraw[GM][P], graw[GM][P];
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    {
#pragma unroll
      for (int j = 0; j < P; ++j) {
        const int64_t row = row0 + (int64_t)g * R;
        const int c = s + j * S;
        const int64_t rc = row < N ? row : N - 1;
        const int cc = c < C ? c : C - 1;
        wv[g][j] = load_nt16(packed + rc * rowK2 + (int64_t)cc * 16);
        const int64_t blk = rc * nkb + (cc >> 1);
        if (DQ) {
          qraw[g][j] = ((const int8_t*)absmax)[blk];
          graw[g][j] = absmax2[blk >> 8];
          sraw[g][j] = 0.0f;
        } else {
          qraw[g][j] = 0;
          sraw[g][j] = ((const float*)absmax)[blk];
          graw[g][j] = 0.0f;
        }
      }
    }
  }
  if (BNBX_GEMV_W_FIRST) load_x();
  const float mu = DQ ? *mean : 0.0f;
  // 2. replicated byte -> bf16-pair table
  for (int e = t; e < 256 * kCopies / 4; e += T) {
    const uint32_t b = (uint32_t)e / (kCopies / 4);
    const uint32_t v = pack_bf16x2(level_lookup(lvl, b >> 4), level_lookup(lvl, b & 15u));
    ((uint4*)tab)[b * 16 + (uint32_t)e % (kCopies / 4)] = make_uint4(v, v, v, v);
  }
  __syncthreads();

  // 3. dequant-in-register dot products, one block scale per 32 weights
  const uint32_t lanebyte = (uint32_t)(t & (kCopies - 1)) << 2;
  const unsigned char* tabb = (const unsigned char*)tab;
  float acc[GM][MM];
#pragma unroll
  for (int g = 0; g < GM; ++g) {
#pragma unroll
    for (int m = 0; m < MM; ++m) acc[g][m] = 0.0f;
  }
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    {
#pragma unroll
      for (int j = 0; j < P; ++j) {
        const int64_t row = row0 + (int64_t)g * R;
        const bool ok = row < N && s + j * S < C;
        float sc = DQ ? __builtin_fmaf((float)qraw[g][j], graw[g][j] * (1.0f / 127.0f), mu)
                      : sraw[g][j];
        sc = ok ? sc : 0.0f;
        const uint32_t d[4] = {wv[g][j].x, wv[g][j].y, wv[g][j].z, wv[g][j].w};
        float part[MM];
#pragma unroll
        for (int m = 0; m < MM; ++m) part[m] = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t addr = perm(d[q], lanebyte, 0x0c0c0000u | ((4u + i) << 8));
            const uint32_t pair = *(const uint32_t*)(tabb + addr);
#pragma unroll
            for (int m = 0; m < MM; ++m) part[m] = dot2_bf16(pair, xr[m][j][4 * q + i], part[m]);
          }
        }
#pragma unroll
        for (int m = 0; m < MM; ++m) acc[g][m] = __builtin_fmaf(part[m], sc, acc[g][m]);
      }
    }
  }

  // 4. reduce each row over its team: waves first, then across the team's waves
  const int nw = T >> 6, wave = t >> 6, wpt = S >> 6;
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    {
#pragma unroll
      for (int m = 0; m < MM; ++m) {
        const float v = wave_sum(acc[g][m]);
        if ((t & 63) == 0) red[(g * MM + m) * nw + wave] = v;
      }
    }
  }
  __syncthreads();
  const int nout = G * R * MM;
  for (int o = t; o < nout; o += T) {
    const int g = o / (R * MM);
    const int rem = o - g * R * MM;
    const int tm = rem / MM, m = rem - tm * MM;
    const int64_t row = (int64_t)blockIdx.x * R * G + (int64_t)g * R + tm;
    if (row < N) {
      float v = 0.0f;
      for (int w = tm * wpt; w < (tm + 1) * wpt; ++w) v += red[(g * MM + m) * nw + w];
      y[(int64_t)m * ldy + row] = f32_to_bf16(v);
    }
  }
}

template <int MM, int P, int G>
hipError_t launch_valu_g(const uint16_t* x, int64_t ldx, const uint8_t* packed,
                         const void* absmax, const float* absmax2, const float* mean, int dq,
                         int N, int K, uint16_t* y, int64_t ldy, int S, int R,
                         hipStream_t stream) {
  const int64_t grid = ((int64_t)N + R * G - 1) / (R * G);
  if (dq)
    hipLaunchKernelGGL((gemv_valu_kernel<MM, P, true, G>), dim3((unsigned)grid), dim3(S * R), 0,
                       stream, x, ldx, packed, absmax, absmax2, mean, N, K, y, ldy, S, R,
                       level_table());
  else
    hipLaunchKernelGGL((gemv_valu_kernel<MM, P, false, G>), dim3((unsigned)grid), dim3(S * R), 0,
                       stream, x, ldx, packed, absmax, absmax2, mean, N, K, y, ldy, S, R,
                       level_table());
  return hipGetLastError();
}

// Team size S covers a row's chunks (P per thread); R teams per workgroup;
// G rows per team, picked so that about 512 workgroups (two per CU, the LDS
// limit) cover N.
template <int MM, int P>
hipError_t launch_valu(const uint16_t* x, int64_t ldx, const uint8_t* packed, const void* absmax,
                       const float* absmax2, const float* mean, int dq, int N, int K,
                       uint16_t* y, int64_t ldy, hipStream_t stream) {
  const int C = K >> 5;
  const int S = ((C + P - 1) / P + 63) / 64 * 64;
  const int R = kMaxThreads / S >= 1 ? kMaxThreads / S : 1;
  const int64_t need = ((int64_t)N + (int64_t)R * BNBX_GEMV_WG_TARGET - 1) /
                       ((int64_t)R * BNBX_GEMV_WG_TARGET);
  const int gmax = kGMax / P;
  const int G = need <= 4 ? (int)(need < 1 ? 1 : need) : need <= 6 ? 6 : 8;
  const int Gc = G < gmax ? G : gmax;
#define BNBX_GEMV_G(GV)                                                                     \
  if (Gc == GV)                                                                             \
    return launch_valu_g<MM, P, (GV * P <= kGMax ? GV : 1)>(x, ldx, packed, absmax, absmax2, \
                                                           mean, dq, N, K, y, ldy, S, R, stream);
  BNBX_GEMV_G(1)
  BNBX_GEMV_G(2)
  BNBX_GEMV_G(3)
  BNBX_GEMV_G(4)
  BNBX_GEMV_G(6)
  BNBX_GEMV_G(8)
#undef BNBX_GEMV_G
  return hipErrorNotSupported;
}

template <int P>
hipError_t launch_valu_m(int MM, const uint16_t* x, int64_t ldx, const uint8_t* packed,
                         const void* absmax, const float* absmax2, const float* mean, int dq,
                         int N, int K, uint16_t* y, int64_t ldy, hipStream_t stream) {
  switch (MM) {
    case 1: return launch_valu<1, P>(x, ldx, packed, absmax, absmax2, mean, dq, N, K, y, ldy, stream);
    case 2: return launch_valu<2, P>(x, ldx, packed, absmax, absmax2, mean, dq, N, K, y, ldy, stream);
    case 3: return launch_valu<3, P>(x, ldx, packed, absmax, absmax2, mean, dq, N, K, y, ldy, stream);
    default: return launch_valu<4, P>(x, ldx, packed, absmax, absmax2, mean, dq, N, K, y, ldy, stream);
  }
}

}  // namespace

hipError_t launch_gemv(const uint16_t* x, int64_t ldx, const uint8_t* packed, const void* absmax,
                       const float* absmax2, const float* mean, int double_quant, int M, int N,
                       int K, uint16_t* y, int64_t ldy, hipStream_t stream) {
  const int C = K >> 5;
  const int P = C <= kMaxThreads ? 1 : C <= 2 * kMaxThreads ? 2 : C <= 4 * kMaxThreads ? 4 : 0;
  if (P == 0) return hipErrorNotSupported;
  // Rows of X in groups of at most 4 (each group streams W once); with two
  // chunks per thread one row at a time keeps the X slice in registers.
  const int mstep = P == 1 ? 4 : 1;
  for (int m0 = 0; m0 < M; m0 += mstep) {
    const int mm = M - m0 < mstep ? M - m0 : mstep;
    const hipError_t e =
        P == 1 ? launch_valu_m<1>(mm, x + (int64_t)m0 * ldx, ldx, packed, absmax, absmax2, mean,
                                  double_quant, N, K, y + (int64_t)m0 * ldy, ldy, stream)
      : P == 2 ? launch_valu<1, 2>(x + (int64_t)m0 * ldx, ldx, packed, absmax, absmax2, mean,
                                   double_quant, N, K, y + (int64_t)m0 * ldy, ldy, stream)
               : launch_valu<1, 4>(x + (int64_t)m0 * ldx, ldx, packed, absmax, absmax2, mean,
                                   double_quant, N, K, y + (int64_t)m0 * ldy, ldy, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bnbx

// Prefill GEMM with NF4 weights for gfx950: Y[M, N] = X[M, K] . W_hat[N, K]^T
// (mlqm.cn bitsandbytes article, sec. 3.4: 4-bit storage, dequantize to BF16,
// multiply in 16-bit with fp32 accumulation).
//
// Tiling.  A workgroup (4 waves, one per SIMD) owns a 256 x 256 tile of Y;
// each wave a 128 x 128 quarter, i.e. 4 x 4 tiles of
// v_mfma_f32_32x32x16_bf16 with the 256 accumulators per lane in AGPRs.  K is
// walked in steps of 64 = one NF4 block per weight row, so a weight-tile row
// shares one block scale per step.
//
// Pipeline.  LDS holds two buffers of the X tile and of the dequantized
// weight tile, and a byte -> (L[hi], L[lo]) binary32 level-pair table.
//   - X goes from global memory straight into LDS (global_load_lds, 16 B per
//     lane, no registers).  Its rows are 128 B with the eight 16-byte chunks
//     of row r rotated by (r / 2) % 8, so that 16 lanes reading the same
//     chunk of 16 consecutive rows hit 64 distinct banks.
//   - Each thread owns one weight row: it stages the row's 32 packed bytes
//     and block scale of a K step in registers (two staging sets, the loop
//     unrolled twice so that neither is ever copied) and writes the row
//     dequantized into LDS (pair lookup, binary32 multiply by the block
//     scale, v_cvt_pk_bf16_f32; rows padded to 144 B).
// In step t a wave issues the X copy of step t+1 and the weight loads of step
// t+2, then runs its 64 MFMAs on buffer t%2 and, between them, dequantizes
// step t+1's weights into buffer (t+1)%2; one barrier ends the step (it also
// waits for everything issued at the start of the step).  Scheduling-group
// barriers lay the instruction stream out as one MFMA followed by a share of
// the LDS reads, vector ops and LDS writes, so that vector and LDS work issues
// while the matrix core is busy.  Steps past the end of K load and write
// clamped (redundant) data into a buffer no MFMA reads, so the loop body has
// no branches.
//
// Tile order is XCD-aware: workgroup b runs on XCD b % 8, so consecutive
// tile ids (which share the same 256 rows of X) are given to the same XCD
// and meet in its L2.
#include <type_traits>

#include "bnbx_device.hpp"
#include "bnbx_internal.hpp"

namespace bnbx {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int LDS_ROW = BK + 8;             // bf16 per weight-tile LDS row (144 B)
constexpr int kThreads = 256;
constexpr int kTabCopies = 4;
constexpr int kXcds = 8;
constexpr int kABuf = BM * BK;              // bf16 elements per X buffer (128 B rows)
constexpr int kBBuf = BN * LDS_ROW;         // bf16 elements per weight buffer

// Scheduling-group masks (AMDGPU sched_group_barrier).
constexpr int kSgMfma = 0x008, kSgValu = 0x002, kSgDsRead = 0x100, kSgDsWrite = 0x200;

// One thread's weight row for one K step.
struct Stage {
  uint4 w[2];   // 32 packed bytes (64 weights)
  int q;        // int8 block code (double quant)
  float s;      // group scale (double quant) or block absmax
};

template <bool DQ>
__device__ __forceinline__ void load_stage(Stage& st, const uint8_t* __restrict__ packed,
                                           const void* __restrict__ absmax,
                                           const float* __restrict__ absmax2, int64_t gn,
                                           int64_t rowK2, int64_t nkb, int64_t kb) {
  kb = kb < nkb ? kb : nkb - 1;   // past the end: the last step again (never used)
  const int64_t k0 = kb * BK;
  const uint4* src = (const uint4*)(packed + gn * rowK2 + (k0 >> 1));
  st.w[0] = src[0];
  st.w[1] = src[1];
  const int64_t blk = gn * nkb + kb;
  if (DQ) {
    st.q = ((const int8_t*)absmax)[blk];
    st.s = absmax2[blk >> 8];
  } else {
    st.q = 0;
    st.s = ((const float*)absmax)[blk];
  }
}

template <bool DQ>
__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ packed,
    const void* __restrict__ absmax, const float* __restrict__ absmax2,
    const float* __restrict__ mean, int M, int N, int K, uint16_t* __restrict__ y, int64_t ldy,
    int tiles_m, int tiles_n, LevelTable lv) {
  // Every buffer is an LDS object of its own and is picked at compile time,
  // so that the compiler can tell reads of one buffer from the X copies in
  // flight into another (a read that might alias a copy waits for all of them).
  __shared__ __attribute__((aligned(16))) uint16_t As0[kABuf], As1[kABuf];   // X, rotated chunks
  __shared__ __attribute__((aligned(16))) uint16_t Bs0[kBBuf], Bs1[kBBuf];   // weights, padded rows
  __shared__ float2 tabs[kTabCopies * 256];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS bases in SGPRs
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

  const int64_t gnr = n0 + tid;
  const bool bok = gnr < N;
  const int64_t gn = bok ? gnr : N - 1;

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  auto load = [&](Stage& st, int64_t kb) {
    load_stage<DQ>(st, packed, absmax, absmax2, gn, rowK2, nkb, kb);
  };
  // X copy of one K step into LDS buffer `buf`: wave w copies rows
  // [64 w, 64 w + 64) in 8 instructions of 8 rows; lane l fills chunk slot
  // l % 8 of row l / 8 with the chunk that the rotation puts there.  Rows past
  // M are clamped to row M-1 (they only feed rows of Y that are never stored).
  const int xr_l = lane >> 3, xslot = lane & 7;
  auto copy_x = [&](uint16_t* xbuf, int64_t kb) {
    kb = kb < nkb ? kb : nkb - 1;
    const int64_t k0 = kb * BK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = wave * 64 + i * 8 + xr_l;
      const int chunk = xslot ^ ((r >> 1) & 7);
      int64_t gm = m0 + r;
      gm = gm < M ? gm : M - 1;
      __builtin_amdgcn_global_load_lds((const void*)(x + gm * ldx + k0 + chunk * 8),
                                       (void __attribute__((address_space(3)))*)(xbuf + (wave * 64 + i * 8) * BK),
                                       16, 0, 0);
    }
  };
  // Quarter p (0..3) of the weight row (16 weights), dequantized.
  auto scale_of = [&](const Stage& st) {
    const float sc = DQ ? __builtin_fmaf((float)st.q, st.s * (1.0f / 127.0f), mu) : st.s;
    return bok ? sc : 0.0f;
  };
  auto put_w = [&](const Stage& st, uint16_t* wbuf, int p, float sc) {
    // dwords 2p, 2p+1 of the 32 packed bytes = weights 16p .. 16p+15
    const uint32_t d0 = p == 0 ? st.w[0].x : p == 1 ? st.w[0].z : p == 2 ? st.w[1].x : st.w[1].z;
    const uint32_t d1 = p == 0 ? st.w[0].y : p == 1 ? st.w[0].w : p == 2 ? st.w[1].y : st.w[1].w;
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float2 l0 = tab[(d0 >> (8 * i)) & 0xffu];
      const float2 l1 = tab[(d1 >> (8 * i)) & 0xffu];
      o[i] = pack_bf16x2(l0.x * sc, l0.y * sc);
      o[4 + i] = pack_bf16x2(l1.x * sc, l1.y * sc);
    }
    uint16_t* bw = wbuf + tid * LDS_ROW + p * 16;
    *(uint4*)(bw) = make_uint4(o[0], o[1], o[2], o[3]);
    *(uint4*)(bw + 8) = make_uint4(o[4], o[5], o[6], o[7]);
  };

  // Prologue: step 0 into buffer 0; step 1's weights staged in set 1.
  Stage s0, s1;
  copy_x(As0, 0);
  load(s0, 0);
  {
    const float sc = scale_of(s0);
#pragma unroll
    for (int p = 0; p < 4; ++p) put_w(s0, Bs0, p, sc);
  }
  load(s1, 1);
  __syncthreads();

  // MFMA operands.  A: lane l reads row wm*128 + i*32 + l%32, 16-byte chunk
  // 2*ks + l/32, at its rotated slot (the rotation (r/2)%8 is the same for
  // all i).  B: weight rows wn*128 + j*32 + l%32, padded rows.
  const int arow_op = wm * 128 + (lane & 31);
  const int akey = (arow_op >> 1) & 7;
  uint32_t aoff[BK / 16];
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks)
    aoff[ks] = (uint32_t)(arow_op * BK + (((2 * ks + (lane >> 5)) ^ akey) << 3));
  const int brow_op = wn * 128 + (lane & 31);
  const int kcol = (lane >> 5) * 8;

  // One K step: MFMAs on buffer kb%2 with the writes of `sn` (step kb+1)
  // into the other buffer between them; `sl` is refilled with step kb+2.
  auto step = [&](auto buf_tag, int64_t kb, Stage& sn, Stage& sl) {
    constexpr int buf = decltype(buf_tag)::value;   // kb % 2
    uint16_t* const a = buf ? As1 : As0;
    uint16_t* const bb = buf ? Bs1 : Bs0;
    uint16_t* const an = buf ? As0 : As1;
    uint16_t* const bn = buf ? Bs0 : Bs1;
    // The staged registers of step kb+1 arrived before the last barrier.  Using
    // them here, before this step's copies and loads are issued, makes the
    // compiler's wait for them land where nothing is outstanding; a first use
    // after the copies would wait for the copies too (the counter is in order).
    asm volatile("" ::"v"(sn.w[0].x), "v"(sn.w[0].y), "v"(sn.w[0].z), "v"(sn.w[0].w),
                 "v"(sn.w[1].x), "v"(sn.w[1].y), "v"(sn.w[1].z), "v"(sn.w[1].w), "v"(sn.q),
                 "v"(sn.s));
    copy_x(an, kb + 1);
    load(sl, kb + 2);
    const float sc = scale_of(sn);
    bf16x8_t av[2][4], bv[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      av[0][i] = *(const bf16x8_t*)(a + aoff[0] + i * 32 * BK);
      bv[0][i] = *(const bf16x8_t*)(bb + (brow_op + i * 32) * LDS_ROW + kcol);
    }
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < BK / 16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          av[cur ^ 1][i] = *(const bf16x8_t*)(a + aoff[ks + 1] + i * 32 * BK);
          bv[cur ^ 1][i] = *(const bf16x8_t*)(bb + (brow_op + i * 32) * LDS_ROW + (ks + 1) * 16 + kcol);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[cur][i], bv[cur][j], acc[i][j], 0, 0, 0);
      // this substep's quarter of step kb+1's weight row
      put_w(sn, bn, ks, sc);
      // Lay out the substep as 8 x {1 MFMA, address ops, 2 LDS reads (operands
      // of the next substep and table lookups)} then 8 x {1 MFMA, multiplies
      // and conversions, 1 LDS write}: the lookups have eight MFMAs' time to
      // return before they are used.
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgValu, 2, 0);
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
      }
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgValu, 3, 0);
        __builtin_amdgcn_sched_group_barrier(kSgDsWrite, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);   // one substep per scheduling region
    }
    __syncthreads();
  };
  int64_t kb = 0;
  for (; kb + 1 < nkb; kb += 2) {
    step(std::integral_constant<int, 0>{}, kb, s1, s0);
    step(std::integral_constant<int, 1>{}, kb + 1, s0, s1);
  }
  if (kb < nkb) step(std::integral_constant<int, 0>{}, kb, s1, s0);

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


}  // namespace

hipError_t launch_gemm(const uint16_t* x, int64_t ldx, const uint8_t* packed, const void* absmax,
                       const float* absmax2, const float* mean, int double_quant, int M, int N,
                       int K, uint16_t* y, int64_t ldy, hipStream_t stream) {
  const int64_t tm = ((int64_t)M + BM - 1) / BM, tn = ((int64_t)N + BN - 1) / BN;
  const int64_t ntiles = tm * tn;
  if (ntiles > (int64_t)1 << 30) return hipErrorNotSupported;
  const int64_t per_xcd = (ntiles + kXcds - 1) / kXcds;
  const unsigned grid = (unsigned)(per_xcd * kXcds);
  if (double_quant)
    hipLaunchKernelGGL(gemm_kernel<true>, dim3(grid), dim3(kThreads), 0, stream, x, ldx,
                       packed, absmax, absmax2, mean, M, N, K, y, ldy, (int)tm, (int)tn,
                       level_table());
  else
    hipLaunchKernelGGL(gemm_kernel<false>, dim3(grid), dim3(kThreads), 0, stream, x, ldx,
                       packed, absmax, absmax2, mean, M, N, K, y, ldy, (int)tm, (int)tn,
                       level_table());
  return hipGetLastError();
}

}  // namespace bnbx

// Input gradient of the 4-bit linear layer for gfx950:
// dX[M, K] = dY[M, N] . W_hat[N, K], with W_hat the dequantized 4-bit weight
// (NF4 or FP4 levels, bf16 or FP16 compute), frozen.  The pomoai.com overview
// has the 4-bit base weights frozen under QLoRA (the trained adapters need
// the gradient that flows through the base layer); mlqm.cn bitsandbytes
// article, sec. 3.4: 4-bit storage, dequantize to 16 bits, multiply.
//
// The contraction now runs over the weight rows n, so an MFMA B operand (8
// consecutive contraction values for one output column k) needs one value
// from each of 8 rows: the weights are transposed on the way through LDS.
//
// Tiling.  A workgroup (4 waves, one per SIMD) owns a 256 x 256 tile of dX
// and walks N in steps of 64.  Wave w owns all 256 rows m and the columns
// [64 w, 64 w + 64) of the tile: 8 x 2 tiles of v_mfma_f32_32x32x16, 256
// accumulators per lane.  Per step two LDS tiles of 256 rows x 64 values
// (128-byte rows whose eight 16-byte chunks are rotated by (row / 2) % 8, so
// that 16 lanes reading one chunk of 16 consecutive rows hit 64 banks):
//   A: dY[m0 + r][n0 .. n0 + 64), copied from global memory straight into
//      LDS (buffer_load ... lds, 16 bytes per lane);
//   B: W_hat[n0 .. n0 + 64][k0 + r] (row r of the tile is column k0 + r of
//      the weight).  Each thread dequantizes two units of 4 weight rows x 8
//      columns (four packed dwords and four block scales): a byte table in
//      LDS gives the two fp32 levels of each packed byte, times the block
//      scale in fp32, rounded to the compute type; the values of rows
//      (n, n+1) and (n+2, n+3) at one column form one 8-byte LDS write.
// Both tiles are double-buffered: while the MFMAs of step t read buffer t % 2,
// the dY copy and the dequantized weights of step t + 1 go to the other one;
// one wait and one barrier end the step.
//
// Requirements checked on the host: N a multiple of 64 (whole contraction
// steps), K a multiple of 64.  Columns past K in the last tile read clamped
// or range-checked (zero) data and are never stored; rows past M likewise.
#include "bnbx_device.hpp"
#include "bnbx_internal.hpp"

namespace bnbx {
namespace {

constexpr int TM = 256, TK = 256, TN = 64;
constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr int kTile = 256 * TN;   // 16-bit elements per LDS tile (128-byte rows)
constexpr int kCopies = 4;        // byte-table copies (lane & 3) against bank conflicts

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Byte offset of 16-bit element (row r, column c) in a rotated tile.
__device__ __forceinline__ uint32_t tile_off(int r, int c) {
  return (uint32_t)(r * (TN * 2) + (((c >> 3) ^ ((r >> 1) & 7)) << 4) + ((c & 7) << 1));
}

template <bool DQ, bool F16>
__global__ __launch_bounds__(kThreads) void gemm_dx_kernel(
    const uint16_t* __restrict__ dy, int64_t lddy, const uint8_t* __restrict__ packed,
    const void* __restrict__ absmax, const float* __restrict__ absmax2,
    const float* __restrict__ mean, int M, int N, int K, uint16_t* __restrict__ dx,
    int64_t lddx, int tiles_m, int tiles_k, LevelTable lv) {
  __shared__ __attribute__((aligned(16))) uint16_t As0[kTile], As1[kTile], Bs0[kTile], Bs1[kTile];
  __shared__ float2 tabs[kCopies][256];   // byte -> (L[high nibble], L[low nibble])

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;

  // XCD-aware tile id: workgroups b, b+8, ... share an XCD, so consecutive
  // tile ids (the same rows of dY) meet in one L2.
  const int ntiles = tiles_m * tiles_k;
  const int per_xcd = (ntiles + kXcds - 1) / kXcds;
  const int b = blockIdx.x;
  const int tile = (b % kXcds) * per_xcd + b / kXcds;
  if (tile >= ntiles) return;
  const int m0 = (tile / tiles_k) * TM;
  const int k0 = (tile % tiles_k) * TK;

  {
    const int lvl = level_lanes(lv);
    for (int e = tid; e < kCopies * 256; e += kThreads) {
      const uint32_t bb = (uint32_t)e & 255u;
      tabs[e >> 8][bb] = make_float2(level_lookup(lvl, bb >> 4), level_lookup(lvl, bb & 15u));
    }
  }
  const float2* tab = tabs[lane & (kCopies - 1)];
  const float mu = DQ ? *mean : 0.0f;
  const int nkb = K >> 6;
  const uint32_t rowK2 = (uint32_t)K >> 1;

  // dY copy of one step: wave w copies rows [64 w, 64 w + 64) of the tile in
  // 8 instructions of 8 rows; lane l fills chunk slot l % 8 of row l / 8
  // with the chunk the rotation puts there.  Rows past M are clamped.
  const rsrc_t ry = make_rsrc(dy, (uint32_t)((int64_t)(M - 1) * lddy * 2 + (int64_t)N * 2));
  uint32_t yoff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = wave * 64 + i * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ ((r >> 1) & 7);
    int gm = m0 + r;
    gm = gm < M ? gm : M - 1;
    yoff[i] = (uint32_t)(((int64_t)gm * lddy + chunk * 8) * 2);
  }
  auto copy_dy = [&](uint16_t* buf, int step) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ry, (void __attribute__((address_space(3)))*)(buf + (wave * 64 + i * 8) * TN), 16,
          yoff[i], (uint32_t)step * (TN * 2), 0, 0);
  };

  // Weight units of this thread: unit v covers rows 4 rg .. 4 rg + 3 of the
  // step and columns 8 kg .. 8 kg + 7 of the tile (rg = tid % 16, kg =
  // tid / 16 + 16 v): 16 lanes of one kg write one 128-byte LDS row.
  const int rg = tid & 15;
  int kgs[2];
  uint32_t woff[2], qidx[2];
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    kgs[v] = (tid >> 4) + 16 * v;
    const int kcol = k0 + 8 * kgs[v];
    woff[v] = (uint32_t)(4 * rg) * rowK2 + (uint32_t)(kcol >> 1);
    int kblk = kcol >> 6;
    kblk = kblk < nkb ? kblk : nkb - 1;
    qidx[v] = (uint32_t)(4 * rg) * (uint32_t)nkb + (uint32_t)kblk;
  }
  const uint32_t nblocks = (uint32_t)N * (uint32_t)nkb;
  const rsrc_t rw = make_rsrc(packed, (uint32_t)N * rowK2);
  const rsrc_t rq = make_rsrc(absmax, DQ ? nblocks : nblocks * 4u);
  const rsrc_t rg2 = make_rsrc(absmax2, DQ ? (nblocks + 255u) / 256u * 4u : 4u);

  struct WUnit {
    uint32_t d[4];
    uint32_t q[4];
    float s[4];
  };
  auto load_units = [&](WUnit* u, int step) {
    const uint32_t rows = (uint32_t)step * TN;
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u[v].d[i] = __builtin_amdgcn_raw_buffer_load_b32(rw, woff[v] + (rows + i) * rowK2, 0, 0);
        const uint32_t blk = qidx[v] + (rows + i) * (uint32_t)nkb;
        if (DQ) {
          u[v].q[i] = __builtin_amdgcn_raw_buffer_load_b8(rq, blk, 0, 0);
          u[v].s[i] = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(rg2, (blk >> 8) * 4u, 0, 0));
        } else {
          u[v].q[i] = __builtin_amdgcn_raw_buffer_load_b32(rq, blk * 4u, 0, 0);
          u[v].s[i] = 0.0f;
        }
      }
  };
  // Block scale exactly as stored: a_b, or fl32(fl32(q * fl32(s_g / 127)) + mean).
  auto scale_of = [&](uint32_t q, float s) {
    if (!DQ) return __builtin_bit_cast(float, q);
    const float qf = (float)(int8_t)(uint8_t)q;
    const float step = s / 127.0f;
    const float prod = qf * step;
    return prod + mu;
  };
  auto put_units = [&](const WUnit* u, uint16_t* buf) {
    char* base = (char*)buf;
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      float sc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] = scale_of(u[v].q[i], u[v].s[i]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {   // packed byte j: columns 2j (high nibble), 2j + 1
        float2 lp[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) lp[i] = tab[(u[v].d[i] >> (8 * j)) & 0xffu];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r = 8 * kgs[v] + 2 * j + h;   // tile row = column of the weight
          const float w0 = (h ? lp[0].y : lp[0].x) * sc[0], w1 = (h ? lp[1].y : lp[1].x) * sc[1];
          const float w2 = (h ? lp[2].y : lp[2].x) * sc[2], w3 = (h ? lp[3].y : lp[3].x) * sc[3];
          uint2 p;
          p.x = pack16x2<F16>(w0, w1);
          p.y = pack16x2<F16>(w2, w3);
          *(uint2*)(base + tile_off(r, 4 * rg)) = p;
        }
      }
    }
  };

  // Operand offsets (bytes) of lane (col, half) in substep s: row 32 i + col
  // (A) or 32 j + 64 w + col (B), 16-bit columns 16 s + 8 half .. + 8.
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    aoff[s] = tile_off(col, 16 * s + 8 * half);
    boff[s] = tile_off(64 * wave + col, 16 * s + 8 * half);
  }
  // Rows 32 i + col and 32 i + 64 w + col share the rotation ((r / 2) % 8 is
  // the same for r and r + 32), so only the row base changes.

  f32x16_t acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int nsteps = N / TN;
  WUnit wu[2];
  load_units(wu, 0);
  copy_dy(As0, 0);
  __syncthreads();   // byte table complete
  put_units(wu, Bs0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  auto mma_step = [&](const uint16_t* A, const uint16_t* B) {
    const char* a = (const char*)A;
    const char* bq = (const char*)B;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4_t av[8], bv[2];
#pragma unroll
      for (int i = 0; i < 8; ++i) av[i] = *(const u32x4_t*)(a + aoff[s] + i * 32 * TN * 2);
#pragma unroll
      for (int j = 0; j < 2; ++j) bv[j] = *(const u32x4_t*)(bq + boff[s] + j * 32 * TN * 2);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma_32x32x16<F16>(av[i], bv[j], acc[i][j]);
      // one substep's operands live at a time (hoisting all four spilled)
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The loads, copy and dequant of the next step are unconditional (the last
  // step repeats itself into the idle buffers), so no branch separates the
  // loads from their use and they stay in flight across the MFMAs.
  for (int t = 0; t < nsteps; ++t) {
    const int next = t + 1 < nsteps ? t + 1 : t;
    load_units(wu, next);
    copy_dy((t & 1) ? As0 : As1, next);
    mma_step((t & 1) ? As1 : As0, (t & 1) ? Bs1 : Bs0);
    put_units(wu, (t & 1) ? Bs0 : Bs1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // D layout of a 32x32 MFMA tile: lane l, value v -> column l % 32, row
  // 8 (v / 4) + 4 (l / 32) + v % 4.
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = k0 + wave * 64 + 32 * j + col;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = m0 + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
        if (r < M && c < K) dx[(int64_t)r * lddx + c] = f32_to_16<F16>(acc[i][j][v]);
      }
    }
}

}  // namespace

hipError_t launch_gemm_dx(const uint16_t* dy, int64_t lddy, const uint8_t* packed,
                          const void* absmax, const float* absmax2, const float* mean,
                          int double_quant, int quant_type, bool f16, int M, int N, int K,
                          uint16_t* dx, int64_t lddx, hipStream_t stream) {
  const int64_t kLimit = (int64_t)1 << 31;
  if (N % TN != 0 || K % 64 != 0) return hipErrorNotSupported;
  if ((int64_t)N * (K / 2) >= kLimit) return hipErrorNotSupported;
  // dY offsets are 32-bit: walk M in slabs whose rows fit.
  int64_t slab = (kLimit - (int64_t)N * 2) / (lddy * 2);
  slab = slab / TM * TM;
  if (slab < TM) return hipErrorNotSupported;
  const LevelTable& lv = level_table(quant_type);
  for (int64_t r0 = 0; r0 < M; r0 += slab) {
    const int m = (int)(M - r0 < slab ? M - r0 : slab);
    const int tm = (m + TM - 1) / TM, tk = (K + TK - 1) / TK;
    const int per_xcd = (tm * tk + kXcds - 1) / kXcds;
    const uint16_t* dys = dy + r0 * lddy;
    uint16_t* dxs = dx + r0 * lddx;
    auto go = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, dim3((unsigned)(per_xcd * kXcds)), dim3(kThreads), 0, stream,
                         dys, lddy, packed, absmax, absmax2, mean, m, N, K, dxs, lddx, tm, tk,
                         lv);
    };
    if (double_quant) {
      if (f16) go(gemm_dx_kernel<true, true>);
      else go(gemm_dx_kernel<true, false>);
    } else {
      if (f16) go(gemm_dx_kernel<false, true>);
      else go(gemm_dx_kernel<false, false>);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bnbx

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
// Tiling.  A workgroup of 8 waves (two per SIMD) owns a 256 x 256 tile of dX
// and walks N in steps of 64.  Wave w owns rows [128 (w / 4), +128) and
// columns [64 (w % 4), +64) of the tile: 4 x 2 tiles of
// v_mfma_f32_32x32x16, 128 accumulators per lane.  Two waves per SIMD let one
// issue MFMAs while the other waits on LDS for its dequant work (with one
// wave per SIMD every such wait stopped the matrix core).  Per step two LDS
// tiles of 256 rows x 64 values (128-byte rows whose eight 16-byte chunks are
// rotated by (row / 2) % 8, so that 16 lanes reading one chunk of 16
// consecutive rows hit 64 banks):
//   A: dY[m0 + r][n0 .. n0 + 64), copied from global memory straight into
//      LDS (buffer_load ... lds, 16 bytes per lane);
//   B: W_hat[n0 .. n0 + 64][k0 + r'] (row r of the tile is column k0 + r'
//      of the weight, r' = r with the two columns of each pair swapped in
//      odd groups of 8, which spreads the writes over both bank halves).
//      Each thread dequantizes one unit of 4 weight rows x 8 columns (four
//      packed dwords; the rows' block scales come from a small LDS table
//      that 256 threads fill per step): a byte table in LDS gives the two
//      fp32 levels of each packed byte, times the block scale in fp32,
//      rounded to the compute type; the values of rows (n, n+1) and
//      (n+2, n+3) at one column form one 8-byte LDS write.
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
constexpr int kThreads = 512;     // 8 waves, two per SIMD
constexpr int kXcds = 8;
constexpr int kTile = 256 * TN;   // 16-bit elements per LDS tile (128-byte rows)
constexpr int kCopies = 8;        // byte-table copies, interleaved per entry (lane & 7)

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Byte offset of 16-bit element (row r, column c) in a rotated tile.
__device__ __forceinline__ uint32_t tile_off(int r, int c) {
  return (uint32_t)(r * (TN * 2) + (((c >> 3) ^ ((r >> 1) & 7)) << 4) + ((c & 7) << 1));
}

template <int DQ, bool F16>
__global__ __launch_bounds__(kThreads) void gemm_dx_kernel(
    const uint16_t* __restrict__ dy, int64_t lddy, const uint8_t* __restrict__ packed,
    const void* __restrict__ absmax, const float* __restrict__ absmax2,
    const float* __restrict__ mean, int M, int N, int K, uint16_t* __restrict__ dx,
    int64_t lddx, int tiles_m, int tiles_k, LevelTable lv) {
  // One LDS array for the four tiles (A0, A1, B0, B1 at 0, 32, 64, 96 KB), so
  // that which buffer an access goes to is an immediate offset from one base
  // address (separate arrays made the compiler keep an address register per
  // buffer and spill them).
  __shared__ __attribute__((aligned(16))) uint16_t lds[4 * kTile];
  uint16_t* const As0 = lds;
  uint16_t* const As1 = lds + kTile;
  uint16_t* const Bs0 = lds + 2 * kTile;
  uint16_t* const Bs1 = lds + 3 * kTile;
  // byte -> (L[high nibble], L[low nibble]); entry e of copy c at e * 8 + c,
  // so lanes of different copies read different banks whatever e they read
  __shared__ float2 tabs[256][kCopies];
  __shared__ float scl[2][4][TN];   // block scales of a step: [block][row]
  constexpr bool DYN = DQ == kDqDynamic;
  __shared__ float dmap[DYN ? 256 : 1];   // the dynamic 8-bit map (DYN)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mh = wave >> 2, wk = wave & 3;   // rows [128 mh, +128), columns [64 wk, +64)
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

  if (DYN && tid < 256) dmap[tid] = kDynMapDev.v[tid];
  {
    const int lvl = level_lanes(lv);
    for (int e = tid; e < kCopies * 256; e += kThreads) {
      const uint32_t bb = (uint32_t)e / kCopies;
      tabs[bb][e % kCopies] =
          make_float2(level_lookup(lvl, bb >> 4), level_lookup(lvl, bb & 15u));
    }
  }
  const float2* tab = &tabs[0][lane & (kCopies - 1)];   // entry e at tab[e * kCopies]
  const float mu = DQ ? *mean : 0.0f;
  const int nkb = K >> 6;
  const uint32_t rowK2 = (uint32_t)K >> 1;

  // dY copy of one step: wave w copies rows [32 w, 32 w + 32) of the tile in
  // 4 instructions of 8 rows; lane l fills chunk slot l % 8 of row l / 8
  // with the chunk the rotation puts there.  Rows past M are clamped.
  const rsrc_t ry = make_rsrc(dy, (uint32_t)((int64_t)(M - 1) * lddy * 2 + (int64_t)N * 2));
  uint32_t yoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wave * 32 + i * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ ((r >> 1) & 7);
    int gm = m0 + r;
    gm = gm < M ? gm : M - 1;
    yoff[i] = (uint32_t)(((int64_t)gm * lddy + chunk * 8) * 2);
  }
  auto copy_dy = [&](uint16_t* buf, int step) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ry, (void __attribute__((address_space(3)))*)(buf + (wave * 32 + i * 8) * TN), 16,
          yoff[i], (uint32_t)step * (TN * 2), 0, 0);
  };

  // The thread's weight unit: rows 4 rg .. 4 rg + 3 of the step and columns
  // 8 kg .. 8 kg + 7 of the tile (rg = tid % 16, kg = tid / 16): 16 lanes of
  // one kg write one 128-byte LDS row.  One packed dword per row; the
  // per-lane offset is fixed, the step's rows come as a scalar offset.
  const int rg = tid & 15, kg = tid >> 4;
  const rsrc_t rw = make_rsrc(packed, (uint32_t)N * rowK2);
  uint32_t wvo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    wvo[i] = (uint32_t)(4 * rg + i) * rowK2 + (uint32_t)((k0 + 8 * kg) >> 1);
  struct WUnit {
    uint32_t d[4];
  };
  auto load_unit = [&](WUnit& u, int step) {
    const uint32_t so = (uint32_t)step * TN * rowK2;
#pragma unroll
    for (int i = 0; i < 4; ++i) u.d[i] = __builtin_amdgcn_raw_buffer_load_b32(rw, wvo[i], so, 0);
  };

  // Block scales of a step: 64 rows x the tile's 4 blocks, one per thread of
  // the first 256 (row tid / 4, block tid % 4).  Exactly as stored: a_b, or
  // fl32(fl32(q * fl32(s_g / 127)) + mean) (dq_scale), or with the dynamic
  // map fl32(fl32(map[q] * s_g) + mean).
  const uint32_t nblocks = (uint32_t)N * (uint32_t)nkb;
  const rsrc_t rq = make_rsrc(absmax, DQ ? nblocks : nblocks * 4u);
  const rsrc_t rg2 = make_rsrc(absmax2, DQ ? (nblocks + 255u) / 256u * 4u : 4u);
  const bool scaler = tid < 4 * TN;   // uniform per wave
  const int srow = (tid >> 2) & (TN - 1), sblk = tid & 3;
  int sk = (k0 >> 6) + sblk;
  sk = sk < nkb ? sk : nkb - 1;
  const uint32_t sidx = (uint32_t)srow * (uint32_t)nkb + (uint32_t)sk;
  struct SRaw {
    uint32_t q;
    float s;
  };
  auto load_scale = [&](int step) {
    SRaw r{0u, 0.0f};
    if (scaler) {
      const uint32_t blk = sidx + (uint32_t)step * TN * (uint32_t)nkb;
      if (DQ) {
        r.q = __builtin_amdgcn_raw_buffer_load_b8(rq, blk, 0, 0);
        r.s = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rg2, (blk >> 8) * 4u, 0, 0));
      } else {
        r.q = __builtin_amdgcn_raw_buffer_load_b32(rq, blk * 4u, 0, 0);
      }
    }
    return r;
  };
  auto put_scale = [&](const SRaw& r, int buf) {
    if (!scaler) return;
    float sc;
    if (DYN) {
      const float prod = dmap[r.q & 0xffu] * r.s;
      sc = prod + mu;
    } else if (DQ) {
      sc = dq_scale((float)(int8_t)(uint8_t)r.q, r.s, mu);
    } else {
      sc = __builtin_bit_cast(float, r.q);
    }
    scl[buf][sblk][srow] = sc;
  };

  // Piece p (0..3) of the dequant into a B tile: packed byte p of the unit's
  // four rows (columns 8 kg + 2 p and 8 kg + 2 p + 1).
  // The four block scales of the thread's unit (the same for all four
  // pieces of a step: its 8 columns lie in one block), read once per step.
  auto scales4 = [&](int sbuf) { return *(const float4*)&scl[sbuf][kg >> 3][4 * rg]; };
  auto put_piece = [&](const WUnit& u, const float4 sc4, int p, uint16_t* buf) {
    char* base = (char*)buf;
    float2 lp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) lp[i] = tab[((u.d[i] >> (8 * p)) & 0xffu) * kCopies];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // tile row of column 8 kg + 2 p + h: odd kg swap the columns of each
      // pair, so the four kg of a wave write both 128-byte halves of the banks
      const int r = 8 * kg + 2 * p + (h ^ (kg & 1));
      const float w0 = (h ? lp[0].y : lp[0].x) * sc4.x;
      const float w1 = (h ? lp[1].y : lp[1].x) * sc4.y;
      const float w2 = (h ? lp[2].y : lp[2].x) * sc4.z;
      const float w3 = (h ? lp[3].y : lp[3].x) * sc4.w;
      uint2 pk;
      pk.x = pack16x2<F16>(w0, w1);
      pk.y = pack16x2<F16>(w2, w3);
      *(uint2*)(base + tile_off(r, 4 * rg)) = pk;
    }
  };

  // Operand offsets (bytes) of lane (col, half) in substep s: rows
  // 128 mh + 32 i + col (A) and 64 wk + 32 j + col (B), 16-bit columns
  // 16 s + 8 half .. + 8.  Rows 32 apart share the rotation.
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    aoff[s] = tile_off(128 * mh + col, 16 * s + 8 * half);
    boff[s] = tile_off(64 * wk + col, 16 * s + 8 * half);
  }

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Pipeline.  Step t reads A/B buffer t % 2; during it the dY copy of step
  // t + 1 goes to the other A buffer, the weights of step t + 1 (loaded one
  // step earlier, so already in registers, with their scales in LDS) are
  // dequantized into the other B buffer in four pieces, one after the MFMAs
  // of each substep, and the weights and scale inputs of step t + 2 are
  // loaded.  The step ends with a wait to zero (a copy's arrival in LDS is not
  // ordered with later loads), the scales of step t + 2 into LDS, and one
  // barrier.  Steps past the end repeat the last one into idle buffers.
  const int nsteps = N / TN;
  auto clampstep = [&](int t) { return t < nsteps ? t : nsteps - 1; };
  WUnit wa, wb;
  load_unit(wa, 0);
  copy_dy(As0, 0);
  const SRaw r0 = load_scale(0), r1 = load_scale(clampstep(1));
  load_unit(wb, clampstep(1));
  __builtin_amdgcn_s_waitcnt(0);
  if (DYN) __syncthreads();   // the map in LDS
  put_scale(r0, 0);
  put_scale(r1, 1);
  __syncthreads();   // byte table and first scales complete
  {
    const float4 sc4 = scales4(0);
#pragma unroll
    for (int p = 0; p < 4; ++p) put_piece(wa, sc4, p, Bs0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  auto step = [&](int t, const uint16_t* A, const uint16_t* B, uint16_t* Anext, uint16_t* Bnext,
                  const WUnit& wput, WUnit& wload) {
    const int sb = (t + 1) & 1;                 // scale buffer of step t + 1
    const SRaw rr = load_scale(clampstep(t + 2));
    load_unit(wload, clampstep(t + 2));
    copy_dy(Anext, clampstep(t + 1));
    const char* a = (const char*)A;
    const char* bq = (const char*)B;
    const float4 sc4 = scales4(sb);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4_t av[4], bv[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = *(const u32x4_t*)(a + aoff[s] + i * 32 * TN * 2);
#pragma unroll
      for (int j = 0; j < 2; ++j) bv[j] = *(const u32x4_t*)(bq + boff[s] + j * 32 * TN * 2);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma_32x32x16<F16>(av[i], bv[j], acc[i][j]);
      put_piece(wput, sc4, s, Bnext);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    put_scale(rr, t & 1);                       // step t + 2 uses buffer t % 2
    __syncthreads();
  };
  for (int t = 0; t < nsteps; t += 2) {
    step(t, As0, Bs0, As1, Bs1, wb, wa);       // puts step t + 1 (set b), loads t + 2 (set a)
    if (t + 1 < nsteps) step(t + 1, As1, Bs1, As0, Bs0, wa, wb);
  }

  // D layout of a 32x32 MFMA tile: lane l, value v -> column l % 32, row
  // 8 (v / 4) + 4 (l / 32) + v % 4.  Tile row 64 wk + 32 j + col of B holds
  // column 64 wk + 32 j + (col ^ ((col / 8) % 2)).
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = k0 + wk * 64 + 32 * j + (col ^ ((col >> 3) & 1));
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = m0 + 128 * mh + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
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
    if (double_quant == kDqDynamic) {
      if (f16) go(gemm_dx_kernel<kDqDynamic, true>);
      else go(gemm_dx_kernel<kDqDynamic, false>);
    } else if (double_quant) {
      if (f16) go(gemm_dx_kernel<kDqLinear, true>);
      else go(gemm_dx_kernel<kDqLinear, false>);
    } else {
      if (f16) go(gemm_dx_kernel<kDqNone, true>);
      else go(gemm_dx_kernel<kDqNone, false>);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bnbx

// Decode GEMV with 4-bit (NF4 or FP4) weights for gfx950:
// Y[M, N] = X[M, K] . W_hat[N, K]^T,
// M <= 16 (mlqm.cn bitsandbytes article, sec. 3.4 "4-bit storage, 16-bit
// compute", and the sec. 7 pitfall that 4-bit only pays off when the layer is
// bound by weight traffic: so the packed weight is streamed exactly once per
// group of up to four rows of X).
//
// Work layout.  A row of W is C = K/32 chunks of 16 packed bytes (32
// weights, half of one 64-block).  A row is owned by a team of TW waves
// (S = 64 TW lanes); lane s of a team owns chunks s, s+S, ..., s+(NI-1)S of
// every row the team takes, so its slice of X is read once into registers.
// A workgroup is 16 waves and the grid has at most one workgroup per CU; a
// team takes RR rows per pass, so for the decode shapes one pass covers the
// matrix.  The first row's loads go out before the lookup table is built,
// the others right after the workgroup barrier (a wave stalled issuing loads
// into a full memory pipeline would otherwise hold the barrier for all).
//
// Loads are buffer loads whose resource is the row (a scalar base and a
// length), with a per-lane offset fixed for the whole kernel.  The hardware
// range check returns zero past the end of the row (the ragged last chunks)
// and for rows past N, so there is no per-load address arithmetic or bounds
// branch.  With double quant a row's int8 codes come in one dword per lane and
// reach the lanes that need them by ds_bpermute, and its (at most two) group
// scales by scalar loads.  X is staged once per workgroup in LDS.
//
// Dequant in registers.  An LDS table maps each packed byte to the level pair
// (L[high nibble], L[low nibble]) in the compute type (bf16, or FP16 with
// v_dot2_f32_f16 and the _f16 MFMA); it is replicated in 32 lane columns with a
// 256-byte stride so that the lanes of each half-wave read distinct banks, and
// the byte address (byte << 8 | lane << 2) is one v_perm_b32.  The pair feeds
// v_dot2_f32_bf16 against the matching X pair and the 32-weight partial sum
// is scaled once by its block scale, so dequant costs one VALU instruction per
// weight plus one LDS read per two.  Chunks are consumed one at a time in
// load order (scheduling barriers keep the compiler from hoisting work above
// the waits).  Sums over a wave use DPP row shifts and row broadcasts; a
// multi-wave team adds its waves' sums through LDS.
#include "bnbx_device.hpp"
#include "bnbx_internal.hpp"

namespace bnbx {
namespace {

constexpr int kWaves = 16;                  // waves per workgroup (one workgroup per CU)
constexpr int kThreads = kWaves * 64;
constexpr int kCopies = 32;                 // lane columns of the byte table (128 B)
constexpr int kTabBytes = 256 * 256;        // 256 B per byte value
// X staged in LDS when MM*K*2 fits (the table takes 64 KB of the CU's 160 KB).
constexpr int kXBytes = 64 * 1024;
constexpr int kMaxMM = 4;
constexpr int kMaxRR = 4;
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer, 32-bit data format

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           (int)kRsrcWord3);
}
template <int AUX>
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int CTRL, int ROWMASK, bool BOUND_ZERO>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWMASK, 0xf, BOUND_ZERO));
}
// Sum over the 64 lanes of a wave, left in lane 63: prefix sums within each
// row of 16 lanes (row_shr 1, 2, 4, 8), then row_bcast:15 and row_bcast:31
// carry the row totals up to lane 63.
__device__ __forceinline__ float wave_sum_to_63(float v) {
  v += dpp<0x111, 0xf, true>(v);
  v += dpp<0x112, 0xf, true>(v);
  v += dpp<0x114, 0xf, true>(v);
  v += dpp<0x118, 0xf, true>(v);
  v += dpp<0x142, 0xa, false>(v);
  v += dpp<0x143, 0xc, false>(v);
  return v;
}

// Block-scale storage: fp32 absmax, or double quant (int8 code + fp32 group
// scale + mean) read per lane, or double quant read per row.  The row-wise
// read loads whole dwords of codes, and the buffer range check zeroes a dword
// that is only partly inside the row, so it needs a row of 4k blocks (at most
// 256: K <= 16384, K % 256 == 0) and 4-byte aligned codes.
enum ScaleMode { kScaleF32 = 0, kScaleDqLane = 1, kScaleDqRow = 2 };

// MM rows of X per launch (rows >= mvalid are zero), NI chunks per lane, RR
// rows of W per team and pass.  TW = 1 << twl waves per team.
template <int MM, int NI, int RR, int SM, bool F16>
__global__ __launch_bounds__(kThreads, 4) void gemv_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ packed,
    const void* __restrict__ absmax, const float* __restrict__ absmax2,
    const float* __restrict__ mean, int mvalid, int N, int K, uint16_t* __restrict__ y,
    int64_t ldy, int twl, int xlds, LevelTable lv) {
  constexpr bool DQ = SM != kScaleF32;
  // One LDS block with the table at offset 0, so that a table address is the
  // v_perm result itself (the ds_read offset field cannot hold a 64 KB base),
  // then X, then the team sums.  X is stored in 64-byte chunks whose four
  // 16-byte pieces are rotated by (chunk / 4) % 4: piece q of chunk c sits at
  // 64 c + 16 (q ^ ((c >> 2) & 3)), so that 16 lanes reading piece q of 16
  // consecutive chunks hit 64 distinct banks.
  __shared__ __attribute__((aligned(16))) unsigned char smem[kTabBytes + kXBytes +
                                                             kWaves * MM * RR * 4];
  unsigned char* const tab = smem;
  unsigned char* const xs = smem + kTabBytes;
  float* const red = (float*)(smem + kTabBytes + kXBytes);

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int TW = 1 << twl;
  const int tpw = kWaves >> twl;              // teams per workgroup
  const int team_l = wave >> twl;
  const int wit = wave - (team_l << twl);     // wave within team
  const int S = 64 << twl;
  const int s = wit * 64 + lane;              // lane slot within team
  const int C = K >> 5;
  const uint32_t rowK2 = (uint32_t)K >> 1;
  const uint32_t nkb = (uint32_t)K >> 6;
  const uint32_t xbytes = (uint32_t)K * 2u;
  const int64_t pass_rows = (int64_t)gridDim.x * tpw * RR;
  const int64_t rb_first = (int64_t)blockIdx.x * tpw * RR;   // workgroup's first row
  const uint32_t ng_bytes = DQ ? (uint32_t)((((uint64_t)N * nkb + 255) >> 8) * 4) : 0u;
  const rsrc_t rg = make_rsrc(absmax2, ng_bytes);

  // Fixed per-lane offsets: chunk c of the row (bytes), its block (index).
  uint32_t woff[NI], boff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint32_t c = (uint32_t)(s + i * S);
    woff[i] = c * 16u;
    boff[i] = c >> 1;
  }

  // 1. X: staging loads (LDS path) or the lane's slice directly.
  uint32_t xr[MM][NI][16];
  constexpr int kStage = kXBytes / 16 / kThreads;   // 16-byte pieces per thread (max)
  uint4 xst[kStage];
  const int xpieces = (int)(xbytes >> 4);          // per row of X
  if (xlds) {
    // One resource over the valid rows of X; rows at or past mvalid (and
    // pieces past MM rows) fall outside it and read as zero.
    const rsrc_t rx = make_rsrc(x, (uint32_t)((int64_t)(mvalid - 1) * ldx * 2) + xbytes);
#pragma unroll
    for (int k = 0; k < kStage; ++k) {
      const int e = t + k * kThreads;
      if (e < MM * xpieces) {          // whole waves drop out: no idle loads
        const int m = e / xpieces;
        const int p = e - m * xpieces;
        xst[k] = buf_load16<0>(rx, (uint32_t)((int64_t)m * ldx * 2) + (uint32_t)p * 16u);
      }
    }
  } else {
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      const rsrc_t rx = make_rsrc(x + (int64_t)m * ldx, m < mvalid ? xbytes : 0u);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 v = buf_load16<0>(rx, woff[i] * 4u + q * 16u);
          xr[m][i][4 * q] = v.x;
          xr[m][i][4 * q + 1] = v.y;
          xr[m][i][4 * q + 2] = v.z;
          xr[m][i][4 * q + 3] = v.w;
        }
      }
    }
  }

  // 2. Weight and scale loads of RR rows.  Rows past N get an empty resource.
  //    Double quant with rows of at most 256 blocks (K <= 16384) loads a
  //    row's int8 codes with one dword per lane (lane l: blocks 4l..4l+3,
  //    handed to the lanes that need them by ds_bpermute) and its group
  //    scales with scalar loads (a row spans at most two groups); otherwise
  //    every lane loads its own block's scales.
  constexpr bool rowsc = SM == kScaleDqRow;
  const uint32_t ng = DQ ? (uint32_t)(((uint64_t)N * nkb + 255) >> 8) : 1u;
  uint4 w[RR][NI];
  int qv[RR][NI];
  float gv[RR][NI];
  int qd[RR];
  float gs0[RR], gs1[RR];
  uint32_t split[RR];
  auto issue_part = [&](int64_t rb, int lo, int hi) {
#pragma unroll
    for (int j = 0; j < RR; ++j) {
      if ((j + 1) * NI <= lo || j * NI >= hi) continue;
      const int64_t row = rb + j;
      const bool ok = row < N;
      const rsrc_t rw = make_rsrc(packed + row * rowK2, ok ? rowK2 : 0u);
#pragma unroll
      for (int i = 0; i < NI; ++i)
        if (j * NI + i >= lo && j * NI + i < hi) w[j][i] = buf_load16<2>(rw, woff[i]);   // nt
      if (j * NI < lo) continue;              // the row's scales went with its first chunk
      if (rowsc) {
        const rsrc_t rq = make_rsrc((const int8_t*)absmax + row * nkb, ok ? nkb : 0u);
        qd[j] = (int)__builtin_amdgcn_raw_buffer_load_b32(rq, (uint32_t)lane * 4u, 0, 0);
        const uint32_t blk0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(row * nkb));
        uint32_t g0 = blk0 >> 8;
        g0 = g0 < ng ? g0 : ng - 1u;
        const uint32_t g1 = g0 + 1u < ng ? g0 + 1u : ng - 1u;
        gs0[j] = absmax2[g0];
        gs1[j] = absmax2[g1];
        split[j] = 256u - (blk0 & 255u);     // blocks of the row in group g0
      } else if (DQ) {
        const rsrc_t rq = make_rsrc((const int8_t*)absmax + row * nkb, ok ? nkb : 0u);
        const uint32_t blk0 = (uint32_t)(row * nkb);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          qv[j][i] = (int8_t)__builtin_amdgcn_raw_buffer_load_b8(rq, boff[i], 0, 0);
          gv[j][i] = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(rg, ((blk0 + boff[i]) >> 8) * 4u, 0, 0));
        }
      } else {
        const rsrc_t ra = make_rsrc((const float*)absmax + row * nkb, ok ? nkb * 4u : 0u);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          qv[j][i] = 0;
          gv[j][i] = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(ra, boff[i] * 4u, 0, 0));
        }
      }
    }
  };
  auto issue = [&](int64_t rb) { issue_part(rb, 0, RR * NI); };
  // The first row of the first pass goes out now, before the table build;
  // the other rows after the barrier, so that a wave held up issuing loads
  // into a full memory pipeline does not hold the barrier for the others.
  issue_part(rb_first + (int64_t)team_l * RR, 0, NI);

  // 3. Byte -> level-pair table (compute type), then X into LDS.
  const int lvl = level_lanes(lv);
  for (int e = t; e < 256 * kCopies / 4; e += kThreads) {
    const uint32_t b = (uint32_t)e / (kCopies / 4);
    const uint32_t v = pack16x2<F16>(level_lookup(lvl, b >> 4), level_lookup(lvl, b & 15u));
    *(uint4*)(tab + b * 256u + ((uint32_t)e % (kCopies / 4)) * 16u) = make_uint4(v, v, v, v);
  }
  if (xlds) {
#pragma unroll
    for (int k = 0; k < kStage; ++k) {
      const int e = t + k * kThreads;
      if (e < MM * xpieces) {
        const uint32_t c = (uint32_t)e >> 2, q = (uint32_t)e & 3u;   // chunk and piece
        *(uint4*)(xs + c * 64u + ((q ^ ((c >> 2) & 3u)) << 4)) = xst[k];
      }
    }
  }
  // Nothing may move across the barrier: a weight use hoisted above it would
  // make every wave wait there for its first row.
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
  // X slice of this lane (LDS path), read up front.
  auto read_x = [&](int i) {
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      {
        const int c = s + i * S;
        const bool in = c < C;
        const uint32_t cg = (uint32_t)(m * C + (in ? c : 0));   // chunk of the staged X
        const unsigned char* src = xs + cg * 64u;
        const uint32_t rot = (cg >> 2) & 3u;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 v = *(const uint4*)(src + (((uint32_t)q ^ rot) << 4));
          xr[m][i][4 * q] = in ? v.x : 0u;
          xr[m][i][4 * q + 1] = in ? v.y : 0u;
          xr[m][i][4 * q + 2] = in ? v.z : 0u;
          xr[m][i][4 * q + 3] = in ? v.w : 0u;
        }
      }
    }
  };
  if (xlds) {
#pragma unroll
    for (int i = 0; i < NI; ++i) read_x(i);
  }

  issue_part(rb_first + (int64_t)team_l * RR, NI, RR * NI);
  const float mu = DQ ? *mean : 0.0f;
  const uint32_t lanebyte = (uint32_t)(lane & (kCopies - 1)) << 2;
  // 4. Dequant-in-register dot products of one pass, one chunk at a time in
  //    load order, then the sums over the team and the stores.
  auto pass = [&](int64_t rb) {
    float acc[MM][RR];
#pragma unroll
    for (int j = 0; j < RR; ++j) {
#pragma unroll
      for (int m = 0; m < MM; ++m) acc[m][j] = 0.0f;
      // the row's (at most two) group steps fl32(s_g / 127), once per row
      const float step0 = rowsc ? dq_step_normal(gs0[j]) : 0.0f;
      const float step1 = rowsc ? dq_step_normal(gs1[j]) : 0.0f;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float sc;
        if (rowsc) {
          const int qw = __builtin_amdgcn_ds_bpermute((int)((boff[i] >> 2) << 2), qd[j]);
          const int q = __builtin_amdgcn_sbfe(qw, (boff[i] & 3u) * 8u, 8);
          const float prod = (float)q * (boff[i] < split[j] ? step0 : step1);
          sc = prod + mu;
        } else {
          sc = DQ ? (float)qv[j][i] * dq_step_normal(gv[j][i]) + mu : gv[j][i];
        }
        const uint32_t d[4] = {w[j][i].x, w[j][i].y, w[j][i].z, w[j][i].w};
        float part[MM];
#pragma unroll
        for (int m = 0; m < MM; ++m) part[m] = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const uint32_t addr = perm(d[q], lanebyte, 0x0c0c0000u | ((4u + b) << 8));
            const uint32_t pair = *(const uint32_t*)(tab + addr);
#pragma unroll
            for (int m = 0; m < MM; ++m) part[m] = dot2_16<F16>(pair, xr[m][i][4 * q + b], part[m]);
          }
        }
#pragma unroll
        for (int m = 0; m < MM; ++m) acc[m][j] = __builtin_fmaf(part[m], sc, acc[m][j]);
        // Only one chunk's table addresses and pairs live at a time.
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int j = 0; j < RR; ++j)
#pragma unroll
      for (int m = 0; m < MM; ++m) acc[m][j] = wave_sum_to_63(acc[m][j]);
    if (TW == 1) {
      if (lane == 63) {
#pragma unroll
        for (int j = 0; j < RR; ++j)
#pragma unroll
          for (int m = 0; m < MM; ++m)
            if (rb + j < N && m < mvalid) y[(int64_t)m * ldy + rb + j] = f32_to_16<F16>(acc[m][j]);
      }
    } else {
      if (lane == 63) {
#pragma unroll
        for (int j = 0; j < RR; ++j)
#pragma unroll
          for (int m = 0; m < MM; ++m) red[(wave * MM + m) * RR + j] = acc[m][j];
      }
      __syncthreads();
      if (wit == 0 && lane < MM * RR) {
        const int m = lane / RR, j = lane - (lane / RR) * RR;
        float v = 0.0f;
        for (int u = 0; u < TW; ++u) v += red[((team_l * TW + u) * MM + m) * RR + j];
        if (rb + j < N && m < mvalid) y[(int64_t)m * ldy + rb + j] = f32_to_16<F16>(v);
      }
      __syncthreads();
    }
  };
  // The first pass uses the loads issued before the table build; later
  // passes (more rows than the grid holds at once) issue their own.  The
  // loop condition is the workgroup's, so its barriers are uniform.
  pass(rb_first + (int64_t)team_l * RR);
  for (int64_t rb0 = rb_first + pass_rows; rb0 < N; rb0 += pass_rows) {
    issue(rb0 + (int64_t)team_l * RR);
    pass(rb0 + (int64_t)team_l * RR);
  }
}

// ---------------------------------------------------------------------------
// 4 < M <= 16: the weights streamed once into v_mfma_f32_16x16x32_bf16 (or
// _f16 with the FP16 compute dtype).
//
// A workgroup of 16 waves takes groups of 16 weight rows (16 columns of Y)
// in turn; wave w owns the K slice of blocks [w nkb / 16, (w+1) nkb / 16)
// (BPW = 4 blocks: K = 4096) and keeps its X slice for all 16
// rows of X in registers as MFMA A operands.  In an MFMA, lane l supplies
// column l % 16 and eight k of the 32; the 32 k of each MFMA are one half of
// one block, lane quarter q taking k [16q + 8h, 16q + 8h + 8) of half h, so
// every MFMA sits inside one block.  The B operand is the bf16 levels from
// the byte -> pair table (as in gemv_kernel, no per-weight arithmetic); a
// block's two MFMAs go to a zeroed accumulator that is then scaled by the
// block scale of the lane's column (its own row's) and added to the running
// sums.  The 16 waves' partial sums meet in LDS once per round of GD row
// groups.
//
// Weights and X are loaded row-contiguous (16 bytes per lane, eight lanes
// per 128-byte line: an MFMA layout would touch 16 rows per load) and turned
// into the MFMA layout through a 512 BPW-byte LDS region private to the
// wave: 16-byte pieces of a row are stored at piece ^ f(row), which makes
// the layout reads conflict-free.
// ---------------------------------------------------------------------------
constexpr int kMfWaves = 16;

template <int BPW, int GD, int SM, bool F16>
__global__ __launch_bounds__(kMfWaves * 64, 1) void gemv_mfma_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ packed,
    const void* __restrict__ absmax, const float* __restrict__ absmax2,
    const float* __restrict__ mean, int M, int N, int K, uint16_t* __restrict__ y, int64_t ldy,
    LevelTable lv) {
  constexpr bool DQ = SM != kScaleF32;
  constexpr int kPieces = 2 * BPW;                 // 16-byte pieces per row of a slice
  constexpr int kRow = 16 * kPieces;               // bytes per row of a slice
  constexpr int kLoads = 16 * kPieces / 64;        // row-contiguous loads per 16 rows
  constexpr int kRegion = 16 * kRow;               // bytes of a wave's region
  // Table at LDS offset 0 (its addresses are v_perm results), then the
  // waves' partial sums of GD row groups (16 waves x 64 lanes x 4 values
  // each), then the waves' transpose regions.
  __shared__ __attribute__((aligned(16))) unsigned char
      smem[kTabBytes + GD * kMfWaves * 1024 + kMfWaves * kRegion];
  unsigned char* const tab = smem;
  float* const red = (float*)(smem + kTabBytes);

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  unsigned char* const reg = smem + kTabBytes + GD * kMfWaves * 1024 + wave * kRegion;
  const int c = lane & 15, q = lane >> 4;
  const int nkb = K >> 6;
  const int b0 = wave * BPW;                       // nkb == 16 BPW
  const uint32_t rowK2 = (uint32_t)K >> 1;
  const int ngroups = (N + 15) >> 4;

  // Region layout: piece p of row r at r * kRow + 16 (p ^ swz(r)).
  static_assert(BPW == 4, "slices of 4 blocks");
  auto swz = [](int r) { return (r >> 1) & 7; };
  // A row-contiguous load covers 64 / kPieces rows: lane l of load u takes
  // piece (64 u + l) % kPieces of row (64 u + l) / kPieces.
  auto put = [&](const u32x4_t (&v)[kLoads]) {
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int e = 64 * u + lane, r = e / kPieces, p = e % kPieces;
      *(u32x4_t*)(reg + r * kRow + 16 * (p ^ swz(r))) = v[u];
    }
  };

  // X slice, A operand of half h of block i, lane (row l % 16, quarter q):
  // X[row][64 (b0 + i) + 16 q + 8 h ..+8] = piece 8 i + 2 q + h of the
  // row's slice; rows >= M read as zero.
  const rsrc_t rx = make_rsrc(x, (uint32_t)((int64_t)(M - 1) * ldx * 2 + (int64_t)K * 2));
  u32x4_t xa[BPW][2];
  {
    // The slice is 16 rows x 8 BPW pieces; it passes through the region in
    // four rounds of kPieces pieces per row (BPW / 4 blocks), whose loads all
    // go out first (every workgroup reads all of X at once, so a round often
    // waits for a miss; two rounds in flight took 3% longer).
    constexpr int kBr = BPW / 4;
    u32x4_t xv[4][kLoads];
    auto xload = [&](int R) {
#pragma unroll
      for (int u = 0; u < kLoads; ++u) {
        const int e = 64 * u + lane, r = e / kPieces, p = e % kPieces;
        xv[R][u] = __builtin_amdgcn_raw_buffer_load_b128(
            rx, (uint32_t)((int64_t)r * ldx * 2) + (uint32_t)(128 * b0 + 16 * (R * kPieces + p)), 0, 0);
      }
    };
#pragma unroll
    for (int R = 0; R < 4; ++R) xload(R);
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      put(xv[R]);
#pragma unroll
      for (int ib = 0; ib < kBr; ++ib)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int pc = 8 * ib + 2 * q + h;     // piece within this round
          xa[R * kBr + ib][h] = *(const u32x4_t*)(reg + c * kRow + 16 * (pc ^ swz(c)));
        }
    }
  }

  // Weights of row group g: row-contiguous 16-byte pieces of the 16 rows'
  // slices (rows past N read as zero and are never stored), and the block
  // scales of the lane's own row 16 g + l % 16.
  const rsrc_t rw = make_rsrc(packed, (uint32_t)N * rowK2);
  const uint32_t nblocks = (uint32_t)N * (uint32_t)nkb;
  const rsrc_t rq = make_rsrc(absmax, DQ ? nblocks : nblocks * 4u);
  const rsrc_t rg = make_rsrc(absmax2, DQ ? (nblocks + 255u) / 256u * 4u : 4u);
  const float mu = DQ ? *mean : 0.0f;
  struct Stage {
    u32x4_t w[kLoads];
    uint32_t qc[BPW];   // block codes (DQ per block), or 4 codes per dword (row mode)
    float s[BPW];       // group scale (DQ), or fp32 absmax
  };
  auto load = [&](Stage& st, int g) {
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int e = 64 * u + lane, r = e / kPieces, p = e % kPieces;
      st.w[u] = __builtin_amdgcn_raw_buffer_load_b128(
          rw, (uint32_t)(16 * g + r) * rowK2 + (uint32_t)(32 * b0 + 16 * p), 0, 0);
    }
    const uint32_t blk0 = (uint32_t)(16 * g + c) * (uint32_t)nkb + (uint32_t)b0;
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      if (SM == kScaleDqRow) {
        // BPW is a multiple of 4 and the wave's blocks sit in one group.
        if ((i & 3) == 0) st.qc[i] = __builtin_amdgcn_raw_buffer_load_b32(rq, blk0 + i, 0, 0);
        if (i == 0)
          st.s[0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, (blk0 >> 8) * 4u, 0, 0));
      } else if (DQ) {
        st.qc[i] = __builtin_amdgcn_raw_buffer_load_b8(rq, blk0 + i, 0, 0);
        st.s[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, ((blk0 + i) >> 8) * 4u, 0, 0));
      } else {
        st.s[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rq, (blk0 + i) * 4u, 0, 0));
      }
    }
  };
  auto scale = [&](const Stage& st, int i) {
    if (!DQ) return st.s[i];
    int code;
    float g;
    if (SM == kScaleDqRow) {
      code = __builtin_amdgcn_sbfe((int)st.qc[i & ~3], (i & 3) * 8, 8);
      g = st.s[0];
    } else {
      code = (int)(int8_t)st.qc[i];
      g = st.s[i];
    }
    const float prod = (float)code * dq_step_normal(g);
    return prod + mu;
  };

  // The loads of the first GD groups go out first (for the decode shapes
  // that is every group of the workgroup), then the byte -> pair table.
  Stage st[GD];
#pragma unroll
  for (int j = 0; j < GD; ++j)
    if ((int)blockIdx.x + j * (int)gridDim.x < ngroups) load(st[j], blockIdx.x + j * gridDim.x);
  const int lvl = level_lanes(lv);
  for (int e = t; e < 256 * kCopies / 4; e += kMfWaves * 64) {
    const uint32_t b = (uint32_t)e / (kCopies / 4);
    const uint32_t v = pack16x2<F16>(level_lookup(lvl, b >> 4), level_lookup(lvl, b & 15u));
    *(uint4*)(tab + b * 256u + ((uint32_t)e % (kCopies / 4)) * 16u) = make_uint4(v, v, v, v);
  }
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
  const uint32_t lanebyte = (uint32_t)(lane & (kCopies - 1)) << 2;

  // One row group: the wave's partial sums over its blocks.  Lane l holds
  // Y[4 (l / 16) + v][16 g + l % 16], v = 0..3.
  auto group = [&](const Stage& st) {
    put(st.w);
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      // Bytes [8 q, 8 q + 8) of block i of the lane's row: piece 2 i + q / 2.
      const int pc = 2 * i + (q >> 1);
      const uint2 d2 = *(const uint2*)(reg + c * kRow + 16 * (pc ^ swz(c)) + 8 * (q & 1));
      f32x4_t blk = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t d = h ? d2.y : d2.x;
        u32x4_t bw;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t addr = perm(d, lanebyte, 0x0c0c0000u | ((4u + j) << 8));
          bw[j] = *(const uint32_t*)(tab + addr);
        }
        blk = mfma_16x16x32<F16>(xa[i][h], bw, blk);
      }
      const float sc = scale(st, i);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(blk[v], sc, acc[v]);
    }
    return acc;
  };
  // Rounds of GD row groups: group blockIdx.x + k * grid uses stage k % GD,
  // which then takes the loads of group k + GD.  The waves run a round's
  // groups without synchronizing (their LDS regions are private), then add
  // up the round's partial sums in one pass.  The loop condition is the
  // workgroup's, so its barriers are uniform.
  for (int k0 = 0; (int)blockIdx.x + k0 * (int)gridDim.x < ngroups; k0 += GD) {
#pragma unroll
    for (int j = 0; j < GD; ++j) {
      const int gg = (int)blockIdx.x + (k0 + j) * (int)gridDim.x;
      if (gg < ngroups) {
        *(f32x4_t*)(red + (j * kMfWaves + wave) * 256 + lane * 4) = group(st[j]);
        const int gn = gg + GD * (int)gridDim.x;
        if (gn < ngroups) load(st[j], gn);
      }
    }
    __syncthreads();
    for (int e = t; e < GD * 256; e += kMfWaves * 64) {
      const int j = e >> 8, m = (e >> 4) & 15, cc = e & 15;
      const int gg = (int)blockIdx.x + (k0 + j) * (int)gridDim.x;
      const int n = 16 * gg + cc;
      if (gg < ngroups && m < M && n < N) {
        const int src = (((m >> 2) * 16 + cc) << 2) + (m & 3);
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < kMfWaves; ++w) sum += red[(j * kMfWaves + w) * 256 + src];
        y[(int64_t)m * ldy + n] = f32_to_16<F16>(sum);
      }
    }
    __syncthreads();
  }
}

// Row-wise scales in the MFMA path: every wave's four blocks are one dword of
// codes inside one group; needs 4-byte aligned codes.
template <bool F16>
hipError_t launch_mfma(int grid, const uint16_t* x, int64_t ldx, const uint8_t* packed,
                       const void* absmax, const float* absmax2, const float* mean, int dq,
                       int M, int N, int K, uint16_t* y, int64_t ldy, const LevelTable& lv,
                       hipStream_t stream) {
  if (dq && ((uintptr_t)absmax & 3u) == 0)
    hipLaunchKernelGGL((gemv_mfma_kernel<4, 4, kScaleDqRow, F16>), dim3(grid),
                       dim3(kMfWaves * 64), 0, stream, x, ldx, packed, absmax, absmax2, mean, M, N,
                       K, y, ldy, lv);
  else if (dq)
    hipLaunchKernelGGL((gemv_mfma_kernel<4, 2, kScaleDqLane, F16>), dim3(grid),
                       dim3(kMfWaves * 64), 0, stream, x, ldx, packed, absmax, absmax2, mean, M, N,
                       K, y, ldy, lv);
  else
    hipLaunchKernelGGL((gemv_mfma_kernel<4, 2, kScaleF32, F16>), dim3(grid), dim3(kMfWaves * 64),
                       0, stream, x, ldx, packed, absmax, absmax2, mean, M, N, K, y, ldy, lv);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// host side: plan and dispatch
// ---------------------------------------------------------------------------
struct Plan {
  int mm, ni, rr, twl, grid, xlds;
};

int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}

// Largest rows-per-pass the registers allow for (mm, ni): the X slice takes
// 16*mm*ni VGPRs and each row 6*ni more (weights and scales), within the
// 128 VGPRs of four waves per SIMD.
int rr_max(int mm, int ni) {
  int r = (100 - 16 * mm * ni) / (6 * ni);
  if (r > kMaxRR) r = kMaxRR;
  if (r < 1) r = 1;
  if (mm == 1 && ni == 3) r = 2;
  if (mm == 1 && ni == 4) r = 1;
  if (mm == 2 && ni == 2) r = 2;
  return r;
}

bool make_plan(int mm, int N, int K, Plan& p) {
  const int C = K >> 5;
  const int nimax = 4 / mm;
  int best_twl = -1, best_ni = 0;
  double best_util = 0.0;
  for (int twl = 0; (1 << twl) <= kWaves; ++twl) {
    const int S = 64 << twl;
    const int ni = (C + S - 1) / S;
    if (ni > nimax) continue;
    const double util = (double)C / ((double)S * ni);
    if (util > best_util + 1e-9) {
      best_util = util;
      best_twl = twl;
      best_ni = ni;
    }
  }
  if (best_twl < 0) return false;
  const int tpw = kWaves >> best_twl;
  const int cus = cu_count();
  const int rmax = rr_max(mm, best_ni);
  const int64_t slots = (int64_t)cus * tpw;   // teams resident at once
  int64_t rr = ((int64_t)N + slots - 1) / slots;
  if (rr < 1) rr = 1;
  if (rr > rmax) rr = rmax;
  int64_t grid = ((int64_t)N + tpw * rr - 1) / (tpw * rr);
  if (grid > (int64_t)cus) grid = (int64_t)cus;
  p.mm = mm;
  p.ni = best_ni;
  p.rr = (int)rr;
  p.twl = best_twl;
  p.grid = (int)grid;
  p.xlds = (int64_t)mm * K * 2 <= kXBytes ? 1 : 0;
  return true;
}

template <int MM, int NI, int RR, bool F16>
hipError_t launch_k(const Plan& p, const uint16_t* x, int64_t ldx, const uint8_t* packed,
                    const void* absmax, const float* absmax2, const float* mean, int dq,
                    int mvalid, int N, int K, uint16_t* y, int64_t ldy, const LevelTable& lv,
                    hipStream_t stream) {
  if (!dq)
    hipLaunchKernelGGL((gemv_kernel<MM, NI, RR, kScaleF32, F16>), dim3(p.grid), dim3(kThreads), 0,
                       stream, x, ldx, packed, absmax, absmax2, mean, mvalid, N, K, y, ldy, p.twl,
                       p.xlds, lv);
  else if ((K >> 6) <= 256 && (K >> 6) % 4 == 0 && ((uintptr_t)absmax & 3u) == 0)
    hipLaunchKernelGGL((gemv_kernel<MM, NI, RR, kScaleDqRow, F16>), dim3(p.grid), dim3(kThreads),
                       0, stream, x, ldx, packed, absmax, absmax2, mean, mvalid, N, K, y, ldy,
                       p.twl, p.xlds, lv);
  else
    hipLaunchKernelGGL((gemv_kernel<MM, NI, RR, kScaleDqLane, F16>), dim3(p.grid), dim3(kThreads),
                       0, stream, x, ldx, packed, absmax, absmax2, mean, mvalid, N, K, y, ldy,
                       p.twl, p.xlds, lv);
  return hipGetLastError();
}

hipError_t dispatch(const Plan& p, const uint16_t* x, int64_t ldx, const uint8_t* packed,
                    const void* absmax, const float* absmax2, const float* mean, int dq,
                    int mvalid, int N, int K, uint16_t* y, int64_t ldy, const LevelTable& lv,
                    bool f16, hipStream_t stream) {
#define BNBX_GEMV_CASE(MM, NI, RR)                                                              \
  if (p.mm == MM && p.ni == NI && p.rr == RR)                                                   \
    return f16 ? launch_k<MM, NI, RR, true>(p, x, ldx, packed, absmax, absmax2, mean, dq, mvalid, \
                                            N, K, y, ldy, lv, stream)                           \
               : launch_k<MM, NI, RR, false>(p, x, ldx, packed, absmax, absmax2, mean, dq,      \
                                             mvalid, N, K, y, ldy, lv, stream);
  BNBX_GEMV_CASE(1, 1, 1) BNBX_GEMV_CASE(1, 1, 2) BNBX_GEMV_CASE(1, 1, 3) BNBX_GEMV_CASE(1, 1, 4)
  BNBX_GEMV_CASE(1, 2, 1) BNBX_GEMV_CASE(1, 2, 2) BNBX_GEMV_CASE(1, 2, 3) BNBX_GEMV_CASE(1, 2, 4)
  BNBX_GEMV_CASE(1, 3, 1) BNBX_GEMV_CASE(1, 3, 2)
  BNBX_GEMV_CASE(1, 4, 1)
  BNBX_GEMV_CASE(2, 1, 1) BNBX_GEMV_CASE(2, 1, 2) BNBX_GEMV_CASE(2, 1, 3) BNBX_GEMV_CASE(2, 1, 4)
  BNBX_GEMV_CASE(2, 2, 1) BNBX_GEMV_CASE(2, 2, 2)
  BNBX_GEMV_CASE(4, 1, 1) BNBX_GEMV_CASE(4, 1, 2) BNBX_GEMV_CASE(4, 1, 3) BNBX_GEMV_CASE(4, 1, 4)
#undef BNBX_GEMV_CASE
  return hipErrorNotSupported;
}

}  // namespace

hipError_t launch_gemv(const uint16_t* x, int64_t ldx, const uint8_t* packed, const void* absmax,
                       const float* absmax2, const float* mean, int double_quant, int quant_type,
                       bool f16, int M, int N, int K, uint16_t* y, int64_t ldy,
                       hipStream_t stream) {
  const int64_t rowK2 = K >> 1, nkb = K >> 6;
  const LevelTable& lv = level_table(quant_type);
  // 4 < M <= 16 at K = 4096 (each wave's K slice in its registers): one
  // MFMA launch streams the weights once, when the offsets fit 32 bits.
  if (M > 4) {
    const bool fits = nkb == 64 &&
                      (int64_t)N * rowK2 < ((int64_t)1 << 31) &&
                      15 * ldx * 2 + (int64_t)K * 2 < ((int64_t)1 << 31);
    if (fits) {
      const int ngroups = (N + 15) / 16;
      const int grid = ngroups < cu_count() ? ngroups : cu_count();
      return f16 ? launch_mfma<true>(grid, x, ldx, packed, absmax, absmax2, mean, double_quant, M,
                                     N, K, y, ldy, lv, stream)
                 : launch_mfma<false>(grid, x, ldx, packed, absmax, absmax2, mean, double_quant, M,
                                      N, K, y, ldy, lv, stream);
    }
  }
  // Slabs of rows keep every byte offset of a launch below 2^31.
  int64_t slab = ((int64_t)1 << 30) / rowK2;
  slab -= slab % 256;
  // Rows of X in groups of up to four (each group streams W once); a group
  // of three runs the four-row kernel with its last row empty.  Long rows
  // take smaller groups (the X slice must fit the registers).
  for (int m0 = 0; m0 < M;) {
    const int left = M - m0;
    Plan p;
    int mv = 0;
    for (int mm : {4, 2, 1}) {
      if (left < (mm == 4 ? 3 : mm)) continue;       // a group of 3 uses mm = 4
      if (make_plan(mm, N < slab ? N : (int)slab, K, p)) {
        mv = left < mm ? left : mm;
        break;
      }
    }
    if (mv == 0) return hipErrorNotSupported;
    for (int64_t r0 = 0; r0 < N; r0 += slab) {
      const int n = (int)(N - r0 < slab ? N - r0 : slab);
      if (!make_plan(p.mm, n, K, p)) return hipErrorNotSupported;
      const void* am = double_quant ? (const void*)((const int8_t*)absmax + r0 * nkb)
                                    : (const void*)((const float*)absmax + r0 * nkb);
      const float* am2 = double_quant ? absmax2 + (r0 * nkb) / 256 : absmax2;
      const hipError_t e =
          dispatch(p, x + (int64_t)m0 * ldx, ldx, packed + r0 * rowK2, am, am2, mean,
                   double_quant, mv, n, K, y + (int64_t)m0 * ldy + r0, ldy, lv, f16, stream);
      if (e != hipSuccess) return e;
    }
    m0 += mv;
  }
  return hipSuccess;
}

}  // namespace bnbx

// Shared by the decode GEMV translation units of libbnbx: constants, buffer
// and DPP helpers, the scale modes, the M <= 4 kernel (gemv_kernel) and its
// host-side planner.  Everything here has internal linkage, one copy per
// translation unit.
//
// Decode GEMV with 4-bit (NF4 or FP4) weights for gfx950:
// Y[M, N] = X[M, K] . W_hat[N, K]^T,
// M <= 16 (mlqm.cn bitsandbytes article, sec. 3.4 "4-bit storage, 16-bit
// compute", and the sec. 7 pitfall that 4-bit only pays off when the layer is
// bound by weight traffic: so the packed weight is streamed exactly once:
// gemv_kernel below for up to four rows of X, gemv16_kernel in bnbx_gemv16.hip
// for 4 < M <= 16).
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
// scales in one vector load.  Nothing the table build needs waits on a
// memory load: the kernel issues no scalar loads from memory (the table
// build's wait for its scalar kernel-argument loads would cover them too),
// and the mean is loaded first so that its use waits for nothing else.  X is
// staged once per workgroup in LDS.
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
#pragma once

#include <type_traits>

#include "bnbx_device.hpp"
#include "bnbx_internal.hpp"

namespace bnbx {
namespace {

constexpr int kWaves = 16;                  // waves per workgroup (one workgroup per CU)
constexpr int kThreads = kWaves * 64;
// The single-weight M = 1 kernel may instead run 8-wave workgroups, two per
// CU (their X stage is then 8 KB, so that both fit the LDS).
constexpr int kWavesHalf = 8;
constexpr int kCopies = 32;                 // lane columns of the byte table (128 B)
constexpr int kTabBytes = 256 * 256;        // 256 B per byte value
// X staged in LDS when MM*K*2 fits (the table takes 64 KB of the CU's 160 KB).
constexpr int kXBytes = 64 * 1024;
constexpr int x_stage_bytes(int wv) { return wv == kWaves ? kXBytes : 8 * 1024; }
constexpr int kMaxMM = 4;
constexpr int kMaxRR = 4;
// Rows per team in a grouped launch: more spill registers (the item lookups
// of the rolling row window).
constexpr int kMaxGroupRR = 3;
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

// Block-scale storage: fp32 absmax, or double quant (code byte + fp32 group
// scale + mean) read per lane, or double quant read per row; the code bytes
// are int8 steps of s_g / 127 (linear map) or indices into the dynamic 8-bit
// map (Dyn modes, a copy of the map in LDS).  The row-wise read loads whole
// dwords of codes, and the buffer range check zeroes a dword that is only
// partly inside the row, so it needs a row of 4k blocks (at most 256:
// K <= 16384, K % 256 == 0) and 4-byte aligned codes.
enum ScaleMode {
  kScaleF32 = 0,
  kScaleDqLane = 1,
  kScaleDqRow = 2,
  kScaleDynLane = 3,
  kScaleDynRow = 4
};
constexpr bool scale_dyn(int sm) { return sm == kScaleDynLane || sm == kScaleDynRow; }
constexpr bool scale_row(int sm) { return sm == kScaleDqRow || sm == kScaleDynRow; }
constexpr int kMapBytes = 256 * 4;

// Lane t % 256's value of the dynamic map, one load per lane with no
// condition (so that the wait for it, in load order, names nothing later).
__device__ __forceinline__ float dyn_map_value(int t) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(kDynMapDev.v, (uint32_t)kMapBytes),
                                                  (uint32_t)(t & 255) * 4u, 0, 0));
}

// The weights of one launch: one (GemvOne), or (GRP) up to kMaxItems
// weights that multiply the same X (GemvItems), their rows concatenated in
// item order: item w owns rows [end[w-1], end[w]) (end[-1] = 0; entries
// past the last item hold INT_MAX).  Y of item w, row m, is at
// y[w] + m * ldy[w].  A single weight keeps the short argument block.
constexpr int kMaxItems = 4;
struct GemvOne {
  const uint8_t* packed;
  const void* absmax;
  const float* absmax2;
  const float* mean;
  uint16_t* y;
  int64_t ldy;
};
struct GemvItems {
  int end[kMaxItems];
  const uint8_t* packed[kMaxItems];
  const void* absmax[kMaxItems];
  const float* absmax2[kMaxItems];
  const float* mean[kMaxItems];
  uint16_t* y[kMaxItems];
  int64_t ldy[kMaxItems];
};

// Field of item w by selects (indexing the argument struct with a run-time
// w would copy it to scratch memory).
template <typename T>
__device__ __forceinline__ T pick_item(const T (&a)[kMaxItems], int w) {
  return w == 0 ? a[0] : w == 1 ? a[1] : w == 2 ? a[2] : a[3];
}

// A single weight with a LoRA term (LORA): Y += XA . B^T with XA [M, r] and
// the up-projection B [N, r] in the compute type, r a multiple of 16 up to
// 256.
struct GemvOneLora : GemvOne {
  const uint16_t* xa;
  int64_t ldxa;
  const uint16_t* lb;
  int64_t ldb;
  int r;
};

template <bool GRP, bool LORA = false>
using GemvArgs = typename std::conditional<
    GRP, GemvItems, typename std::conditional<LORA, GemvOneLora, GemvOne>::type>::type;

// 16-bit value (bf16 or binary16) to binary32, exactly.
template <bool F16>
__device__ __forceinline__ float half_to_f32(uint32_t h) {
  if constexpr (F16)
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
  else
    return __uint_as_float(h << 16);
}
constexpr uint32_t kLoraFar = 0x80000000u;   // an offset past every buffer resource
constexpr int kLoraPer = 4;                  // ranks per lane slot: r <= 256, 64 slots or more
constexpr int kLoraMaxRR = 3;                // rows per team with a LoRA term (registers)

// MM rows of X per launch (rows >= mvalid are zero), NI chunks per lane, RR
// rows of W per team and pass.  TW = 1 << twl waves per team.  N rows in
// all (of every item).  LP: ranks of the LoRA term per lane slot.
template <int MM, int NI, int RR, int SM, bool F16, bool GRP, int WV, bool LORA = false,
          int LP = 1>
__global__ __launch_bounds__(WV * 64, 4) void gemv_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, GemvArgs<GRP, LORA> items, int nitems, int mvalid,
    int N, int K, int twl, int xlds, LevelTable lv) {
  constexpr bool DQ = SM != kScaleF32;
  constexpr bool DYN = scale_dyn(SM);
  constexpr int kWaves = WV;                 // this instantiation's workgroup
  constexpr int kThreads = WV * 64;
  constexpr int kXBytes = x_stage_bytes(WV);
  // One LDS block with the table at offset 0, so that a table address is the
  // v_perm result itself (the ds_read offset field cannot hold a 64 KB base),
  // then X, then the team sums, then the dynamic map (DYN).  X is stored in 64-byte chunks whose four
  // 16-byte pieces are rotated by (chunk / 4) % 4: piece q of chunk c sits at
  // 64 c + 16 (q ^ ((c >> 2) & 3)), so that 16 lanes reading piece q of 16
  // consecutive chunks hit 64 distinct banks.
  __shared__ __attribute__((aligned(16))) unsigned char smem[kTabBytes + kXBytes +
                                                             kWaves * MM * RR * 4 +
                                                             (DYN ? kMapBytes : 0)];
  unsigned char* const tab = smem;
  unsigned char* const xs = smem + kTabBytes;
  float* const red = (float*)(smem + kTabBytes + kXBytes);
  unsigned char* const dmap = smem + kTabBytes + kXBytes + kWaves * MM * RR * 4;

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

  // The item of a row, the item's first and end rows, and its fields (item
  // 0 and the single weight's fields without GRP).
  auto item_of = [&](int64_t row) -> int {
    if constexpr (GRP)
      return (int)(row >= items.end[0]) + (int)(row >= items.end[1]) + (int)(row >= items.end[2]);
    else
      return 0;
  };
  auto item_start = [&](int wi) -> int64_t {
    if constexpr (GRP)
      return wi == 0 ? 0 : wi == 1 ? items.end[0] : wi == 2 ? items.end[1] : items.end[2];
    else
      return 0;
  };
  auto item_end = [&](int wi) -> int64_t {
    if constexpr (GRP) return pick_item(items.end, wi); else return N;
  };
#define BNBX_ITEM_FIELD(NAME, T)                                   \
  auto item_##NAME = [&](int wi) -> T {                            \
    if constexpr (GRP) return pick_item(items.NAME, wi);           \
    else return items.NAME;                                        \
  };
  BNBX_ITEM_FIELD(packed, const uint8_t*)
  BNBX_ITEM_FIELD(absmax, const void*)
  BNBX_ITEM_FIELD(absmax2, const float*)
  BNBX_ITEM_FIELD(mean, const float*)
  BNBX_ITEM_FIELD(y, uint16_t*)
  BNBX_ITEM_FIELD(ldy, int64_t)
#undef BNBX_ITEM_FIELD

  // Fixed per-lane offsets: chunk c of the row (bytes), its block (index).
  uint32_t woff[NI], boff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint32_t c = (uint32_t)(s + i * S);
    woff[i] = c * 16u;
    boff[i] = c >> 1;
  }

  // 0. The mean, by lane 0 alone and before every other load: loads
  //    complete in issue order, so its first use (broadcast with
  //    v_readfirstlane) then waits for nothing else.
  //    With GRP, lane w loads item w's mean.
  float mul = 0.0f;
  if (GRP) {
    if (DQ && lane < nitems) mul = *item_mean(lane);
  } else if (DQ && lane == 0) {
    mul = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(item_mean(0), 4u), 0u, 0, 0));
  }
  const float dmv = DYN ? dyn_map_value(t) : 0.0f;

  // LoRA term: lane slot s takes ranks s, s + S, ... of XA's rows (binary32)
  // and of each row of B; unused ranks read zero from an offset past the
  // buffers, so no load sits behind a branch.
  constexpr int kLP = LORA ? LP : 1;
  uint32_t lof[kLP];
  float xav[MM][kLP];
  if constexpr (LORA) {
#pragma unroll
    for (int i = 0; i < kLP; ++i) {
      const int j = s + i * S;
      lof[i] = j < items.r ? (uint32_t)j * 2u : kLoraFar;
    }
    const rsrc_t rxa =
        make_rsrc(items.xa, (uint32_t)(((int64_t)(mvalid - 1) * items.ldxa + items.r) * 2));
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
      for (int i = 0; i < kLP; ++i)
        xav[m][i] = half_to_f32<F16>(__builtin_amdgcn_raw_buffer_load_b16(
            rxa, lof[i] + (uint32_t)((int64_t)m * items.ldxa * 2), 0, 0));
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
  constexpr bool rowsc = scale_row(SM);
  uint4 w[RR][NI];
  int qv[RR][NI];
  float gv[RR][NI];
  int qd[RR];
  float gsl[RR];      // the row's group scales: g0 in even lanes, g1 in odd ones
  uint32_t split[RR];
  uint32_t lbv[RR][kLP];   // LoRA: the row's ranks of B (16-bit values)
  // Loads of the team's rows that start at row rb (rows at or past N get
  // empty resources).
  auto issue_part = [&](int64_t rb, int lo, int hi) {
#pragma unroll
    for (int j = 0; j < RR; ++j) {
      if ((j + 1) * NI <= lo || j * NI >= hi) continue;
      const bool ok = rb + j < N;
      const int wi = item_of(ok ? rb + j : 0);
      const int64_t row = rb + j - item_start(wi);   // row within its item
      const uint32_t ng =
          DQ ? (uint32_t)(((uint64_t)(item_end(wi) - item_start(wi)) * nkb + 255) >> 8) : 1u;
      const rsrc_t rg = make_rsrc(item_absmax2(wi), DQ ? ng * 4u : 0u);
      const void* const absmax = item_absmax(wi);
      const rsrc_t rw = make_rsrc(item_packed(wi) + row * rowK2, ok ? rowK2 : 0u);
#pragma unroll
      for (int i = 0; i < NI; ++i)
        if (j * NI + i >= lo && j * NI + i < hi) w[j][i] = buf_load16<2>(rw, woff[i]);   // nt
      if (j * NI < lo) continue;              // the row's scales went with its first chunk
      if constexpr (LORA) {
        const rsrc_t rbl = make_rsrc(items.lb + row * items.ldb, ok ? (uint32_t)items.r * 2u : 0u);
#pragma unroll
        for (int i = 0; i < kLP; ++i) lbv[j][i] = __builtin_amdgcn_raw_buffer_load_b16(rbl, lof[i], 0, 0);
      }
      if (rowsc) {
        const rsrc_t rq = make_rsrc((const int8_t*)absmax + row * nkb, ok ? nkb : 0u);
        qd[j] = (int)__builtin_amdgcn_raw_buffer_load_b32(rq, (uint32_t)lane * 4u, 0, 0);
        const uint32_t blk0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(row * nkb));
        uint32_t g0 = blk0 >> 8;
        g0 = g0 < ng ? g0 : ng - 1u;
        const uint32_t g1 = g0 + 1u < ng ? g0 + 1u : ng - 1u;
        // Both group scales in one vector load, g0 in the even lanes and g1
        // in the odd ones, spread to every lane by DPP where they are used.
        // (A scalar load here would make the table build, which waits for all
        // scalar loads, wait for a memory latency: 4.5 against 4.1 us per
        // 4096^2 launch.  Loading them with two lanes active, or broadcasting
        // with v_readlane, measured slower still.)
        gsl[j] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rg, ((lane & 1) ? g1 : g0) * 4u, 0, 0));
        split[j] = 256u - (blk0 & 255u);     // blocks of the row in group g0
      } else if (DQ) {
        const rsrc_t rq = make_rsrc((const int8_t*)absmax + row * nkb, ok ? nkb : 0u);
        const uint32_t blk0 = (uint32_t)(row * nkb);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const uint32_t cb = __builtin_amdgcn_raw_buffer_load_b8(rq, boff[i], 0, 0);
          qv[j][i] = DYN ? (int)(uint8_t)cb : (int)(int8_t)(uint8_t)cb;
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
  if (DYN && t < 256) *(float*)(dmap + t * 4) = dmv;
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

  // In the first pass at most kRowWindow rows per team are in flight: the
  // next ones are requested as rows are consumed, which keeps the memory
  // pipeline fed evenly instead of with one burst per wave.
  constexpr int kRowWindow = 2;
  constexpr int kFirstRows = RR < kRowWindow ? RR : kRowWindow;
  issue_part(rb_first + (int64_t)team_l * RR, NI, kFirstRows * NI);
  const uint32_t lanebyte = (uint32_t)(lane & (kCopies - 1)) << 2;
  // 4. Dequant-in-register dot products of one pass, one chunk at a time in
  //    load order, then the sums over the team and the stores.
  auto pass = [&](int64_t rb, bool first) {
    float acc[MM][RR];
#pragma unroll
    for (int j = 0; j < RR; ++j) {
      const float mu =
          !DQ ? 0.0f
              : GRP ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mul),
                                                               item_of(rb + j < N ? rb + j : 0)))
                    : __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(mul)));
#pragma unroll
      for (int m = 0; m < MM; ++m) acc[m][j] = 0.0f;
      // the row's (at most two) group factors, once per row: the steps
      // fl32(s_g / 127) (linear map) or s_g itself (dynamic map);
      // quad_perm(0,0,0,0) / (1,1,1,1): every lane takes its quad's g0 / g1
      auto factor = [&](float g) { return DYN ? g : dq_step_normal(g); };
      const float step0 =
          rowsc ? factor(__int_as_float(__builtin_amdgcn_update_dpp(
                      0, __float_as_int(gsl[j]), 0x00, 0xF, 0xF, false)))
                : 0.0f;
      const float step1 =
          rowsc ? factor(__int_as_float(__builtin_amdgcn_update_dpp(
                      0, __float_as_int(gsl[j]), 0x55, 0xF, 0xF, false)))
                : 0.0f;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float sc;
        if (rowsc) {
          const int qw = __builtin_amdgcn_ds_bpermute((int)((boff[i] >> 2) << 2), qd[j]);
          float qf;
          if (DYN)
            qf = *(const float*)(dmap + __builtin_amdgcn_ubfe((uint32_t)qw, (boff[i] & 3u) * 8u, 8) * 4u);
          else
            qf = (float)(int)__builtin_amdgcn_sbfe(qw, (boff[i] & 3u) * 8u, 8);   // signed
          const float prod = qf * (boff[i] < split[j] ? step0 : step1);
          sc = prod + mu;
        } else if (DYN) {
          const float prod = *(const float*)(dmap + (uint32_t)qv[j][i] * 4u) * gv[j][i];
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
      if constexpr (LORA) {
        // the lane's ranks of XA . B^T join the row's partial sums before
        // the reduction, so that Y is rounded once
#pragma unroll
        for (int m = 0; m < MM; ++m)
#pragma unroll
          for (int i = 0; i < kLP; ++i)
            acc[m][j] = __builtin_fmaf(xav[m][i], half_to_f32<F16>(lbv[j][i]), acc[m][j]);
      }
      if (first && j + kRowWindow < RR)
        issue_part(rb, (j + kRowWindow) * NI, (j + kRowWindow + 1) * NI);
    }
#pragma unroll
    for (int j = 0; j < RR; ++j)
#pragma unroll
      for (int m = 0; m < MM; ++m) acc[m][j] = wave_sum_to_63(acc[m][j]);
    if (TW == 1) {
      if (lane == 63) {
#pragma unroll
        for (int j = 0; j < RR; ++j) {
          if (rb + j >= N) continue;
          const int wi = item_of(rb + j);
          uint16_t* const yw = item_y(wi) + (rb + j - item_start(wi));
          const int64_t ldw = item_ldy(wi);
#pragma unroll
          for (int m = 0; m < MM; ++m)
            if (m < mvalid) yw[(int64_t)m * ldw] = f32_to_16<F16>(acc[m][j]);
        }
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
        const int64_t row = rb + j;   // differs across these lanes
        if (row < N && m < mvalid) {
          // item_of and the fields by per-lane selects (row is not uniform)
          const int wi = item_of(row);
          item_y(wi)[(int64_t)m * item_ldy(wi) + (row - item_start(wi))] = f32_to_16<F16>(v);
        }
      }
      __syncthreads();
    }
  };
  // The first pass uses the loads issued before the table build; later
  // passes (more rows than the grid holds at once) issue their own.  The
  // loop condition is the workgroup's, so its barriers are uniform.
  pass(rb_first + (int64_t)team_l * RR, true);
  for (int64_t rb0 = rb_first + pass_rows; rb0 < N; rb0 += pass_rows) {
    issue(rb0 + (int64_t)team_l * RR);
    pass(rb0 + (int64_t)team_l * RR, false);
  }
}

// ---------------------------------------------------------------------------
// host side: plan and dispatch
// ---------------------------------------------------------------------------
struct Plan {
  int mm, ni, rr, twl, grid, xlds;
  int wv;   // waves per workgroup: kWaves, or kWavesHalf (two workgroups per CU)
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
  if (mm == 1 && ni == 2) r = 6;   // 116-125 VGPRs, no spills (K = 4096 decode rows)
  if (mm == 2 && ni == 2) r = 2;
  return r;
}

// nicap: at most this many chunks per lane (see launch_k).  half: the
// 8-wave workgroups may be chosen (M = 1).
bool make_plan(int mm, int N, int K, Plan& p, int nicap = 4, bool half = false) {
  const int C = K >> 5;
  const int nimax = (4 / mm) < nicap ? (4 / mm) : nicap;
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
  p.wv = kWaves;
  // Rows chained three or more deep per wave: two 8-wave workgroups per CU,
  // each with its own table and barrier, when X still fits their 8 KB stage
  // (measured at M = 1 on 11008 x 4096: 6.46 against 6.86 us; with one row
  // per wave, 4096 x 4096, or X not staged, 4096 x 11008, they were slower).
  if (half && mm == 1 && best_ni <= 2 && rr >= 3 && (int64_t)K * 2 <= x_stage_bytes(kWavesHalf)) {
    const int tpw8 = kWavesHalf >> best_twl;
    const int64_t slots8 = (int64_t)cus * 2 * tpw8;
    int64_t rr8 = ((int64_t)N + slots8 - 1) / slots8;
    if (rr8 < 1) rr8 = 1;
    if (tpw8 >= 1 && rr8 <= rmax && rr8 == rr) {
      p.wv = kWavesHalf;
      p.grid = (int)(((int64_t)N + tpw8 * rr8 - 1) / (tpw8 * rr8));
      p.xlds = 1;
    }
  }
  return true;
}

template <int MM, int NI, int RR, bool F16, bool GRP, bool LORA = false>
hipError_t launch_k(const Plan& p, const uint16_t* x, int64_t ldx, const GemvArgs<GRP, LORA>& it,
                    int nitems, int dq, bool rowq, int mvalid, int N, int K, const LevelTable& lv,
                    hipStream_t stream) {
  if constexpr ((GRP && RR > kMaxGroupRR) || (LORA && (GRP || RR > kLoraMaxRR))) {
    return hipErrorNotSupported;   // planned out (launch_gemv_grouped, launch_gemv_lora)
  } else {
  int sm = kScaleF32;
  if (dq == kDqDynamic)
    sm = rowq ? kScaleDynRow : kScaleDynLane;
  else if (dq)
    sm = rowq ? kScaleDqRow : kScaleDqLane;
  // The 8-wave form is instantiated for the plans that can choose it.
  constexpr bool kHalfOk = MM == 1 && NI <= 2;
  // A LoRA term of rank 64 or less takes one rank per lane slot (a team has
  // 64 slots or more), of rank 128 or less two: one or two loads of XA and
  // per row of B instead of kLoraPer, most of them past the buffers.
  bool lp1 = false, lp2 = false;
  if constexpr (LORA) {
    lp1 = it.r <= 64;
    lp2 = !lp1 && it.r <= 128;
  }
#define BNBX_GEMV_WV(SMV, LPV)                                                                 \
  if (kHalfOk && p.wv == kWavesHalf)                                                           \
    hipLaunchKernelGGL((gemv_kernel<MM, NI, RR, SMV, F16, GRP, kHalfOk ? kWavesHalf : kWaves,  \
                                    LORA, LPV>),                                               \
                       dim3(p.grid), dim3(kWavesHalf * 64), 0, stream, x, ldx, it, nitems,     \
                       mvalid, N, K, p.twl, p.xlds, lv);                                       \
  else                                                                                         \
    hipLaunchKernelGGL((gemv_kernel<MM, NI, RR, SMV, F16, GRP, kWaves, LORA, LPV>),            \
                       dim3(p.grid), dim3(kThreads), 0, stream, x, ldx, it, nitems, mvalid, N, \
                       K, p.twl, p.xlds, lv);
#define BNBX_GEMV_SM(SMV)                                                                      \
  if (sm == SMV) {                                                                             \
    if (lp1) {                                                                                 \
      BNBX_GEMV_WV(SMV, 1)                                                                     \
    } else if (lp2) {                                                                          \
      BNBX_GEMV_WV(SMV, LORA ? 2 : 1)                                                          \
    } else {                                                                                   \
      BNBX_GEMV_WV(SMV, LORA ? kLoraPer : 1)                                                   \
    }                                                                                          \
  }
  // Four chunks per lane with per-lane scales spill registers for the
  // dynamic map, and for both maps with GRP: those plans are capped at three
  // chunks (nicap) and the variants not built.
  BNBX_GEMV_SM(kScaleF32)
  if constexpr (NI < 4 || !GRP) {
    BNBX_GEMV_SM(kScaleDqLane)
  } else {
    if (sm == kScaleDqLane) return hipErrorNotSupported;
  }
  BNBX_GEMV_SM(kScaleDqRow)
  if constexpr (NI < 4) {
    BNBX_GEMV_SM(kScaleDynLane)
  } else {
    if (sm == kScaleDynLane) return hipErrorNotSupported;
  }
  BNBX_GEMV_SM(kScaleDynRow)
#undef BNBX_GEMV_SM
#undef BNBX_GEMV_WV
  return hipGetLastError();
  }
}

// Launch of the plan's (MM, NI, RR) instantiation over the items.  rowq:
// the row-wise code reads apply (every item's codes 4-byte aligned, K/64 a
// multiple of 4 and at most 256).
template <bool GRP, bool LORA = false>
hipError_t dispatch(const Plan& p, const uint16_t* x, int64_t ldx, const GemvArgs<GRP, LORA>& it,
                    int nitems, int dq, bool rowq, int mvalid, int N, int K, const LevelTable& lv,
                    bool f16, hipStream_t stream) {
#define BNBX_GEMV_CASE(MM, NI, RR)                                                              \
  if (p.mm == MM && p.ni == NI && p.rr == RR)                                                   \
    return f16 ? launch_k<MM, NI, RR, true, GRP, LORA>(p, x, ldx, it, nitems, dq, rowq, mvalid, \
                                                       N, K, lv, stream)                        \
               : launch_k<MM, NI, RR, false, GRP, LORA>(p, x, ldx, it, nitems, dq, rowq, mvalid,\
                                                        N, K, lv, stream);
  BNBX_GEMV_CASE(1, 1, 1) BNBX_GEMV_CASE(1, 1, 2) BNBX_GEMV_CASE(1, 1, 3) BNBX_GEMV_CASE(1, 1, 4)
  BNBX_GEMV_CASE(1, 2, 1) BNBX_GEMV_CASE(1, 2, 2) BNBX_GEMV_CASE(1, 2, 3) BNBX_GEMV_CASE(1, 2, 4)
  BNBX_GEMV_CASE(1, 2, 5) BNBX_GEMV_CASE(1, 2, 6)
  BNBX_GEMV_CASE(1, 3, 1) BNBX_GEMV_CASE(1, 3, 2)
  BNBX_GEMV_CASE(1, 4, 1)
  BNBX_GEMV_CASE(2, 1, 1) BNBX_GEMV_CASE(2, 1, 2) BNBX_GEMV_CASE(2, 1, 3) BNBX_GEMV_CASE(2, 1, 4)
  BNBX_GEMV_CASE(2, 2, 1) BNBX_GEMV_CASE(2, 2, 2)
  BNBX_GEMV_CASE(4, 1, 1) BNBX_GEMV_CASE(4, 1, 2) BNBX_GEMV_CASE(4, 1, 3) BNBX_GEMV_CASE(4, 1, 4)
#undef BNBX_GEMV_CASE
  return hipErrorNotSupported;
}

// Row groups of X for one launch each (up to four rows; a group of three
// runs the four-row kernel with its last row empty; long rows take smaller
// groups, the X slice must fit the registers): the next group's size and
// its plan for N rows, or 0.
int next_x_group(int left, int N, int K, int nicap, Plan& p, bool half = false) {
  for (int mm : {4, 2, 1}) {
    if (left < (mm == 4 ? 3 : mm)) continue;
    if (make_plan(mm, N, K, p, nicap, half)) return left < mm ? left : mm;
  }
  return 0;
}

}  // namespace
}  // namespace bnbx

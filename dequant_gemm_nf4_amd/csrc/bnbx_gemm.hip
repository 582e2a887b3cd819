// Prefill GEMM with NF4 weights for gfx950: Y[M, N] = X[M, K] . W_hat[N, K]^T
// (mlqm.cn bitsandbytes article, sec. 3.4: 4-bit storage, dequantize to BF16,
// multiply in 16-bit with fp32 accumulation).
//
// Tiling.  A workgroup (4 waves, one per SIMD) owns a 256 x 256 tile of Y.
// Wave w owns all 256 rows and the 64 columns [64 w, 64 w + 64): 8 x 2 tiles
// of v_mfma_f32_32x32x16_bf16, 256 accumulators per lane in AGPRs.  K is
// walked in steps of 64 = one NF4 block per weight row, so a weight row
// shares one block scale per step; a step is four 16-wide substeps.
//
// Weights never touch LDS.  The B operand of a 32x32x16 MFMA gives lane l
// column l % 32 and eight consecutive k of the 16; which eight k of the step
// feed which lane half and substep is free, as long as X uses the same
// assignment.  Lane half h takes, in substep s, the 8-wide k chunk 4h + s, so
// over a step it needs bytes [16h, 16h + 16) of each of its two weight rows'
// 32 packed bytes: one 16-byte load per row, whose four dwords are the four
// substeps' operands.  Each wave therefore dequantizes exactly the weights it
// multiplies, straight into MFMA operand registers, and every weight is
// dequantized once per workgroup.  The dequant is vector-only: the 16 values
// bf16(L[i] * scale) of a row's block form a byte table in 8 registers that
// v_perm_b32 indexes by the 4-bit codes.
//
// X goes from global memory straight into LDS (buffer_load ... lds, 16 B per
// lane, no registers), two buffers.  Its rows are 128 B with the eight
// 16-byte chunks of row r rotated by (r / 2) % 8, so that 16 lanes reading
// the same chunk of 16 consecutive rows hit 64 distinct banks.
//
// Pipeline of step t (one scheduling region per substep, each laid out as
// single MFMAs interleaved with LDS reads and vector ops):
//   region 0: weight loads of step t+3, half the X copy of step t+1 (other
//             buffer), operand reads of (t, 0), MFMAs of (t-1, 3), dequant of
//             (t, 0);
//   region s = 1..3: operand reads of (t, s), MFMAs of (t, s-1), dequant of
//             (t, s); the rest of the X copy in region 1, the block tables of
//             step t+1 in regions 2 (own row) and 3 (shared);
//   then a wait for all of this wave's loads, X copies and LDS reads, and one
//   barrier.  The weight loads go out before the copies: a copy's arrival in
//   LDS is not ordered with later loads, so the memory counter can only be
//   trusted down to zero.
// Block codes come four steps at a time (one dword of four code bytes per
// row) when the shape allows it; codes into the dynamic 8-bit map are looked
// up in a copy of the map in LDS.  Each LDS buffer is its own object, picked
// at compile time, so the compiler can tell reads of one buffer from copies
// in flight into another.  Steps past the end of K load clamped (redundant)
// data that no MFMA uses.
//
// Addresses are 32-bit offsets from buffer resources (per-lane parts fixed,
// the per-step part a scalar); the host splits M so that the X offsets fit.
// Tile order is XCD-aware: workgroup b runs on XCD b % 8, so consecutive tile
// ids (which share the same 256 rows of X) go to the same XCD and meet in
// its L2.
#include <type_traits>

#include "bnbx_device.hpp"
#include "bnbx_internal.hpp"

namespace bnbx {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr int kABuf = BM * BK;   // bf16 elements per X buffer (128 B rows)
constexpr int kMaxLoraRank = 256;   // the largest r bnbx_gemm_nf4_lora takes

// Scheduling-group masks (AMDGPU sched_group_barrier).
constexpr int kSgMfma = 0x008, kSgValu = 0x002, kSgSalu = 0x004, kSgVmem = 0x010,
              kSgDsRead = 0x100;

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// The 16 values bf16(L[i] * scale) of one row block, split into a table of
// their high bytes (h[j] holds entries 4j..4j+3) and one of their low bytes.
struct Tab16 {
  uint32_t h[4], l[4];
};

// Levels that are exactly -1, +0, -0 or +1 need no multiply: their products
// are -sc, a zero with sc's sign, one with the opposite sign, and sc.  NF4:
// L[0] = -1, L[7] = 0, L[15] = +1.  FP4 (E2M1 / 6, by code): L[0] = +0,
// L[7] = +1, L[8] = -0, L[15] = -1.
template <bool FP4, bool F16>
__device__ __forceinline__ Tab16 make_tab16(const LevelTable& lv, float sc) {
  const uint32_t sb = __builtin_bit_cast(uint32_t, sc);
  const float neg = __builtin_bit_cast(float, sb ^ 0x80000000u);
  const float zero = __builtin_bit_cast(float, sb & 0x80000000u);
  const float nzero = __builtin_bit_cast(float, (sb ^ 0x80000000u) & 0x80000000u);
  uint32_t pk[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    float a, b;
    if (FP4) {
      a = k == 0 ? zero : k == 4 ? nzero : lv.level[2 * k] * sc;
      b = k == 3 ? sc : k == 7 ? neg : lv.level[2 * k + 1] * sc;
    } else {
      a = k == 0 ? neg : lv.level[2 * k] * sc;
      b = k == 3 ? zero : k == 7 ? sc : lv.level[2 * k + 1] * sc;
    }
    pk[k] = pack16x2<F16>(a, b);
  }
  Tab16 t;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    t.h[j] = perm(pk[2 * j + 1], pk[2 * j], 0x07050301u);
    t.l[j] = perm(pk[2 * j + 1], pk[2 * j], 0x06040200u);
  }
  return t;
}

// 8 weights (one packed dword: byte j = codes of weights 2j (high nibble) and
// 2j+1) -> 4 dwords of bf16 pairs in weight order.  Four 4-bit codes held one
// per byte select their entries with v_perm_b32 from each half of the table
// (entries 0-7 and 8-15); a per-byte mask made from bit 3 of the codes
// (v_perm's sign-replicating selectors 8-11) picks between the halves.  The
// codes are grouped as weights (0, 1, 4, 5) and (2, 3, 6, 7), so each output
// dword is one v_perm of a high-byte and a low-byte pick (26 vector
// instructions per 8 weights; grouping even and odd weights took 28).
__device__ __forceinline__ void decode8(uint32_t d, const Tab16& t, uint32_t* o) {
  auto pick = [&](uint32_t sel, uint32_t m, const uint32_t* tt) {
    const uint32_t a = perm(tt[1], tt[0], sel), b = perm(tt[3], tt[2], sel);
    return (m & b) | (~m & a);
  };
  // selectors in weight order: (0, 1, 4, 5) and (2, 3, 6, 7)
  const uint32_t lo3 = d & 0x07070707u, hi3 = (d >> 4) & 0x07070707u;
  const uint32_t sA = perm(hi3, lo3, 0x02060004u), sB = perm(hi3, lo3, 0x03070105u);
  // bit 3 of each selected code: d bits 7, 3, 23, 19 and 15, 11, 31, 27
  const uint32_t mA = perm(d << 12, d << 8, 0x0B090A08u);
  const uint32_t mB = perm(d << 4, d, 0x0B090A08u);
  const uint32_t hiA = pick(sA, mA, t.h), loA = pick(sA, mA, t.l);
  const uint32_t hiB = pick(sB, mB, t.h), loB = pick(sB, mB, t.l);
  o[0] = perm(hiA, loA, 0x05010400u);
  o[1] = perm(hiB, loB, 0x05010400u);
  o[2] = perm(hiA, loA, 0x07030602u);
  o[3] = perm(hiB, loB, 0x07030602u);
}

// One K step of a lane's weights: 16 packed bytes (32 weights) of each of
// its two rows.
struct WSet {
  u32x4_t w[2];
};
// Block scale of a lane's own row: the block code byte(s) as loaded (one per
// step, or four per dword) and the group scale (double quant), or the fp32
// block absmax bits (no double quant).
struct QSet {
  uint32_t q;
  float s;
};

// Both rows' tables from each lane's own one: lanes l and l + 32 hold the
// tables of rows 0 and 1 of lane l % 32; v_permlane32_swap exchanges the
// upper half of its first operand with the lower half of its second, so
// with both operands the own table its two results are row 0's table and
// row 1's table in every lane.
__device__ __forceinline__ void share_tab16(const Tab16& own, Tab16* t) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const auto h = __builtin_amdgcn_permlane32_swap(own.h[k], own.h[k], false, false);
    const auto l = __builtin_amdgcn_permlane32_swap(own.l[k], own.l[k], false, false);
    t[0].h[k] = h[0];
    t[1].h[k] = h[1];
    t[0].l[k] = l[0];
    t[1].l[k] = l[1];
  }
}

// Low-rank term accumulated before the main loop (LoRA: Y += XA . B^T,
// XA = s X A^T given as [M, r], B the up-projection [N, r]); r a multiple of
// 16.
struct LoraArgs {
  const uint16_t* xa;
  int64_t ldxa;
  const uint16_t* b;
  int64_t ldb;
  int r;
};

// Split K (SPLIT).  Workgroups [0, tile0) take tiles [0, tile0) whole (tile0
// a multiple of 8, XCD-aware as without SPLIT); the others take the tail
// tiles [tile0, tiles) in nsplit ranges of K: workgroup tile0 + s W + l
// (W = 8 per_xcd workgroups per split) takes K steps [s kb_per, (s + 1)
// kb_per) of tail tile tile0 + (l % 8) per_xcd + l / 8, both splits of a
// tile on one XCD, and stores its fp32 partial tile (256 x 256, row-major)
// at part + ((s ntail + t) 256 + r) 256 + c for tail tile t;
// split_reduce_kernel adds the splits in order and rounds once.
struct SplitArgs {
  int kb_per;    // K steps per split, a multiple of 4
  int tile0;     // tiles run whole
  int per_xcd;   // tail tiles per XCD
  int ntail;     // tail tiles
  float* part;
};

template <int DQ, bool Q4, bool FP4, bool F16, bool LORA, bool SPLIT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ packed,
    const void* __restrict__ absmax, const float* __restrict__ absmax2,
    const float* __restrict__ mean, int M, int N, int K, uint16_t* __restrict__ y, int64_t ldy,
    int tiles_m, int tiles_n, LevelTable lv, LoraArgs la, SplitArgs sp) {
  __shared__ __attribute__((aligned(16))) uint16_t As0[kABuf], As1[kABuf];
  constexpr bool DYN = DQ == kDqDynamic;
  __shared__ float dmap[DYN ? 256 : 1];   // the dynamic 8-bit map (DYN)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS bases in SGPRs
  const int half = lane >> 5, col = lane & 31;

  // XCD-aware tile id: workgroups b, b+8, b+16, ... share an XCD.
  const int ntiles = tiles_m * tiles_n;
  const int per_xcd = (ntiles + kXcds - 1) / kXcds;
  const int b = blockIdx.x;
  int split = -1;   // -1: the whole tile
  int tile;
  if constexpr (SPLIT) {
    if (b < sp.tile0) {
      tile = (b % kXcds) * (sp.tile0 / kXcds) + b / kXcds;
    } else {
      int l = b - sp.tile0;
      split = l / (sp.per_xcd * kXcds);
      l -= split * sp.per_xcd * kXcds;
      tile = sp.tile0 + (l % kXcds) * sp.per_xcd + l / kXcds;
    }
  } else {
    tile = (b % kXcds) * per_xcd + b / kXcds;
  }
  if (tile >= ntiles) return;
  const int m0 = (tile / tiles_n) * BM;
  const int n0 = (tile % tiles_n) * BN;

  if (DYN) {
    dmap[tid] = kDynMapDev.v[tid];
    __syncthreads();
  }
  const float mu = DQ ? *mean : 0.0f;
  const uint32_t rowK2 = (uint32_t)K >> 1;   // packed bytes per weight row
  const int nkb = K >> 6;
  // This workgroup's K steps [kb0, kb1) (all of them without SPLIT).
  const int kb0 = SPLIT && split >= 0 ? split * sp.kb_per : 0;
  const int kb1 = SPLIT && split >= 0 ? (kb0 + sp.kb_per < nkb ? kb0 + sp.kb_per : nkb) : nkb;

  // The lane's weight rows (B columns) n0 + 64 w + 32 j + l % 32, j = 0, 1;
  // rows past N are clamped to N-1 (their tables are zero).
  uint32_t gn[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wave * 64 + 32 * j + col;
    gn[j] = (uint32_t)(n < N ? n : N - 1);
  }
  // The lane's own row for block scales and tables: n0 + 64 w + l (row j = h
  // of lane l % 32).
  const int no = n0 + wave * 64 + lane;
  const bool boko = no < N;
  const uint32_t qvoff = (uint32_t)(boko ? no : N - 1) * (uint32_t)nkb;   // its first block
  const uint32_t nblocks = (uint32_t)N * (uint32_t)nkb;
  const rsrc_t rw = make_rsrc(packed, (uint32_t)N * rowK2);
  const rsrc_t rq = make_rsrc(absmax, DQ ? nblocks : nblocks * 4u);
  const rsrc_t rg = make_rsrc(absmax2, DQ ? (nblocks + 255u) / 256u * 4u : 4u);
  uint32_t wvoff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) wvoff[j] = gn[j] * rowK2 + 16u * (uint32_t)half;

  // X copy of one K step into an LDS buffer: wave w copies rows
  // [64 w, 64 w + 64) in 8 instructions of 8 rows; lane l fills chunk slot
  // l % 8 of row l / 8 with the chunk that the rotation puts there.  Rows past
  // M are clamped to row M-1 (they only feed rows of Y that are never stored).
  const rsrc_t rx = make_rsrc(x, (uint32_t)((int64_t)(M - 1) * ldx * 2 + (int64_t)K * 2));
  uint32_t xvoff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = wave * 64 + i * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ ((r >> 1) & 7);
    int gm = m0 + r;
    gm = gm < M ? gm : M - 1;
    xvoff[i] = (uint32_t)(((int64_t)gm * ldx + chunk * 8) * 2);
  }
  auto copy_x = [&](uint16_t* xbuf, int kb, int i0, int i1) {
    kb = kb < kb1 ? kb : kb1 - 1;
#pragma unroll
    for (int i = i0; i < i1; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (void __attribute__((address_space(3)))*)(xbuf + (wave * 64 + i * 8) * BK), 16,
          xvoff[i], (uint32_t)kb * (BK * 2), 0, 0);
  };
  auto load_w = [&](WSet& s, int kb) {
    kb = kb < kb1 ? kb : kb1 - 1;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      s.w[j] = __builtin_amdgcn_raw_buffer_load_b128(rw, wvoff[j], (uint32_t)kb * 32u, 0);
  };
  // Own-row scale of one step (Q4 = false) or of the four steps 4g..4g+3 (Q4).
  auto load_q = [&](QSet& s, int idx) {
    if (Q4) {
      const int g = idx < (kb1 >> 2) ? idx : (kb1 >> 2) - 1;
      const uint32_t blk = qvoff + 4u * (uint32_t)g;
      s.q = __builtin_amdgcn_raw_buffer_load_b32(rq, blk, 0, 0);
      s.s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, (blk >> 8) * 4u, 0, 0));
    } else {
      const int kb = idx < kb1 ? idx : kb1 - 1;
      const uint32_t blk = qvoff + (uint32_t)kb;
      if (DQ) {
        // Kept as the raw byte; the sign extension is done where the scale
        // is formed.
        s.q = __builtin_amdgcn_raw_buffer_load_b8(rq, blk, 0, 0);
        s.s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, (blk >> 8) * 4u, 0, 0));
      } else {
        s.q = __builtin_amdgcn_raw_buffer_load_b32(rq, blk * 4u, 0, 0);
        s.s = 0.0f;
      }
    }
  };
  // Own-row block scale from code byte `byte` of the set.
  auto scale_of = [&](const QSet& s, int byte) {
    float sc;
    if (DYN) {
      // fl32(fl32(map[q] * s_g) + mean)
      const float prod = dmap[(s.q >> (8 * byte)) & 0xffu] * s.s;
      sc = prod + mu;
    } else if (DQ) {
      // (float)(int8)q = (float)(int32)(q << 24) * 2^-24, both steps exact
      const uint32_t t = (s.q >> (8 * byte)) << 24;
      const float qf = (float)(int32_t)t * 0x1p-24f;
      sc = dq_scale(qf, s.s, mu);
    } else {
      sc = __builtin_bit_cast(float, s.q);
    }
    return boko ? sc : 0.0f;
  };

  f32x16_t acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // A operands: lane l reads row 32 i + l % 32, chunk 4 h + s at its rotated
  // slot (the rotation (r / 2) % 8 does not depend on i).
  uint32_t aoff[BK / 16];
#pragma unroll
  for (int s = 0; s < BK / 16; ++s)
    aoff[s] = (uint32_t)(col * BK + (((4 * half + s) ^ ((col >> 1) & 7)) << 3));
  u32x4_t av[2][8], bv[2][2];
  auto read_ops = [&](const uint16_t* a, int s, int r) {
#pragma unroll
    for (int i = 0; i < 8; ++i) av[r][i] = *(const u32x4_t*)(a + aoff[s] + i * 32 * BK);
  };
  auto mfmas = [&](int r) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = mfma_32x32x16<F16>(av[r][i], bv[r][j], acc[i][j]);
  };
  auto dequant = [&](const WSet& w, const Tab16* t, int s, int r) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t o[4];
      decode8(w.w[j][s], t[j], o);
      bv[r][j] = u32x4_t{o[0], o[1], o[2], o[3]};
    }
  };

  // Staging: four weight sets (step t in set t % 4), scales either four
  // per-step sets alike or two 4-step groups (current and next).
  WSet ws0, ws1, ws2, ws3;
  QSet qs0, qs1, qs2, qs3;
  Tab16 tA[2], tB[2];
  auto wset = [&](int i) -> WSet& { return i == 0 ? ws0 : i == 1 ? ws1 : i == 2 ? ws2 : ws3; };
  auto qset = [&](int i) -> QSet& { return i == 0 ? qs0 : i == 1 ? qs1 : i == 2 ? qs2 : qs3; };

  if constexpr (LORA) {
    // The low-rank term first, as r / 16 MFMAs per tile into the zeroed
    // accumulators, with XA rows as A and rows of B as B operands in the same
    // lane layout as X and the weights (lane half h takes k 8h .. 8h + 8 of
    // each 16); rows past M or N read zero through the buffer range check.
    const rsrc_t ra = make_rsrc(la.xa, (uint32_t)((int64_t)(M - 1) * la.ldxa * 2 + la.r * 2));
    const rsrc_t rb = make_rsrc(la.b, (uint32_t)((int64_t)(N - 1) * la.ldb * 2 + la.r * 2));
    auto load_lr = [&](u32x4_t (&xa)[8], u32x4_t (&lb)[2], int k0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t row = m0 + 32 * i + col;
        xa[i] = __builtin_amdgcn_raw_buffer_load_b128(
            ra, (uint32_t)((row * la.ldxa + k0 + 8 * half) * 2), 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t n = n0 + wave * 64 + 32 * j + col;
        lb[j] = __builtin_amdgcn_raw_buffer_load_b128(
            rb, (uint32_t)((n * la.ldb + k0 + 8 * half) * 2), 0, 0);
      }
    };
    auto mfma_lr = [&](const u32x4_t (&xa)[8], const u32x4_t (&lb)[2]) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma_32x32x16<F16>(xa[i], lb[j], acc[i][j]);
    };
    // Two operand sets: the loads of step s + 1 go out before the MFMAs of
    // step s.  Unrolled over the largest rank with the two sets named apart
    // (a loop carrying the accumulators, or one array of sets indexed by the
    // step, spilled); steps past r are skipped by uniform branches.
    u32x4_t xa0[8], lb0[2], xa1[8], lb1[2];
    load_lr(xa0, lb0, 0);
#pragma unroll
    for (int st = 0; st < kMaxLoraRank / 16; st += 2) {
      if (16 * st >= la.r) break;
      if (16 * (st + 1) < la.r) load_lr(xa1, lb1, 16 * (st + 1));
      mfma_lr(xa0, lb0);
      if (16 * (st + 1) >= la.r) break;
      if (16 * (st + 2) < la.r) load_lr(xa0, lb0, 16 * (st + 2));
      mfma_lr(xa1, lb1);
    }
  }

  // Prologue: X of step kb0, weights of steps kb0..kb0+2, scales, tables of
  // step kb0 (kb0 is a multiple of 4, so step t's sets are those of t % 4).
  copy_x(As0, kb0, 0, 8);
  load_w(ws0, kb0);
  load_w(ws1, kb0 + 1);
  load_w(ws2, kb0 + 2);
  if (Q4) {
    load_q(qs0, kb0 / 4);       // current group
    load_q(qs1, kb0 / 4 + 1);   // next group
  } else {
    load_q(qs0, kb0);
    load_q(qs1, kb0 + 1);
    load_q(qs2, kb0 + 2);
  }
  share_tab16(make_tab16<FP4, F16>(lv, scale_of(qs0, 0)), tA);
  Tab16 own;
  __syncthreads();

  // One K step t with t % 4 == KM (so that every set is fixed at compile
  // time).  `tc` holds step t's tables, `tn` receives step t+1's.
  auto step = [&](auto km_tag, auto first_tag, int kb, Tab16* tc, Tab16* tn) {
    constexpr int KM = decltype(km_tag)::value;
    constexpr bool first = decltype(first_tag)::value;   // no step t-1
    uint16_t* const a = (KM & 1) ? As1 : As0;
    uint16_t* const an = (KM & 1) ? As0 : As1;
    WSet& wc = wset(KM);
    WSet& wl = wset((KM + 3) & 3);
    constexpr int kn = (KM + 1) & 3;   // (t + 1) % 4: code byte of step t+1
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      if (s == 0) {
        // Loads first, then the X copies, all waited for at the end of the
        // step (the copies' completion into LDS is not ordered with the
        // loads', so no wait may leave loads in flight).
        load_w(wl, kb + 3);
        if (Q4) {
          if (kn == 0) {
            // Step t+1 opens a new group of four: move to the next group's
            // codes (loaded four steps ago) and fetch the one after it.
            qs0 = qs1;
            load_q(qs1, (kb + 1) / 4 + 1);
          }
        } else {
          load_q(qset((KM + 3) & 3), kb + 3);
        }
        __builtin_amdgcn_sched_barrier(0);
        copy_x(an, kb + 1, 0, 4);
      }
      if (s == 1) copy_x(an, kb + 1, 4, 8);
      read_ops(a, s, s & 1);                      // substep s of step t
      if (!first || s > 0) mfmas((s + 1) & 1);    // substep 3 of t-1, then 0..2 of t
      dequant(wc, tc, s, s & 1);
      // Tables of step t+1: the own row's in region 2, shared in region 3.
      if (s == 2) own = make_tab16<FP4, F16>(lv, Q4 ? scale_of(qs0, kn) : scale_of(qset(kn), 0));
      if (s == 3) share_tab16(own, tn);
      // 16 x {1 MFMA, an operand read (first 8), copies, vector ops}.
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        if (g < 8) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
        // A copy with the scalar move that sets its LDS address.
        if (s < 2 && (g & (s == 0 ? 1 : 3)) == 0) {
          __builtin_amdgcn_sched_group_barrier(kSgSalu, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSgVmem, 1, 0);
        }
        if (s == 2)
          __builtin_amdgcn_sched_group_barrier(kSgValu, 6, 0);
        else
          __builtin_amdgcn_sched_group_barrier(kSgValu, 4, 0);
      }
      __builtin_amdgcn_sched_barrier(0);   // one substep per scheduling region
    }
    // End of step: this wave's X copies landed (with the loads issued before
    // them) and its operand reads done.  The memory wait is a builtin, so
    // that the compiler knows the copies are complete; the LDS wait and the
    // barrier are inline asm: the compiler relaxes a builtin wait to what it
    // believes this wave needs, and it does not count the other waves.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  using K0 = std::integral_constant<int, 0>;
  using K1 = std::integral_constant<int, 1>;
  using K2 = std::integral_constant<int, 2>;
  using K3 = std::integral_constant<int, 3>;
  using F0 = std::integral_constant<bool, false>;
  using F1 = std::integral_constant<bool, true>;
  step(K0{}, F1{}, kb0, tA, tB);
  int kb = kb0 + 1;
  for (; kb + 3 < kb1; kb += 4) {
    step(K1{}, F0{}, kb, tB, tA);
    step(K2{}, F0{}, kb + 1, tA, tB);
    step(K3{}, F0{}, kb + 2, tB, tA);
    step(K0{}, F0{}, kb + 3, tA, tB);
  }
  if (kb < kb1) step(K1{}, F0{}, kb, tB, tA);
  if (kb + 1 < kb1) step(K2{}, F0{}, kb + 1, tA, tB);
  if (kb + 2 < kb1) step(K3{}, F0{}, kb + 2, tB, tA);
  mfmas(1);   // substep 3 of the last step

  // The lane's position again, from an instruction the compiler cannot see
  // through: values derived from it before the K loop would otherwise stay
  // live across the loop (where every register is in use) only to address
  // the stores of Y, and the LoRA variant spilled them.
  int lane_e;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_e));
  const int col_e = lane_e & 31, half_e = lane_e >> 5;

  // D layout of a 32x32 MFMA tile: lane l, value v -> column l%32,
  // row 8*(v/4) + 4*(l/32) + v%4.
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = n0 + wave * 64 + 32 * j + col_e;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = m0 + i * 32 + 8 * (v >> 2) + 4 * half_e + (v & 3);
        if constexpr (SPLIT) {
          if (split >= 0) {
            const int64_t t = (int64_t)split * sp.ntail + (tile - sp.tile0);
            sp.part[((t * BM) + (r - m0)) * BN + (c - n0)] = acc[i][j][v];
          } else if (r < M && c < N) {
            y[(int64_t)r * ldy + c] = f32_to_16<F16>(acc[i][j][v]);
          }
        } else {
          if (r < M && c < N) y[(int64_t)r * ldy + c] = f32_to_16<F16>(acc[i][j][v]);
        }
      }
    }
}

// Split K: the fp32 partial tiles of the tail tiles, added in split order
// and rounded once; four columns per thread, only rows and columns inside
// Y are stored.
template <bool F16>
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part,
                                                           int nsplit, int ntail, int tile0,
                                                           int tiles_n, int M, int N,
                                                           uint16_t* __restrict__ y,
                                                           int64_t ldy) {
  constexpr int kQuads = BM * BN / 4;   // per tile
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int t = (int)(idx / kQuads);
  if (t >= ntail) return;
  const int e = (int)(idx - (int64_t)t * kQuads) * 4;
  const int tile = tile0 + t;
  const int r = (tile / tiles_n) * BM + e / BN;
  const int c = (tile % tiles_n) * BN + e % BN;
  if (r >= M) return;
  float4 a = *(const float4*)(part + (int64_t)t * BM * BN + e);
  for (int s = 1; s < nsplit; ++s) {
    const float4 b4 = *(const float4*)(part + ((int64_t)s * ntail + t) * BM * BN + e);
    a.x += b4.x;
    a.y += b4.y;
    a.z += b4.z;
    a.w += b4.w;
  }
  const float v[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (c + k < N) y[(int64_t)r * ldy + c + k] = f32_to_16<F16>(v[k]);
}

int device_cus() {
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

// Split-K plan (K of at least 32 blocks).  Tiles that fill at most half of
// the CUs all split, into up to four ranges; more tiles than CUs but fewer
// than twice as many run the first round whole (tile0 = the CUs, rounded
// down to a multiple of 8) and split the tail tiles, whose round would
// otherwise leave most CUs idle.  Ranges are multiples of 4 steps, at least
// 16.  Returns the partial tiles' bytes, 0 without a split.
struct SplitPlan {
  int nsplit, kb_per, tile0, ntail, per_xcd;
};
size_t split_plan(int M, int N, int K, SplitPlan& sp) {
  sp = SplitPlan{1, 0, 0, 0, 0};
  const int64_t tiles = (int64_t)((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int nkb = K / 64;
  const int cus = device_cus();
  if (nkb < 32) return 0;
  int64_t tile0 = 0;
  if (tiles * 2 > cus) {
    if (tiles <= cus || tiles >= 2 * (int64_t)cus) return 0;
    tile0 = cus / kXcds * kXcds;
  }
  const int64_t ntail = tiles - tile0;
  if (ntail < 1 || ntail * 2 > cus) return 0;
  int s = (int)(cus / ntail);
  s = s < 4 ? s : 4;
  s = s < nkb / 16 ? s : nkb / 16;
  if (s < 2) return 0;
  const int kb_per = ((nkb + s - 1) / s + 3) / 4 * 4;
  const int n = (nkb + kb_per - 1) / kb_per;
  if (n < 2) return 0;
  sp.nsplit = n;
  sp.kb_per = kb_per;
  sp.tile0 = (int)tile0;
  sp.ntail = (int)ntail;
  sp.per_xcd = (int)((ntail + kXcds - 1) / kXcds);
  return (size_t)n * (size_t)ntail * BM * BN * sizeof(float);
}

template <int DQ, bool Q4, bool LORA>
void launch_one(const uint16_t* x, int64_t ldx, const uint8_t* packed, const void* absmax,
                const float* absmax2, const float* mean, int M, int N, int K, uint16_t* y,
                int64_t ldy, int quant_type, bool f16, const LoraArgs& la, const SplitPlan& plan,
                float* part, hipStream_t stream) {
  const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
  const int per_xcd = (tm * tn + kXcds - 1) / kXcds;
  const LevelTable& lv = level_table(quant_type);
  if constexpr (!LORA) {
    if (plan.nsplit > 1) {
      const SplitArgs sa{plan.kb_per, plan.tile0, plan.per_xcd, plan.ntail, part};
      const unsigned grid = (unsigned)(plan.tile0 + plan.nsplit * plan.per_xcd * kXcds);
      auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, stream, x, ldx, packed,
                           absmax, absmax2, mean, M, N, K, y, ldy, tm, tn, lv, la, sa);
      };
      if (quant_type == kQuantFP4) {
        if (f16) go(gemm_kernel<DQ, Q4, true, true, false, true>);
        else go(gemm_kernel<DQ, Q4, true, false, false, true>);
      } else {
        if (f16) go(gemm_kernel<DQ, Q4, false, true, false, true>);
        else go(gemm_kernel<DQ, Q4, false, false, false, true>);
      }
      const int64_t quads = (int64_t)plan.ntail * (BM * BN / 4);
      const unsigned rgrid = (unsigned)((quads + 255) / 256);
      if (f16)
        hipLaunchKernelGGL(split_reduce_kernel<true>, dim3(rgrid), dim3(256), 0, stream, part,
                           plan.nsplit, plan.ntail, plan.tile0, tn, M, N, y, ldy);
      else
        hipLaunchKernelGGL(split_reduce_kernel<false>, dim3(rgrid), dim3(256), 0, stream, part,
                           plan.nsplit, plan.ntail, plan.tile0, tn, M, N, y, ldy);
      return;
    }
  }
  const SplitArgs none{0, 0, 0, 0, nullptr};
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)(per_xcd * kXcds)), dim3(kThreads), 0, stream, x,
                       ldx, packed, absmax, absmax2, mean, M, N, K, y, ldy, tm, tn, lv, la, none);
  };
  if (quant_type == kQuantFP4) {
    if (f16) go(gemm_kernel<DQ, Q4, true, true, LORA, false>);
    else go(gemm_kernel<DQ, Q4, true, false, LORA, false>);
  } else {
    if (f16) go(gemm_kernel<DQ, Q4, false, true, LORA, false>);
    else go(gemm_kernel<DQ, Q4, false, false, LORA, false>);
  }
}

// The M-slab loop of both entry points.  Split K (no LoRA term) needs one
// slab and a workspace of split_plan's size; otherwise the tiles run whole.
template <bool LORA>
hipError_t launch_gemm_any(const uint16_t* x, int64_t ldx, const uint8_t* packed,
                           const void* absmax, const float* absmax2, const float* mean,
                           int double_quant, int quant_type, bool f16, int M, int N, int K,
                           uint16_t* y, int64_t ldy, LoraArgs la, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  // Buffer offsets are 32-bit: the weights and their scales must fit, and M
  // is walked in slabs whose X (and XA) rows do.
  const int64_t kLimit = (int64_t)1 << 31;
  if ((int64_t)N * (K / 2) >= kLimit) return hipErrorNotSupported;
  if (LORA && (int64_t)N * la.ldb * 2 >= kLimit) return hipErrorNotSupported;
  int64_t slab = (kLimit - (int64_t)K * 2) / (ldx * 2);
  if (LORA) {
    const int64_t s2 = (kLimit - (int64_t)la.r * 2) / (la.ldxa * 2);
    slab = s2 < slab ? s2 : slab;
  }
  slab = slab / BM * BM;
  if (slab < BM) return hipErrorNotSupported;
  SplitPlan plan;
  const size_t need = LORA ? 0 : split_plan(M, N, K, plan);
  if (need == 0 || M > slab || workspace == nullptr || workspace_bytes < need ||
      ((uintptr_t)workspace & 15) != 0)
    plan = SplitPlan{1, 0, 0, 0, 0};
  const int nkb = K / 64;
  // Four block codes per dword load: needs whole groups of four blocks per
  // row (then four blocks never straddle a group of 256) and an aligned
  // code array.
  const bool q4 = double_quant && nkb % 4 == 0 && ((uintptr_t)absmax & 3) == 0;
  float* part = (float*)workspace;
  for (int64_t r0 = 0; r0 < M; r0 += slab) {
    const int m = (int)(M - r0 < slab ? M - r0 : slab);
    const uint16_t* xs = x + r0 * ldx;
    uint16_t* ys = y + r0 * ldy;
    LoraArgs ls = la;
    if (LORA) ls.xa = la.xa + r0 * la.ldxa;
    if (!double_quant)
      launch_one<kDqNone, false, LORA>(xs, ldx, packed, absmax, absmax2, mean, m, N, K, ys, ldy,
                                       quant_type, f16, ls, plan, part, stream);
    else if (double_quant == kDqDynamic && q4)
      launch_one<kDqDynamic, true, LORA>(xs, ldx, packed, absmax, absmax2, mean, m, N, K, ys,
                                         ldy, quant_type, f16, ls, plan, part, stream);
    else if (double_quant == kDqDynamic)
      launch_one<kDqDynamic, false, LORA>(xs, ldx, packed, absmax, absmax2, mean, m, N, K, ys,
                                          ldy, quant_type, f16, ls, plan, part, stream);
    else if (q4)
      launch_one<kDqLinear, true, LORA>(xs, ldx, packed, absmax, absmax2, mean, m, N, K, ys, ldy,
                                        quant_type, f16, ls, plan, part, stream);
    else
      launch_one<kDqLinear, false, LORA>(xs, ldx, packed, absmax, absmax2, mean, m, N, K, ys,
                                         ldy, quant_type, f16, ls, plan, part, stream);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

size_t gemm_workspace_bytes(int M, int N, int K) {
  SplitPlan plan;
  return split_plan(M, N, K, plan);
}

hipError_t launch_gemm(const uint16_t* x, int64_t ldx, const uint8_t* packed, const void* absmax,
                       const float* absmax2, const float* mean, int double_quant, int quant_type,
                       bool f16, int M, int N, int K, uint16_t* y, int64_t ldy, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  return launch_gemm_any<false>(x, ldx, packed, absmax, absmax2, mean, double_quant, quant_type,
                                f16, M, N, K, y, ldy, LoraArgs{nullptr, 0, nullptr, 0, 0},
                                workspace, workspace_bytes, stream);
}

hipError_t launch_gemm_lora(const uint16_t* x, int64_t ldx, const uint8_t* packed,
                            const void* absmax, const float* absmax2, const float* mean,
                            int double_quant, int quant_type, bool f16, int M, int N, int K,
                            const uint16_t* xa, int64_t ldxa, const uint16_t* lora_b,
                            int64_t ldb, int r, uint16_t* y, int64_t ldy, hipStream_t stream) {
  return launch_gemm_any<true>(x, ldx, packed, absmax, absmax2, mean, double_quant, quant_type,
                               f16, M, N, K, y, ldy, LoraArgs{xa, ldxa, lora_b, ldb, r}, nullptr,
                               0, stream);
}

}  // namespace bnbx

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
// weight tile.
//   - X goes from global memory straight into LDS (global_load_lds, 16 B per
//     lane, no registers).  Its rows are 128 B with the eight 16-byte chunks
//     of row r rotated by (r / 2) % 8, so that 16 lanes reading the same
//     chunk of 16 consecutive rows hit 64 distinct banks.
//   - Each thread owns one weight row: it stages the row's 32 packed bytes
//     and block code/scale of a K step in registers, four steps ahead (four
//     staging sets), and writes the row dequantized into LDS (rows padded to
//     144 B).  The dequant is vector-only: the 16 values bf16(L[i] * scale)
//     of the row's block form a byte table in 8 registers that v_perm_b32
//     indexes by the 4-bit codes (no LDS lookups).
// In step t a wave issues the X copy of step t+1 and the weight loads of step
// t+4, then runs 64 MFMAs - the last substep of step t-1 (its operands were
// read before the barrier, so the first MFMAs after the barrier wait for no
// LDS read) and substeps 0..2 of step t - and between them dequantizes step
// t+1's weights into the other buffer.  The step ends with one barrier
// preceded by a wait for this wave's LDS writes and X copies only: the weight
// loads, issued after the copies, stay in flight (the memory counter retires
// in order).  Scheduling-group barriers lay each substep out as one MFMA
// followed by a share of the LDS reads, vector ops and LDS writes, so that
// vector and LDS work issues while the matrix core is busy.  Each LDS buffer
// is its own object, picked at compile time, so the compiler can tell reads
// of one buffer from copies in flight into another.  Steps past the end of K
// load and write clamped (redundant) data into a buffer no MFMA reads.
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
constexpr int kXcds = 8;
constexpr int kABuf = BM * BK;              // bf16 elements per X buffer (128 B rows)
constexpr int kBBuf = BN * LDS_ROW;         // bf16 elements per weight buffer

// Scheduling-group masks (AMDGPU sched_group_barrier).
constexpr int kSgMfma = 0x008, kSgValu = 0x002, kSgDsRead = 0x100, kSgDsWrite = 0x200;

// One thread's weight row for one K step.
struct Stage {
  uint4 w[2];   // 32 packed bytes (64 weights)
  uint32_t q;   // int8 block code (double quant), as loaded (zero-extended byte)
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
    // Kept as the raw byte: a sign extension here would be an instruction on
    // the loaded value that the compiler may place before the step's barrier
    // (making it wait for these loads); it is done where the scale is formed.
    st.q = ((const uint8_t*)absmax)[blk];
    st.s = absmax2[blk >> 8];
  } else {
    st.q = 0u;
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
    // (float)(int8)q = (float)(int32)(q << 24) * 2^-24, both steps exact
    const float qf = (float)(int32_t)(st.q << 24) * 0x1p-24f;
    const float sc = DQ ? __builtin_fmaf(qf, st.s * (1.0f / 127.0f), mu) : st.s;
    return bok ? sc : 0.0f;
  };
  // Vector-only dequant.  The 16 values bf16(L[i] * scale) of the row's block
  // are split into a table of their high bytes (h[j] holds entries 4j..4j+3)
  // and one of their low bytes; four 4-bit codes held one per byte select
  // their entries with v_perm_b32 from each half (entries 0-7 and 8-15) and a
  // per-byte mask made from bit 3 of the codes (v_perm's sign-replicating
  // selectors 8-11) picks between the halves.
  struct Tab16 {
    uint32_t h[4], l[4];
  };
  auto make_tab16 = [&](float sc) {
    uint32_t pk[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) pk[k] = pack_bf16x2(lv.level[2 * k] * sc, lv.level[2 * k + 1] * sc);
    Tab16 t;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      t.h[j] = perm(pk[2 * j + 1], pk[2 * j], 0x07050301u);
      t.l[j] = perm(pk[2 * j + 1], pk[2 * j], 0x06040200u);
    }
    return t;
  };
  // 8 weights (one packed dword: byte j = codes of weights 2j (high nibble)
  // and 2j+1) -> 4 dwords of bf16 pairs in weight order.
  auto decode8 = [&](uint32_t d, const Tab16& t, uint32_t* o) {
    auto pick = [&](uint32_t sel, uint32_t m, const uint32_t* tt) {
      const uint32_t a = perm(tt[1], tt[0], sel), b = perm(tt[3], tt[2], sel);
      return (m & b) | (~m & a);
    };
    const uint32_t sE = (d >> 4) & 0x07070707u, sO = d & 0x07070707u;
    const uint32_t mE = perm(d << 8, d, 0x090B080Au);          // bit 7 of each byte
    const uint32_t d4 = d << 4;
    const uint32_t mO = perm(d4 << 8, d4, 0x090B080Au);        // bit 3 of each byte
    const uint32_t hiE = pick(sE, mE, t.h), loE = pick(sE, mE, t.l);
    const uint32_t hiO = pick(sO, mO, t.h), loO = pick(sO, mO, t.l);
    const uint32_t t0 = perm(hiE, loE, 0x05010400u), t1 = perm(hiE, loE, 0x07030602u);
    const uint32_t u0 = perm(hiO, loO, 0x05010400u), u1 = perm(hiO, loO, 0x07030602u);
    o[0] = perm(u0, t0, 0x05040100u);
    o[1] = perm(u0, t0, 0x07060302u);
    o[2] = perm(u1, t1, 0x05040100u);
    o[3] = perm(u1, t1, 0x07060302u);
  };
  auto put_w_valu = [&](const Stage& st, uint16_t* wbuf, int p, const Tab16& t) {
    const uint32_t d0 = p == 0 ? st.w[0].x : p == 1 ? st.w[0].z : p == 2 ? st.w[1].x : st.w[1].z;
    const uint32_t d1 = p == 0 ? st.w[0].y : p == 1 ? st.w[0].w : p == 2 ? st.w[1].y : st.w[1].w;
    uint32_t o[8];
    decode8(d0, t, o);
    decode8(d1, t, o + 4);
    uint16_t* bw = wbuf + tid * LDS_ROW + p * 16;
    *(uint4*)(bw) = make_uint4(o[0], o[1], o[2], o[3]);
    *(uint4*)(bw + 8) = make_uint4(o[4], o[5], o[6], o[7]);
  };
  // Prologue: step 0 into buffer 0; the weights of steps 1..3 staged in sets
  // 1..3.
  Stage s0, s1, s2, s3;
  copy_x(As0, 0);
  load(s0, 0);
  {
    const Tab16 t = make_tab16(scale_of(s0));
#pragma unroll
    for (int p = 0; p < 4; ++p) put_w_valu(s0, Bs0, p, t);
  }
  load(s1, 1);
  load(s2, 2);
  load(s3, 3);
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

  // One K step.  Its MFMAs are the last substep of step kb-1 (operands read
  // before the barrier) and substeps 0..2 of step kb; substep 3 of step kb
  // opens the next step.  So each barrier is followed by 16 MFMAs that need
  // no LDS read, while the first operands of the new buffer are read.
  // Between the MFMAs: the dequantized weights of step kb+1 (from staging set
  // `sn`) are written to the other buffer; `sl` is refilled with step kb+4.
  // R[0] / R[1] hold operands, R[0] holding substep 3 of the previous step.
  bf16x8_t av[2][4], bv[2][4];
  auto read_ops = [&](const uint16_t* a, const uint16_t* bb, int ks, int r) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      av[r][i] = *(const bf16x8_t*)(a + aoff[ks] + i * 32 * BK);
      bv[r][i] = *(const bf16x8_t*)(bb + (brow_op + i * 32) * LDS_ROW + ks * 16 + kcol);
    }
  };
  auto mfmas = [&](int r) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[r][i], bv[r][j], acc[i][j], 0, 0, 0);
  };
  auto step = [&](auto buf_tag, auto first_tag, int64_t kb, Stage& sn, Stage& sl) {
    constexpr int buf = decltype(buf_tag)::value;      // kb % 2
    constexpr bool first = decltype(first_tag)::value; // no step kb-1
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
    __builtin_amdgcn_sched_barrier(0);   // the weight loads go out after the X copies
    load(sl, kb + 4);
    const Tab16 t16 = make_tab16(scale_of(sn));
#pragma unroll
    for (int ss = 0; ss < BK / 16; ++ss) {
      read_ops(a, bb, ss, (ss + 1) & 1);          // substep ss of step kb
      if (!first || ss > 0) mfmas(ss & 1);        // substep 3 of kb-1, then 0..2 of kb
      put_w_valu(sn, bn, ss, t16);                // a quarter of step kb+1's weights
      // 16 x {1 MFMA, an operand read (first 8), 4 vector ops}; the two LDS
      // writes after MFMAs 10 and 11, so that they have retired when the next
      // substep waits for its operands (the LDS counter is in order).
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        if (g < 8) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgValu, 4, 0);
        if (g == 10 || g == 11) __builtin_amdgcn_sched_group_barrier(kSgDsWrite, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);   // one substep per scheduling region
    }
    // End of step: this step's LDS writes done and its X copies landed.  The
    // copies were issued before the weight loads of step kb+4 and the memory
    // counter retires in order, so waiting until only those loads are left
    // (4 instructions, 3 without double quant) covers the copies while the
    // weight loads stay in flight across the barrier.  Written as inline asm:
    // the compiler relaxes a builtin wait to what it believes this wave needs,
    // and it does not count the other waves reading these LDS writes.
    if (DQ)
      __builtin_amdgcn_s_waitcnt(0x0F74);   // vmcnt(4)
    else
      __builtin_amdgcn_s_waitcnt(0x0F73);   // vmcnt(3)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using F0 = std::integral_constant<bool, false>;
  using F1 = std::integral_constant<bool, true>;
  // Four staging sets rotate (step t writes set (t+1)%4 and refills set t%4),
  // two LDS buffers alternate: after the first step, the loop is unrolled four
  // times so that both are fixed at compile time.
  step(B0{}, F1{}, 0, s1, s0);
  int64_t kb = 1;
  for (; kb + 3 < nkb; kb += 4) {
    step(B1{}, F0{}, kb, s2, s1);
    step(B0{}, F0{}, kb + 1, s3, s2);
    step(B1{}, F0{}, kb + 2, s0, s3);
    step(B0{}, F0{}, kb + 3, s1, s0);
  }
  if (kb < nkb) step(B1{}, F0{}, kb, s2, s1);
  if (kb + 1 < nkb) step(B0{}, F0{}, kb + 1, s3, s2);
  if (kb + 2 < nkb) step(B1{}, F0{}, kb + 2, s0, s3);
  mfmas(0);   // substep 3 of the last step

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

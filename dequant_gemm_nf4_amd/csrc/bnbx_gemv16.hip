// Batched decode GEMV, 4 < M <= 16, with 4-bit (NF4 or FP4) weights for
// gfx950 (mlqm.cn bitsandbytes article, sec. 3.4 and the sec. 7 pitfall: the
// packed weight is streamed once, whatever K).
#include "bnbx_gemv_common.hpp"

namespace bnbx {
namespace {

// ---------------------------------------------------------------------------
// 4 < M <= 16: one launch for any K; the weights are streamed once into
// v_mfma_f32_16x16x32_bf16 (or _f16) operands.
//
// MFMA roles: A is X (lane l: row l % 16, eight k), B is the dequantized
// weight (lane l: weight row l % 16 of a group of 16, eight k), and lane l
// ends with Y[4 (l / 16) + v][16 g + l % 16], v = 0..3.
//
// Loads are quad-coalesced: lane x reads 16 bytes of row x / 4 at piece
// x % 4, so the four lanes of a quad read 64 contiguous bytes and one
// instruction covers 16 rows x 64 bytes.  (MFMA-layout loads, where
// neighbouring lanes read different rows, made every lane its own memory
// request; the address path then held the kernel at 17 us on 14336 x 4096.)
// A per-wave 1 KB LDS stage turns that into the MFMA layout: lane x writes
// its piece to slot 16 p + ((r + 4 p) mod 16) and lane (q, r) reads slot
// 16 q + ((r + 4 q) mod 16), both bank-conflict free; lane (q, r) then holds
// piece q of row r.  For the weights, a 4 x 4 transpose across the quarters
// (two v_permlane32_swap, two v_permlane16_swap) then gives lane (q, r) the
// dword q of every piece m: MFMA m covers the 32 k [128 h + 32 m, +32) of
// the slice, half of block 2 h + m / 2, and its B operand is four byte ->
// level-pair lookups in the LDS table of gemv_kernel.  The two MFMAs of a
// block go to a zeroed accumulator scaled by the block scale of the lane's
// weight row; scales are formed where they load (lane x: row x / 4, block
// x % 4) and fetched with ds_bpermute.
//
// Work split.  K is cut into slices of 256 k (4 blocks); wave w of the
// 16-wave workgroup owns slices w, w + 16, ... (one per chunk of 4096 k)
// and keeps the X operands of its current slice in registers.  The
// workgroup owns row groups blockIdx.x + j * gridDim.x and takes NB of them
// at a time.  Every load is unconditional (items past the end get offsets
// outside their buffer, which read as zero), so each wait names exactly the
// loads it needs.  With one chunk (K <= 4096) all of a batch's loads go out
// at once; with more, each half of the next chunk's X goes into the
// registers of the half just multiplied, and the weights two chunks ahead
// into the set just used.  The 16 waves' partial sums meet in LDS, two row
// groups at a time.
// ---------------------------------------------------------------------------
constexpr int k16Waves = 16;
constexpr int k16SliceK = 256;    // k per wave slice (4 blocks)
constexpr int k16ChunkK = k16Waves * k16SliceK;
constexpr uint32_t kFar = 0x80000000u;   // an offset past every buffer resource

// LoRA term (LORA): Y += XA . B^T with XA [M, r] and B [N, r] in the
// compute type, r a multiple of 16 up to 256 (at most 8 chunks of 32 ranks).
struct Gemv16Lora {
  const uint16_t* xa;
  int64_t ldxa;
  const uint16_t* lb;
  int64_t ldb;
  int r;
};
struct NoLora {};

template <int SM, bool F16, int NB, bool MULTI, bool LORA = false>
__global__ __launch_bounds__(k16Waves * 64, 1) void gemv16_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ packed,
    const void* __restrict__ absmax, const float* __restrict__ absmax2,
    const float* __restrict__ mean, int M, int N, int K, uint16_t* __restrict__ y, int64_t ldy,
    LevelTable lv, typename std::conditional<LORA, Gemv16Lora, NoLora>::type la) {
  constexpr bool DQ = SM != kScaleF32;
  constexpr bool DYN = scale_dyn(SM);
  constexpr int kSets = MULTI ? 2 : 1;
  constexpr int kRed = NB < 2 ? NB : 2;   // row groups reduced at once
  static_assert(!MULTI || NB == 1, "several chunks take one row group at a time");
  // Table at LDS offset 0 (its addresses are v_perm results), then the
  // waves' 1 KB stages, then the partial sums, then the dynamic map (DYN).
  __shared__ __attribute__((aligned(16))) unsigned char
      smem[kTabBytes + k16Waves * 1024 + kRed * k16Waves * 256 * 4 + (DYN ? kMapBytes : 0)];
  unsigned char* const tab = smem;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  unsigned char* const stage = smem + kTabBytes + wave * 1024;
  float* const red = (float*)(smem + kTabBytes + k16Waves * 1024);
  unsigned char* const dmap = smem + kTabBytes + k16Waves * 1024 + kRed * k16Waves * 256 * 4;
  const int r = lane & 15, q = lane >> 4;        // MFMA layout
  const int lr = lane >> 2, lp = lane & 3;       // load layout: row, piece
  const uint32_t wslot = 16u * (uint32_t)(16 * lp + ((lr + 4 * lp) & 15));
  const uint32_t rslot = 16u * (uint32_t)(16 * q + ((r + 4 * q) & 15));
  const uint32_t rowK2 = (uint32_t)K >> 1;
  const uint32_t nkb = (uint32_t)K >> 6;
  const int nchunks = (K + k16ChunkK - 1) / k16ChunkK;
  const int ngroups = (N + 15) >> 4;
  const int nrg = ngroups > (int)blockIdx.x
                      ? (ngroups - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x
                      : 0;

  // The mean first, by lane 0 (loads complete in issue order, so its use
  // waits for nothing else); broadcast where it is used.
  float mul = 0.0f;
  if (DQ && lane == 0)
    mul = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(mean, 4u), 0u, 0, 0));
  const float dmv = DYN ? dyn_map_value(t) : 0.0f;

  const rsrc_t rw = make_rsrc(packed, (uint32_t)N * rowK2);
  const uint32_t nblocks = (uint32_t)N * nkb;
  const rsrc_t rq = make_rsrc(absmax, DQ ? nblocks : nblocks * 4u);
  const rsrc_t rg = make_rsrc(absmax2, DQ ? (nblocks + 255u) / 256u * 4u : 4u);
  const rsrc_t rx = make_rsrc(x, (uint32_t)((int64_t)(M - 1) * ldx * 2 + (int64_t)K * 2));
  const uint32_t xrow = (uint32_t)((int64_t)lr * ldx * 2);

  // One item (a row group's piece of one slice), in the load layout: the
  // lane's two 16-byte weight pieces (row 16 g + x / 4, bytes 64 h + 16 (x %
  // 4) of the slice) and the raw scale of block x % 4 of that row.
  struct Item {
    u32x4_t w[2];
    uint32_t qc;   // code byte(s): the row modes hold the row's four codes
    float gs;      // group scale, or the fp32 absmax
  };
  struct Set {
    Item it[NB];
  };
  // X of slice u, half h, in the load layout: xa[h][m] holds row x / 4,
  // k [256 u + 128 h + 32 m + 8 (x % 4), +8) (zero past K; rows past M read
  // as zero through the resource).
  u32x4_t xa[2][4];
  auto load_x = [&](int u, int h) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int k0 = u * k16SliceK + 128 * h + 32 * m;
      xa[h][m] = __builtin_amdgcn_raw_buffer_load_b128(
          rx, k0 < K ? xrow + (uint32_t)(k0 + 8 * lp) * 2u : kFar, 0, 0);
    }
  };
  // Item of slice u, row group j of the workgroup.
  auto load_item = [&](Item& it, int u, int j) {
    {
      const bool uin = u * k16SliceK < K;
      const int g = (int)blockIdx.x + j * (int)gridDim.x;
      const bool in = uin && j < nrg;
      const uint32_t row = (uint32_t)(16 * g + lr);
      const uint32_t wo = in ? row * rowK2 + (uint32_t)u * (k16SliceK / 2) + 16u * (uint32_t)lp : kFar;
#pragma unroll
      for (int h = 0; h < 2; ++h) it.w[h] = __builtin_amdgcn_raw_buffer_load_b128(rw, wo + 64u * h, 0, 2);
      const uint32_t blk = row * nkb + 4u * (uint32_t)u;   // the slice's first block in the row
      if (scale_row(SM)) {
        it.qc = __builtin_amdgcn_raw_buffer_load_b32(rq, in ? blk : kFar, 0, 0);
        it.gs = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rg, in ? (blk >> 8) * 4u : kFar, 0, 0));
      } else if (DQ) {
        const uint32_t b = blk + (uint32_t)lp;
        it.qc = __builtin_amdgcn_raw_buffer_load_b8(rq, in ? b : kFar, 0, 0);
        it.gs = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rg, in ? (b >> 8) * 4u : kFar, 0, 0));
      } else {
        it.qc = 0u;
        it.gs = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rq, in ? (blk + lp) * 4u : kFar, 0, 0));
      }
    }
  };
  auto load_set = [&](Set& st, int u, int j0) {
#pragma unroll
    for (int jj = 0; jj < NB; ++jj) load_item(st.it[jj], u, j0 + jj);
  };
  // Scale of block x % 4 of row x / 4 (load layout).
  auto load_scale = [&](const Item& it, float mu) {
    if (!DQ) return it.gs;
    if (DYN) {
      const uint32_t code = scale_row(SM) ? __builtin_amdgcn_ubfe(it.qc, lp * 8, 8) : it.qc & 0xffu;
      const float prod = *(const float*)(dmap + code * 4u) * it.gs;
      return prod + mu;
    }
    const int code = scale_row(SM) ? __builtin_amdgcn_sbfe((int)it.qc, lp * 8, 8)
                                   : (int)(int8_t)(uint8_t)it.qc;
    const float prod = (float)code * dq_step_normal(it.gs);
    return prod + mu;
  };
  // Load layout -> lane (q, r) holds piece q of row r, through the stage.
  auto relayout = [&](u32x4_t& v) {
    *(u32x4_t*)(stage + wslot) = v;
    v = *(const u32x4_t*)(stage + rslot);
  };

  const uint32_t lanebyte = (uint32_t)(lane & (kCopies - 1)) << 2;
  auto lut = [&](uint32_t d) {
    u32x4_t b;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = *(const uint32_t*)(tab + perm(d, lanebyte, 0x0c0c0000u | ((4u + j) << 8)));
    return b;
  };
  // One item's half h (128 k of its row group) into its sums; X must be in
  // the MFMA layout.
  auto mul_item_half = [&](Item& it, int h, f32x4_t& acc, float sl) {
    relayout(it.w[h]);
    const auto a = __builtin_amdgcn_permlane32_swap(it.w[h][0], it.w[h][2], false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(it.w[h][1], it.w[h][3], false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    const auto e = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    const uint32_t E[4] = {c[0], c[1], e[0], e[1]};
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      f32x4_t blk = {0.0f, 0.0f, 0.0f, 0.0f};
      blk = mfma_16x16x32<F16>(xa[h][2 * hb], lut(E[2 * hb]), blk);
      blk = mfma_16x16x32<F16>(xa[h][2 * hb + 1], lut(E[2 * hb + 1]), blk);
      // block 2 h + hb of row r was formed by lane 4 r + 2 h + hb
      const float sc = __int_as_float(
          __builtin_amdgcn_ds_bpermute((4 * r + 2 * h + hb) << 2, __float_as_int(sl)));
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(blk[v], sc, acc[v]);
    }
  };
  // A set's slice into the batch's sums, item by item (each item's work
  // starts as soon as its own loads are in).
  auto mul_set = [&](Set& st, f32x4_t (&acc)[NB], float mu) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int m = 0; m < 4; ++m) relayout(xa[h][m]);
#pragma unroll
    for (int jj = 0; jj < NB; ++jj) {
      const float sl = load_scale(st.it[jj], mu);
      mul_item_half(st.it[jj], 0, acc[jj], sl);
      mul_item_half(st.it[jj], 1, acc[jj], sl);
    }
  };

  Set sets[kSets];
  for (int j0 = 0; j0 < nrg; j0 += NB) {   // the workgroup's loop: barriers are uniform
    // Only the first item's loads go out before the table build: the
    // barrier after it waits for the slowest wave, and a wave issuing many
    // loads into a full memory pipeline stalls for microseconds.  Then X
    // (cache hits) and the other items.
    load_item(sets[0].it[0], wave, j0);
    if (j0 == 0) {
      // byte -> level-pair table, behind the first loads (no memory waits)
      const int lvl = level_lanes(lv);
      for (int e = t; e < 256 * kCopies / 4; e += k16Waves * 64) {
        const uint32_t b = (uint32_t)e / (kCopies / 4);
        const uint32_t v = pack16x2<F16>(level_lookup(lvl, b >> 4), level_lookup(lvl, b & 15u));
        *(uint4*)(tab + b * 256u + ((uint32_t)e % (kCopies / 4)) * 16u) = make_uint4(v, v, v, v);
      }
      if (DYN && t < 256) *(float*)(dmap + t * 4) = dmv;
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    }
    load_x(wave, 0);
    load_x(wave, 1);
#pragma unroll
    for (int jj = 1; jj < NB; ++jj) load_item(sets[0].it[jj], wave, j0 + jj);
    // LoRA: wave w takes ranks [32 w, 32 w + 32) of XA . B^T for each row
    // group of the batch, in the MFMA layout (lane (q, r): row r, ranks
    // 32 w + 8 q .. +8); ranks past r, rows past M or N read zero.
    u32x4_t lxa, lbo[LORA ? NB : 1];
    if constexpr (LORA) {
      const int k8 = 32 * wave + 8 * q;
      const bool kin = k8 < la.r;
      const rsrc_t rxa = make_rsrc(la.xa, (uint32_t)(((int64_t)(M - 1) * la.ldxa + la.r) * 2));
      lxa = __builtin_amdgcn_raw_buffer_load_b128(
          rxa, kin ? (uint32_t)(((int64_t)r * la.ldxa + k8) * 2) : kFar, 0, 0);
      const rsrc_t rlb = make_rsrc(la.lb, (uint32_t)(((int64_t)(N - 1) * la.ldb + la.r) * 2));
#pragma unroll
      for (int jj = 0; jj < NB; ++jj) {
        const int64_t n = 16 * ((int64_t)blockIdx.x + (int64_t)(j0 + jj) * gridDim.x) + r;
        lbo[jj] = __builtin_amdgcn_raw_buffer_load_b128(
            rlb, kin && j0 + jj < nrg ? (uint32_t)((n * la.ldb + k8) * 2) : kFar, 0, 0);
      }
    }
    if (MULTI) load_set(sets[kSets - 1], k16Waves + wave, j0);
    const float mu = DQ ? __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(mul))) : 0.0f;
    f32x4_t acc[NB];
#pragma unroll
    for (int jj = 0; jj < NB; ++jj) acc[jj] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    if (!MULTI) {
      mul_set(sets[0], acc, mu);
    } else {
      // Chunk c uses weight set c % 2 (one row group).  Once half h of
      // chunk c is multiplied, half h of chunk c + 1's X goes into the same
      // registers; once the whole chunk is, chunk c + 2's weights go into its
      // set.
      for (int c = 0; c < nchunks; c += 2) {
        const int u = c * k16Waves + wave;
#pragma unroll
        for (int m = 0; m < 4; ++m) relayout(xa[0][m]);
        const float s0 = load_scale(sets[0].it[0], mu);
        mul_item_half(sets[0].it[0], 0, acc[0], s0);
        load_x(u + k16Waves, 0);
#pragma unroll
        for (int m = 0; m < 4; ++m) relayout(xa[1][m]);
        mul_item_half(sets[0].it[0], 1, acc[0], s0);
        load_x(u + k16Waves, 1);
        load_set(sets[0], u + 2 * k16Waves, j0);
        if (c + 1 < nchunks) {   // workgroup-uniform, no loads inside
#pragma unroll
          for (int m = 0; m < 4; ++m) relayout(xa[0][m]);
          const float s1 = load_scale(sets[kSets - 1].it[0], mu);
          mul_item_half(sets[kSets - 1].it[0], 0, acc[0], s1);
        }
        load_x(u + 2 * k16Waves, 0);
        if (c + 1 < nchunks) {
#pragma unroll
          for (int m = 0; m < 4; ++m) relayout(xa[1][m]);
          const float s1 = load_scale(sets[kSets - 1].it[0], mu);
          mul_item_half(sets[kSets - 1].it[0], 1, acc[0], s1);
        }
        load_x(u + 2 * k16Waves, 1);
        load_set(sets[kSets - 1], u + 3 * k16Waves, j0);
      }
    }

    if constexpr (LORA) {
#pragma unroll
      for (int jj = 0; jj < NB; ++jj) acc[jj] = mfma_16x16x32<F16>(lxa, lbo[jj], acc[jj]);
    }
    // the batch's partial sums meet in LDS, kRed row groups at a time;
    // Y[m][16 g + n] sits at lane 16 (m / 4) + n, value m % 4 of every
    // wave's fragment
#pragma unroll
    for (int j1 = 0; j1 < NB; j1 += kRed) {
#pragma unroll
      for (int jj = 0; jj < kRed; ++jj)
        *(f32x4_t*)(red + (jj * k16Waves + wave) * 256 + lane * 4) = acc[j1 + jj];
      __syncthreads();
      for (int e = t; e < kRed * 256; e += k16Waves * 64) {
        const int jj = e >> 8, m = (e >> 4) & 15, nn = e & 15;
        const int n = 16 * ((int)blockIdx.x + (j0 + j1 + jj) * (int)gridDim.x) + nn;
        if (j0 + j1 + jj < nrg && m < M && n < N) {
          const int src = ((m >> 2) * 16 + nn) * 4 + (m & 3);
          float sum = 0.0f;
#pragma unroll
          for (int w = 0; w < k16Waves; ++w) sum += red[(jj * k16Waves + w) * 256 + src];
          y[(int64_t)m * ldy + n] = f32_to_16<F16>(sum);
        }
      }
      __syncthreads();
    }
  }
}

// Scale layout of the M > 4 kernel: the four codes of a slice as one dword
// (shared by a quad) when every row holds a multiple of 4 blocks and the
// codes are 4-byte aligned (the four blocks then share one group), else one
// code per lane.  NB, the
// row groups a workgroup multiplies at once: up to 4 with one chunk of K,
// 1 with several (two weight sets); larger counts spill registers.
template <int SM, bool F16, bool LORA = false>
hipError_t launch_gemv16_sm(int grid, int nb, bool multi, const uint16_t* x, int64_t ldx,
                            const uint8_t* packed, const void* absmax, const float* absmax2,
                            const float* mean, int M, int N, int K, uint16_t* y, int64_t ldy,
                            const LevelTable& lv, hipStream_t stream,
                            typename std::conditional<LORA, Gemv16Lora, NoLora>::type la = {}) {
#define BNBX_G16(NB, MULTI)                                                                    \
  hipLaunchKernelGGL((gemv16_kernel<SM, F16, NB, MULTI, LORA>), dim3(grid), dim3(k16Waves * 64), \
                     0, stream, x, ldx, packed, absmax, absmax2, mean, M, N, K, y, ldy, lv, la)
  if (multi) {
    BNBX_G16(1, true);
  } else if (nb == 1) {
    BNBX_G16(1, false);
  } else if (nb == 2 || LORA) {   // four row groups with the LoRA operands spill registers
    BNBX_G16(2, false);
  } else {
    if constexpr (!LORA) BNBX_G16(4, false);
  }
#undef BNBX_G16
  return hipGetLastError();
}

template <bool F16, bool LORA = false>
hipError_t launch_gemv16(int grid, const uint16_t* x, int64_t ldx, const uint8_t* packed,
                         const void* absmax, const float* absmax2, const float* mean, int dq,
                         int M, int N, int K, uint16_t* y, int64_t ldy, const LevelTable& lv,
                         hipStream_t stream,
                         typename std::conditional<LORA, Gemv16Lora, NoLora>::type la = {}) {
  const bool multi = K > k16ChunkK;
  const int ngroups = (N + 15) / 16;
  const int per_wg = (ngroups + grid - 1) / grid;
  const int nb = multi ? 1 : (per_wg >= 3 ? 4 : per_wg);
  const bool rowq = dq && ((K >> 6) % 4 == 0) && ((uintptr_t)absmax & 3u) == 0;
  if (dq == kDqDynamic && rowq)
    return launch_gemv16_sm<kScaleDynRow, F16, LORA>(grid, nb, multi, x, ldx, packed, absmax,
                                                     absmax2, mean, M, N, K, y, ldy, lv, stream,
                                                     la);
  if (dq == kDqDynamic)
    return launch_gemv16_sm<kScaleDynLane, F16, LORA>(grid, nb, multi, x, ldx, packed, absmax,
                                                      absmax2, mean, M, N, K, y, ldy, lv, stream,
                                                      la);
  if (rowq)
    return launch_gemv16_sm<kScaleDqRow, F16, LORA>(grid, nb, multi, x, ldx, packed, absmax,
                                                    absmax2, mean, M, N, K, y, ldy, lv, stream,
                                                    la);
  if (dq)
    return launch_gemv16_sm<kScaleDqLane, F16, LORA>(grid, nb, multi, x, ldx, packed, absmax,
                                                     absmax2, mean, M, N, K, y, ldy, lv, stream,
                                                     la);
  return launch_gemv16_sm<kScaleF32, F16, LORA>(grid, nb, multi, x, ldx, packed, absmax, absmax2,
                                                mean, M, N, K, y, ldy, lv, stream, la);
}

}  // namespace

hipError_t launch_gemv16_lora_batch(int grid, const uint16_t* x, int64_t ldx,
                                    const uint8_t* packed, const void* absmax,
                                    const float* absmax2, const float* mean, int dq, bool f16,
                                    int M, int N, int K, const uint16_t* xa, int64_t ldxa,
                                    const uint16_t* lora_b, int64_t ldb, int r, uint16_t* y,
                                    int64_t ldy, const LevelTable& lv, hipStream_t stream) {
  const Gemv16Lora la{xa, ldxa, lora_b, ldb, r};
  return f16 ? launch_gemv16<true, true>(grid, x, ldx, packed, absmax, absmax2, mean, dq, M, N,
                                         K, y, ldy, lv, stream, la)
             : launch_gemv16<false, true>(grid, x, ldx, packed, absmax, absmax2, mean, dq, M, N,
                                          K, y, ldy, lv, stream, la);
}

hipError_t launch_gemv16_batch(int grid, const uint16_t* x, int64_t ldx, const uint8_t* packed,
                               const void* absmax, const float* absmax2, const float* mean,
                               int dq, bool f16, int M, int N, int K, uint16_t* y, int64_t ldy,
                               const LevelTable& lv, hipStream_t stream) {
  return f16 ? launch_gemv16<true>(grid, x, ldx, packed, absmax, absmax2, mean, dq, M, N, K, y,
                                   ldy, lv, stream)
             : launch_gemv16<false>(grid, x, ldx, packed, absmax, absmax2, mean, dq, M, N, K, y,
                                    ldy, lv, stream);
}

}  // namespace bnbx

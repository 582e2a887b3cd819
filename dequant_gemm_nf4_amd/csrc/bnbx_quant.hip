// Blockwise 4-bit (NF4 or FP4) quantize-on-load and double quantization of
// the block scales for gfx950.
//
// mlqm.cn bitsandbytes article (news/394670): sec. 2.2 (weights are quantized
// while they are loaded, with no calibration data), sec. 3.2 (nearest of 16
// NormalFloat levels), sec. 3.3 (one FP32 absmax scale per block; double
// quantization compresses those scales a second time), sec. 4 (fp4, the
// other 4-bit quant type: the same kernel with the FP4 encode tables).
//
// quantize_kernel streams the bf16 weight once (16-byte loads, 8 weights per
// lane, 8 lanes per 64-weight block), reduces the block absmax with DPP,
// normalises with the block's fp32 reciprocal and encodes each weight with one
// bucket lookup plus one compare (see EncodeTable), packs two codes per byte
// and writes 4 bytes per lane.  With double quantization it also writes the
// fp32 absmax to the workspace and, per workgroup, an exact exponent
// histogram of its absmax values (sum of the 8-bit significands per binary
// exponent) in LDS, which it turns into its exact partial sum (an integer in
// base-2^32 digits) and writes to its own workspace slot; double_quant_kernel
// adds the slots and forms the exactly rounded mean.
//
// The grouped kernels do the same for up to kMaxQItems tensors per call:
// quantize_group_kernel walks the tensors one after another with one
// histogram and one slot per tensor (the single kernel's per-tensor device
// function), dq_mean_kernel forms each tensor's exact mean in one workgroup,
// and dq_codes_kernel gives each group of 256 block scales one wave (group
// max by a wave reduction, no workgroup barrier), with the arithmetic of
// double_quant_groups.
#include "bnbx_device.hpp"
#include "bnbx_internal.hpp"

namespace bnbx {
namespace {

constexpr int kQThreads = 1024;
constexpr int kQWaves = kQThreads / 64;
constexpr int kTabStride = 256;   // LDS bytes per bucket: 32 copies of an 8-byte entry
constexpr int kUnroll = 2;        // 512-weight tiles per wave per round (2 measured faster than 4)
constexpr int kTile = 512;        // weights per wave per tile (8 blocks)

__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v, int ctrl_id) {
  uint32_t o;
  switch (ctrl_id) {
    case 0: o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false); break;   // quad_perm 1,0,3,2
    case 1: o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false); break;   // quad_perm 2,3,0,1
    default: o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false); break; // row_half_mirror
  }
  return v > o ? v : o;
}

// Code of one normalised value x in [-1, 1].  NF4 codes are level
// indices (bucket base + 1 past the threshold); FP4 picks one of the two
// codes the bucket entry holds.
template <bool FP4>
__device__ __forceinline__ uint32_t encode_one(float x, const unsigned char* tab, uint32_t lanebase) {
  // 2^23 + 16 + 16 x rounded once to an integer: the low byte is the bucket.
  const float f = __builtin_fmaf(x, 16.0f, 8388624.0f);
  const uint32_t addr = perm(__float_as_uint(f), lanebase, 0x0c0c0400u);
  const uint2 e = *(const uint2*)(tab + addr);
  if (FP4) return __builtin_amdgcn_ubfe(e.y, x >= __uint_as_float(e.x) ? 4u : 0u, 4u);
  return e.y + (x >= __uint_as_float(e.x) ? 1u : 0u);
}

// One lane's 8 consecutive weights (4 bf16 pairs) -> one packed word; also
// returns the block absmax (bf16 bits in m, value in amax).  All 64 lanes of
// the wave must execute this together (DPP reduction over 8-lane groups).
template <bool FP4>
__device__ __forceinline__ uint32_t encode8(const uint32_t d[4], const unsigned char* tab,
                                            uint32_t lanebase,
                                            uint32_t& m_out, float& amax_out) {
  // |w| as bf16 bits: for non-negative floats integer order is value order.
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t a = d[k] & 0x7fff7fffu;
    m = max(m, max(a & 0xffffu, a >> 16));
  }
  m = dpp_max_u32(m, 0);
  m = dpp_max_u32(m, 1);
  m = dpp_max_u32(m, 2);   // now the max over this lane's 8-lane block
  const float amax = __uint_as_float(m << 16);
  // A nonzero absmax below 2^-100 is scaled by 2^64 together with its
  // weights (exact), so that its reciprocal stays finite; for any absmax
  // above 2^-128 this gives the same x as the plain product.  Such blocks
  // are rare, so the scaled form runs only in waves that hold one.
  const bool tiny = amax < 0x1p-100f && amax != 0.0f;
  const float pre = tiny ? 0x1p64f : 1.0f;
  const float r = (amax == 0.0f) ? 0.0f : 1.0f / (amax * pre);
  uint32_t word = 0;
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(tiny) == 0, 1)) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float x0 = bf16lo_to_f32(d[k]) * r;   // even element -> high nibble
      const float x1 = bf16hi_to_f32(d[k]) * r;
      const uint32_t c0 = encode_one<FP4>(x0, tab, lanebase);
      const uint32_t c1 = encode_one<FP4>(x1, tab, lanebase);
      word |= ((c0 << 4) | c1) << (8 * k);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float x0 = (bf16lo_to_f32(d[k]) * pre) * r;
      const float x1 = (bf16hi_to_f32(d[k]) * pre) * r;
      const uint32_t c0 = encode_one<FP4>(x0, tab, lanebase);
      const uint32_t c1 = encode_one<FP4>(x1, tab, lanebase);
      word |= ((c0 << 4) | c1) << (8 * k);
    }
  }
  m_out = m;
  amax_out = amax;
  return word;
}

__device__ __forceinline__ void record_block(int lane, int64_t e, uint32_t m, float amax,
                                             float* absmax, uint32_t* lhist, bool dq) {
  if ((lane & 7) == 0) {
    absmax[e / kBlock] = amax;
    if (dq && m != 0) {
      const uint32_t ex = m >> 7;   // binary exponent field
      atomicAdd(&lhist[ex], (m & 0x7fu) | (ex ? 0x80u : 0u));
    }
  }
}

// Tile pairs wv, wv + nwaves, ... of one tensor for one wave, and its ragged
// last tile (fewer than 512 weights) when `ragged` is set for this wave.
// Each round a wave loads kUnroll whole tiles (addresses clamped, so no
// per-lane branches), then encodes them; only the stores are skipped for
// tiles past the end.  Latency is hidden by the many resident waves.
template <bool DQ, bool FP4>
__device__ __forceinline__ void quantize_tensor(const uint16_t* __restrict__ w,
                                                uint8_t* __restrict__ packed,
                                                float* __restrict__ absmax, int64_t n,
                                                uint32_t* lhist, int64_t wv, int64_t nwaves,
                                                bool ragged, const unsigned char* tab,
                                                uint32_t lanebase, int lane) {
  const int64_t full = n / kTile;                       // whole 512-weight tiles
  for (int64_t t0 = wv * kUnroll; t0 < full; t0 += nwaves * kUnroll) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t tile = t0 + u < full ? t0 + u : full - 1;
      v[u] = load_nt16(w + tile * kTile + lane * 8);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t d[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      uint32_t m;
      float amax;
      const uint32_t word = encode8<FP4>(d, tab, lanebase, m, amax);
      if (t0 + u < full) {   // wave-uniform
        const int64_t e = (t0 + u) * kTile + lane * 8;
        *(uint32_t*)(packed + (e >> 1)) = word;
        record_block(lane, e, m, amax, absmax, lhist, DQ);
      }
    }
  }

  if (n % kTile != 0 && ragged) {
    const int64_t e = full * kTile + lane * 8;
    uint16_t h[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) h[k] = (e + k < n) ? w[e + k] : (uint16_t)0;
    const uint32_t d[4] = {h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
                           h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16)};
    uint32_t m;
    float amax;
    const uint32_t word = encode8<FP4>(d, tab, lanebase, m, amax);
    if (e < n) {
      const int nbytes = (int)((n - e) < 8 ? (n - e) >> 1 : 4);
      for (int k = 0; k < nbytes; ++k) packed[(e >> 1) + k] = (uint8_t)(word >> (8 * k));
      record_block(lane, e, m, amax, absmax, lhist, DQ);
    }
  }
}

// The workgroup's partial sum I_w = sum_e lhist[e] * 2^(max(e,1)-1) (see
// exact_mean) into the base-2^32 digits ldig (zero on entry): a bin (below
// 2^32) shifted by less than 32 spans two digits.
__device__ __forceinline__ void histogram_digits(const uint32_t* lhist, unsigned long long* ldig,
                                                 int tid) {
  for (int e = tid; e < (int)kHistBins; e += kQThreads) {
    const unsigned long long h = lhist[e];
    if (h) {
      const int sh = (e > 1 ? e : 1) - 1;
      const int k = sh >> 5, bit = sh & 31;
      const unsigned long long p = h << bit;
      atomicAdd(&ldig[k], p & 0xffffffffull);
      if (p >> 32) atomicAdd(&ldig[k + 1], p >> 32);
    }
  }
}

// Replicated bucket table in LDS (entry (b, copy) at b*256 + copy*8).
__device__ __forceinline__ void fill_table(unsigned char* tab, const EncodeTable& et, int tid) {
  for (int e = tid; e < kBuckets * 32; e += kQThreads) {
    uint2 t;
    t.x = __float_as_uint(et.thr[e >> 5]);
    t.y = et.base[e >> 5];
    *(uint2*)(tab + (e >> 5) * kTabStride + (e & 31) * 8) = t;
  }
}

template <bool DQ, bool FP4>
__global__ __launch_bounds__(kQThreads, 2) void quantize_kernel(
    const uint16_t* __restrict__ w, uint8_t* __restrict__ packed, float* __restrict__ absmax,
    unsigned long long* __restrict__ slots, int64_t n, EncodeTable et) {
  __shared__ __attribute__((aligned(16))) unsigned char tab[kBuckets * kTabStride];
  __shared__ uint32_t lhist[kHistBins];
  __shared__ unsigned long long ldig[kSumDigits];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t gw = (int64_t)blockIdx.x * kQWaves + (tid >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kQWaves;

  fill_table(tab, et, tid);
  if (DQ) {
    for (int e = tid; e < (int)kHistBins; e += kQThreads) lhist[e] = 0;
    if (tid < kSumDigits) ldig[tid] = 0ull;
  }
  __syncthreads();
  const uint32_t lanebase = (uint32_t)(lane & 31) << 3;
  // The ragged last tile goes to the last wave.
  quantize_tensor<DQ, FP4>(w, packed, absmax, n, lhist, gw, nwaves, gw == nwaves - 1, tab,
                           lanebase, lane);
  if (DQ) {
    // Every workgroup writes its whole slot.
    __syncthreads();
    histogram_digits(lhist, ldig, tid);
    __syncthreads();
    if (tid < kSumDigits) slots[(int64_t)blockIdx.x * kSumDigits + tid] = ldig[tid];
  }
}

// The tensors of one grouped launch (entries past `count` unused).  Tensor
// i's 512-weight tile pairs continue the round-robin over the grid's waves
// where tensor i - 1's left off: wave v takes pairs p = v - rot[i] (mod the
// wave count) of tensor i.
struct QuantItems {
  int count;
  int64_t n[kMaxQItems];
  int64_t rot[kMaxQItems];
  const uint16_t* w[kMaxQItems];
  uint8_t* packed[kMaxQItems];
  float* absmax[kMaxQItems];
};

// Entry i of a per-tensor argument array, by selects (indexing the argument
// block with a run-time i would copy it to scratch memory).
template <typename T>
__device__ __forceinline__ T pick_item(const T (&a)[kMaxQItems], int i) {
  T r = a[0];
#pragma unroll
  for (int k = 1; k < kMaxQItems; ++k) r = i == k ? a[k] : r;
  return r;
}

// Slots: tensor i's slot of workgroup b at slots + (i * grid + b) * kSumDigits.
template <bool DQ, bool FP4>
__global__ __launch_bounds__(kQThreads, 2) void quantize_group_kernel(
    QuantItems it, unsigned long long* __restrict__ slots, EncodeTable et) {
  __shared__ __attribute__((aligned(16))) unsigned char tab[kBuckets * kTabStride];
  __shared__ uint32_t lhist[DQ ? kMaxQItems : 1][kHistBins];
  __shared__ unsigned long long ldig[DQ ? kMaxQItems : 1][kSumDigits];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t gw = (int64_t)blockIdx.x * kQWaves + __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kQWaves;

  fill_table(tab, et, tid);
  if (DQ) {
    for (int e = tid; e < it.count * (int)kHistBins; e += kQThreads)
      lhist[e / kHistBins][e % kHistBins] = 0;
    if (tid < it.count * kSumDigits) ldig[tid / kSumDigits][tid % kSumDigits] = 0ull;
  }
  __syncthreads();
  const uint32_t lanebase = (uint32_t)(lane & 31) << 3;
  for (int i = 0; i < it.count; ++i) {
    int64_t wv = gw - pick_item(it.rot, i);
    wv = wv < 0 ? wv + nwaves : wv;
    // Tensor i's ragged last tile goes to wave nwaves - 1 - i.
    quantize_tensor<DQ, FP4>(pick_item(it.w, i), pick_item(it.packed, i), pick_item(it.absmax, i),
                             pick_item(it.n, i), lhist[DQ ? i : 0], wv, nwaves,
                             gw == nwaves - 1 - i, tab, lanebase, lane);
  }
  if (DQ) {
    __syncthreads();
    for (int i = 0; i < it.count; ++i) histogram_digits(lhist[i], ldig[i], tid);
    __syncthreads();
    if (tid < it.count * kSumDigits) {
      const int i = tid / kSumDigits, d = tid % kSumDigits;
      slots[((int64_t)i * gridDim.x + blockIdx.x) * kSumDigits + d] = ldig[i][d];
    }
  }
}

// Exact mean of the block absmax values.  absmax = sig * 2^(max(e,1) - 134)
// for binary exponent field e and 8-bit significand sig, so
// sum = I * 2^-133 with I = sum_e hist[e] * 2^(max(e,1)-1), an integer below
// 2^320.  I arrives as the quantize workgroups' partial sums in ten base-2^32
// digits each (digits below 2^40); they are added digit-wise, carried,
// rounded once to binary64 (nearest even), divided by nb in binary64 and
// rounded to binary32.
__device__ float exact_mean(const unsigned long long* __restrict__ slots, int nslots, int64_t nb,
                            unsigned long long* digits /* LDS[kSumDigits], 256 threads */) {
  const int tid = threadIdx.x;
  if (tid < kSumDigits) digits[tid] = 0ull;
  __syncthreads();
  // Thread t adds digit t % 10 of slots t / 10, t / 10 + P, ... (P = 25
  // threads per digit of a 256-thread block) in a register, all loads in
  // flight at once, then one LDS add per thread.
  constexpr int P = 256 / kSumDigits;
  constexpr int kPer = (kMaxQGrid + P - 1) / P;
  if (tid < P * kSumDigits) {
    const int d = tid % kSumDigits, j0 = tid / kSumDigits;
    unsigned long long v = 0ull;
    // Unconditional loads (an index past nslots reads slot 0 and is
    // discarded), so that none waits for another.
    unsigned long long x[kPer];
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int j = j0 + r * P;
      x[r] = slots[(j < nslots ? j : 0) * kSumDigits + d];
    }
#pragma unroll
    for (int r = 0; r < kPer; ++r) v += j0 + r * P < nslots ? x[r] : 0ull;
    if (v) atomicAdd(&digits[d], v);
  }
  __syncthreads();
  double S = 0.0;
  if (tid == 0) {
    // Every digit index below is a compile-time constant (unrolled loops and
    // selects), so the digits stay in registers: a private array indexed at
    // run time would live in scratch memory.
    uint32_t dig[kSumDigits];
    unsigned long long carry = 0;
#pragma unroll
    for (int j = 0; j < kSumDigits; ++j) {
      const unsigned long long t = digits[j] + carry;
      dig[j] = (uint32_t)t;
      carry = t >> 32;
    }
    int hj = -1;   // the highest nonzero digit
#pragma unroll
    for (int j = 0; j < kSumDigits; ++j) hj = dig[j] != 0u ? j : hj;
    if (hj >= 0) {
      uint32_t d2 = 0u, d1 = 0u, d0 = 0u;   // digits hj, hj - 1, hj - 2
      bool sticky = false;                   // any nonzero digit below hj - 2
#pragma unroll
      for (int j = 0; j < kSumDigits; ++j) {
        d2 = j == hj ? dig[j] : d2;
        d1 = j == hj - 1 ? dig[j] : d1;
        d0 = j == hj - 2 ? dig[j] : d0;
        sticky |= j < hj - 2 && dig[j] != 0u;
      }
      const int lz = __clz(d2);
      const unsigned long long whi = ((unsigned long long)d2 << 32) | d1;
      const uint32_t wlo = d0;
      const unsigned long long top = lz ? (whi << lz) | (wlo >> (32 - lz)) : whi;
      const uint32_t rest = lz ? (wlo << lz) : wlo;
      sticky |= rest != 0u;
      unsigned long long m = top >> 11;
      const uint32_t drop = (uint32_t)(top & 0x7ffu);
      if (drop > 0x400u || (drop == 0x400u && (sticky || (m & 1ull)))) ++m;
      S = ldexp((double)m, 32 * (hj - 1) - lz + 11 - 133);
    }
    const double mean = S / (double)nb;
    digits[0] = __double_as_longlong(mean);  // hand the result to the block
  }
  __syncthreads();
  const double mean = __longlong_as_double((long long)digits[0]);
  return (float)mean;
}

// Groups per double_quant workgroup; their absmax values are loaded before
// the mean is formed, so that one memory latency covers both.
constexpr int kDqGroups = 4;

// Second level of the double quantization (mlqm.cn article, sec. 3.3) for
// groups g0 .. g0 + kDqGroups - 1 of one tensor: the exact mean, the group
// scales s_g = max |a_b - mean|, and per block the code of t = fl32((a_b -
// mean) / s_g): linear, round-half-even(fl32(t * 127)) as int8; DYN, the
// index of the nearest value of the dynamic 8-bit map (exact ties to the
// lower index), found by binary search over the exact binary64 midpoints of
// neighbouring values.  A group with s_g = 0 stores the code of the value 0.
// The mean goes to mean_out when write_mean is set.
template <bool DYN>
__device__ __forceinline__ void double_quant_groups(
    const float* __restrict__ a, const unsigned long long* __restrict__ slots, int nslots,
    int64_t nb, uint8_t* __restrict__ q, float* __restrict__ s_out, float* __restrict__ mean_out,
    bool write_mean, int64_t g0, unsigned long long* digits, float (*red)[4], double* mids) {
  const int tid = threadIdx.x;
  float v[kDqGroups];
#pragma unroll
  for (int i = 0; i < kDqGroups; ++i) {
    const int64_t b = (g0 + i) * kGroup + tid;
    v[i] = b < nb ? a[b] : 0.0f;
  }
  if (DYN && tid < 255) mids[tid] = kDynMapDev.mid[tid];   // visible after exact_mean's barriers
  const float mu = exact_mean(slots, nslots, nb, digits);
  if (write_mean && tid == 0) *mean_out = mu;
  const int64_t ng = (nb + kGroup - 1) / kGroup;
  float c[kDqGroups];
#pragma unroll
  for (int i = 0; i < kDqGroups; ++i) {
    const int64_t b = (g0 + i) * kGroup + tid;
    c[i] = b < nb ? v[i] - mu : 0.0f;
    const float m = wave_max(fabsf(c[i]));
    if ((tid & 63) == 0) red[i][tid >> 6] = m;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kDqGroups; ++i) {
    const int64_t g = g0 + i;
    if (g >= ng) break;   // uniform
    const int64_t b = g * kGroup + tid;
    const float s = fmaxf(fmaxf(red[i][0], red[i][1]), fmaxf(red[i][2], red[i][3]));
    int qv = DYN ? kDynZeroCode : 0;
    if (s > 0.0f) {
      const float t = c[i] / s;       // correctly rounded binary32 division
      if (DYN) {
        // #{k : t > mid[k]} over the 255 ascending midpoints
        int idx = 0;
#pragma unroll
        for (int step = 128; step >= 1; step >>= 1)
          if ((double)t > mids[idx + step - 1]) idx += step;
        qv = idx;
      } else {
        const float u = t * 127.0f;
        qv = (int)rintf(u);           // round half to even
      }
    }
    if (b < nb) q[b] = (uint8_t)qv;
    if (tid == 0) s_out[g] = s;
  }
}

template <bool DYN>
__global__ __launch_bounds__(256) void double_quant_kernel(
    const float* __restrict__ a, const unsigned long long* __restrict__ slots, int nslots,
    int64_t nb, uint8_t* __restrict__ q, float* __restrict__ s_out, float* __restrict__ mean_out) {
  __shared__ unsigned long long digits[kSumDigits];
  __shared__ float red[kDqGroups][4];
  __shared__ double mids[DYN ? 256 : 1];
  double_quant_groups<DYN>(a, slots, nslots, nb, q, s_out, mean_out, blockIdx.x == 0,
                           (int64_t)blockIdx.x * kDqGroups, digits, red, mids);
}

// The tensors of the grouped second level: tensor i owns global groups
// [gend[i-1], gend[i]) (gend[-1] = 0, entries past `count` hold INT64_MAX);
// its quantize slots start at slots + i * nslots * kSumDigits.
struct DqItems {
  int count;
  int64_t gend[kMaxQItems];
  int64_t nb[kMaxQItems];
  const float* a[kMaxQItems];
  uint8_t* q[kMaxQItems];
  float* s[kMaxQItems];
  float* mean[kMaxQItems];
};

// Grouped second level, first launch: workgroup i forms tensor i's exact
// mean and writes it to the tensor's state.
__global__ __launch_bounds__(256) void dq_mean_kernel(
    DqItems it, const unsigned long long* __restrict__ slots, int nslots) {
  __shared__ unsigned long long digits[kSumDigits];
  const int i = blockIdx.x;
  const float mu = exact_mean(slots + (int64_t)i * nslots * kSumDigits, nslots,
                              pick_item(it.nb, i), digits);
  if (threadIdx.x == 0) *pick_item(it.mean, i) = mu;
}

constexpr int kDqcThreads = 1024;

// Grouped second level, second launch: one wave per group of 256 blocks,
// lane l taking blocks 4l .. 4l + 3 (one 16-byte load), the group max |a_b -
// mean| by a wave reduction, then the codes of the double_quant_groups rule
// (the same operations on the same values); four codes per lane leave in one
// dword store when the code array allows it.  Wave w of the grid takes the
// global groups w, w + W, ... (W waves).
template <bool DYN>
__global__ __launch_bounds__(kDqcThreads) void dq_codes_kernel(DqItems it, int64_t total_groups) {
  __shared__ double mids[DYN ? 256 : 1];
  if (DYN) {
    for (int e = threadIdx.x; e < 255; e += kDqcThreads) mids[e] = kDynMapDev.mid[e];
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * (kDqcThreads / 64);
  for (int64_t gg = (int64_t)blockIdx.x * (kDqcThreads / 64) +
                    __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
       gg < total_groups; gg += nw) {
    int i = 0;
#pragma unroll
    for (int k = 0; k < kMaxQItems - 1; ++k) i += gg >= it.gend[k] ? 1 : 0;
    const int64_t g = gg - (i == 0 ? 0 : pick_item(it.gend, i - 1));
    const int64_t nb = pick_item(it.nb, i);
    const float* const a = pick_item(it.a, i);
    uint8_t* const q = pick_item(it.q, i);
    const float mu = *pick_item(it.mean, i);
    const int64_t b0 = g * kGroup + lane * 4;
    const bool whole = b0 + 4 <= nb;
    float v[4];
    if (whole) {
      const float4 t = *(const float4*)(a + b0);
      v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = b0 + k < nb ? a[b0 + k] : 0.0f;
    }
    float c[4], m = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      c[k] = b0 + k < nb ? v[k] - mu : 0.0f;
      m = fmaxf(m, fabsf(c[k]));
    }
    const float s = wave_max(m);
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      int qv = DYN ? kDynZeroCode : 0;
      if (s > 0.0f) {
        const float t = c[k] / s;       // correctly rounded binary32 division
        if (DYN) {
          int idx = 0;
#pragma unroll
          for (int step = 128; step >= 1; step >>= 1)
            if ((double)t > mids[idx + step - 1]) idx += step;
          qv = idx;
        } else {
          const float u = t * 127.0f;
          qv = (int)rintf(u);           // round half to even
        }
      }
      word |= ((uint32_t)qv & 0xffu) << (8 * k);
    }
    if (whole && ((uintptr_t)q & 3u) == 0) {
      *(uint32_t*)(q + b0) = word;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (b0 + k < nb) q[b0 + k] = (uint8_t)(word >> (8 * k));
    }
    if (lane == 0) pick_item(it.s, i)[g] = s;
  }
}

int grid_for(int64_t work_items, int per_block, int cap) {
  int64_t g = (work_items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (int)g;
}

int quantize_grid(int64_t n) {
  const int64_t ntiles = (n + kTile - 1) / kTile;
  return grid_for(ntiles, kQWaves * kUnroll, kMaxQGrid);
}

hipError_t launch_single(const QuantJob& j, unsigned long long* slots, int dq, int quant_type,
                         hipStream_t stream) {
  const int grid = quantize_grid(j.n);
  const EncodeTable& et = encode_table(quant_type);
  const bool fp4 = quant_type == kQuantFP4;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kQThreads), 0, stream, j.w, j.packed,
                       j.absmax_f32, slots, j.n, et);
  };
  if (dq == kDqNone) {
    if (fp4) go(quantize_kernel<false, true>);
    else go(quantize_kernel<false, false>);
    return hipGetLastError();
  }
  if (fp4) go(quantize_kernel<true, true>);
  else go(quantize_kernel<true, false>);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nb = (j.n + kBlock - 1) / kBlock;
  const int64_t ng = (nb + kGroup - 1) / kGroup;
  const int64_t wgs = (ng + kDqGroups - 1) / kDqGroups;
  if (wgs > 0x7fffffff) return hipErrorInvalidValue;
  if (dq == kDqDynamic)
    hipLaunchKernelGGL(double_quant_kernel<true>, dim3((unsigned)wgs), dim3(256), 0, stream,
                       j.absmax_f32, slots, grid, nb, j.q, j.absmax2, j.mean);
  else
    hipLaunchKernelGGL(double_quant_kernel<false>, dim3((unsigned)wgs), dim3(256), 0, stream,
                       j.absmax_f32, slots, grid, nb, j.q, j.absmax2, j.mean);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const QuantJob* jobs, int count, unsigned long long* slots, int dq,
                           int quant_type, hipStream_t stream) {
  if (count < 1 || count > kMaxQItems) return hipErrorInvalidValue;
  if (count == 1) return launch_single(jobs[0], slots, dq, quant_type, stream);
  int64_t total = 0;
  for (int i = 0; i < count; ++i) total += jobs[i].n;
  const int grid = quantize_grid(total);
  const int64_t nwaves = (int64_t)grid * kQWaves;
  QuantItems it{};
  it.count = count;
  int64_t pairs = 0;   // tile pairs of the tensors before i
  for (int i = 0; i < count; ++i) {
    it.n[i] = jobs[i].n;
    it.rot[i] = pairs % nwaves;
    it.w[i] = jobs[i].w;
    it.packed[i] = jobs[i].packed;
    it.absmax[i] = jobs[i].absmax_f32;
    pairs += (jobs[i].n / kTile + kUnroll - 1) / kUnroll;
  }
  const EncodeTable& et = encode_table(quant_type);
  const bool fp4 = quant_type == kQuantFP4;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kQThreads), 0, stream, it, slots, et);
  };
  if (dq == kDqNone) {
    if (fp4) go(quantize_group_kernel<false, true>);
    else go(quantize_group_kernel<false, false>);
    return hipGetLastError();
  }
  if (fp4) go(quantize_group_kernel<true, true>);
  else go(quantize_group_kernel<true, false>);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  DqItems dqi{};
  dqi.count = count;
  int64_t groups = 0;
  for (int i = 0; i < kMaxQItems; ++i) {
    if (i < count) {
      const int64_t nb = (jobs[i].n + kBlock - 1) / kBlock;
      groups += (nb + kGroup - 1) / kGroup;
      dqi.gend[i] = groups;
      dqi.nb[i] = nb;
      dqi.a[i] = jobs[i].absmax_f32;
      dqi.q[i] = jobs[i].q;
      dqi.s[i] = jobs[i].absmax2;
      dqi.mean[i] = jobs[i].mean;
    } else {
      dqi.gend[i] = INT64_MAX;
    }
  }
  hipLaunchKernelGGL(dq_mean_kernel, dim3(count), dim3(256), 0, stream, dqi, slots, grid);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t per_wg = kDqcThreads / 64;
  int64_t cgrid = (groups + per_wg - 1) / per_wg;
  cgrid = cgrid < 1024 ? cgrid : 1024;
  if (dq == kDqDynamic)
    hipLaunchKernelGGL(dq_codes_kernel<true>, dim3((unsigned)cgrid), dim3(kDqcThreads), 0, stream,
                       dqi, groups);
  else
    hipLaunchKernelGGL(dq_codes_kernel<false>, dim3((unsigned)cgrid), dim3(kDqcThreads), 0,
                       stream, dqi, groups);
  return hipGetLastError();
}

}  // namespace bnbx

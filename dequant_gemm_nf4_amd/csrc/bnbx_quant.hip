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
#include <float.h>

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

// Code of one normalised value x in [-1, 1] (or +-inf / NaN when the block
// reciprocal overflowed, handled by the caller).  NF4 codes are level
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
                                            uint32_t lanebase, uint32_t cmin, uint32_t cmax,
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
  const float r = (amax == 0.0f) ? 0.0f : 1.0f / amax;
  uint32_t word = 0;
  if (__builtin_expect(r <= FLT_MAX, 1)) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float x0 = bf16lo_to_f32(d[k]) * r;   // even element -> high nibble
      const float x1 = bf16hi_to_f32(d[k]) * r;
      const uint32_t c0 = encode_one<FP4>(x0, tab, lanebase);
      const uint32_t c1 = encode_one<FP4>(x1, tab, lanebase);
      word |= ((c0 << 4) | c1) << (8 * k);
    }
  } else {
    // Reciprocal overflowed (absmax below 2^-128): x is +inf, -inf or NaN,
    // which are at or above every threshold (+inf: the highest level) or
    // none (the lowest level).
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float x0 = bf16lo_to_f32(d[k]) * r;
      const float x1 = bf16hi_to_f32(d[k]) * r;
      const uint32_t c0 = x0 > 1.0f ? cmax : cmin, c1 = x1 > 1.0f ? cmax : cmin;
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

template <bool DQ, bool FP4>
__global__ __launch_bounds__(kQThreads, 2) void quantize_kernel(
    const uint16_t* __restrict__ w, uint8_t* __restrict__ packed, float* __restrict__ absmax,
    unsigned long long* __restrict__ slots, int64_t n, EncodeTable et) {
  __shared__ __attribute__((aligned(16))) unsigned char tab[kBuckets * kTabStride];
  __shared__ uint32_t lhist[kHistBins];
  __shared__ unsigned long long ldig[kSumDigits];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t full = n / kTile;                       // whole 512-weight tiles
  const int64_t gw = (int64_t)blockIdx.x * kQWaves + (tid >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kQWaves;

  // Replicated bucket table in LDS (entry (b, copy) at b*256 + copy*8).
  for (int e = tid; e < kBuckets * 32; e += kQThreads) {
    uint2 t;
    t.x = __float_as_uint(et.thr[e >> 5]);
    t.y = et.base[e >> 5];
    *(uint2*)(tab + (e >> 5) * kTabStride + (e & 31) * 8) = t;
  }
  if (DQ) {
    for (int e = tid; e < (int)kHistBins; e += kQThreads) lhist[e] = 0;
    if (tid < kSumDigits) ldig[tid] = 0ull;
  }
  __syncthreads();
  const uint32_t lanebase = (uint32_t)(lane & 31) << 3;

  // Each round a wave loads kUnroll whole tiles (addresses clamped, so no
  // per-lane branches), then encodes them; only the stores are skipped for
  // tiles past the end.  Latency is hidden by the many resident waves.
  for (int64_t t0 = gw * kUnroll; t0 < full; t0 += nwaves * kUnroll) {
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
      const uint32_t word = encode8<FP4>(d, tab, lanebase, et.code_min, et.code_max, m, amax);
      if (t0 + u < full) {   // wave-uniform
        const int64_t e = (t0 + u) * kTile + lane * 8;
        *(uint32_t*)(packed + (e >> 1)) = word;
        record_block(lane, e, m, amax, absmax, lhist, DQ);
      }
    }
  }

  // The ragged last tile (fewer than 512 weights) goes to the last wave.
  if (n % kTile != 0 && gw == nwaves - 1) {
    const int64_t e = full * kTile + lane * 8;
    uint16_t h[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) h[k] = (e + k < n) ? w[e + k] : (uint16_t)0;
    const uint32_t d[4] = {h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
                           h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16)};
    uint32_t m;
    float amax;
    const uint32_t word = encode8<FP4>(d, tab, lanebase, et.code_min, et.code_max, m, amax);
    if (e < n) {
      const int nbytes = (int)((n - e) < 8 ? (n - e) >> 1 : 4);
      for (int k = 0; k < nbytes; ++k) packed[(e >> 1) + k] = (uint8_t)(word >> (8 * k));
      record_block(lane, e, m, amax, absmax, lhist, DQ);
    }
  }

  if (DQ) {
    // The workgroup's partial sum I_w = sum_e lhist[e] * 2^(max(e,1)-1) (see
    // exact_mean) in base-2^32 digits: a bin (below 2^32) shifted by less
    // than 32 spans two digits.  Every workgroup writes its whole slot.
    __syncthreads();
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
    __syncthreads();
    if (tid < kSumDigits) slots[(int64_t)blockIdx.x * kSumDigits + tid] = ldig[tid];
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
    uint32_t dig[10];
    unsigned long long carry = 0;
    for (int j = 0; j < 10; ++j) {
      const unsigned long long t = digits[j] + carry;
      dig[j] = (uint32_t)t;
      carry = t >> 32;
    }
    int hj = 9;
    while (hj >= 0 && dig[hj] == 0) --hj;
    if (hj >= 0) {
      const int lz = __clz(dig[hj]);
      const unsigned long long whi = ((unsigned long long)dig[hj] << 32) | (hj >= 1 ? dig[hj - 1] : 0u);
      const uint32_t wlo = hj >= 2 ? dig[hj - 2] : 0u;
      bool sticky = false;
      for (int j = 0; j < hj - 2; ++j) sticky |= dig[j] != 0u;
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

__global__ __launch_bounds__(256) void double_quant_kernel(
    const float* __restrict__ a, const unsigned long long* __restrict__ slots, int nslots,
    int64_t nb, int8_t* __restrict__ q, float* __restrict__ s_out, float* __restrict__ mean_out) {
  __shared__ unsigned long long digits[kSumDigits];
  __shared__ float red[kDqGroups][4];
  const int tid = threadIdx.x;
  const int64_t g0 = (int64_t)blockIdx.x * kDqGroups;
  float v[kDqGroups];
#pragma unroll
  for (int i = 0; i < kDqGroups; ++i) {
    const int64_t b = (g0 + i) * kGroup + tid;
    v[i] = b < nb ? a[b] : 0.0f;
  }
  const float mu = exact_mean(slots, nslots, nb, digits);
  if (blockIdx.x == 0 && tid == 0) *mean_out = mu;
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
    int qv = 0;
    if (s > 0.0f) {
      const float t = c[i] / s;       // correctly rounded binary32 division
      const float u = t * 127.0f;
      qv = (int)rintf(u);             // round half to even
    }
    if (b < nb) q[b] = (int8_t)qv;
    if (tid == 0) s_out[g] = s;
  }
}

int grid_for(int64_t work_items, int per_block, int cap) {
  int64_t g = (work_items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (int)g;
}

}  // namespace

int quantize_grid(int64_t n) {
  const int64_t ntiles = (n + kTile - 1) / kTile;
  return grid_for(ntiles, kQWaves * kUnroll, kMaxQGrid);
}

hipError_t launch_quantize(const uint16_t* w, uint8_t* packed, int64_t n, float* absmax_f32,
                           unsigned long long* slots, int quant_type, hipStream_t stream) {
  const int grid = quantize_grid(n);
  const EncodeTable& et = encode_table(quant_type);
  const bool dq = slots != nullptr;
  if (quant_type == kQuantFP4) {
    if (dq)
      hipLaunchKernelGGL((quantize_kernel<true, true>), dim3(grid), dim3(kQThreads), 0, stream, w,
                         packed, absmax_f32, slots, n, et);
    else
      hipLaunchKernelGGL((quantize_kernel<false, true>), dim3(grid), dim3(kQThreads), 0, stream, w,
                         packed, absmax_f32, slots, n, et);
  } else {
    if (dq)
      hipLaunchKernelGGL((quantize_kernel<true, false>), dim3(grid), dim3(kQThreads), 0, stream, w,
                         packed, absmax_f32, slots, n, et);
    else
      hipLaunchKernelGGL((quantize_kernel<false, false>), dim3(grid), dim3(kQThreads), 0, stream,
                         w, packed, absmax_f32, slots, n, et);
  }
  return hipGetLastError();
}

hipError_t launch_double_quant(const float* absmax_f32, const unsigned long long* slots,
                               int nslots, int64_t nb, int8_t* q, float* absmax2, float* mean,
                               hipStream_t stream) {
  const int64_t ng = (nb + kGroup - 1) / kGroup;
  const int64_t grid = (ng + kDqGroups - 1) / kDqGroups;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(double_quant_kernel, dim3((unsigned)grid), dim3(256), 0, stream, absmax_f32,
                     slots, nslots, nb, q, absmax2, mean);
  return hipGetLastError();
}

}  // namespace bnbx

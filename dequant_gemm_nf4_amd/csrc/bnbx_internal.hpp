// Internal declarations shared by the host entry points and the kernel
// translation units of libbnbx.  Not part of the public ABI (include/bnbx.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bnbx {

constexpr int kBlock = 64;    // weights per first-level block
constexpr int kGroup = 256;   // first-level scales per second-level group
constexpr int kBuckets = 33;  // encode buckets: round(16 x + 16), x in [-1, 1]

// The two 4-bit quant types (mlqm.cn bitsandbytes article, sec. 4: nf4 or
// fp4); values of bnbx_nf4_state.quant_type.
constexpr int kQuantNF4 = 0;
constexpr int kQuantFP4 = 1;

// Host-computed tables derived from a quant type's 16 levels (mlqm.cn
// bitsandbytes article, sec. 3.2).  Passed to kernels by value.
struct EncodeTable {
  // Bucket b holds the values x with round-half-even(16 x + 16) == b.  At most
  // one decision threshold falls in a bucket (the thresholds are more than
  // 1/16 apart).  NF4 (codes in level order): code(x) = base[b] + (x >=
  // thr[b]).  FP4: base[b] holds the codes below and above the bucket's
  // threshold in bits 0-3 and 4-7, and code(x) is the field (x >= thr[b])
  // selects.  thr is +inf when the bucket holds no threshold.
  float thr[kBuckets];
  uint32_t base[kBuckets];
  uint32_t code_min, code_max;   // codes of the lowest and highest level
};

struct LevelTable {
  float level[16];       // level of each code, binary32 (NF4: ascending)
};

// The one-time host tables (built on first use, immutable afterwards).
const float* levels_f32(int quant_type);   // float[16], by code
const EncodeTable& encode_table(int quant_type);
const LevelTable& level_table(int quant_type);

// Workspace layout of the double-quant quantize: one slot per quantize
// workgroup (at most kMaxQGrid) holding that workgroup's exact partial sum of
// its block absmax values as kSumDigits base-2^32 digits (each slot is fully
// overwritten by every call, so nothing needs clearing), then the fp32
// absmax of every block.
constexpr int kMaxQGrid = 512;
constexpr int kSumDigits = 10;
constexpr size_t kHistBins = 256;   // binary exponent fields of a bf16 absmax
constexpr size_t kSlotBytes = (size_t)kMaxQGrid * kSumDigits * sizeof(unsigned long long);
inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline size_t dq_workspace_bytes(int64_t nb) {
  return round_up(kSlotBytes, 256) + round_up((size_t)nb * sizeof(float), 256);
}

// ---- kernel launchers (return hipError_t of the launch) ----
// quantize_grid(n) workgroups write slots [0, quantize_grid(n)) when
// `slots` is given (double quant); double_quant reads as many.
int quantize_grid(int64_t n);
hipError_t launch_quantize(const uint16_t* w, uint8_t* packed, int64_t n, float* absmax_f32,
                           unsigned long long* slots, int quant_type, hipStream_t stream);
hipError_t launch_double_quant(const float* absmax_f32, const unsigned long long* slots,
                               int nslots, int64_t nb, int8_t* q, float* absmax2, float* mean,
                               hipStream_t stream);
// `f16`: the 16-bit compute type is IEEE binary16 instead of bfloat16.
hipError_t launch_dequantize(const uint8_t* packed, int64_t n, const void* absmax,
                             const float* absmax2, const float* mean, int double_quant,
                             int quant_type, bool f16, uint16_t* out, hipStream_t stream);
// Returns hipErrorNotSupported if no GEMV variant covers (M, K).
hipError_t launch_gemv(const uint16_t* x, int64_t ldx, const uint8_t* packed, const void* absmax,
                       const float* absmax2, const float* mean, int double_quant, int quant_type,
                       bool f16, int M, int N, int K, uint16_t* y, int64_t ldy,
                       hipStream_t stream);
hipError_t launch_gemm(const uint16_t* x, int64_t ldx, const uint8_t* packed, const void* absmax,
                       const float* absmax2, const float* mean, int double_quant, int quant_type,
                       bool f16, int M, int N, int K, uint16_t* y, int64_t ldy,
                       hipStream_t stream);
// Y = X . W_hat^T + XA . B^T (XA [M, r], B [N, r], r % 16 == 0).
hipError_t launch_gemm_lora(const uint16_t* x, int64_t ldx, const uint8_t* packed,
                            const void* absmax, const float* absmax2, const float* mean,
                            int double_quant, int quant_type, bool f16, int M, int N, int K,
                            const uint16_t* xa, int64_t ldxa, const uint16_t* lora_b,
                            int64_t ldb, int r, uint16_t* y, int64_t ldy, hipStream_t stream);
// dX[M, K] = dY[M, N] . W_hat[N, K]; hipErrorNotSupported unless N % 64 == 0
// and the offsets fit 32 bits.
hipError_t launch_gemm_dx(const uint16_t* dy, int64_t lddy, const uint8_t* packed,
                          const void* absmax, const float* absmax2, const float* mean,
                          int double_quant, int quant_type, bool f16, int M, int N, int K,
                          uint16_t* dx, int64_t lddx, hipStream_t stream);

}  // namespace bnbx

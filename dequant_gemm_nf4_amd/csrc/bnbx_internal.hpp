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
};

struct LevelTable {
  float level[16];       // level of each code, binary32 (NF4: ascending)
};

// Second-level code maps (bnbx_nf4_state.double_quant): linear int8 codes,
// or byte codes into the dynamic 8-bit map.
constexpr int kDqNone = 0;
constexpr int kDqLinear = 1;
constexpr int kDqDynamic = 2;

// The dynamic 8-bit map.  The csdn.net bitsandbytes feature page (sec. 1,
// item 5) lists dynamic 8-bit quantization among the library's types and
// the mlqm.cn article (sec. 3.3) quantizes the fp32 block scales a second
// time; no page defines the map.  It is read as dynamic tree quantization
// (Dettmers, 8-bit approximations for parallelism in deep learning, 2016):
// after the sign bit, E zero bits give the decimal exponent 10^-E, a one
// bit ends them, and the remaining 6 - E bits f pick one of 2^(6-E) equal
// bins of [0.1, 1], valued at its midpoint: |v| = 10^-E (0.1 + 0.9 (f +
// 1/2) / 2^(6-E)), E = 0..6; with 0 and 1 that makes 256 values.  Each is
// formed in binary64 and rounded once to binary32.  In ascending order the
// code of a value is its index: 0..126 negative, 127 zero, 128..254
// positive, 255 one.  The decades are disjoint, so the positive values
// ascend with the decade (E from 6 down to 0) and then with f.
//
// mid[i] is the midpoint of v[i] and v[i+1], exact in binary64 (neighbours
// are within a factor of 10 of each other, or one of them is 0).  The code
// of a binary32 t is #{i : t > mid[i]}: the nearest value, an exact tie
// going to the lower code.
struct DynMap {
  float v[256];
  double mid[255];
};
constexpr DynMap make_dyn_map() {
  // 10^-E as the binary64 nearest each power (decimal literals round once)
  const double p10[7] = {1.0, 0.1, 0.01, 0.001, 1e-4, 1e-5, 1e-6};
  DynMap m{};
  int i = 128;
  for (int e = 6; e >= 0; --e) {
    const int nf = 1 << (6 - e);
    for (int f = 0; f < nf; ++f) {
      const double mag = p10[e] * (0.1 + 0.9 * (f + 0.5) / nf);
      m.v[i] = (float)mag;
      m.v[254 - i] = -(float)mag;
      ++i;
    }
  }
  m.v[127] = 0.0f;
  m.v[255] = 1.0f;
  for (int k = 0; k < 255; ++k) m.mid[k] = ((double)m.v[k] + (double)m.v[k + 1]) / 2.0;
  return m;
}
constexpr int kDynZeroCode = 127;
// The device copy (constant memory, one per translation unit).
static __constant__ DynMap kDynMapDev = make_dyn_map();

// The one-time host tables (built on first use, immutable afterwards).
const float* levels_f32(int quant_type);   // float[16], by code
const EncodeTable& encode_table(int quant_type);
const LevelTable& level_table(int quant_type);

// Workspace layout of the double-quant quantize, for a call on `count`
// tensors: per tensor, one slot per quantize workgroup (at most kMaxQGrid)
// holding that workgroup's exact partial sum of the tensor's block absmax
// values as kSumDigits base-2^32 digits (every slot is fully overwritten by
// every call, so nothing needs clearing); then the fp32 absmax of every
// block of each tensor, each tensor's array 256-byte aligned.
constexpr int kMaxQGrid = 512;
constexpr int kMaxQItems = 8;   // tensors per grouped quantize call
constexpr int kSumDigits = 10;
constexpr size_t kHistBins = 256;   // binary exponent fields of a bf16 absmax
constexpr size_t kSlotBytes = (size_t)kMaxQGrid * kSumDigits * sizeof(unsigned long long);
constexpr size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
constexpr size_t dq_slot_bytes(int count) { return round_up((size_t)count * kSlotBytes, 256); }
constexpr size_t dq_absmax_bytes(int64_t nb) { return round_up((size_t)nb * sizeof(float), 256); }
constexpr size_t dq_workspace_bytes(int64_t nb) { return dq_slot_bytes(1) + dq_absmax_bytes(nb); }

// ---- kernel launchers (return hipError_t of the launch) ----
// One tensor of a (grouped) quantize call.
struct QuantJob {
  const uint16_t* w;    // bf16[n]
  uint8_t* packed;      // uint8[n / 2]
  int64_t n;
  float* absmax_f32;    // fp32 block absmax: the state's absmax without double
                        // quant, the tensor's workspace array with it
  uint8_t* q;           // double quant: code bytes (the state's absmax),
  float* absmax2;       //   group scales
  float* mean;          //   and the mean
};
// Quantizes `count` (1..kMaxQItems) tensors of one quant type in one launch;
// with double quant (dq = kDqLinear or kDqDynamic; `slots` the workspace's
// slot region, dq_slot_bytes(count) bytes) a second launch forms every
// tensor's mean, group scales and codes.
hipError_t launch_quantize(const QuantJob* jobs, int count, unsigned long long* slots, int dq,
                           int quant_type, hipStream_t stream);
// `f16`: the 16-bit compute type is IEEE binary16 instead of bfloat16.
hipError_t launch_dequantize(const uint8_t* packed, int64_t n, const void* absmax,
                             const float* absmax2, const float* mean, int double_quant,
                             int quant_type, bool f16, uint16_t* out, hipStream_t stream);
// Returns hipErrorNotSupported if no GEMV variant covers (M, K).
hipError_t launch_gemv(const uint16_t* x, int64_t ldx, const uint8_t* packed, const void* absmax,
                       const float* absmax2, const float* mean, int double_quant, int quant_type,
                       bool f16, int M, int N, int K, uint16_t* y, int64_t ldy,
                       hipStream_t stream);
// One weight of a grouped GEMV (device pointers; Y row m at y + m * ldy).
struct GemvItem {
  const uint8_t* packed;
  const void* absmax;
  const float* absmax2;
  const float* mean;
  int N;
  uint16_t* y;
  int64_t ldy;
};
// Up to four weights with the same K, quant type, compute type and second
// level that multiply the same X.
hipError_t launch_gemv_grouped(const uint16_t* x, int64_t ldx, const GemvItem* items, int count,
                               int double_quant, int quant_type, bool f16, int M, int K,
                               hipStream_t stream);
// 4 < M <= 16 rows of X over one slab of rows, one launch of `grid`
// workgroups (bnbx_gemv16.hip).
hipError_t launch_gemv16_batch(int grid, const uint16_t* x, int64_t ldx, const uint8_t* packed,
                               const void* absmax, const float* absmax2, const float* mean,
                               int dq, bool f16, int M, int N, int K, uint16_t* y, int64_t ldy,
                               const LevelTable& lv, hipStream_t stream);
// The same with a LoRA term, Y += XA . B^T (XA [M, r], B [N, r], r a multiple
// of 16 up to 256).
hipError_t launch_gemv16_lora_batch(int grid, const uint16_t* x, int64_t ldx,
                                    const uint8_t* packed, const void* absmax,
                                    const float* absmax2, const float* mean, int dq, bool f16,
                                    int M, int N, int K, const uint16_t* xa, int64_t ldxa,
                                    const uint16_t* lora_b, int64_t ldb, int r, uint16_t* y,
                                    int64_t ldy, const LevelTable& lv, hipStream_t stream);
// Workspace of the GEMM's split-K path for (M, N, K) on the current device
// (fp32 partial tiles; 0 when the tiles already fill the GPU).
size_t gemm_workspace_bytes(int M, int N, int K);
// Splits K when the workspace holds gemm_workspace_bytes(M, N, K) bytes
// (16-byte aligned); otherwise runs the tiles whole.
hipError_t launch_gemm(const uint16_t* x, int64_t ldx, const uint8_t* packed, const void* absmax,
                       const float* absmax2, const float* mean, int double_quant, int quant_type,
                       bool f16, int M, int N, int K, uint16_t* y, int64_t ldy, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);
// Y = X . W_hat^T + XA . B^T (XA [M, r], B [N, r], r % 16 == 0).
// Y = X . W_hat^T + XA . B^T for 1 <= M <= 16 (the decode GEMVs with the
// low-rank term added before their reductions; bnbx_gemv_lora.hip).
hipError_t launch_gemv_lora(const uint16_t* x, int64_t ldx, const uint8_t* packed,
                            const void* absmax, const float* absmax2, const float* mean,
                            int double_quant, int quant_type, bool f16, int M, int N, int K,
                            const uint16_t* xa, int64_t ldxa, const uint16_t* lora_b, int64_t ldb,
                            int r, uint16_t* y, int64_t ldy, hipStream_t stream);
hipError_t launch_gemm_lora(const uint16_t* x, int64_t ldx, const uint8_t* packed,
                            const void* absmax, const float* absmax2, const float* mean,
                            int double_quant, int quant_type, bool f16, int M, int N, int K,
                            const uint16_t* xa, int64_t ldxa, const uint16_t* lora_b,
                            int64_t ldb, int r, uint16_t* y, int64_t ldy, hipStream_t stream);
// XA[M, r] = rnd(fl32(s * X . A^T)), A [r, K], 16 <= r <= 256, r % 16 == 0,
// K % 32 == 0.
hipError_t launch_lora_down(const uint16_t* x, int64_t ldx, const uint16_t* a, int64_t lda,
                            int M, int K, int r, float scale, bool f16, uint16_t* xa,
                            int64_t ldxa, hipStream_t stream);
// dX[M, K] = dY[M, N] . W_hat[N, K]; hipErrorNotSupported unless N % 64 == 0
// and the offsets fit 32 bits.
hipError_t launch_gemm_dx(const uint16_t* dy, int64_t lddy, const uint8_t* packed,
                          const void* absmax, const float* absmax2, const float* mean,
                          int double_quant, int quant_type, bool f16, int M, int N, int K,
                          uint16_t* dx, int64_t lddx, hipStream_t stream);

}  // namespace bnbx

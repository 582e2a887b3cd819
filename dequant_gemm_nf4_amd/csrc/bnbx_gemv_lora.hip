// Decode form of the 4-bit linear layer with a LoRA term, at most 16 rows
// of X: Y = X . W_hat^T + XA . B^T (the pomoai.com overview, QLoRA: low-rank
// adapters beside the frozen 4-bit base; mlqm.cn bitsandbytes article,
// sec. 3.4: 4-bit storage, 16-bit compute).  Up to 4 rows, gemv_kernel with
// its LORA flag streams the packed weight once, as for the plain layer, and
// each lane slot adds its ranks of XA . B^T to a row's partial sums before
// the wave reduction; from 5 to 16 rows gemv16_kernel with its LORA flag
// adds one MFMA of 32 ranks per wave and row group before the reduction
// over waves.  Either way Y is rounded once.
#include "bnbx_gemv_common.hpp"

namespace bnbx {

hipError_t launch_gemv_lora(const uint16_t* x, int64_t ldx, const uint8_t* packed,
                            const void* absmax, const float* absmax2, const float* mean,
                            int double_quant, int quant_type, bool f16, int M, int N, int K,
                            const uint16_t* xa, int64_t ldxa, const uint16_t* lora_b, int64_t ldb,
                            int r, uint16_t* y, int64_t ldy, hipStream_t stream) {
  if (M < 1 || M > 16) return hipErrorNotSupported;
  const int64_t rowK2 = K >> 1, nkb = K >> 6;
  const LevelTable& lv = level_table(quant_type);
  // Slabs of rows keep every byte offset of a launch below 2^31 (whole
  // 256-row multiples, so the slabs' double-quant groups stay whole).
  int64_t slab = ((int64_t)1 << 30) / rowK2;
  slab -= slab % 256;
  if (slab < 256) return hipErrorNotSupported;
  // XA and each slab's rows of B are addressed by 32-bit offsets too
  const int64_t slab_rows = N < slab ? N : slab;
  if ((int64_t)(M - 1) * ldxa * 2 + (int64_t)r * 2 >= ((int64_t)1 << 31) ||
      (slab_rows - 1) * ldb * 2 + (int64_t)r * 2 >= ((int64_t)1 << 31))
    return hipErrorNotSupported;
  // 4 < M <= 16: the batched kernel, each wave adding a 32-rank chunk of the
  // term by one more MFMA per row group before the reduction over waves.
  if (M > 4) {
    if (15 * ldx * 2 + (int64_t)K * 2 >= ((int64_t)1 << 31)) return hipErrorNotSupported;
    for (int64_t r0 = 0; r0 < N; r0 += slab) {
      const int n = (int)(N - r0 < slab ? N - r0 : slab);
      const int ngroups = (n + 15) / 16;
      const int grid = ngroups < cu_count() ? ngroups : cu_count();
      const void* am = double_quant ? (const void*)((const int8_t*)absmax + r0 * nkb)
                                    : (const void*)((const float*)absmax + r0 * nkb);
      const float* am2 = double_quant ? absmax2 + (r0 * nkb) / 256 : absmax2;
      const hipError_t e = launch_gemv16_lora_batch(
          grid, x, ldx, packed + r0 * rowK2, am, am2, mean, double_quant, f16, M, n, K, xa, ldxa,
          lora_b + r0 * ldb, ldb, r, y + r0, ldy, lv, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const bool rowq = nkb <= 256 && nkb % 4 == 0 && ((uintptr_t)absmax & 3u) == 0;
  const int nicap = double_quant == kDqDynamic && !rowq ? 3 : 4;
  Plan p;
  if (next_x_group(M, N < slab ? N : (int)slab, K, nicap, p, true) < M)
    return hipErrorNotSupported;
  for (int64_t r0 = 0; r0 < N; r0 += slab) {
    const int n = (int)(N - r0 < slab ? N - r0 : slab);
    if (!make_plan(p.mm, n, K, p, nicap, true)) return hipErrorNotSupported;
    // at most kLoraMaxRR rows per team (the adapter's values take registers);
    // rows past one pass are taken by further passes of the same launch, in
    // 16-wave workgroups
    if (p.rr > kLoraMaxRR) {
      p.wv = kWaves;
      p.xlds = (int64_t)p.mm * K * 2 <= kXBytes ? 1 : 0;
      const int tpw = kWaves >> p.twl;
      p.rr = kLoraMaxRR;
      const int64_t g = ((int64_t)n + tpw * p.rr - 1) / (tpw * p.rr);
      p.grid = (int)(g < cu_count() ? g : cu_count());
    }
    GemvOneLora it;
    it.packed = packed + r0 * rowK2;
    it.absmax = double_quant ? (const void*)((const int8_t*)absmax + r0 * nkb)
                             : (const void*)((const float*)absmax + r0 * nkb);
    it.absmax2 = double_quant ? absmax2 + (r0 * nkb) / 256 : absmax2;
    it.mean = mean;
    it.y = y + r0;
    it.ldy = ldy;
    it.xa = xa;
    it.ldxa = ldxa;
    it.lb = lora_b + r0 * ldb;
    it.ldb = ldb;
    it.r = r;
    const hipError_t e = dispatch<false, true>(p, x, ldx, it, 1, double_quant, rowq, M, n, K, lv,
                                               f16, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bnbx

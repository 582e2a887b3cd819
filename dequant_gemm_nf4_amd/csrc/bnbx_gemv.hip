// Decode GEMV entry (bnbx_gemv_nf4): M <= 4 rows of X per launch of
// gemv_kernel (bnbx_gemv_common.hpp), 4 < M <= 16 in one launch of the
// batched kernel (bnbx_gemv16.hip).  mlqm.cn bitsandbytes article, sec. 3.4.
#include "bnbx_gemv_common.hpp"

namespace bnbx {

hipError_t launch_gemv(const uint16_t* x, int64_t ldx, const uint8_t* packed, const void* absmax,
                       const float* absmax2, const float* mean, int double_quant, int quant_type,
                       bool f16, int M, int N, int K, uint16_t* y, int64_t ldy,
                       hipStream_t stream) {
  const int64_t rowK2 = K >> 1, nkb = K >> 6;
  const LevelTable& lv = level_table(quant_type);
  // Slabs of rows keep every byte offset of a launch below 2^31 (whole
  // 256-row multiples, so the slabs' double-quant groups stay whole).
  int64_t slab = ((int64_t)1 << 30) / rowK2;
  slab -= slab % 256;
  if (slab < 256) return hipErrorNotSupported;
  // 4 < M <= 16: one launch per slab streams the weights once.
  if (M > 4) {
    if (15 * ldx * 2 + (int64_t)K * 2 >= ((int64_t)1 << 31)) return hipErrorNotSupported;
    for (int64_t r0 = 0; r0 < N; r0 += slab) {
      const int n = (int)(N - r0 < slab ? N - r0 : slab);
      const int ngroups = (n + 15) / 16;
      const int grid = ngroups < cu_count() ? ngroups : cu_count();
      const void* am = double_quant ? (const void*)((const int8_t*)absmax + r0 * nkb)
                                    : (const void*)((const float*)absmax + r0 * nkb);
      const float* am2 = double_quant ? absmax2 + (r0 * nkb) / 256 : absmax2;
      const hipError_t e = launch_gemv16_batch(grid, x, ldx, packed + r0 * rowK2, am, am2, mean,
                                               double_quant, f16, M, n, K, y + r0, ldy, lv,
                                               stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  // Rows of X in groups of up to four (each group streams W once); a group
  // of three runs the four-row kernel with its last row empty.  Long rows
  // take smaller groups (the X slice must fit the registers).
  const bool rowq = nkb <= 256 && nkb % 4 == 0 && ((uintptr_t)absmax & 3u) == 0;
  const int nicap = double_quant == kDqDynamic && !rowq ? 3 : 4;
  for (int m0 = 0; m0 < M;) {
    Plan p;
    const int mv = next_x_group(M - m0, N < slab ? N : (int)slab, K, nicap, p);
    if (mv == 0) return hipErrorNotSupported;
    for (int64_t r0 = 0; r0 < N; r0 += slab) {
      const int n = (int)(N - r0 < slab ? N - r0 : slab);
      if (!make_plan(p.mm, n, K, p, nicap, true)) return hipErrorNotSupported;
      GemvOne it;
      it.packed = packed + r0 * rowK2;
      it.absmax = double_quant ? (const void*)((const int8_t*)absmax + r0 * nkb)
                               : (const void*)((const float*)absmax + r0 * nkb);
      it.absmax2 = double_quant ? absmax2 + (r0 * nkb) / 256 : absmax2;
      it.mean = mean;
      it.y = y + (int64_t)m0 * ldy + r0;
      it.ldy = ldy;
      const hipError_t e = dispatch<false>(p, x + (int64_t)m0 * ldx, ldx, it, 1, double_quant,
                                           rowq, mv, n, K, lv, f16, stream);
      if (e != hipSuccess) return e;
    }
    m0 += mv;
  }
  return hipSuccess;
}

}  // namespace bnbx

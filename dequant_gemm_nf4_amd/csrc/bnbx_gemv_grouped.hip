// Grouped decode GEMV (bnbx_gemv_nf4_grouped): up to four weights that
// multiply the same X (the q, k and v projections of a layer, or gate and
// up) in one launch of gemv_kernel per group of up to four rows of X, their
// rows concatenated, so that the fixed part of a launch (argument and X
// loads, the byte-table build, the barrier, the tail) is paid once.
// mlqm.cn bitsandbytes article, sec. 3.4 and the sec. 7 pitfall (4-bit pays
// off when the layer is bound by weight traffic).
#include "bnbx_gemv_common.hpp"

namespace bnbx {
namespace {

// One grouped launch per group of up to four rows of X over `count` items
// whose `rows` rows fit one pass.
hipError_t launch_group(const uint16_t* x, int64_t ldx, const GemvItem* items, int count,
                        int double_quant, bool rowq, int nicap, const LevelTable& lv, bool f16,
                        int M, int K, int rows, hipStream_t stream) {
  GemvItems it{};
  int64_t total = 0;
  for (int w = 0; w < kMaxItems; ++w) it.end[w] = 0x7fffffff;
  for (int w = 0; w < count; ++w) {
    total += items[w].N;
    it.end[w] = (int)total;
    it.packed[w] = items[w].packed;
    it.absmax[w] = items[w].absmax;
    it.absmax2[w] = items[w].absmax2;
    it.mean[w] = items[w].mean;
    it.y[w] = items[w].y;
    it.ldy[w] = items[w].ldy;
  }
  for (int m0 = 0; m0 < M;) {
    Plan p;
    const int mv = next_x_group(M - m0, rows, K, nicap, p, true);
    if (mv == 0) return hipErrorNotSupported;
    GemvItems im = it;
    for (int w = 0; w < count; ++w) im.y[w] = it.y[w] + (int64_t)m0 * it.ldy[w];
    const hipError_t e = dispatch<true>(p, x + (int64_t)m0 * ldx, ldx, im, count, double_quant,
                                        rowq, mv, rows, K, lv, f16, stream);
    if (e != hipSuccess) return e;
    m0 += mv;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_gemv_grouped(const uint16_t* x, int64_t ldx, const GemvItem* items, int count,
                               int double_quant, int quant_type, bool f16, int M, int K,
                               hipStream_t stream) {
  if (count < 1 || count > kMaxItems) return hipErrorInvalidValue;
  const int64_t rowK2 = K >> 1, nkb = K >> 6;
  const LevelTable& lv = level_table(quant_type);
  // 4 < M <= 16: the batched kernel, one launch per weight (each streams its
  // weight once).
  if (M > 4) {
    for (int w = 0; w < count; ++w) {
      const hipError_t e = launch_gemv(x, ldx, items[w].packed, items[w].absmax,
                                       items[w].absmax2, items[w].mean, double_quant, quant_type,
                                       f16, M, items[w].N, K, items[w].y, items[w].ldy, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  bool rowq = nkb <= 256 && nkb % 4 == 0;
  for (int w = 0; w < count; ++w) {
    // every byte offset within an item must fit 31 bits
    if ((int64_t)items[w].N * rowK2 >= ((int64_t)1 << 31)) return hipErrorNotSupported;
    rowq = rowq && ((uintptr_t)items[w].absmax & 3u) == 0;
  }
  const int nicap = double_quant && !rowq ? 3 : 4;
  // Consecutive items go into one launch while their rows fit one pass of
  // at most kMaxGroupRR rows per team (for the decode shapes: q, k and v
  // together; gate and up, 11008 rows each, apart).  An item alone runs
  // the single-weight kernel.
  auto fits = [&](int64_t rows) {
    Plan p;
    if (rows >= ((int64_t)1 << 31) || next_x_group(M, (int)rows, K, nicap, p, true) == 0)
      return false;
    return p.rr <= kMaxGroupRR && rows <= (int64_t)p.grid * (p.wv >> p.twl) * p.rr;
  };
  for (int w0 = 0; w0 < count;) {
    int w1 = w0 + 1;
    int64_t rows = items[w0].N;
    while (w1 < count && fits(rows + items[w1].N)) rows += items[w1++].N;
    hipError_t e;
    if (w1 - w0 == 1) {
      e = launch_gemv(x, ldx, items[w0].packed, items[w0].absmax, items[w0].absmax2,
                      items[w0].mean, double_quant, quant_type, f16, M, items[w0].N, K,
                      items[w0].y, items[w0].ldy, stream);
    } else {
      e = launch_group(x, ldx, items + w0, w1 - w0, double_quant, rowq, nicap, lv, f16, M, K,
                       (int)rows, stream);
    }
    if (e != hipSuccess) return e;
    w0 = w1;
  }
  return hipSuccess;
}

}  // namespace bnbx

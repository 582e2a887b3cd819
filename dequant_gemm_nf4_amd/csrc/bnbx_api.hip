// C entry points of libbnbx (declared in include/bnbx.h): argument checks on
// the host, the one-time codebook and encode tables, and kernel launches.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "../../include/bnbx.h"
#include "bnbx_internal.hpp"

namespace bnbx {
namespace {

// Standard normal CDF and density in binary64 (C library erfc / exp).
double normal_cdf(double x) { return 0.5 * erfc(-x * 0.70710678118654752440); }
double normal_pdf(double x) { return exp(-0.5 * x * x) * 0.39894228040143267794; }

// Upper-half standard normal quantile by Newton's method on the CDF from 0.
// The CDF is concave on [0, inf), so from the left every Newton step stays at
// or below the root and the iterates rise monotonically to it; stop when a
// step no longer moves x up.
double normal_quantile_upper(double p) {
  double x = 0.0;
  for (int it = 0; it < 200; ++it) {
    const double nx = x - (normal_cdf(x) - p) / normal_pdf(x);
    if (!(nx > x)) break;
    x = nx;
  }
  return x;
}

struct Tables {
  float levels[16];   // level of each code
  EncodeTable enc;
  LevelTable lv;
};

// NF4 codebook (mlqm.cn bitsandbytes article, sec. 3.2: 16 levels laid out
// by the normal density, dense near 0, with exact 0 and ends at +-1): 8
// positive quantiles of probabilities evenly spaced from the offset toward
// 1/2, 7 mirrored negative ones over the same span, and 0, all divided by the
// outermost quantile.  The offset averages the 1/30 and 1/32 tail masses.
// Codes are in ascending level order.
void nf4_levels(float* levels) {
  const double off = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0);
  const double top = normal_quantile_upper(off);
  double v[16];
  int k = 0;
  for (int i = 0; i < 7; ++i) v[k++] = -normal_quantile_upper(off + i * (0.5 - off) / 7.0);
  v[k++] = 0.0;
  for (int i = 0; i < 8; ++i) v[k++] = normal_quantile_upper(off + i * (0.5 - off) / 8.0);
  std::sort(v, v + 16);
  for (int i = 0; i < 16; ++i) levels[i] = (float)(v[i] / top);   // ends: +-top/top = +-1
}

// FP4 (mlqm.cn article, sec. 4: the plain 4-bit float quant type; the pages
// give no layout, E2M1 is taken): code bit 3 is the sign, bits 2-1 the
// exponent e, bit 0 the mantissa m; magnitude m/2 for e = 0, else
// 2^(e-1) (1 + m/2), i.e. 0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0-7, divided by
// 6 so the block absmax maps to +-1.
void fp4_levels(float* levels) {
  for (int c = 0; c < 16; ++c) {
    const int e = (c >> 1) & 3, m = c & 1;
    const double mag = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    levels[c] = (float)((c & 8 ? -mag : mag) / 6.0);
  }
}

// Encode tables of a codebook.  `order` lists the codes of the distinct
// levels by ascending value (count of them in `nl`; FP4 leaves out -0, code
// 8, which the encoder never emits).  Thresholds: the smallest float strictly
// above each midpoint of neighbouring levels, so the nearest level wins and
// an exact tie takes the lower one.  Returns false if the codebook does not
// fit the bucket scheme (never for the two fixed codebooks; checked anyway,
// and reported by every call as BNBX_E_INTERNAL).
bool build_encode(const float* levels, const int* order, int nl, bool in_order, EncodeTable& enc) {
  float thr[15];
  for (int i = 0; i + 1 < nl; ++i) {
    const double mid = ((double)levels[order[i]] + (double)levels[order[i + 1]]) * 0.5;
    float th = (float)mid;
    if ((double)th <= mid) th = nextafterf(th, INFINITY);
    thr[i] = th;
  }
  // Encode buckets: bucket b holds x with round-half-even(16x + 16) == b,
  // i.e. x in [(b - 1/2)/16 - 1, (b + 1/2)/16 - 1].  Each bucket must hold at
  // most one threshold and no threshold may sit near a bucket edge (the
  // rounding of 16x + 16 moves an edge by far less than the margin checked).
  for (int b = 0; b < kBuckets; ++b) {
    const double lo = (b - 0.5) / 16.0 - 1.0, hi = (b + 0.5) / 16.0 - 1.0;
    uint32_t below = 0;
    float inside = INFINITY;
    int count = 0;
    for (int i = 0; i + 1 < nl; ++i) {
      const double th = thr[i];
      if (fabs(th - lo) < 1e-4 || fabs(th - hi) < 1e-4) return false;   // too near an edge
      if (th < lo) ++below;
      else if (th < hi) { inside = thr[i]; ++count; }
    }
    if (count > 1) return false;   // two thresholds in one bucket
    enc.thr[b] = inside;
    if (in_order) {
      enc.base[b] = below;
    } else {
      const uint32_t c0 = (uint32_t)order[below];
      const uint32_t c1 = count ? (uint32_t)order[below + 1] : c0;
      enc.base[b] = c0 | (c1 << 4);
    }
  }
  return true;
}

bool build_tables(int quant_type, Tables& t) {
  int order[16];
  int nl = 0;
  if (quant_type == kQuantNF4) {
    nf4_levels(t.levels);
    for (int c = 0; c < 16; ++c) order[nl++] = c;
  } else {
    fp4_levels(t.levels);
    for (int c = 0; c < 16; ++c)
      if (c != 8) order[nl++] = c;
    std::sort(order, order + nl, [&](int a, int b) { return t.levels[a] < t.levels[b]; });
  }
  for (int i = 0; i < 16; ++i) t.lv.level[i] = t.levels[i];
  return build_encode(t.levels, order, nl, quant_type == kQuantNF4, t.enc);
}

struct AllTables {
  Tables t[2];
  bool ok;
};

const AllTables& all_tables() {
  static AllTables a;
  static std::once_flag once;
  std::call_once(once, [] {
    const bool nf4 = build_tables(kQuantNF4, a.t[0]);
    const bool fp4 = build_tables(kQuantFP4, a.t[1]);
    a.ok = nf4 && fp4;
  });
  return a;
}

const Tables& tables(int quant_type) { return all_tables().t[quant_type == kQuantFP4 ? 1 : 0]; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int64_t nblocks(int64_t n) { return (n + kBlock - 1) / kBlock; }
int64_t ngroups(int64_t nb) { return (nb + kGroup - 1) / kGroup; }

int check_state(const bnbx_nf4_state* st) {
  if (!all_tables().ok) return BNBX_E_INTERNAL;
  if (st == nullptr) return BNBX_E_INVAL;
  if (st->n < 2 || (st->n & 1)) return BNBX_E_INVAL;
  if (st->blocksize != kBlock) return BNBX_E_UNSUPPORTED;
  if (st->double_quant != kDqNone && st->double_quant != kDqLinear &&
      st->double_quant != kDqDynamic)
    return BNBX_E_INVAL;
  if (st->quant_type != BNBX_QUANT_NF4 && st->quant_type != BNBX_QUANT_FP4) return BNBX_E_INVAL;
  if (st->compute_dtype != BNBX_DTYPE_BF16 && st->compute_dtype != BNBX_DTYPE_F16)
    return BNBX_E_INVAL;
  if (st->absmax == nullptr) return BNBX_E_INVAL;
  if (st->double_quant && (st->absmax2 == nullptr || st->absmax_mean == nullptr))
    return BNBX_E_INVAL;
  return BNBX_OK;
}

int check_matmul(const uint16_t* x, int64_t ldx, const uint8_t* packed, const bnbx_nf4_state* st,
                 int M, int N, int K, const uint16_t* y, int64_t ldy) {
  if (x == nullptr || packed == nullptr || y == nullptr) return BNBX_E_INVAL;
  const int s = check_state(st);
  if (s != BNBX_OK) return s;
  if (M < 1 || N < 1 || K < kBlock) return BNBX_E_INVAL;
  if (K % kBlock != 0) return BNBX_E_INVAL;
  if (st->n != (int64_t)N * (int64_t)K) return BNBX_E_INVAL;
  if (ldx < K || ldy < N) return BNBX_E_INVAL;
  if (ldx % 8 != 0) return BNBX_E_ALIGN;
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(y, 2)) return BNBX_E_ALIGN;
  return BNBX_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? BNBX_OK : BNBX_E_HIP; }

// The double-quant quantize with a library-owned workspace
// (bnbx_quantize_nf4_noalloc): a file-scope device array, one copy per GPU
// the library runs on, held until the process ends.  Its size is the
// workspace of BNBX_NOALLOC_MAX_WEIGHTS weights.
constexpr size_t kNoAllocScratchBytes = dq_slot_bytes(1) +
                                        (size_t)(BNBX_NOALLOC_MAX_WEIGHTS / kBlock) * sizeof(float);
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device.  In host code the array's
// name is only a stand-in for the symbol, so kernels get this address instead;
// it is looked up once per device.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// The job of one tensor: fp32 block absmax into the state (no double
// quant) or into the workspace at `a32`.
QuantJob job_of(const uint16_t* w, uint8_t* packed, const bnbx_nf4_state* st, float* a32) {
  QuantJob j;
  j.w = w;
  j.packed = packed;
  j.n = st->n;
  j.absmax_f32 = st->double_quant ? a32 : (float*)st->absmax;
  j.q = (uint8_t*)st->absmax;
  j.absmax2 = st->absmax2;
  j.mean = st->absmax_mean;
  return j;
}

// One tensor with double quant: slots, then its fp32 absmax, in the workspace.
int quantize_dq(const uint16_t* w, uint8_t* packed, const bnbx_nf4_state* st, void* workspace,
                hipStream_t hs) {
  unsigned long long* slots = (unsigned long long*)workspace;
  const QuantJob j = job_of(w, packed, st, (float*)((char*)workspace + dq_slot_bytes(1)));
  return hip_status(launch_quantize(&j, 1, slots, st->double_quant, st->quant_type, hs));
}

// The dynamic map ascends strictly, holds 0 at its zero code and 1 at the
// top, and is symmetric below the top.
constexpr bool dyn_map_ok() {
  constexpr DynMap m = make_dyn_map();
  for (int i = 0; i < 255; ++i)
    if (!(m.v[i] < m.v[i + 1]) || !(m.v[i] < m.mid[i] && m.mid[i] < m.v[i + 1])) return false;
  for (int i = 0; i < 127; ++i)
    if (m.v[i] != -m.v[254 - i]) return false;
  return m.v[kDynZeroCode] == 0.0f && m.v[255] == 1.0f;
}
static_assert(dyn_map_ok(), "dynamic 8-bit map");
static_assert(BNBX_QUANTIZE_MAX_ITEMS == kMaxQItems, "grouped quantize bound");

}  // namespace

const float* levels_f32(int quant_type) { return tables(quant_type).levels; }
const EncodeTable& encode_table(int quant_type) { return tables(quant_type).enc; }
const LevelTable& level_table(int quant_type) { return tables(quant_type).lv; }

}  // namespace bnbx

using namespace bnbx;

extern "C" {

const char* bnbx_status_str(int status) {
  switch (status) {
    case BNBX_OK: return "BNBX_OK";
    case BNBX_E_INVAL: return "BNBX_E_INVAL: invalid argument";
    case BNBX_E_ALIGN: return "BNBX_E_ALIGN: misaligned pointer or leading dimension";
    case BNBX_E_UNSUPPORTED: return "BNBX_E_UNSUPPORTED: unsupported configuration";
    case BNBX_E_WORKSPACE: return "BNBX_E_WORKSPACE: workspace missing or too small";
    case BNBX_E_HIP: return "BNBX_E_HIP: HIP runtime error at launch";
    case BNBX_E_INTERNAL: return "BNBX_E_INTERNAL: codebook tables failed their self-check";
    default: return "BNBX: unknown status";
  }
}

int bnbx_nf4_codebook(float levels_host[16]) {
  if (levels_host == nullptr) return BNBX_E_INVAL;
  if (!all_tables().ok) return BNBX_E_INTERNAL;
  const float* l = levels_f32(kQuantNF4);
  for (int i = 0; i < 16; ++i) levels_host[i] = l[i];
  return BNBX_OK;
}

int bnbx_fp4_codebook(float levels_host[16]) {
  if (levels_host == nullptr) return BNBX_E_INVAL;
  if (!all_tables().ok) return BNBX_E_INTERNAL;
  const float* l = levels_f32(kQuantFP4);
  for (int i = 0; i < 16; ++i) levels_host[i] = l[i];
  return BNBX_OK;
}

int bnbx_dynamic_map(float values_host[256]) {
  if (values_host == nullptr) return BNBX_E_INVAL;
  constexpr DynMap m = make_dyn_map();
  for (int i = 0; i < 256; ++i) values_host[i] = m.v[i];
  return BNBX_OK;
}

size_t bnbx_quantize_nf4_workspace_bytes(int64_t n, int blocksize, int double_quant) {
  if (n < 2 || (n & 1) || blocksize != kBlock) return 0;
  if (!double_quant) return 0;
  return dq_workspace_bytes(nblocks(n));
}

int bnbx_quantize_nf4(const uint16_t* w, uint8_t* packed, const bnbx_nf4_state* st,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (w == nullptr || packed == nullptr) return BNBX_E_INVAL;
  const int s = check_state(st);
  if (s != BNBX_OK) return s;
  if (!aligned(w, 16) || !aligned(packed, 16)) return BNBX_E_ALIGN;
  const int64_t n = st->n, nb = nblocks(n);
  hipStream_t hs = (hipStream_t)stream;
  if (!st->double_quant) {
    const QuantJob j = job_of(w, packed, st, nullptr);
    return hip_status(launch_quantize(&j, 1, nullptr, kDqNone, st->quant_type, hs));
  }
  const size_t need = dq_workspace_bytes(nb);
  if (workspace == nullptr || workspace_bytes < need) return BNBX_E_WORKSPACE;
  if (!aligned(workspace, 256)) return BNBX_E_ALIGN;
  return quantize_dq(w, packed, st, workspace, hs);
}

int bnbx_quantize_nf4_noalloc(const uint16_t* w, uint8_t* packed, const bnbx_nf4_state* st,
                              void* stream) {
  if (w == nullptr || packed == nullptr) return BNBX_E_INVAL;
  const int s = check_state(st);
  if (s != BNBX_OK) return s;
  if (!aligned(w, 16) || !aligned(packed, 16)) return BNBX_E_ALIGN;
  hipStream_t hs = (hipStream_t)stream;
  if (!st->double_quant) {
    const QuantJob j = job_of(w, packed, st, nullptr);
    return hip_status(launch_quantize(&j, 1, nullptr, kDqNone, st->quant_type, hs));
  }
  if (st->n > BNBX_NOALLOC_MAX_WEIGHTS) return BNBX_E_WORKSPACE;
  static_assert(kNoAllocScratchBytes >= dq_slot_bytes(1), "scratch holds the slots");
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return BNBX_E_HIP;
  if (dq_workspace_bytes((st->n + kBlock - 1) / kBlock) > kNoAllocScratchBytes) return BNBX_E_WORKSPACE;
  return quantize_dq(w, packed, st, ws, hs);
}

size_t bnbx_quantize_nf4_grouped_workspace_bytes(const int64_t* n, int count, int blocksize,
                                                 int double_quant) {
  if (n == nullptr || count < 1 || count > BNBX_QUANTIZE_MAX_ITEMS || blocksize != kBlock)
    return 0;
  size_t bytes = dq_slot_bytes(count);
  for (int i = 0; i < count; ++i) {
    if (n[i] < 2 || (n[i] & 1)) return 0;
    bytes += dq_absmax_bytes(nblocks(n[i]));
  }
  return double_quant ? bytes : 0;
}

int bnbx_quantize_nf4_grouped(const bnbx_quantize_item* items, int count, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (items == nullptr || count < 1 || count > BNBX_QUANTIZE_MAX_ITEMS) return BNBX_E_INVAL;
  const bnbx_nf4_state* s0 = items[0].st;
  int64_t ns[BNBX_QUANTIZE_MAX_ITEMS];
  for (int i = 0; i < count; ++i) {
    const bnbx_quantize_item& a = items[i];
    if (a.w == nullptr || a.packed == nullptr) return BNBX_E_INVAL;
    const int s = check_state(a.st);
    if (s != BNBX_OK) return s;
    if (!aligned(a.w, 16) || !aligned(a.packed, 16)) return BNBX_E_ALIGN;
    if (a.st->quant_type != s0->quant_type || a.st->double_quant != s0->double_quant)
      return BNBX_E_INVAL;
    ns[i] = a.st->n;
  }
  QuantJob jobs[BNBX_QUANTIZE_MAX_ITEMS];
  unsigned long long* slots = nullptr;
  if (s0->double_quant) {
    const size_t need = bnbx_quantize_nf4_grouped_workspace_bytes(ns, count, kBlock, 1);
    if (workspace == nullptr || workspace_bytes < need) return BNBX_E_WORKSPACE;
    if (!aligned(workspace, 256)) return BNBX_E_ALIGN;
    slots = (unsigned long long*)workspace;
  }
  char* a32 = (char*)workspace + dq_slot_bytes(count);
  for (int i = 0; i < count; ++i) {
    jobs[i] = job_of(items[i].w, items[i].packed, items[i].st,
                     s0->double_quant ? (float*)a32 : nullptr);
    if (s0->double_quant) a32 += dq_absmax_bytes(nblocks(ns[i]));
  }
  return hip_status(launch_quantize(jobs, count, slots, s0->double_quant, s0->quant_type,
                                    (hipStream_t)stream));
}

int bnbx_dequantize_nf4(const uint8_t* packed, const bnbx_nf4_state* st, uint16_t* out,
                        void* stream) {
  if (packed == nullptr || out == nullptr) return BNBX_E_INVAL;
  const int s = check_state(st);
  if (s != BNBX_OK) return s;
  if (!aligned(packed, 16) || !aligned(out, 16)) return BNBX_E_ALIGN;
  return hip_status(launch_dequantize(packed, st->n, st->absmax, st->absmax2, st->absmax_mean,
                                      st->double_quant, st->quant_type,
                                      st->compute_dtype == BNBX_DTYPE_F16, out,
                                      (hipStream_t)stream));
}

int bnbx_gemv_nf4(const uint16_t* x, int64_t ldx, const uint8_t* packed,
                  const bnbx_nf4_state* st, int M, int N, int K, uint16_t* y, int64_t ldy,
                  void* stream) {
  const int s = check_matmul(x, ldx, packed, st, M, N, K, y, ldy);
  if (s != BNBX_OK) return s;
  if (M > 16) return BNBX_E_INVAL;
  const hipError_t e = launch_gemv(x, ldx, packed, st->absmax, st->absmax2, st->absmax_mean,
                                   st->double_quant, st->quant_type,
                                   st->compute_dtype == BNBX_DTYPE_F16, M, N, K, y, ldy,
                                   (hipStream_t)stream);
  if (e == hipErrorNotSupported) return BNBX_E_UNSUPPORTED;
  return hip_status(e);
}

int bnbx_gemv_nf4_grouped(const uint16_t* x, int64_t ldx, const bnbx_gemv_item* items,
                          int count, int M, int K, void* stream) {
  if (items == nullptr || count < 1 || count > BNBX_GEMV_MAX_ITEMS) return BNBX_E_INVAL;
  static_assert(BNBX_GEMV_MAX_ITEMS <= 4, "the grouped kernel takes at most four weights");
  GemvItem it[BNBX_GEMV_MAX_ITEMS];
  for (int w = 0; w < count; ++w) {
    const bnbx_gemv_item& a = items[w];
    const int s = check_matmul(x, ldx, a.packed, a.st, M, a.N, K, a.y, a.ldy);
    if (s != BNBX_OK) return s;
    const bnbx_nf4_state* s0 = items[0].st;
    if (a.st->quant_type != s0->quant_type || a.st->compute_dtype != s0->compute_dtype ||
        a.st->double_quant != s0->double_quant)
      return BNBX_E_INVAL;
    it[w] = GemvItem{a.packed, a.st->absmax, a.st->absmax2, a.st->absmax_mean, a.N, a.y, a.ldy};
  }
  if (M > 16) return BNBX_E_INVAL;
  const bnbx_nf4_state* s0 = items[0].st;
  const hipError_t e = launch_gemv_grouped(x, ldx, it, count, s0->double_quant, s0->quant_type,
                                           s0->compute_dtype == BNBX_DTYPE_F16, M, K,
                                           (hipStream_t)stream);
  if (e == hipErrorNotSupported) return BNBX_E_UNSUPPORTED;
  return hip_status(e);
}

int bnbx_lora_down(const uint16_t* x, int64_t ldx, const uint16_t* lora_a, int64_t lda, int M,
                   int K, int r, float scale, int compute_dtype, uint16_t* xa, int64_t ldxa,
                   void* stream) {
  if (x == nullptr || lora_a == nullptr || xa == nullptr) return BNBX_E_INVAL;
  if (compute_dtype != BNBX_DTYPE_BF16 && compute_dtype != BNBX_DTYPE_F16) return BNBX_E_INVAL;
  if (M < 1 || K < 32 || K % 32 != 0 || r < 16 || r > 256 || r % 16 != 0) return BNBX_E_INVAL;
  if (ldx < K || lda < K || ldxa < r) return BNBX_E_INVAL;
  if (ldx % 8 != 0 || lda % 8 != 0) return BNBX_E_ALIGN;
  if (!aligned(x, 16) || !aligned(lora_a, 16) || !aligned(xa, 2)) return BNBX_E_ALIGN;
  const hipError_t e = launch_lora_down(x, ldx, lora_a, lda, M, K, r, scale,
                                        compute_dtype == BNBX_DTYPE_F16, xa, ldxa,
                                        (hipStream_t)stream);
  if (e == hipErrorNotSupported) return BNBX_E_UNSUPPORTED;
  return hip_status(e);
}

size_t bnbx_gemm_nf4_workspace_bytes(int M, int N, int K) {
  if (M < 1 || N < 1 || K < kBlock || K % kBlock != 0) return 0;
  return gemm_workspace_bytes(M, N, K);
}

int bnbx_gemm_nf4(const uint16_t* x, int64_t ldx, const uint8_t* packed,
                  const bnbx_nf4_state* st, int M, int N, int K, uint16_t* y, int64_t ldy,
                  void* workspace, size_t workspace_bytes, void* stream) {
  const int s = check_matmul(x, ldx, packed, st, M, N, K, y, ldy);
  if (s != BNBX_OK) return s;
  if (workspace != nullptr && workspace_bytes > 0 && !aligned(workspace, 16)) return BNBX_E_ALIGN;
  const hipError_t e = launch_gemm(x, ldx, packed, st->absmax, st->absmax2, st->absmax_mean,
                                   st->double_quant, st->quant_type,
                                   st->compute_dtype == BNBX_DTYPE_F16, M, N, K, y, ldy,
                                   workspace, workspace_bytes, (hipStream_t)stream);
  if (e == hipErrorNotSupported) return BNBX_E_UNSUPPORTED;
  return hip_status(e);
}

int bnbx_gemm_nf4_lora(const uint16_t* x, int64_t ldx, const uint8_t* packed,
                       const bnbx_nf4_state* st, int M, int N, int K, const uint16_t* xa,
                       int64_t ldxa, const uint16_t* lora_b, int64_t ldb, int r, uint16_t* y,
                       int64_t ldy, void* stream) {
  const int s = check_matmul(x, ldx, packed, st, M, N, K, y, ldy);
  if (s != BNBX_OK) return s;
  if (xa == nullptr || lora_b == nullptr) return BNBX_E_INVAL;
  if (r < 16 || r > 256 || r % 16 != 0) return BNBX_E_INVAL;
  if (ldxa < r || ldb < r) return BNBX_E_INVAL;
  if (ldxa % 8 != 0 || ldb % 8 != 0) return BNBX_E_ALIGN;
  if (!aligned(xa, 16) || !aligned(lora_b, 16)) return BNBX_E_ALIGN;
  // Up to 16 rows of X: the decode GEMVs with the low-rank term; else the GEMM.
  const bool f16 = st->compute_dtype == BNBX_DTYPE_F16;
  const hipError_t e =
      M <= 16 ? launch_gemv_lora(x, ldx, packed, st->absmax, st->absmax2, st->absmax_mean,
                                st->double_quant, st->quant_type, f16, M, N, K, xa, ldxa, lora_b,
                                ldb, r, y, ldy, (hipStream_t)stream)
             : launch_gemm_lora(x, ldx, packed, st->absmax, st->absmax2, st->absmax_mean,
                                st->double_quant, st->quant_type, f16, M, N, K, xa, ldxa, lora_b,
                                ldb, r, y, ldy, (hipStream_t)stream);
  if (e == hipErrorNotSupported) return BNBX_E_UNSUPPORTED;
  return hip_status(e);
}

int bnbx_gemm_nf4_dx(const uint16_t* dy, int64_t lddy, const uint8_t* packed,
                     const bnbx_nf4_state* st, int M, int N, int K, uint16_t* dx, int64_t lddx,
                     void* stream) {
  // dY [M, N] plays the part of X (ld >= N) and dX [M, K] that of Y (ld >= K).
  if (dy == nullptr || packed == nullptr || dx == nullptr) return BNBX_E_INVAL;
  const int s = check_state(st);
  if (s != BNBX_OK) return s;
  if (M < 1 || N < 1 || K < kBlock || K % kBlock != 0) return BNBX_E_INVAL;
  if (st->n != (int64_t)N * (int64_t)K) return BNBX_E_INVAL;
  if (lddy < N || lddx < K) return BNBX_E_INVAL;
  if (lddy % 8 != 0) return BNBX_E_ALIGN;
  if (!aligned(dy, 16) || !aligned(packed, 16) || !aligned(dx, 2)) return BNBX_E_ALIGN;
  const hipError_t e = launch_gemm_dx(dy, lddy, packed, st->absmax, st->absmax2, st->absmax_mean,
                                      st->double_quant, st->quant_type,
                                      st->compute_dtype == BNBX_DTYPE_F16, M, N, K, dx, lddx,
                                      (hipStream_t)stream);
  if (e == hipErrorNotSupported) return BNBX_E_UNSUPPORTED;
  return hip_status(e);
}

}  // extern "C"

/*
 * bnbx.h -- C ABI of the MI355X (gfx950) NF4 4-bit weight library.
 *
 * Blockwise NF4 (or FP4) quantize-on-load with double quantization of the
 * block scales, dequantize to bfloat16 (or FP16), and the "4-bit storage,
 * 16-bit compute" linear layer Y = X . W_hat^T as a decode GEMV (M <= 16) and
 * a prefill GEMM (any M).
 *
 * Sources (five web pages about bitsandbytes, cited by page and section):
 *   mlqm.cn bitsandbytes article (news/394670), sec. 2.2 (quantize while
 *     loading, no calibration data), 3.2 (NF4: 16 levels placed by the normal
 *     density), 3.3 (one FP32 scale per block; double quantization quantizes
 *     the scales again), 3.4 (store 4-bit, dequantize to FP16/BF16, multiply),
 *     4 (loading options: 4-bit quant type nf4 or fp4, compute dtype BF16 or
 *     FP16);
 *   pomoai.com bitsandbytes overview, module list (Linear4bit replaces
 *     torch.nn.Linear: weight [out_features, in_features]; the functional
 *     module holds blockwise quantization and the NF4 format).
 *
 * Conventions shared by every call
 * --------------------------------
 * - 16-bit values (bf16, or IEEE binary16 where the state's compute_dtype
 *   says so) are passed as uint16_t bit patterns.
 * - Pointers named "device" are device (HBM) addresses; the caller allocates
 *   and frees every buffer.  The library never allocates device memory, never
 *   frees, and never synchronises: work is enqueued on `stream` (a
 *   hipStream_t; NULL means the null stream) and results are ready when the
 *   caller synchronises that stream.
 * - Every call validates its arguments on the host before enqueueing anything
 *   and returns a negative bnbx_status without side effects on failure.  A
 *   launch failure reported by the HIP runtime returns BNBX_E_HIP.  Faults
 *   during execution surface at the caller's next synchronisation.
 * - The library keeps no mutable global state after its one-time codebook
 *   initialisation, so calls on different streams may run concurrently.
 *   Calls that share output or workspace buffers must be ordered by the caller.
 * - Inputs must be finite.  A non-finite weight gives unspecified codes.
 *
 * Quantized tensor format (the "quant state")
 * -------------------------------------------
 * A weight of n elements (row-major [N, K] for a linear layer, n = N*K, n
 * even) is split into nb = ceil(n / 64) blocks of 64 consecutive elements of
 * the flat array (the last block may be short).
 *   packed   uint8[n/2]   two 4-bit codes per byte; element 2j in the HIGH
 *                         nibble of byte j, element 2j+1 in the low nibble.
 *   Without double quant:
 *     absmax   float[nb]  a_b = max |w| over block b.
 *   With double quant (second-level groups of 256 consecutive blocks,
 *   ng = ceil(nb / 256)), t_b = fl32((a_b - mean) / s_g):
 *     absmax      linear map (double_quant 1): int8_t[nb], q_b =
 *                 round-half-even(fl32(t_b * 127)), the block scale minus
 *                 the mean in units of s_g / 127;
 *                 dynamic map (double_quant 2): uint8_t[nb], q_b = the code
 *                 of the value of the dynamic 8-bit map nearest t_b, exact
 *                 ties to the lower code (bnbx_dynamic_map);
 *                 a group with s_g = 0 stores the code of 0 (0, or 127)
 *     absmax2     float[ng]   s_g = max |a_b - mean| over group g
 *     absmax_mean float[1]    mean = fl32(fl64(sum_b a_b) / nb), the sum exact
 *   Dequantized scale: without DQ a_b; with the linear map
 *     fl32(fl32(q_b * fl32(s_g / 127)) + mean); with the dynamic map
 *     fl32(fl32(map[q_b] * s_g) + mean).
 *   Code of element j: x = fl32(w_j * fl32(1 / a_b)) (for a nonzero a_b
 *   below 2^-100, w_j and a_b are first multiplied by 2^64, exactly, so the
 *   reciprocal stays finite); s = #{i : x >= T_i}
 *   where T_i is the smallest float above the midpoint of the i-th and
 *   (i+1)-th smallest distinct levels (nearest level, exact ties to the lower
 *   level); c is the code of the s-th smallest level.  An all-zero block
 *   takes the code of the 0.0 level.
 *   NF4 (quant_type 0): codes are the levels in ascending order, L[0] = -1,
 *   L[7] = 0, L[15] = +1 (bnbx_nf4_codebook).
 *   FP4 (quant_type 1; the pages give no layout, E2M1 is taken): bit 3 the
 *   sign, bits 2-1 the exponent e, bit 0 the mantissa m; L[c] =
 *   fl32(+-mag / 6) with mag = m/2 for e = 0, else 2^(e-1) (1 + m/2), i.e.
 *   0, 1/12, 1/6, 1/4, 1/3, 1/2, 2/3, 1 for codes 0-7 and their negatives for
 *   8-15 (bnbx_fp4_codebook).  The encoder never emits code 8 (-0); zero
 *   blocks take code 0.
 *   Dequantized weight: W_hat_j = rnd(fl32(L[c_j] * scale_b)), rnd = round
 *   to nearest even into the compute dtype (bf16 or binary16; binary16
 *   keeps subnormals and overflows to infinity).
 */
#ifndef BNBX_H
#define BNBX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Only the entry points below are exported from libbnbx.so. */
#define BNBX_API __attribute__((visibility("default")))

typedef enum {
  BNBX_OK = 0,
  BNBX_E_INVAL = -1,        /* bad size, null pointer, out-of-range argument   */
  BNBX_E_ALIGN = -2,        /* a pointer or leading dimension is misaligned    */
  BNBX_E_UNSUPPORTED = -3,  /* valid request the library does not implement    */
  BNBX_E_WORKSPACE = -4,    /* workspace missing or smaller than required      */
  BNBX_E_HIP = -5,          /* the HIP runtime reported an error at launch     */
  BNBX_E_INTERNAL = -6      /* the library's codebook tables failed their
                               one-time self-check (not expected to happen)    */
} bnbx_status;

/* 4-bit quant types (bnbx_nf4_state.quant_type). */
enum { BNBX_QUANT_NF4 = 0, BNBX_QUANT_FP4 = 1 };
/* Second-level maps of the block scales (bnbx_nf4_state.double_quant). */
enum { BNBX_DQ_NONE = 0, BNBX_DQ_LINEAR = 1, BNBX_DQ_DYNAMIC = 2 };
/* 16-bit compute types (bnbx_nf4_state.compute_dtype). */
enum { BNBX_DTYPE_BF16 = 0, BNBX_DTYPE_F16 = 1 };

/* Caller-owned descriptor of one quantized tensor (host memory; the pointers
 * inside are device addresses).  The library reads it during the call only. */
typedef struct {
  int64_t n;             /* number of weights, even, >= 2                      */
  int32_t blocksize;     /* weights per block; only 64 is supported            */
  int32_t double_quant;  /* BNBX_DQ_NONE (0): absmax is float[nb];
                            BNBX_DQ_LINEAR (1): int8 codes + absmax2 + mean;
                            BNBX_DQ_DYNAMIC (2): uint8 codes into the dynamic
                            8-bit map + absmax2 + mean                        */
  int32_t quant_type;    /* BNBX_QUANT_NF4 (0) or BNBX_QUANT_FP4 (1)            */
  int32_t compute_dtype; /* BNBX_DTYPE_BF16 (0) or BNBX_DTYPE_F16 (1): the type
                            of dequantized weights and of X and Y; the quantize
                            input is always bf16 and ignores it               */
  void*   absmax;        /* device: float[nb] (dq=0), int8_t[nb] (dq=1) or
                            uint8_t[nb] (dq=2)                                */
  float*  absmax2;       /* device: float[ng] (dq=1), else NULL                */
  float*  absmax_mean;   /* device: float[1]  (dq=1), else NULL                */
} bnbx_nf4_state;

/* Human-readable name of a status code (static string, never NULL). */
BNBX_API const char* bnbx_status_str(int status);

/* The 16 NF4 levels, ascending, into host memory.
 * mlqm.cn article sec. 3.2: 16 levels at standard-normal quantiles, dense
 * near zero and sparse at the ends; here 8 positive quantiles of probabilities
 * evenly spaced from 1 - (1/30 + 1/32)/2 toward 1/2, 7 mirrored negative ones
 * over the same span, and 0, divided by the outermost quantile so that
 * L[0] = -1, L[7] = 0, L[15] = +1 exactly.  Host-only, synchronous.
 * Returns BNBX_E_INVAL if levels_host is NULL. */
BNBX_API int bnbx_nf4_codebook(float levels_host[16]);

/* The 16 FP4 levels by code (E2M1 divided by 6, see the format notes above)
 * into host memory.  mlqm.cn article sec. 4: fp4, the plain 4-bit float
 * quant type offered beside nf4.  Host-only, synchronous.
 * Returns BNBX_E_INVAL if levels_host is NULL. */
BNBX_API int bnbx_fp4_codebook(float levels_host[16]);

/* The 256 values of the dynamic 8-bit map, ascending (the value of code c
 * is values_host[c]), into host memory.  The csdn.net bitsandbytes feature
 * page (sec. 1, item 5) lists dynamic 8-bit quantization among the library's
 * types and the mlqm.cn article (sec. 3.3) quantizes the fp32 block scales a
 * second time; no page defines the map.  It is read as dynamic tree
 * quantization (Dettmers, 2016): a sign bit, then E zero bits for the decimal
 * exponent 10^-E, a one bit, and 6 - E bits f of a linear fraction, valued at
 * the bin midpoint: |v| = 10^-E (0.1 + 0.9 (f + 1/2) / 2^(6-E)), E = 0..6,
 * formed in binary64 and rounded once to binary32; with 0 and 1 that makes
 * 256 values: codes 0-126 negative, 127 zero, 128-254 positive, 255 one.
 * Host-only, synchronous.  Returns BNBX_E_INVAL if values_host is NULL. */
BNBX_API int bnbx_dynamic_map(float values_host[256]);

/* Bytes of device workspace bnbx_quantize_nf4 needs for (n, blocksize,
 * double_quant); 0 without double quant.  Returns 0 for invalid arguments. */
BNBX_API size_t bnbx_quantize_nf4_workspace_bytes(int64_t n, int blocksize, int double_quant);

/* Blockwise 4-bit quantize-on-load, NF4 or FP4 by st->quant_type (mlqm.cn
 * article sec. 2.2, 3.2, 3.3, 4).
 *   w          device, bf16[n], 16-byte aligned (read only)
 *   packed     device, uint8[n/2], 16-byte aligned (written)
 *   st         host descriptor; st->absmax (and absmax2, absmax_mean with
 *              double quant) are written
 *   workspace  device, >= bnbx_quantize_nf4_workspace_bytes(...) bytes,
 *              256-byte aligned (may be NULL when that is 0); contents are
 *              scratch, overwritten by the call
 * Errors: BNBX_E_INVAL (null pointer, n odd or < 2, quant_type or
 * compute_dtype out of range; blocksize != 64 is BNBX_E_UNSUPPORTED),
 * BNBX_E_ALIGN, BNBX_E_WORKSPACE. */
BNBX_API int bnbx_quantize_nf4(const uint16_t* w, uint8_t* packed, const bnbx_nf4_state* st,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Largest weight count bnbx_quantize_nf4_noalloc takes with double quant
 * (2^28: every linear of a 70B-class model fits). */
#define BNBX_NOALLOC_MAX_WEIGHTS ((int64_t)1 << 28)

/* bnbx_quantize_nf4 for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the double-quant scratch (per-workgroup exact partial sums of
 * the block scales and the fp32 block scales, the workspace
 * bnbx_quantize_nf4 takes from its caller) lives in a fixed device array of
 * the library instead, 16 MiB plus 40 KiB on each GPU the library runs on,
 * held until the process ends.  The call allocates nothing: no hipMalloc, no
 * hipFree.  Results are identical to bnbx_quantize_nf4's.
 *   w, packed, st  as bnbx_quantize_nf4
 * Every call on one GPU shares that GPU's array, and nothing in it needs to
 * start at zero (each call overwrites what it reads).  Calls that overlap in
 * time on one GPU (different streams, or different host threads) race on it
 * and give undefined results: the caller must order them.
 * Errors: as bnbx_quantize_nf4; BNBX_E_WORKSPACE with double quant when
 * st->n > BNBX_NOALLOC_MAX_WEIGHTS; BNBX_E_HIP if the array's device address
 * cannot be obtained. */
BNBX_API int bnbx_quantize_nf4_noalloc(const uint16_t* w, uint8_t* packed,
                                       const bnbx_nf4_state* st, void* stream);

/* One tensor of a grouped quantize. */
typedef struct {
  const uint16_t* w;            /* device: bf16[st->n], 16-byte aligned (read only) */
  uint8_t* packed;              /* device: uint8[st->n / 2], 16-byte aligned (written) */
  const bnbx_nf4_state* st;     /* host descriptor, read during the call; its
                                   device arrays are written                  */
} bnbx_quantize_item;

/* Most tensors one grouped quantize takes (the seven linears of a
 * Llama-style layer fit). */
#define BNBX_QUANTIZE_MAX_ITEMS 8

/* Bytes of device workspace bnbx_quantize_nf4_grouped needs for `count`
 * tensors of n[0..count-1] weights; 0 without double quant.  Returns 0 for
 * invalid arguments. */
BNBX_API size_t bnbx_quantize_nf4_grouped_workspace_bytes(const int64_t* n, int count,
                                                         int blocksize, int double_quant);

/* Grouped quantize-on-load: bnbx_quantize_nf4 on up to
 * BNBX_QUANTIZE_MAX_ITEMS tensors at once, for a loader that quantizes a
 * layer's weights as they arrive (mlqm.cn article sec. 2.2: weights are
 * quantized while they are loaded; sec. 3.2-3.3, 4 as bnbx_quantize_nf4).
 * One launch quantizes every tensor's blocks and, with double quant, two
 * short ones form every tensor's mean and then its group scales and codes,
 * so the fixed cost of the launches is paid once per group of tensors
 * instead of once per tensor.  Each
 * tensor is quantized on its own (its own blocks, mean and groups): its
 * results are bit-identical to a bnbx_quantize_nf4 call on it.
 *   items      host array of `count` items, read during the call
 *   count      1 .. BNBX_QUANTIZE_MAX_ITEMS
 *   workspace  device, >= bnbx_quantize_nf4_grouped_workspace_bytes(...)
 *              bytes, 256-byte aligned (may be NULL without double quant);
 *              contents are scratch, overwritten by the call
 * Every item's state must have the same quant_type and double_quant.
 * Errors: as bnbx_quantize_nf4 for each item; BNBX_E_INVAL if items is NULL,
 * count is out of range or the items' states differ. */
BNBX_API int bnbx_quantize_nf4_grouped(const bnbx_quantize_item* items, int count,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* Dequantize to the compute dtype, bf16 or binary16 (mlqm.cn article
 * sec. 3.4, 4).
 *   packed  device, uint8[n/2], 16-byte aligned
 *   st      host descriptor of the quant state (read)
 *   out     device, 16-bit[n] of st->compute_dtype, 16-byte aligned (written)
 * Errors: BNBX_E_INVAL, BNBX_E_ALIGN, BNBX_E_UNSUPPORTED. */
BNBX_API int bnbx_dequantize_nf4(const uint8_t* packed, const bnbx_nf4_state* st, uint16_t* out,
                        void* stream);

/* Decode GEMV, Y[M, N] = X[M, K] . W_hat[N, K]^T, 1 <= M <= 16
 * (mlqm.cn article sec. 3.4 and the "4-bit is not always faster" pitfall in
 * sec. 7: the weight is streamed once from HBM in 4 bits and dequantized in
 * registers; products accumulate in fp32; Y is rounded to the compute dtype).
 * X, Y and the dequantized weights are of st->compute_dtype (sec. 4).
 *   x       device, 16-bit, row m at x + m*ldx; ldx >= K, ldx % 8 == 0,
 *           16-byte aligned
 *   packed  device, the quantized [N, K] weight (st->n == N*K), 16-byte aligned
 *   y       device, 16-bit, row m at y + m*ldy; ldy >= N, written
 * K must be a multiple of 64 (blocks never straddle rows).
 * Errors: BNBX_E_INVAL (sizes, M outside 1..16, null), BNBX_E_ALIGN,
 * BNBX_E_UNSUPPORTED. */
BNBX_API int bnbx_gemv_nf4(const uint16_t* x, int64_t ldx, const uint8_t* packed,
                  const bnbx_nf4_state* st, int M, int N, int K,
                  uint16_t* y, int64_t ldy, void* stream);

/* One weight of a grouped decode GEMV. */
typedef struct {
  const uint8_t* packed;        /* device: the quantized [N, K] weight, 16-byte aligned */
  const bnbx_nf4_state* st;     /* host descriptor (st->n == N*K), read during the call */
  int32_t N;                    /* rows of this weight, >= 1 */
  uint16_t* y;                  /* device: row m of this weight's Y at y + m*ldy */
  int64_t ldy;                  /* >= N */
} bnbx_gemv_item;

/* Most weights one grouped GEMV takes. */
#define BNBX_GEMV_MAX_ITEMS 4

/* Grouped decode GEMV: Y_i = X . W_hat_i^T for up to BNBX_GEMV_MAX_ITEMS
 * weights that multiply the same X (the q, k and v projections of an
 * attention layer, or the gate and up projections of its MLP), 1 <= M <= 16.
 * Same arithmetic and results as one bnbx_gemv_nf4 call per weight (mlqm.cn
 * article sec. 3.4 and the sec. 7 pitfall: each weight is streamed once).
 * For M <= 4 the weights' rows run as one launch per group of up to four
 * rows of X, so the fixed part of a launch is paid once for all of them; for
 * 4 < M <= 16 each weight gets its own launch of the batched kernel.
 *   x, ldx      as bnbx_gemv_nf4
 *   items       host array of `count` items, read during the call
 *   count       1 .. BNBX_GEMV_MAX_ITEMS
 *   M, K        rows of X and the common K of every weight
 * Every item's state must have the same quant_type, compute_dtype and
 * double_quant; each weight's packed bytes must stay below 2^31.
 * Errors: as bnbx_gemv_nf4 for each item; BNBX_E_INVAL if items is NULL,
 * count is out of range or the items' states differ; BNBX_E_UNSUPPORTED if
 * a weight is too large for one launch. */
BNBX_API int bnbx_gemv_nf4_grouped(const uint16_t* x, int64_t ldx, const bnbx_gemv_item* items,
                                   int count, int M, int K, void* stream);

/* Bytes of device workspace bnbx_gemm_nf4 can use for (M, N, K) on the
 * current device.  With K of at least 32 blocks (2048 values): when the
 * 256 x 256 output tiles fill at most half of the GPU's compute units, the
 * GEMM splits K over up to four workgroups per tile (e.g. M = 2048 with
 * N = 4096: 128 tiles on 256 CUs); when they fill more than one round but
 * less than two, it runs the first round's tiles whole and splits the rest.
 * The split workgroups write fp32 partial tiles here and a second launch
 * adds them in split order and rounds once.  Returns 0 when no split is
 * planned, and for invalid sizes. */
BNBX_API size_t bnbx_gemm_nf4_workspace_bytes(int M, int N, int K);

/* Prefill GEMM, Y[M, N] = X[M, K] . W_hat[N, K]^T for any M >= 1: weights
 * are dequantized in registers straight into 16-bit matrix-core operands
 * (bf16 or binary16 MFMA by st->compute_dtype) with fp32 accumulation; Y is
 * rounded to the compute dtype (mlqm.cn article sec. 3.4, "4-bit storage,
 * 16-bit compute").  Arguments as bnbx_gemv_nf4.
 *   workspace  device, 16-byte aligned, or NULL: with at least
 *              bnbx_gemm_nf4_workspace_bytes(M, N, K) bytes the GEMM may
 *              split K (see there); with less (or none) it runs the tiles
 *              whole.  Either way Y is the fp32 sum rounded once; the split
 *              changes only the order of the fp32 additions.  Contents are
 *              scratch, overwritten by the call.
 * Errors: as bnbx_gemv_nf4 (M >= 1); BNBX_E_ALIGN for a misaligned workspace
 * of nonzero size. */
BNBX_API int bnbx_gemm_nf4(const uint16_t* x, int64_t ldx, const uint8_t* packed,
                  const bnbx_nf4_state* st, int M, int N, int K,
                  uint16_t* y, int64_t ldy, void* workspace, size_t workspace_bytes,
                  void* stream);

/* 4-bit linear layer with a LoRA term fused in (any M):
 * Y = X . W_hat^T + XA . B^T, where XA [M, r] = s . X . A^T is the
 * adapter's down-projection already applied (and scaled) by the caller and
 * B [N, r] its up-projection (the nn.Linear(r, N) weight).  The pomoai.com
 * overview: QLoRA trains low-rank adapters beside the frozen 4-bit base
 * layer.  For M > 16 the adapter term runs as r / 16 more matrix-core
 * products per output tile, into the same fp32 accumulators as the 4-bit
 * product (before it); for M <= 16 the decode GEMVs stream the weight once
 * and add the term to their partial sums before the reduction (M <= 4: each
 * lane's ranks; 4 < M <= 16: one matrix-core product of 32 ranks per wave
 * and group of 16 weight rows).  Either way Y is rounded once to the compute
 * dtype.
 *   x, packed, st, M, N, K, y, ldy  as bnbx_gemm_nf4
 *   xa      device, 16-bit, row m at xa + m*ldxa; ldxa >= r, ldxa % 8 == 0,
 *           16-byte aligned
 *   lora_b  device, 16-bit, row n at lora_b + n*ldb; ldb >= r, ldb % 8 == 0,
 *           16-byte aligned
 *   r       adapter rank, a multiple of 16, 16 <= r <= 256
 * Errors: as bnbx_gemm_nf4 (BNBX_E_INVAL for r or a leading dimension out of
 * range, BNBX_E_ALIGN for xa / lora_b alignment). */
BNBX_API int bnbx_gemm_nf4_lora(const uint16_t* x, int64_t ldx, const uint8_t* packed,
                       const bnbx_nf4_state* st, int M, int N, int K,
                       const uint16_t* xa, int64_t ldxa, const uint16_t* lora_b, int64_t ldb,
                       int r, uint16_t* y, int64_t ldy, void* stream);

/* LoRA down-projection, XA = rnd(fl32(s . X . A^T)) with fp32 accumulation:
 * the adapter input that bnbx_gemm_nf4_lora takes (pomoai.com overview,
 * QLoRA: trainable low-rank adapters beside the frozen 4-bit base; A is the
 * adapter's nn.Linear(K, r) weight, s its scale).  Values are of
 * compute_dtype (BNBX_DTYPE_BF16 or BNBX_DTYPE_F16).
 *   x       device, X [M, K], row m at x + m*ldx; ldx >= K, ldx % 8 == 0,
 *           16-byte aligned
 *   lora_a  device, A [r, K], row j at lora_a + j*lda; lda >= K, lda % 8 == 0,
 *           16-byte aligned
 *   M, K, r M >= 1; K a multiple of 32; r a multiple of 16, 16 <= r <= 256
 *   scale   s, applied once to the fp32 sum before the rounding
 *   xa      device, XA [M, r], row m at xa + m*ldxa; ldxa >= r (written)
 * The sum over K runs in a fixed order, so results repeat bit for bit.
 * Errors: BNBX_E_INVAL (null, sizes, compute_dtype), BNBX_E_ALIGN,
 * BNBX_E_UNSUPPORTED (leading dimensions too large for 32-bit offsets). */
BNBX_API int bnbx_lora_down(const uint16_t* x, int64_t ldx, const uint16_t* lora_a, int64_t lda,
                            int M, int K, int r, float scale, int compute_dtype, uint16_t* xa,
                            int64_t ldxa, void* stream);

/* Input gradient of the 4-bit linear layer, dX[M, K] = dY[M, N] . W_hat[N, K]
 * (the weights stay frozen, as for the 4-bit base layer under QLoRA in the
 * pomoai.com overview; W_hat as in bnbx_dequantize_nf4, mlqm.cn article
 * sec. 3.4): the weights are dequantized into LDS, transposed, and fed to
 * 16-bit matrix cores with fp32 accumulation; dX is rounded to the compute
 * dtype.  dY, dX and W_hat are of st->compute_dtype.
 *   dy      device, 16-bit, row m at dy + m*lddy; lddy >= N, lddy % 8 == 0,
 *           16-byte aligned
 *   packed  device, the quantized [N, K] weight (st->n == N*K), 16-byte aligned
 *   dx      device, 16-bit, row m at dx + m*lddx; lddx >= K, written
 * M >= 1; K must be a multiple of 64 (else BNBX_E_INVAL) and N a multiple
 * of 64 (else BNBX_E_UNSUPPORTED: the kernel takes whole 64-row steps).
 * Errors: BNBX_E_INVAL (sizes, null), BNBX_E_ALIGN, BNBX_E_UNSUPPORTED. */
BNBX_API int bnbx_gemm_nf4_dx(const uint16_t* dy, int64_t lddy, const uint8_t* packed,
                     const bnbx_nf4_state* st, int M, int N, int K,
                     uint16_t* dx, int64_t lddx, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BNBX_H */

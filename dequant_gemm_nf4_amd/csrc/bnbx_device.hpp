// Device-side helpers shared by the kernels of libbnbx (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bnbx {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;

// bfloat16 bits -> binary32 (exact).
__device__ __forceinline__ float bf16lo_to_f32(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t pair) {
  return __uint_as_float(pair & 0xffff0000u);
}

// Two binary32 -> packed bfloat16 pair (lo in bits 0..15), round to nearest
// even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return (uint16_t)(pack_bf16x2(f, 0.0f) & 0xffffu);
}

// The same for the compute type: bfloat16, or IEEE binary16 when F16
// (v_cvt_f16_f32: round to nearest even, subnormals kept, overflow to inf).
template <bool F16>
__device__ __forceinline__ uint32_t pack16x2(float lo, float hi) {
  if constexpr (F16) {
    f16x2_t v;
    v[0] = (_Float16)lo;
    v[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, v);
  } else {
    return pack_bf16x2(lo, hi);
  }
}
template <bool F16>
__device__ __forceinline__ uint16_t f32_to_16(float f) {
  return (uint16_t)(pack16x2<F16>(f, 0.0f) & 0xffffu);
}

// Double-quant block scale as the stored format defines it,
// fl32(fl32(q * fl32(s_g / 127)) + mean), each operation rounded on its own.
// fl32(s_g / 127) is s_g * fl32(1/127) corrected once with its exact
// residual: that equals the correctly rounded quotient for every positive
// binary32 except the smallest subnormals, which take the division.
// dq_step_normal is the corrected product alone: exact for s_g >= 2^-120,
// within one subnormal ulp below.  The GEMV kernels use it (they scale bf16
// levels by the fp32 block scale, so their products are not bit-exact
// anyway, and the division's registers made their larger variants spill).
__device__ __forceinline__ float dq_step_normal(float s) {
  constexpr float kR = 1.0f / 127.0f;
  const float q0 = s * kR;
  return __builtin_fmaf(__builtin_fmaf(-q0, 127.0f, s), kR, q0);
}
__device__ __forceinline__ float dq_step(float s) {
  float st = dq_step_normal(s);
  if (__builtin_expect(s < 0x1p-120f, 0)) st = s / 127.0f;
  return st;
}
__device__ __forceinline__ float dq_scale(float qf, float s, float mean) {
  const float prod = qf * dq_step(s);
  return prod + mean;
}

// v_perm_b32: byte k of the result is byte sel[k] of the 8-byte value
// {hi, lo} (0..3 pick lo's bytes, 4..7 hi's bytes, 0x0c gives 0).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}
// a.lo * b.lo + a.hi * b.hi + c over pairs of the compute type.
template <bool F16>
__device__ __forceinline__ float dot2_16(uint32_t a, uint32_t b, float c) {
  if constexpr (F16)
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                  c, false);
  else
    return dot2_bf16(a, b, c);
}

// Matrix-core products over 8-element operands of the compute type (raw bits).
template <bool F16>
__device__ __forceinline__ f32x4_t mfma_16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
template <bool F16>
__device__ __forceinline__ f32x16_t mfma_32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// 16-byte streaming load / store (non-temporal hint: data used once).
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store_nt16(void* p, uint4 v) {
  u32x4_t t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, (u32x4_t*)p);
}

// The 16 levels held in lanes 0..15 of one VGPR, built from the
// kernel-argument block with scalar loads and v_writelane only; a lookup is
// one ds_bpermute.  Table builds therefore touch no vector memory and never
// wait behind weight loads already in flight.
template <int I>
__device__ __forceinline__ void write_lane(int& v, int s) {
  asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(v) : "s"(s), "n"(I));
}
template <typename LevelTableT>
__device__ __forceinline__ int level_lanes(const LevelTableT& lv) {
  int v = 0;
  int s[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) s[i] = __builtin_amdgcn_readfirstlane(__float_as_int(lv.level[i]));
  write_lane<0>(v, s[0]);   write_lane<1>(v, s[1]);   write_lane<2>(v, s[2]);
  write_lane<3>(v, s[3]);   write_lane<4>(v, s[4]);   write_lane<5>(v, s[5]);
  write_lane<6>(v, s[6]);   write_lane<7>(v, s[7]);   write_lane<8>(v, s[8]);
  write_lane<9>(v, s[9]);   write_lane<10>(v, s[10]); write_lane<11>(v, s[11]);
  write_lane<12>(v, s[12]); write_lane<13>(v, s[13]); write_lane<14>(v, s[14]);
  write_lane<15>(v, s[15]);
  return v;
}
__device__ __forceinline__ float level_lookup(int lanes, uint32_t c) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute((int)(c << 2), lanes));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

}  // namespace bnbx

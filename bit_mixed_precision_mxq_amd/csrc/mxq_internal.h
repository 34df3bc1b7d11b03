// Internal helpers shared by the libmxq kernels and host entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "../../include/mxq.h"

namespace mxq {

// ---- host-side error reporting ---------------------------------------------
void set_error(const std::string& msg);
mxq_status fail(mxq_status s, const std::string& msg);
mxq_status check_launch(const char* what);

#define MXQ_REQUIRE(cond, code, msg) \
  do {                               \
    if (!(cond)) return ::mxq::fail((code), (msg)); \
  } while (0)

inline hipStream_t as_stream(mxq_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

// ---- MFMA operand vector types -----------------------------------------------
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// ---- device number-format helpers --------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// floor(log2(a)) - emax clamped to [-127, 127]; a == 0 or subnormal -> -127.
// Subnormal fp32 amax only arises from subnormal inputs, whose floor(log2) is
// below -126, so the clamp gives -127 there as well.
__device__ __forceinline__ int shared_exponent(float amax, int emax) {
  uint32_t bits = __float_as_uint(amax);
  int ef = static_cast<int>((bits >> 23) & 0xFF);
  if (ef == 0) return -127;
  int e = ef - 127 - emax;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// E2M1 magnitude code of a >= 0 (a = |x| * 2^-e, exact): nearest of
// {0,.5,1,1.5,2,3,4,6}, ties to the even code, saturating at 6.
__device__ __forceinline__ uint32_t e2m1_mag_code(float a) {
  return static_cast<uint32_t>(a > 0.25f) + static_cast<uint32_t>(a >= 0.75f) +
         static_cast<uint32_t>(a > 1.25f) + static_cast<uint32_t>(a >= 1.75f) +
         static_cast<uint32_t>(a > 2.5f) + static_cast<uint32_t>(a >= 3.5f) +
         static_cast<uint32_t>(a > 5.0f);
}

// Two fp32 values rounded to bf16 (round to nearest, ties to even; one
// v_cvt_pk_bf16_f32), a in the low half.
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));
  const v2bf16 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// E2M1 codes of eight block-scaled values (each x * 2^-e, exact), element i
// in nibble i: the nearest of {0,.5,1,1.5,2,3,4,6} with ties to the even code,
// saturating at 6, the sign bit copied from the value (so -0 and negatives
// that round to 0 give code 8).  gfx950's packed FP4 conversion with a unit
// scale does exactly this in one instruction per pair (checked on every
// bf16-representable input against the exactly rounded code).
__device__ __forceinline__ uint32_t e2m1_pack8(const float (&v)[8]) {
  uint32_t w;
  __asm__ volatile("" : "=v"(w));  // every byte is written below
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
  return w;
}

// OCP E4M3 codes of four block-scaled values (x * 2^-e, exact), value i in
// byte i: round to nearest, ties to even, saturating at 448 (the clamp takes
// values beyond 448 to 448, which is also what rounding with saturation
// gives), sign copied.  gfx950's packed FP8 conversion after the clamp does
// exactly this (checked on every bf16-representable input against the
// exactly rounded code).
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  auto cl = [](float x) { return __builtin_fminf(__builtin_fmaxf(x, -448.0f), 448.0f); };
  int w;
  __asm__ volatile("" : "=v"(w));  // both halves are written below
  w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), w, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), w, true);
  return static_cast<uint32_t>(w);
}

// ---- P of low-bit tiles (ThriftAttention, abstract: low-bit blocks merged
// through one online softmax; readings R14, R15, R17) --------------------------
// 1.5 * 2^12: an fp32 in [2^12, 2^13) has a spacing of exactly 2^-11, so one
// fused multiply-add onto it rounds the softmax exponent to the 2^-11 grid.
constexpr float kPGridMagic = 6144.0f;

// Four scores -> four E4M3 codes packed in one word (score i in byte i):
// code_i = E4M3_RNE(2^x_i) with x_i = fl32(s_i * c + off) - 6144, where off =
// 6144 + 8 - m puts the exponent on the grid relative to the reference m with
// P stored as 2^8 times its value (E8M0 2^-8 restores it).  Because x_i is a
// grid point, v_exp_f32 followed by the round-to-nearest-even conversion gives
// the exactly rounded E4M3 code at every grid point a tile can produce.  The
// two conversions write the low and the high half of the word, so its earlier
// contents do not matter: an opaque register spares a zeroing move.
__device__ __forceinline__ int p4_e4m3(const v4f& s4, float c, float off) {
  float y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s4[i], c, off) - kPGridMagic);
  int w;
  __asm__ volatile("" : "=v"(w));
  w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], w, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
}

// Asymmetric 4-bit group of 32 values (reading R19): s = fp16(fl32(max-min)/15),
// z = fp16(min), code = clamp(rint(fl32(x - z) / s), 0, 15), all codes 0 when
// s == 0; codes packed two per byte, element 2k in the low nibble.  Every
// operation rounds on its own (no fused multiply-add can form here).
__device__ __forceinline__ void int4_group(const float (&v)[32], uint32_t (&packed)[4], uint16_t& sbits,
                                           uint16_t& zbits) {
  float mn = v[0], mx = v[0];
#pragma unroll
  for (int i = 1; i < 32; ++i) { mn = fminf(mn, v[i]); mx = fmaxf(mx, v[i]); }
  const float s32 = (mx - mn) / 15.0f;
  const _Float16 sh = static_cast<_Float16>(s32);
  const _Float16 zh = static_cast<_Float16>(mn);
  const float s = static_cast<float>(sh), z = static_cast<float>(zh);
#pragma unroll
  for (int i = 0; i < 4; ++i) packed[i] = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    uint32_t c = 0;
    if (s != 0.0f) {
      float q = __builtin_rintf((v[i] - z) / s);
      q = fminf(fmaxf(q, 0.0f), 15.0f);
      c = static_cast<uint32_t>(q);
    }
    packed[i / 8] |= c << (4 * (i % 8));
  }
  sbits = __builtin_bit_cast(uint16_t, sh);
  zbits = __builtin_bit_cast(uint16_t, zh);
}

// Exact floor division helpers
__host__ __device__ __forceinline__ int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace mxq

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

// OCP E4M3 code of x (|x| < 2^9 after block scaling, exact), round half to
// even, saturating at 448, sign copied.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  uint32_t bits = __float_as_uint(x);
  uint32_t sign = (bits >> 24) & 0x80u;
  float a = __uint_as_float(bits & 0x7FFFFFFFu);
  uint32_t code;
  if (a < 0.015625f) {  // below 2^-6: subnormal grid k * 2^-9, k = 0..8
    code = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
  } else {
    uint32_t ab = bits & 0x7FFFFFFFu;
    uint32_t r = (ab + 0x7FFFFu + ((ab >> 20) & 1u)) >> 20;  // RNE to 3 mantissa bits
    code = r - (120u << 3);                                   // rebias 127 -> 7
    code = code > 126u ? 126u : code;                         // saturate at 448
  }
  return code | sign;
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

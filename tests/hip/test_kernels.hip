// Test-only HIP kernels for the GPU tests (not part of libmxq).
//  - mxqt_p_codes: runs the attention kernel's own P conversion (p4_e4m3 from
//    the library's internal header: fused multiply-add onto the 2^-11 grid,
//    v_exp_f32, round-to-nearest-even E4M3 conversion) on given scores, so a
//    test can compare every grid point with the exactly rounded code.
//  - mxqt_e2m1_codes: runs the quantisers' E2M1 element conversion
//    (e2m1_pack8) on given values, eight to a word.
//  - mxqt_e4m3_codes: runs the V quantiser's E4M3 element conversion
//    (e4m3_pack4) on given values, four to a word.
//  - mxqt_fill_lds: fills the whole LDS of every CU with one 32-bit word, so
//    a kernel launched right after starts on garbage LDS contents (LDS is not
//    cleared between workgroups).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../bit_mixed_precision_mxq_amd/csrc/mxq_internal.h"

#pragma clang fp contract(off)

namespace {

__global__ void k_p_codes(const float* __restrict__ s, const float* __restrict__ c, const float* __restrict__ off,
                          int n4, uint32_t* __restrict__ codes) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const mxq::v4f s4 = {s[4 * i], s[4 * i + 1], s[4 * i + 2], s[4 * i + 3]};
  codes[i] = static_cast<uint32_t>(mxq::p4_e4m3(s4, c[i], off[i]));
}

// e2m1_pack8 (the quantisers' element conversion) on 8 consecutive values
__global__ void k_e2m1_codes(const float* __restrict__ v, int n8, uint32_t* __restrict__ codes) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = v[8 * i + j];
  codes[i] = mxq::e2m1_pack8(x);
}

// e4m3_pack4 (the V quantiser's element conversion) on 4 consecutive values
__global__ void k_e4m3_codes(const float* __restrict__ v, int n4, uint32_t* __restrict__ codes) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  codes[i] = mxq::e4m3_pack4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
}

constexpr int kLdsWords = 160 * 1024 / 4;  // all of a gfx950 CU's LDS

__global__ void __launch_bounds__(1024) k_fill_lds(uint32_t word, int probe, uint32_t* __restrict__ sink) {
  __shared__ uint32_t buf[kLdsWords];
  for (int i = threadIdx.x; i < kLdsWords; i += blockDim.x) buf[i] = word;
  __syncthreads();
  // one read the compiler cannot drop, so the stores stay
  if (threadIdx.x == 0 && buf[probe % kLdsWords] != word) sink[0] = 1u;
}

}  // namespace

extern "C" int mxqt_p_codes(const float* s, const float* c, const float* off, int n4, uint32_t* codes,
                            void* stream) {
  if (n4 <= 0) return 0;
  hipLaunchKernelGGL(k_p_codes, dim3((n4 + 255) / 256), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), s, c,
                     off, n4, codes);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

extern "C" int mxqt_e2m1_codes(const float* v, int n8, uint32_t* codes, void* stream) {
  if (n8 <= 0) return 0;
  hipLaunchKernelGGL(k_e2m1_codes, dim3((n8 + 255) / 256), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), v, n8,
                     codes);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

extern "C" int mxqt_e4m3_codes(const float* v, int n4, uint32_t* codes, void* stream) {
  if (n4 <= 0) return 0;
  hipLaunchKernelGGL(k_e4m3_codes, dim3((n4 + 255) / 256), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), v, n4,
                     codes);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

extern "C" int mxqt_fill_lds(uint32_t word, int n_blocks, uint32_t* sink, void* stream) {
  hipLaunchKernelGGL(k_fill_lds, dim3(n_blocks), dim3(1024), 0, reinterpret_cast<hipStream_t>(stream), word,
                     static_cast<int>(word & 0x3FF), sink);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

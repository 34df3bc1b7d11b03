// attn_quantkv_append: one decode step's update of the 4-bit KV cache.
// HyQuant (summary, abstract) applies its hybrid principle to KV-cache
// compression in decode: the sink tokens and a recent window stay in fp16,
// the rest is stored as 4-bit codes with an fp16 scale and zero per 32
// elements of head_dim.  As a sequence grows, the new token enters the window
// and the token leaving it is quantised from its fp16 copy.
//
// Two kernels:
//  k_kv_append : one workgroup per (kv head, K or V, sequence): quantise the
//                window's first row (one thread per 32-element group), then
//                move the window up by one row (16-byte units, all loads of a
//                slice before its stores) and write the new token as the last
//                row (bf16 -> fp16, round to nearest even), and into the sink
//                copy while t < n_sink;
//  k_kv_bump   : seq_len[b] += 1, after every head of every sequence is done.
#include "mxq_internal.h"

#pragma clang fp contract(off)

namespace mxq {
namespace {

struct AppendArgs {
  const uint16_t* k_new;  // bf16 [B][Hkv][D]
  const uint16_t* v_new;
  mxq_kv_cache_rw c;
  int Hkv, D;
};

__device__ __forceinline__ uint16_t f16_bits_of_bf16(uint16_t b) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(bf16_to_f32(b)));
}

__global__ void __launch_bounds__(256) k_kv_append(AppendArgs a) {
  const int h = blockIdx.x >> 1;
  const bool is_v = blockIdx.x & 1;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int D = a.D;
  const int t = a.c.seq_len[b];
  if (t < 0 || t >= a.c.L_cap) return;  // left unchanged
  const int64_t bh = static_cast<int64_t>(b) * a.Hkv + h;
  const uint16_t* xnew = (is_v ? a.v_new : a.k_new) + bh * D;
  uint16_t* rec = (is_v ? a.c.v_recent : a.c.k_recent);
  uint16_t* sink = (is_v ? a.c.v_sink : a.c.k_sink);
  uint8_t* codes = is_v ? a.c.v_codes : a.c.k_codes;
  uint16_t* scale = is_v ? a.c.v_scale : a.c.k_scale;
  uint16_t* zero = is_v ? a.c.v_zero : a.c.k_zero;
  const int n_recent = a.c.n_recent, n_sink = a.c.n_sink;
  uint16_t* win = n_recent > 0 ? rec + bh * n_recent * D : nullptr;

  // 1) the token leaving the window (or, without a window, the new token)
  const int t_old = t - n_recent;
  if (t_old >= n_sink && t_old >= 0 && tid < D / 32) {
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint16_t hb = n_recent > 0 ? win[32 * tid + i] : f16_bits_of_bf16(xnew[32 * tid + i]);
      v[i] = static_cast<float>(__builtin_bit_cast(_Float16, hb));
    }
    uint32_t packed[4];
    uint16_t sb, zb;
    int4_group(v, packed, sb, zb);
    const int64_t g = (bh * a.c.L_cap + t_old) * (D / 32) + tid;
    reinterpret_cast<uint4*>(codes)[g] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    scale[g] = sb;
    zero[g] = zb;
  }
  __syncthreads();  // row 0 is read before the move overwrites it

  // 2) move the window up by one row, a slice of rows at a time: every unit of
  // rows [r0+1, r0+R] is loaded before any is stored to rows [r0, r0+R-1]
  if (n_recent > 0) {
    const int upr = D / 8;             // 16-byte units per row
    const int R = 256 / upr;           // rows per slice (one unit per thread)
    uint4* w4 = reinterpret_cast<uint4*>(win);
    for (int r0 = 0; r0 < n_recent - 1; r0 += R) {
      const int r = r0 + tid / upr, u = tid % upr;
      const bool live = tid < R * upr && r + 1 < n_recent;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (live) val = w4[(r + 1) * upr + u];
      __syncthreads();
      if (live) w4[r * upr + u] = val;
      __syncthreads();
    }
    // 3) the new token as the last row
    for (int d = tid; d < D; d += blockDim.x) win[(n_recent - 1) * D + d] = f16_bits_of_bf16(xnew[d]);
  }
  if (t < n_sink)
    for (int d = tid; d < D; d += blockDim.x) sink[(bh * n_sink + t) * D + d] = f16_bits_of_bf16(xnew[d]);
}

__global__ void k_kv_bump(int32_t* seq_len, int B, int L_cap) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) {
    const int t = seq_len[b];
    if (t >= 0 && t < L_cap) seq_len[b] = t + 1;
  }
}

// Decode line tokens from the prefill's vertical lines (HyQuant: the prefill's
// principle carried over to the decode cache; reading R36).  One thread per
// (entry, 8-element unit) of one (sequence, kv head): the list of the kv
// group's first query head is copied, and the listed token's K and V rows are
// converted bf16 -> fp16 (round to nearest even); an entry outside [0, L)
// gets zero rows (such an entry never takes part, reading R33).
struct LinesFromPrefillArgs {
  const int32_t* lines_hq;  // [B][Hq][n]
  const uint16_t* k;        // bf16 [B][Hkv][L][D]
  const uint16_t* v;
  int32_t* lines;           // [B][Hkv][n]
  uint16_t* k_lines;        // fp16 [B][Hkv][n][D]
  uint16_t* v_lines;
  int Hq, Hkv, L, D, n;
};

__global__ void __launch_bounds__(256) k_kv_lines_from_prefill(LinesFromPrefillArgs a) {
  const int hk = blockIdx.x, b = blockIdx.y;
  const int G = a.Hq / a.Hkv;
  const int units = a.D / 8;
  const int64_t bhk = static_cast<int64_t>(b) * a.Hkv + hk;
  const int32_t* src = a.lines_hq + (static_cast<int64_t>(b) * a.Hq + hk * G) * a.n;
  for (int idx = threadIdx.x; idx < a.n * units; idx += blockDim.x) {
    const int e = idx / units, u = idx % units;
    const int key = src[e];
    if (u == 0) a.lines[bhk * a.n + e] = key;
    const bool ok = key >= 0 && key < a.L;
    const int64_t row = (bhk * a.L + (ok ? key : 0)) * a.D + 8 * u;
    const int64_t dst = (bhk * a.n + e) * a.D + 8 * u;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      a.k_lines[dst + x] = ok ? f16_bits_of_bf16(a.k[row + x]) : 0;
      a.v_lines[dst + x] = ok ? f16_bits_of_bf16(a.v[row + x]) : 0;
    }
  }
}

}  // namespace
}  // namespace mxq

using namespace mxq;

extern "C" mxq_status attn_quantkv_append(const uint16_t* k_new, const uint16_t* v_new,
                                          const mxq_kv_cache_rw* c, int32_t B, int32_t Hkv, int32_t D,
                                          mxq_stream_t stream) {
  MXQ_REQUIRE(c != nullptr, MXQ_EINVAL, "attn_quantkv_append: cache is NULL");
  MXQ_REQUIRE(B >= 0 && Hkv >= 1 && B <= 65535 && Hkv <= 32767, MXQ_EINVAL,
              "attn_quantkv_append: need 0 <= B <= 65535 and 1 <= Hkv <= 32767");
  MXQ_REQUIRE(D >= 32 && D <= 256 && D % 32 == 0, MXQ_EUNSUPPORTED,
              "attn_quantkv_append: D must be a multiple of 32, at most 256");
  MXQ_REQUIRE(c->L_cap >= 1 && c->n_sink >= 0 && c->n_recent >= 0, MXQ_EINVAL,
              "attn_quantkv_append: need L_cap >= 1, n_sink >= 0, n_recent >= 0");
  MXQ_REQUIRE(k_new && v_new && c->k_codes && c->v_codes && c->k_scale && c->k_zero && c->v_scale && c->v_zero &&
                  c->seq_len,
              MXQ_EINVAL, "attn_quantkv_append: new tokens, codes, scales, zeros and seq_len are required");
  MXQ_REQUIRE(c->n_sink == 0 || (c->k_sink && c->v_sink), MXQ_EINVAL,
              "attn_quantkv_append: sink copies are required when n_sink > 0");
  MXQ_REQUIRE(c->n_recent == 0 || (c->k_recent && c->v_recent), MXQ_EINVAL,
              "attn_quantkv_append: recent copies are required when n_recent > 0");
  if (B == 0) return MXQ_OK;
  hipStream_t st = as_stream(stream);
  AppendArgs a;
  a.k_new = k_new; a.v_new = v_new; a.c = *c; a.Hkv = Hkv; a.D = D;
  hipLaunchKernelGGL(k_kv_append, dim3(2 * Hkv, B), dim3(256), 0, st, a);
  mxq_status s = check_launch("k_kv_append");
  if (s != MXQ_OK) return s;
  hipLaunchKernelGGL(k_kv_bump, dim3((B + 255) / 256), dim3(256), 0, st, c->seq_len, B, c->L_cap);
  return check_launch("k_kv_bump");
}

extern "C" mxq_status mxq_kv_lines_from_prefill(const int32_t* lines_hq, int32_t Hq, const uint16_t* k_bf16,
                                                const uint16_t* v_bf16, int32_t B, int32_t Hkv, int32_t L,
                                                int32_t D, int32_t n_lines, int32_t* lines, uint16_t* k_lines,
                                                uint16_t* v_lines, mxq_stream_t stream) {
  MXQ_REQUIRE(B >= 1 && Hkv >= 1 && Hq >= 1 && Hq % Hkv == 0 && B <= 65535 && Hkv <= 65535, MXQ_EINVAL,
              "mxq_kv_lines_from_prefill: need B, Hkv >= 1 and Hq a multiple of Hkv");
  MXQ_REQUIRE(L >= 1 && D >= 8 && D % 8 == 0, MXQ_EINVAL, "mxq_kv_lines_from_prefill: need L >= 1, D a multiple of 8");
  MXQ_REQUIRE(n_lines >= 1 && n_lines <= 16, MXQ_EINVAL, "mxq_kv_lines_from_prefill: n_lines must be in [1, 16]");
  MXQ_REQUIRE(lines_hq && k_bf16 && v_bf16 && lines && k_lines && v_lines, MXQ_EINVAL,
              "mxq_kv_lines_from_prefill: every array is required");
  LinesFromPrefillArgs a;
  a.lines_hq = lines_hq; a.k = k_bf16; a.v = v_bf16; a.lines = lines; a.k_lines = k_lines; a.v_lines = v_lines;
  a.Hq = Hq; a.Hkv = Hkv; a.L = L; a.D = D; a.n = n_lines;
  hipLaunchKernelGGL(k_kv_lines_from_prefill, dim3(Hkv, B), dim3(256), 0, as_stream(stream), a);
  return check_launch("k_kv_lines_from_prefill");
}

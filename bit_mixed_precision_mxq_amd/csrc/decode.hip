// attn_quantkv_decode: one decode step over a 4-bit group-scaled KV cache.
//
// HyQuant (abstract): in decode the hybrid principle applies to the KV cache,
// with dequantisation fused into attention; the first tokens (vertical-line
// sink) and the recent window stay in fp16.  NOVA-KV (abstract, third page):
// decode reads the whole cache each step and is bandwidth-bound, so the kernel
// is built to stream the cache once at full HBM rate.
//
// Layout of the work:
//   k_decode_split: workgroup = (split s, kv head, sequence); 4 waves, each
//   walking 16-token tiles of the split.  Lane (t = lane/4, g = lane%4) owns
//   token t of the tile and head_dim group g (32 elements, one INT4 scale/zero
//   pair), so one wave reads 16 consecutive tokens' 64-byte code rows as one
//   contiguous 1 KB load.  For the G query heads of the kv head:
//     score   S_h = sum_g [ s_g * sum_{d in g} c_d q_hd + z_g * sum_{d in g} q_hd ]
//             (codes unpacked to exact fp16, products by v_dot2_f32_f16 with
//             fp32 accumulation; the zero term uses a precomputed group sum);
//     softmax fp32 online per head over the wave's tokens (exp2 domain);
//     values  O_hd += (p_h s_g) c_d  plus  Z_hg += p_h z_g, fp32 FMAs.
//   Each wave keeps partial (m, l, O) for its tokens; the 4 waves are merged in
//   wave order at the end of the split and written to the workspace.
//   k_decode_merge: (sequence, query head): merge the splits in ascending order.
#include "mxq_internal.h"

namespace mxq {
namespace {

constexpr int kD = 128;          // head_dim supported by the decode kernel
constexpr int kTokPerWave = 16;  // tokens per wave iteration
constexpr int kWaves = 4;

struct DecodeArgs {
  const uint16_t* q;  // bf16 [B][Hq][D]
  mxq_kv_cache kv;
  float* ws;          // [B][Hq][S][D + 2]
  int Hq, Hkv, S, tokens_per_split;
  float c;            // fl32(scale * log2 e)
};

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }

// 8 INT4 codes (one dword, element e in bits 4e..4e+3) -> four exact fp16 pairs
// in the order (c0,c2), (c4,c6), (c1,c3), (c5,c7).
__device__ __forceinline__ void unpack8_f16(uint32_t x, uint32_t out[4]) {
  const uint32_t lo = x & 0x0F0F0F0Fu;          // c0 c2 c4 c6
  const uint32_t hi = (x >> 4) & 0x0F0F0F0Fu;   // c1 c3 c5 c7
  const uint32_t k64 = 0x64646464u;             // high byte of fp16 1024
  const h2 minus1024 = {static_cast<_Float16>(-1024.0f), static_cast<_Float16>(-1024.0f)};
  uint32_t p0 = __builtin_amdgcn_perm(k64, lo, 0x04010400u);  // (1024+c0, 1024+c2)
  uint32_t p1 = __builtin_amdgcn_perm(k64, lo, 0x04030402u);  // (1024+c4, 1024+c6)
  uint32_t p2 = __builtin_amdgcn_perm(k64, hi, 0x04010400u);  // (1024+c1, 1024+c3)
  uint32_t p3 = __builtin_amdgcn_perm(k64, hi, 0x04030402u);  // (1024+c5, 1024+c7)
  out[0] = __builtin_bit_cast(uint32_t, as_h2(p0) + minus1024);
  out[1] = __builtin_bit_cast(uint32_t, as_h2(p1) + minus1024);
  out[2] = __builtin_bit_cast(uint32_t, as_h2(p2) + minus1024);
  out[3] = __builtin_bit_cast(uint32_t, as_h2(p3) + minus1024);
}

// element index (0..7 within a dword) of pair slot k, half j (see unpack8_f16)
__device__ __forceinline__ int pair_elem(int k, int j) {
  const int base[4] = {0, 4, 1, 5};
  return base[k] + 2 * j;
}

__device__ __forceinline__ float grp_sum(float v) {  // over the 4 lanes of one token
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  return v;
}
__device__ __forceinline__ float tok_max(float v) {  // over the 16 tokens of a wave
  v = fmaxf(v, __shfl_xor(v, 4));
  v = fmaxf(v, __shfl_xor(v, 8));
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float tok_sum(float v) {
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 8);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

template <int G>
__global__ void __launch_bounds__(256) k_decode_split(DecodeArgs a) {
  const int s = blockIdx.x;
  const int hk = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int tl = lane >> 2;  // token within the wave tile
  const int g = lane & 3;    // head_dim group
  const int len = min(a.kv.seq_len[b], a.kv.L_cap);  // never read past the cache
  const int t_begin = s * a.tokens_per_split;
  const int t_end = min(t_begin + a.tokens_per_split, len);
  const int64_t bh = static_cast<int64_t>(b) * a.Hkv + hk;
  const int L = a.kv.L_cap;
  const int n_sink = a.kv.n_sink, n_recent = a.kv.n_recent;
  const int rec0 = len - n_recent;  // first token served from the recent copy

  // query heads hk*G .. hk*G+G-1: fp16 pairs for this lane's 32 elements, in
  // the pair order produced by unpack8_f16, plus the group sums
  uint32_t qp[G][16];
  float qsum[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint16_t* qrow = a.q + (static_cast<int64_t>(b) * a.Hq + hk * G + h) * kD + 32 * g;
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {        // dword w of the code row: elements 8w..8w+7
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const _Float16 lo = static_cast<_Float16>(bf16_to_f32(qrow[8 * w + pair_elem(k, 0)]));
        const _Float16 hi = static_cast<_Float16>(bf16_to_f32(qrow[8 * w + pair_elem(k, 1)]));
        qp[h][4 * w + k] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
                           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
      }
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) acc += bf16_to_f32(qrow[e]);
    qsum[h] = acc;
  }

  float m[G], l[G], Z[G];
  float O[G][32];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -__builtin_inff(); l[h] = 0.0f; Z[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) O[h][e] = 0.0f;
  }
  const float c = a.c;

  for (int t0 = t_begin + wave * kTokPerWave; t0 < t_end; t0 += kWaves * kTokPerWave) {
    const int t = t0 + tl;
    const bool live = t < t_end;
    const bool f16 = live && (t < n_sink || t >= rec0);
    // ---------------- keys
    float part[G];
#pragma unroll
    for (int h = 0; h < G; ++h) part[h] = 0.0f;
    if (live) {
      if (!f16) {
        const int64_t row = bh * L + t;
        const uint4 cw = *reinterpret_cast<const uint4*>(a.kv.k_codes + row * (kD / 2) + 16 * g);
        const float ks = static_cast<float>(__builtin_bit_cast(_Float16, a.kv.k_scale[row * 4 + g]));
        const float kz = static_cast<float>(__builtin_bit_cast(_Float16, a.kv.k_zero[row * 4 + g]));
        const uint32_t cws[4] = {cw.x, cw.y, cw.z, cw.w};
        float x[G];
#pragma unroll
        for (int h = 0; h < G; ++h) x[h] = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t pr[4];
          unpack8_f16(cws[w], pr);
#pragma unroll
          for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int h = 0; h < G; ++h)
              x[h] = __builtin_amdgcn_fdot2(as_h2(pr[k]), as_h2(qp[h][4 * w + k]), x[h], false);
        }
#pragma unroll
        for (int h = 0; h < G; ++h) part[h] = __builtin_fmaf(ks, x[h], kz * qsum[h]);
      } else {
        const uint16_t* src = t < n_sink ? a.kv.k_sink + (bh * n_sink + t) * kD
                                         : a.kv.k_recent + (bh * n_recent + (t - rec0)) * kD;
        const uint4* s4 = reinterpret_cast<const uint4*>(src + 32 * g);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint4 v = s4[w];  // elements 8w..8w+7, fp16
          const uint16_t* e16 = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t kp = static_cast<uint32_t>(e16[pair_elem(k, 0)]) |
                                (static_cast<uint32_t>(e16[pair_elem(k, 1)]) << 16);
#pragma unroll
            for (int h = 0; h < G; ++h)
              part[h] = __builtin_amdgcn_fdot2(as_h2(kp), as_h2(qp[h][4 * w + k]), part[h], false);
          }
        }
      }
    }
    // ---------------- softmax (exp2 domain), per head
    float p[G];
    bool grow = false;
    float fac[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float sc = grp_sum(part[h]) * c;  // every lane takes part in the shuffles
      if (!live) sc = -__builtin_inff();
      const float tm = tok_max(sc);
      const float mn = fmaxf(m[h], tm);
      fac[h] = (m[h] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(m[h] - mn);
      grow |= mn != m[h];
      p[h] = live ? __builtin_amdgcn_exp2f(sc - mn) : 0.0f;
      // lanes of one group g hold the 16 tokens once each
      l[h] = l[h] * fac[h] + tok_sum(p[h]);
      m[h] = mn;
    }
    if (__any(grow)) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        Z[h] *= fac[h];
#pragma unroll
        for (int e = 0; e < 32; ++e) O[h][e] *= fac[h];
      }
    }
    // ---------------- values
    if (live) {
      if (!f16) {
        const int64_t row = bh * L + t;
        const uint4 cw = *reinterpret_cast<const uint4*>(a.kv.v_codes + row * (kD / 2) + 16 * g);
        const float vs = static_cast<float>(__builtin_bit_cast(_Float16, a.kv.v_scale[row * 4 + g]));
        const float vz = static_cast<float>(__builtin_bit_cast(_Float16, a.kv.v_zero[row * 4 + g]));
        float w[G];
#pragma unroll
        for (int h = 0; h < G; ++h) { w[h] = p[h] * vs; Z[h] = __builtin_fmaf(p[h], vz, Z[h]); }
        const uint32_t cws[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const uint32_t lo = cws[q4] & 0x0F0F0F0Fu, hi = (cws[q4] >> 4) & 0x0F0F0F0Fu;
          float cv[8];
#pragma unroll
          for (int j = 0; j < 4; ++j) {  // v_cvt_f32_ubyte{0..3}
            cv[2 * j] = static_cast<float>((lo >> (8 * j)) & 0xFFu);
            cv[2 * j + 1] = static_cast<float>((hi >> (8 * j)) & 0xFFu);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int h = 0; h < G; ++h) O[h][8 * q4 + e] = __builtin_fmaf(w[h], cv[e], O[h][8 * q4 + e]);
        }
      } else {
        const uint16_t* src = t < n_sink ? a.kv.v_sink + (bh * n_sink + t) * kD
                                         : a.kv.v_recent + (bh * n_recent + (t - rec0)) * kD;
        const uint4* s4 = reinterpret_cast<const uint4*>(src + 32 * g);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const uint4 v = s4[q4];
          const _Float16* e16 = reinterpret_cast<const _Float16*>(&v);
#pragma unroll
          for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int h = 0; h < G; ++h)
              O[h][8 * q4 + e] = __builtin_fmaf(p[h], static_cast<float>(e16[e]), O[h][8 * q4 + e]);
        }
      }
    }
  }

  // ---------------- reduce the 16 token lanes, then the 4 waves (in order)
  __shared__ float s_o[kWaves][G][kD];
  __shared__ float s_ml[kWaves][G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    Z[h] = tok_sum(Z[h]);
#pragma unroll
    for (int e = 0; e < 32; ++e) O[h][e] = tok_sum(O[h][e]) + Z[h];
  }
  if (tl == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 32; ++e) s_o[wave][h][32 * g + e] = O[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) { s_ml[wave][h][0] = m[h]; s_ml[wave][h][1] = l[h]; }
  }
  __syncthreads();
  // thread (h, d) merges the 4 waves
  for (int idx = tid; idx < G * kD; idx += 256) {
    const int h = idx / kD, d = idx % kD;
    float M = -__builtin_inff();
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_ml[w][h][0]);
    float lt = 0.0f, ot = 0.0f;
    if (M != -__builtin_inff()) {
      for (int w = 0; w < kWaves; ++w) {
        const float mw = s_ml[w][h][0];
        if (mw == -__builtin_inff()) continue;
        const float f = __builtin_amdgcn_exp2f(mw - M);
        lt = __builtin_fmaf(s_ml[w][h][1], f, lt);
        ot = __builtin_fmaf(s_o[w][h][d], f, ot);
      }
    }
    float* dst = a.ws + ((static_cast<int64_t>(b) * a.Hq + hk * G + h) * a.S + s) * (kD + 2);
    dst[d] = ot;
    if (d == 0) { dst[kD] = M; dst[kD + 1] = lt; }
  }
}

__global__ void k_decode_merge(const float* __restrict__ ws, float* __restrict__ out, int Hq, int S) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const float* base = ws + (static_cast<int64_t>(b) * Hq + h) * S * (kD + 2);
  float M = -__builtin_inff();
  for (int s = 0; s < S; ++s) M = fmaxf(M, base[s * (kD + 2) + kD]);
  float lt = 0.0f, ot = 0.0f;
  for (int s = 0; s < S; ++s) {
    const float ms = base[s * (kD + 2) + kD];
    if (ms == -__builtin_inff()) continue;
    const float f = __builtin_amdgcn_exp2f(ms - M);
    lt = __builtin_fmaf(base[s * (kD + 2) + kD + 1], f, lt);
    ot = __builtin_fmaf(base[s * (kD + 2) + d], f, ot);
  }
  out[(static_cast<int64_t>(b) * Hq + h) * kD + d] = ot / lt;
}

int pick_splits(int max_seq_len, int num_splits) {
  if (num_splits > 0) return num_splits;
  int s = (max_seq_len + 2047) / 2048;
  return s < 1 ? 1 : (s > 64 ? 64 : s);
}

}  // namespace
}  // namespace mxq

using namespace mxq;

extern "C" size_t attn_quantkv_decode_workspace(int32_t B, int32_t Hq, int32_t D, int32_t num_splits,
                                                int32_t max_seq_len) {
  if (B <= 0 || Hq <= 0 || D <= 0) return 0;
  int S = pick_splits(max_seq_len, num_splits);
  return static_cast<size_t>(B) * Hq * S * (D + 2) * sizeof(float);
}

extern "C" mxq_status attn_quantkv_decode(const uint16_t* q, const mxq_kv_cache* kv, int32_t B,
                                          int32_t Hq, int32_t Hkv, int32_t D, int32_t max_seq_len,
                                          float softmax_scale, int32_t num_splits, void* workspace,
                                          size_t ws_bytes, float* out, mxq_stream_t stream) {
  MXQ_REQUIRE(q && kv && out, MXQ_EINVAL, "attn_quantkv_decode: q, cache and out are required");
  MXQ_REQUIRE(B >= 1 && Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0, MXQ_EINVAL,
              "attn_quantkv_decode: need B, Hq, Hkv >= 1 and Hq % Hkv == 0");
  MXQ_REQUIRE(D == kD, MXQ_EUNSUPPORTED, "attn_quantkv_decode: D must be 128");
  const int G = Hq / Hkv;
  MXQ_REQUIRE(G == 1 || G == 2 || G == 4, MXQ_EUNSUPPORTED,
              "attn_quantkv_decode: Hq/Hkv must be 1, 2 or 4");
  MXQ_REQUIRE(kv->seq_len && kv->k_codes && kv->v_codes && kv->k_scale && kv->k_zero &&
                  kv->v_scale && kv->v_zero,
              MXQ_EINVAL, "attn_quantkv_decode: INT4 cache arrays and seq_len are required");
  MXQ_REQUIRE(kv->n_sink >= 0 && kv->n_recent >= 0, MXQ_EINVAL, "attn_quantkv_decode: negative n_sink/n_recent");
  MXQ_REQUIRE(kv->n_sink == 0 || (kv->k_sink && kv->v_sink), MXQ_EINVAL, "attn_quantkv_decode: sink arrays missing");
  MXQ_REQUIRE(kv->n_recent == 0 || (kv->k_recent && kv->v_recent), MXQ_EINVAL,
              "attn_quantkv_decode: recent arrays missing");
  MXQ_REQUIRE(max_seq_len >= 1 && max_seq_len <= kv->L_cap, MXQ_EINVAL,
              "attn_quantkv_decode: need 1 <= max_seq_len <= L_cap");
  MXQ_REQUIRE(num_splits >= 0 && num_splits <= 4096, MXQ_EINVAL, "attn_quantkv_decode: num_splits out of range");
  MXQ_REQUIRE(B <= 65535 && Hkv <= 65535, MXQ_EUNSUPPORTED, "attn_quantkv_decode: B, Hkv must be <= 65535");
  MXQ_REQUIRE(!(softmax_scale != softmax_scale), MXQ_EINVAL, "attn_quantkv_decode: softmax_scale is NaN");
  const int S = pick_splits(max_seq_len, num_splits);
  MXQ_REQUIRE(workspace && ws_bytes >= attn_quantkv_decode_workspace(B, Hq, D, num_splits, max_seq_len),
              MXQ_EINVAL, "attn_quantkv_decode: workspace too small");
  DecodeArgs a;
  a.q = q; a.kv = *kv; a.ws = static_cast<float*>(workspace); a.Hq = Hq; a.Hkv = Hkv; a.S = S;
  int tps = (max_seq_len + S - 1) / S;
  tps = (tps + kWaves * kTokPerWave - 1) / (kWaves * kTokPerWave) * (kWaves * kTokPerWave);
  a.tokens_per_split = tps;
  const double sc = softmax_scale > 0.0f ? static_cast<double>(softmax_scale) : 1.0 / __builtin_sqrt(static_cast<double>(D));
  a.c = static_cast<float>(sc * 1.4426950408889634);
  hipStream_t st = as_stream(stream);
  dim3 grid(S, Hkv, B);
  switch (G) {
    case 1: hipLaunchKernelGGL(k_decode_split<1>, grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL(k_decode_split<2>, grid, dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL(k_decode_split<4>, grid, dim3(256), 0, st, a); break;
  }
  mxq_status stt = check_launch("k_decode_split");
  if (stt != MXQ_OK) return stt;
  hipLaunchKernelGGL(k_decode_merge, dim3(Hq, B), dim3(kD), 0, st, a.ws, out, Hq, S);
  return check_launch("k_decode_merge");
}

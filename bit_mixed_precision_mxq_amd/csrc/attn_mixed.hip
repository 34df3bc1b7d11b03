// attn_mixed_fwd: stage 2 of ThriftAttention (abstract) -- selected query-key
// tiles in FP16, the rest in block-scaled low bit, merged through one online
// softmax into a single output.  HyQuant (abstract): sink and local-window
// tiles are among the high-precision ones (the selection mask carries them).
//
// Work decomposition (gfx950, wave64):
//   workgroup = (batch, query head, query tile of BQ rows), BQ/16 waves;
//   wave      = 16 query rows; the wave walks the key axis in chunks of 128
//               keys (two 64-key selection tiles) in ascending order.
// Per chunk and wave:
//   S^T[128 keys x 16 queries] = K . Q^T with
//     - one v_mfma_scale_f32_16x16x128_f8f6f4 (FP4 x FP4, E8M0 block scales)
//       per 16 keys for low-bit tiles: the whole head_dim (<=128) in one
//       instruction, so S is the exactly rounded dot product whenever the
//       block-exponent spread within a pair is <= 18 bits;
//     - four v_mfma_f32_16x16x32_bf16 per 16 keys for FP16 tiles (bf16 inputs
//       are exact in fp16, so this is the FP16 product);
//   the K rows fed to the MFMA are permuted so that lane group g (lanes
//   16g..16g+15) ends up holding, for its query column, keys {16g+j} of the
//   first tile and {64+16g+j} of the second: exactly the K-operand layout of
//   the 16x16x128 FP8 MFMA used for PV, so P never leaves the registers.
//   Softmax: row max over lanes (2 shuffles), integer-snapped running
//   reference per tile, P = E4M3(2^xq) with xq on the 2^-11 grid (one FMA,
//   one subtraction, v_exp_f32, v_cvt_pk_fp8_f32), FP16 tiles fp16(2^x).
//   O^T[d x 16 queries] += V^T . P^T: v_mfma_scale_f32_16x16x128_f8f6f4 (FP8 x
//   FP8) per 16 head_dim rows; each 64-key tile's reference enters through
//   the E8M0 scale of its K blocks (2^-8 minus the reference gap), and one
//   more MFMA with an all-ones A operand accumulates l = sum(P).  FP16 tiles
//   add their contribution with v_mfma_f32_16x16x32_f16.
// K and V of the low-bit tiles are staged once per chunk in LDS and shared by
// the BQ/16 waves; the FP16 tiles' operands (few) are read straight from
// global memory.
#include "mxq_internal.h"

// Products and sums round on their own unless written as __builtin_fmaf: the
// reference exponent ceil(fl32(rowmax * c)) must be one rounded product.
#pragma clang fp contract(off)

namespace mxq {
mxq_status validate_attn_shape(const mxq_attn_shape* s);

namespace {

struct AttnArgs {
  const uint8_t* q_codes;
  const uint8_t* q_scales;
  const uint8_t* k_codes;
  const uint8_t* k_scales;
  const uint8_t* v_codes;
  const uint8_t* v_scales;
  const uint16_t* q_bf16;
  const uint16_t* k_bf16;
  const uint16_t* v_f16t;
  const uint32_t* mask;
  void* out;
  float* lse;
  int Hq, Hkv, N, n_valid, n_qt, words, causal, mode, out_bf16;
  float c;  // fl32(softmax_scale * log2(e))
};

constexpr float kGridMagic = 6144.0f;  // 1.5 * 2^12: spacing 2^-11 in [2^12, 2^13)
constexpr float kExpOffset = 8.0f;     // P is stored as E4M3(2^(x + 8)) * 2^-8
constexpr int kPScale = 119;           // E8M0 code of 2^-8

// Key (within the 128-key chunk) that A-operand row r of S-block beta holds.
__device__ __forceinline__ int chunk_key(int beta, int r) {
  return 64 * (beta >> 2) + 16 * (r >> 2) + 4 * (beta & 3) + (r & 3);
}

__device__ __forceinline__ float wave_rowmax(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

template <int D, int BQ>
__global__ void __launch_bounds__(BQ * 4) k_attn_mixed(AttnArgs a) {
  constexpr int NW = BQ / 16;    // waves per workgroup
  constexpr int NT = NW * 64;    // threads
  constexpr int KROW = D / 2;    // bytes of one FP4 K row
  constexpr int NDB = D / 16;    // 16-row head_dim blocks of O^T
  constexpr int NSB = D / 32;    // MX blocks per row, and K=32 steps of the bf16 MFMA

  __shared__ __attribute__((aligned(16))) uint8_t s_kc[128 * KROW];
  __shared__ __attribute__((aligned(16))) uint8_t s_ks[128 * NSB];
  __shared__ __attribute__((aligned(16))) uint8_t s_vc[D * 128];
  __shared__ __attribute__((aligned(16))) uint32_t s_vs[D];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;   // query column within the wave's 16 rows
  const int g = lane >> 4;     // lane group 0..3
  const int it = a.n_qt - 1 - static_cast<int>(blockIdx.x);  // longest causal tiles first
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int G = a.Hq / a.Hkv;
  const int64_t bhq = static_cast<int64_t>(b) * a.Hq + h;
  const int64_t bhk = static_cast<int64_t>(b) * a.Hkv + h / G;
  const int qs = it * BQ;
  const int q = qs + wave * 16 + col;  // this lane's query row

  // ---------------------------------------------------------------- epilogue for padding tiles
  if (qs >= a.n_valid) {
    for (int idx = tid; idx < BQ * D; idx += NT) {
      int64_t o = (bhq * a.N + qs) * D + idx;
      if (a.out_bf16) static_cast<uint16_t*>(a.out)[o] = 0;
      else static_cast<float*>(a.out)[o] = 0.0f;
    }
    if (a.lse)
      for (int r = tid; r < BQ; r += NT) a.lse[bhq * a.N + qs + r] = -__builtin_inff();
    return;
  }
  const int qe = min(qs + BQ, a.n_valid) - 1;
  int last_tile = (a.n_valid - 1) / 64;
  if (a.causal) last_tile = min(last_tile, qe / 64);
  const int n_chunks = (last_tile + 2) / 2;

  // ---------------------------------------------------------------- Q fragments (registers)
  v8i qf4 = {0, 0, 0, 0, 0, 0, 0, 0};
  int qsc = 127;
  if (a.mode != MXQ_ALL_FP16 && g < NSB) {
    const uint4 w = *reinterpret_cast<const uint4*>(a.q_codes + (bhq * a.N + q) * KROW + 16 * g);
    qf4[0] = w.x; qf4[1] = w.y; qf4[2] = w.z; qf4[3] = w.w;
    qsc = a.q_scales[(bhq * a.N + q) * NSB + g];
  }
  v8bf qbf[NSB];
  if (a.mode != MXQ_ALL_LOWBIT) {
#pragma unroll
    for (int s = 0; s < NSB; ++s)
      qbf[s] = *reinterpret_cast<const v8bf*>(a.q_bf16 + (bhq * a.N + q) * D + 32 * s + 8 * g);
  }

  v4f O[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) O[i] = v4f{0.f, 0.f, 0.f, 0.f};
  v4f L = {0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  const float c = a.c;
  const uint32_t* mrow = a.mask ? a.mask + (bhq * a.n_qt + it) * a.words : nullptr;

  v8i ones8;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones8[i] = 0x38383838;  // E4M3 1.0
  v8h ones16;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones16[i] = static_cast<_Float16>(1.0f);

  for (int ch = 0; ch < n_chunks; ++ch) {
    const int kc = ch * 128;
    const int j0 = 2 * ch;
    const bool valid1 = j0 + 1 <= last_tile;
    bool prom0, prom1;
    if (a.mode == MXQ_ALL_FP16) {
      prom0 = true; prom1 = valid1;
    } else if (a.mode == MXQ_ALL_LOWBIT) {
      prom0 = false; prom1 = false;
    } else {
      const uint32_t wbits = mrow[j0 >> 5];
      prom0 = (wbits >> (j0 & 31)) & 1u;
      prom1 = valid1 && ((wbits >> ((j0 + 1) & 31)) & 1u);
    }
    const bool low0 = !prom0;
    const bool low1 = valid1 && !prom1;
    const bool need_low = low0 || low1;

    // ------------------------------------------------------------ stage low-bit K, V in LDS
    __syncthreads();
    if (need_low) {
      const uint4* kg = reinterpret_cast<const uint4*>(a.k_codes + (bhk * a.N + kc) * KROW);
      for (int u = tid; u < 128 * KROW / 16; u += NT) reinterpret_cast<uint4*>(s_kc)[u] = kg[u];
      const uint4* ksg = reinterpret_cast<const uint4*>(a.k_scales + (bhk * a.N + kc) * NSB);
      for (int u = tid; u < 128 * NSB / 16; u += NT) reinterpret_cast<uint4*>(s_ks)[u] = ksg[u];
      for (int u = tid; u < D * 8; u += NT) {
        const int d = u >> 3, part = u & 7;
        reinterpret_cast<uint4*>(s_vc)[u] =
            *reinterpret_cast<const uint4*>(a.v_codes + (bhk * D + d) * a.N + kc + 16 * part);
      }
      for (int d = tid; d < D; d += NT)
        s_vs[d] = *reinterpret_cast<const uint32_t*>(a.v_scales + (bhk * D + d) * (a.N / 32) + kc / 32);
    }
    __syncthreads();

    // ------------------------------------------------------------ S^T blocks
    v4f S[8];
#pragma unroll
    for (int beta = 0; beta < 8; ++beta) {
      const int t = beta >> 2;
      const bool valid_t = t == 0 ? true : valid1;
      const bool prom_t = t == 0 ? prom0 : prom1;
      v4f acc = {0.f, 0.f, 0.f, 0.f};
      const int key = chunk_key(beta, col);  // A-operand row of this lane
      if (!valid_t) {
        acc = v4f{-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
      } else if (prom_t) {
        const uint16_t* krow = a.k_bf16 + (bhk * a.N + kc + key) * D;
#pragma unroll
        for (int s = 0; s < NSB; ++s) {
          const v8bf ka = *reinterpret_cast<const v8bf*>(krow + 32 * s + 8 * g);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qbf[s], acc, 0, 0, 0);
        }
      } else {
        v8i ka = {0, 0, 0, 0, 0, 0, 0, 0};
        int ksc = 127;
        if (g < NSB) {
          const uint4 w = *reinterpret_cast<const uint4*>(s_kc + key * KROW + 16 * g);
          ka[0] = w.x; ka[1] = w.y; ka[2] = w.z; ka[3] = w.w;
          ksc = s_ks[key * NSB + g];
        }
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qf4, acc, 4, 4, 0, ksc, 0, qsc);
      }
      S[beta] = acc;
    }

    // ------------------------------------------------------------ masking
    const bool need_mask = (kc + 127 >= a.n_valid) || (a.causal && kc + 127 > qs) || (qe < qs + BQ - 1);
    if (need_mask) {
#pragma unroll
      for (int beta = 0; beta < 8; ++beta) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kc + 64 * (beta >> 2) + 16 * g + 4 * (beta & 3) + i;
          const bool ok = key < a.n_valid && q < a.n_valid && (!a.causal || key <= q);
          if (!ok) S[beta][i] = -__builtin_inff();
        }
      }
    }

    // ------------------------------------------------------------ running reference per tile
    float mx0 = -__builtin_inff(), mx1 = -__builtin_inff();
#pragma unroll
    for (int beta = 0; beta < 4; ++beta)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx0 = fmaxf(mx0, S[beta][i]);
#pragma unroll
    for (int beta = 4; beta < 8; ++beta)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx1 = fmaxf(mx1, S[beta][i]);
    mx0 = wave_rowmax(mx0);
    mx1 = wave_rowmax(mx1);
    const float t0 = ceilf(mx0 * c);
    const float t1 = ceilf(mx1 * c);
    const float m0 = fmaxf(m_run, t0);
    const float m1 = fmaxf(m0, t1);
    if (__any(m1 != m_run)) {
      float f = 1.0f;
      if (m_run != -__builtin_inff() && m1 != m_run)
        f = __builtin_ldexpf(1.0f, static_cast<int>(fmaxf(m_run - m1, -256.0f)));
#pragma unroll
      for (int i = 0; i < NDB; ++i) O[i] *= f;
      L *= f;
    }
    m_run = m1;

    // ------------------------------------------------------------ low-bit P and PV
    if (need_low) {
      v8i pb = {0, 0, 0, 0, 0, 0, 0, 0};
      if (low0) {
        const float off = kGridMagic + kExpOffset - (m0 == -__builtin_inff() ? 0.0f : m0);
#pragma unroll
        for (int beta = 0; beta < 4; ++beta) {
          float y[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            y[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[beta][i], c, off) - kGridMagic);
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
          pb[beta] = w;
        }
      }
      if (low1) {
        const float off = kGridMagic + kExpOffset - (m1 == -__builtin_inff() ? 0.0f : m1);
#pragma unroll
        for (int beta = 4; beta < 8; ++beta) {
          float y[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            y[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[beta][i], c, off) - kGridMagic);
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
          pb[beta] = w;
        }
      }
      // K blocks 0,1 (lane groups 0,1) carry the first tile, blocks 2,3 the second.
      int psc = kPScale;
      if (g < 2) {
        // the first tile's P was formed against m0 <= m1: scale it by 2^-(m1-m0)
        const float gap = m1 - m0;
        psc = (m0 == -__builtin_inff() || gap >= static_cast<float>(kPScale))
                  ? 0
                  : kPScale - static_cast<int>(gap);
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint8_t* vrow = s_vc + (16 * db + col) * 128;
        const uint4 w0 = *reinterpret_cast<const uint4*>(vrow + 16 * g);
        const uint4 w1 = *reinterpret_cast<const uint4*>(vrow + 64 + 16 * g);
        const v8i va = {static_cast<int>(w0.x), static_cast<int>(w0.y), static_cast<int>(w0.z),
                        static_cast<int>(w0.w), static_cast<int>(w1.x), static_cast<int>(w1.y),
                        static_cast<int>(w1.z), static_cast<int>(w1.w)};
        const int vsc = (s_vs[16 * db + col] >> (8 * g)) & 0xFF;
        O[db] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(va, pb, O[db], 0, 0, 0, vsc, 0, psc);
      }
      L = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones8, pb, L, 0, 0, 0, 127, 0, psc);
    }

    // ------------------------------------------------------------ FP16 tiles
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bool prom_t = t == 0 ? prom0 : prom1;
      if (!prom_t) continue;
      const float negm = -(m1 == -__builtin_inff() ? 0.0f : m1);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        v8h ph;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int beta = 4 * t + 2 * s + (e >> 2);
          ph[e] = static_cast<_Float16>(__builtin_amdgcn_exp2f(__builtin_fmaf(S[beta][e & 3], c, negm)));
        }
        const int key0 = kc + 64 * t + 16 * g + 8 * s;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const v8h va = *reinterpret_cast<const v8h*>(a.v_f16t + (bhk * D + 16 * db + col) * a.N + key0);
          O[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, ph, O[db], 0, 0, 0);
        }
        L = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones16, ph, L, 0, 0, 0);
      }
    }
  }

  // ---------------------------------------------------------------- epilogue
  const bool row_ok = q < a.n_valid;
  const float l = L[0];
  const float inv = row_ok ? 1.0f / l : 0.0f;
  const int64_t obase = (bhq * a.N + q) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int d0 = 16 * db + 4 * g;
    const float o0 = O[db][0] * inv, o1 = O[db][1] * inv, o2 = O[db][2] * inv, o3 = O[db][3] * inv;
    if (a.out_bf16) {
      auto bf = [](float x) -> uint32_t {
        uint32_t u = __float_as_uint(x);
        return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
      };
      uint2 pk = make_uint2(bf(o0) | (bf(o1) << 16), bf(o2) | (bf(o3) << 16));
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + obase + d0) = pk;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(a.out) + obase + d0) = make_float4(o0, o1, o2, o3);
    }
  }
  if (a.lse && g == 0) {
    a.lse[bhq * a.N + q] = row_ok ? (m_run + __log2f(l)) * 0.69314718055994531f : -__builtin_inff();
  }
}

template <int D, int BQ>
mxq_status launch(const AttnArgs& a, int n_qt, int Hq, int B, hipStream_t st) {
  hipLaunchKernelGGL((k_attn_mixed<D, BQ>), dim3(n_qt, Hq, B), dim3(BQ * 4), 0, st, a);
  return check_launch("k_attn_mixed");
}

}  // namespace
}  // namespace mxq

using namespace mxq;

extern "C" mxq_status attn_mixed_fwd(const uint8_t* q_codes, const uint8_t* q_scales,
                                     const uint8_t* k_codes, const uint8_t* k_scales,
                                     const uint8_t* v_codes, const uint8_t* v_scales,
                                     const uint16_t* q_bf16, const uint16_t* k_bf16,
                                     const uint16_t* v_f16t, const uint32_t* mask,
                                     const mxq_attn_shape* s, float softmax_scale, mxq_mode mode,
                                     void* out, mxq_out_dtype out_dtype, float* lse,
                                     mxq_stream_t stream) {
  mxq_status st = validate_attn_shape(s);
  if (st != MXQ_OK) return st;
  MXQ_REQUIRE(mode == MXQ_MIXED || mode == MXQ_ALL_LOWBIT || mode == MXQ_ALL_FP16, MXQ_EINVAL,
              "attn_mixed_fwd: bad mode");
  MXQ_REQUIRE(out_dtype == MXQ_OUT_F32 || out_dtype == MXQ_OUT_BF16, MXQ_EINVAL,
              "attn_mixed_fwd: bad out_dtype");
  MXQ_REQUIRE(out != nullptr, MXQ_EINVAL, "attn_mixed_fwd: out is NULL");
  const bool lowbit = mode != MXQ_ALL_FP16;
  const bool hi = mode != MXQ_ALL_LOWBIT;
  MXQ_REQUIRE(!lowbit || (q_codes && q_scales && k_codes && k_scales && v_codes && v_scales),
              MXQ_EINVAL, "attn_mixed_fwd: low-bit operands are required in this mode");
  MXQ_REQUIRE(!hi || (q_bf16 && k_bf16 && v_f16t), MXQ_EINVAL,
              "attn_mixed_fwd: bf16 Q/K and fp16 V^T are required in this mode");
  MXQ_REQUIRE(mode != MXQ_MIXED || mask != nullptr, MXQ_EINVAL, "attn_mixed_fwd: mask required in MIXED mode");
  MXQ_REQUIRE(!(softmax_scale != softmax_scale), MXQ_EINVAL, "attn_mixed_fwd: softmax_scale is NaN");
  double sc = softmax_scale > 0.0f ? static_cast<double>(softmax_scale) : 1.0 / __builtin_sqrt(static_cast<double>(s->D));
  AttnArgs a;
  a.q_codes = q_codes; a.q_scales = q_scales; a.k_codes = k_codes; a.k_scales = k_scales;
  a.v_codes = v_codes; a.v_scales = v_scales; a.q_bf16 = q_bf16; a.k_bf16 = k_bf16;
  a.v_f16t = v_f16t; a.mask = mask; a.out = out; a.lse = lse;
  a.Hq = s->Hq; a.Hkv = s->Hkv; a.N = s->N; a.n_valid = s->n_valid; a.n_qt = s->N / s->Bq;
  a.words = (s->N / s->Bk + 31) / 32; a.causal = s->causal; a.mode = mode;
  a.out_bf16 = out_dtype == MXQ_OUT_BF16;
  a.c = static_cast<float>(sc * 1.4426950408889634);
  hipStream_t strm = as_stream(stream);
  const int n_qt = s->N / s->Bq;
  if (s->D == 128 && s->Bq == 128) return launch<128, 128>(a, n_qt, s->Hq, s->B, strm);
  if (s->D == 128 && s->Bq == 64) return launch<128, 64>(a, n_qt, s->Hq, s->B, strm);
  if (s->D == 64 && s->Bq == 128) return launch<64, 128>(a, n_qt, s->Hq, s->B, strm);
  return launch<64, 64>(a, n_qt, s->Hq, s->B, strm);
}

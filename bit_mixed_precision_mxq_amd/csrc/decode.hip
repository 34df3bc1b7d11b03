// attn_quantkv_decode: one decode step over a 4-bit group-scaled KV cache.
//
// HyQuant (abstract): in decode the hybrid principle applies to the KV cache,
// with dequantisation fused into attention; the first tokens (vertical-line
// sink) and the recent window stay in fp16.  NOVA-KV (abstract, third page):
// decode reads the whole cache each step and is bandwidth-bound, so the kernel
// streams the cache once and keeps the vector ALU work per byte small: both
// contractions run on the matrix cores and no code is dequantised to a wider
// type before the MFMA.
//
// k_decode_split: workgroup = (split s, kv head, sequence), 4 waves.  Splits
// 0..S-1 cover the INT4 tokens [n_sink, len - n_recent) in equal ranges; each
// wave takes 32-token blocks of its split's range in turn.  Split S holds the
// fp16 tokens (sink and recent window), handled with plain fp32 arithmetic.
//
// INT4 block of 32 tokens, per wave (G query heads of the kv head):
//  scores  one v_mfma_scale_f32_16x16x128_f8f6f4 per 16 tokens and q part:
//          the B operand is the token's 128 codes, each nibble widened to a
//          byte, which is exactly the E4M3 value code * 2^-9 (scale 2^9);
//          the A operand is q split into two E4M3 parts (hi + lo reproduce
//          the bf16 value) laid out block-diagonally: row 4h+g holds head h's
//          q on group g's 32 elements only.  So output row (h, g) is the
//          unscaled partial dot product of group g, and each lane (token t,
//          head h) ends up with the four partials of its token, which the
//          fp16 scale and zero of the group turn into the score:
//            S = sum_g s_g * C_g + z_g * sum_{d in g} q_d.
//  softmax fp32 online, exp2 domain, row maxima by DPP within 16 lanes.
//  values  O[(h,g), d] += sum_t (p_t s_t,g) * code_t,d with one
//          v_mfma_f32_16x16x32_f16 per 16 head_dim columns: the A operand
//          p*s (fp16) is written to LDS by the (token, head) lanes and read
//          back transposed with ds_read_b64_tr_b16; the B operand holds the
//          codes as fp16 subnormals 16*code*2^-24 built from the packed cache
//          bytes by one byte permute and a mask (no float conversion).
//          Row (h, g) is meaningful for the head_dim columns of group g; the
//          zero-point term sum_t p_t z_t,g is accumulated on the side.
//  Loads for the next block are issued before the current one is computed.
// Vertical-line tokens (the LINES variant): up to 16 listed tokens of the INT4
// region are read from fp16 rows instead; the INT4 splits mask them out of
// their blocks and split S adds them to its fp16 tokens.
// k_decode_merge: (sequence, query head): merge the S+1 partials in ascending
// split order, 16 at a time.
#include <mutex>
#include <string>

#include "mxq_internal.h"

namespace mxq {
namespace {

constexpr int kD = 128;      // head_dim supported by the decode kernel
constexpr int kWaves = 4;    // waves per workgroup
constexpr int kBlk = 32;     // INT4 tokens per wave block
constexpr int kCodeScale = 136;  // E8M0 of 2^9: a code byte c is the E4M3 value c * 2^-9
constexpr int kMaxLines = 16;    // vertical-line tokens per (sequence, kv head)

struct DecodeArgs {
  const uint16_t* q;  // bf16 [B][Hq][D]
  mxq_kv_cache kv;
  float* ws;          // [B][Hq][S+1][D + 2]
  int Hq, Hkv, S, tokens_per_split;
  float c;            // fl32(scale * log2 e)
};

typedef short s4 __attribute__((ext_vector_type(4)));
typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// max / sum over the 16 lanes of a row (quad_perm 1032, quad_perm 2301, row_half_mirror, row_mirror)
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  return fmaxf(v, dpp<0x140>(v));
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  return v + dpp<0x140>(v);
}
// sum over the 4 rows of 16 lanes (same lane % 16)
__device__ __forceinline__ float rows_sum4(float v) {
  uint32_t u = __float_as_uint(v);
  const auto p16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  u = __float_as_uint(__uint_as_float(p16[0]) + __uint_as_float(p16[1]));
  const auto p32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
}

__device__ __forceinline__ float h_lo(uint32_t u) {
  return static_cast<float>(__builtin_bit_cast(h2, u)[0]);
}
__device__ __forceinline__ float h_hi(uint32_t u) {
  return static_cast<float>(__builtin_bit_cast(h2, u)[1]);
}
__device__ __forceinline__ float half_at(const unsigned int __attribute__((ext_vector_type(2))) u, int g) {
  return g == 0 ? h_lo(u[0]) : g == 1 ? h_hi(u[0]) : g == 2 ? h_lo(u[1]) : h_hi(u[1]);  // fp16 element g of 4
}

typedef unsigned int u4v __attribute__((ext_vector_type(4)));
typedef unsigned int u2v __attribute__((ext_vector_type(2)));

// Buffer resources of one (sequence, kv head) region of the INT4 arrays:
// codes and the four fp16 scale/zero arrays (K scale, K zero, V scale,
// V zero).  Reads past the region (tokens >= L_cap) return zeros instead of
// faulting.
struct Rsrc {
  __amdgpu_buffer_rsrc_t kc, vc;
  __amdgpu_buffer_rsrc_t sz[4];
};
// (bytes is the descriptor's unsigned 32-bit record count: up to 2^31 at
// L_cap = 2^25, so it is carried unsigned and passed as its bit pattern)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t region(const void* base, int64_t off_bytes, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(static_cast<const char*>(base) + off_bytes), 0,
                                           __builtin_bit_cast(int, bytes), 0x00020000);
}

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;

// Per-wave LDS slot of one INT4 block: its V codes [32 rows][64 B].  Four
// slots per wave rotate with the blocks in flight.
constexpr int kSlotBytes = kBlk * (kD / 2);  // 2048
constexpr int kInFlight = 3;                 // blocks whose loads are in flight while one is computed
constexpr int kVmemPerBlk = 8;               // vector-memory instructions issue_blk issues

// Register part of one block: K codes of token t0 + 16*set + (lane%16), group
// lane/16, and dword `lane` of the block's 256-byte span of each scale/zero
// array (token lane/2, half lane%2).
struct KBlk {
  u4v kc[2];
  uint32_t sz[4];
};

// Issue one block's loads (kVmemPerBlk vector-memory instructions): K codes
// and scale/zero spans into registers, the V codes straight into the wave's
// LDS slot (the 16 bytes of lane l land at byte 16 l of each 1 KB half).
// Offsets are formed in 32-bit unsigned arithmetic (the descriptors' range is
// up to 2^31 bytes); t0 = L_cap puts every load past its range: the loads
// still issue (and count) but return zeros without touching memory.
// The slot was last read (LDS reads of the block computed just before) by
// this wave; those reads are waited for before the copies into the slot are
// issued, since a copy's data can land in LDS ahead of a read still queued
// (soon after issue for a load past the range, which never goes to memory).
__device__ __forceinline__ void issue_blk(KBlk& x, const Rsrc& r, int t0, int offk, int lane, lds_char* slot) {
  const uint32_t t = static_cast<uint32_t>(t0);
  const uint32_t ok = static_cast<uint32_t>(offk) + t * (kD / 2);
  x.kc[0] = __builtin_amdgcn_raw_buffer_load_b128(r.kc, __builtin_bit_cast(int, ok), 0, 0);
  x.kc[1] = __builtin_amdgcn_raw_buffer_load_b128(r.kc, __builtin_bit_cast(int, ok + 16u * (kD / 2)), 0, 0);
  const uint32_t os = static_cast<uint32_t>(lane) * 4u + t * 8u;
#pragma unroll
  for (int a = 0; a < 4; ++a)
    x.sz[a] = __builtin_amdgcn_raw_buffer_load_b32(r.sz[a], __builtin_bit_cast(int, os), 0, 0);
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const uint32_t ov = static_cast<uint32_t>(lane) * 16u + t * (kD / 2);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r.vc, (lds_void*)slot, 16, __builtin_bit_cast(int, ov), 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r.vc, (lds_void*)(slot + 1024), 16, __builtin_bit_cast(int, ov + 1024u), 0,
                                          0, 0);
  // keep the block's loads together, ahead of the computation that follows,
  // so that waits for the block being computed never cover these loads
  __builtin_amdgcn_sched_barrier(0);
}

// 32 codes (16 bytes) -> 32 E4M3 bytes: low nibbles (even head_dim elements)
// in dwords 0..3, high nibbles (odd elements) in dwords 4..7.
__device__ __forceinline__ v8i widen_codes(u4v c4) {
  const uint4 c = make_uint4(c4[0], c4[1], c4[2], c4[3]);
  v8i r;
  r[0] = c.x & 0x0F0F0F0F; r[4] = (c.x >> 4) & 0x0F0F0F0F;
  r[1] = c.y & 0x0F0F0F0F; r[5] = (c.y >> 4) & 0x0F0F0F0F;
  r[2] = c.z & 0x0F0F0F0F; r[6] = (c.z >> 4) & 0x0F0F0F0F;
  r[3] = c.w & 0x0F0F0F0F; r[7] = (c.w >> 4) & 0x0F0F0F0F;
  return r;
}

// fp16 sink/recent tokens of one (sequence, kv head): plain fp32 online
// softmax, lane l owns head_dim elements 2l and 2l+1.  Writes the wave's
// partial (m, l, o) to LDS.
template <int G, bool LINES>
__device__ void fp16_tokens(const DecodeArgs& a, int hk, int b, int len, int wave, int lane,
                            float (*s_o)[4][kD], float (*s_ml)[4][2], int lkey) {
  const int64_t bh = static_cast<int64_t>(b) * a.Hkv + hk;
  const int n_sink = a.kv.n_sink, n_recent = a.kv.n_recent;
  const int a0 = min(n_sink, len);
  const int r0 = max(len - n_recent, a0);
  const int nSR = a0 + (len - r0);               // sink and window tokens
  const int nF = nSR + (LINES ? kMaxLines : 0);  // then the line entries (masked when unused)
  const int rec_base = len - n_recent;  // recent row r holds token rec_base + r
  float qf[G][2], m[G], l[G], o[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint32_t qq = *reinterpret_cast<const uint32_t*>(
        a.q + (static_cast<int64_t>(b) * a.Hq + hk * G + h) * kD + 2 * lane);
    qf[h][0] = bf16_to_f32(static_cast<uint16_t>(qq & 0xFFFF));
    qf[h][1] = bf16_to_f32(static_cast<uint16_t>(qq >> 16));
    m[h] = -__builtin_inff(); l[h] = 0.0f; o[h][0] = 0.0f; o[h][1] = 0.0f;
  }
  for (int base = 8 * wave; base < nF; base += 8 * kWaves) {
    uint32_t kk[8], vv[8];
    bool ok[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = base + u;
      kk[u] = 0u; vv[u] = 0u;
      ok[u] = idx < nF;
      if (idx < nSR) {
        const int t = idx < a0 ? idx : r0 + (idx - a0);
        const int64_t off = t < n_sink ? (bh * n_sink + t) * kD : (bh * n_recent + (t - rec_base)) * kD;
        const uint16_t* ks = t < n_sink ? a.kv.k_sink : a.kv.k_recent;
        const uint16_t* vs = t < n_sink ? a.kv.v_sink : a.kv.v_recent;
        kk[u] = *reinterpret_cast<const uint32_t*>(ks + off + 2 * lane);
        vv[u] = *reinterpret_cast<const uint32_t*>(vs + off + 2 * lane);
      } else if (LINES && idx < nF) {
        const int e = idx - nSR;  // line entry (wave-uniform)
        ok[u] = __builtin_amdgcn_readlane(lkey, e) >= 0;
        if (ok[u]) {
          const int64_t off = (bh * a.kv.n_lines + e) * kD + 2 * lane;
          kk[u] = *reinterpret_cast<const uint32_t*>(a.kv.k_lines + off);
          vv[u] = *reinterpret_cast<const uint32_t*>(a.kv.v_lines + off);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool valid = ok[u];
      const float k0 = h_lo(kk[u]), k1 = h_hi(kk[u]), v0 = h_lo(vv[u]), v1 = h_hi(vv[u]);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float sc = __builtin_fmaf(qf[h][0], k0, qf[h][1] * k1);
        sc = rows_sum4(row_sum16(sc));
        const float x = valid ? sc * a.c : -__builtin_inff();
        const float mn = fmaxf(m[h], x);
        const float fac = m[h] == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m[h] - mn);
        const float p = x == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(x - mn);
        l[h] = __builtin_fmaf(l[h], fac, p);
        o[h][0] = __builtin_fmaf(o[h][0], fac, p * v0);
        o[h][1] = __builtin_fmaf(o[h][1], fac, p * v1);
        m[h] = mn;
      }
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    s_o[wave][h][2 * lane] = o[h][0];
    s_o[wave][h][2 * lane + 1] = o[h][1];
    if (lane == 0) { s_ml[wave][h][0] = m[h]; s_ml[wave][h][1] = l[h]; }
  }
}

typedef __attribute__((address_space(3))) s4 lds_s4;

// Softmax state of one wave: running max m_run (log2 units) of head lane/16,
// the lane's partial row sum and zero-point sums, and the PV accumulators.
struct St {
  float m_run, l_run;
  float Z[4];
  v4f O[8];
};
template <int G>
struct Ctx {
  v8i qa_hi, qa_lo;
  int sc_hi, sc_lo;
  float qs[4];
  float c;
  int end, tl, hl;
  lds_s4* rd0;
  lds_s4* rd1;
  uint2* wr;   // this wave's [16 tokens][4 heads] fp16x4 staging of p*s, tokens 0..15
  uint2* wr2;  // tokens 16..31
  int lane;
};

// The LDS pointers are restrict parameters: after inlining, their accesses
// carry alias scopes, which lets the compiler's wait insertion see that reads
// of this block's slot do not depend on loads still landing in other slots.
// lmask bit j: token t0 + j is a vertical line, read elsewhere (masked here)
template <int G>
__device__ __forceinline__ void process_blk(St& S, const Ctx<G>& cx, const KBlk& x,
                                            const lds_char* __restrict__ slot, u2v* __restrict__ szw,
                                            uint2* __restrict__ wr, uint2* __restrict__ wr2,
                                            lds_s4* __restrict__ rd0, lds_s4* __restrict__ rd1, int t0,
                                            uint32_t lmask) {
  // this block's V codes have landed once only the later blocks' loads may
  // still be in flight (vector-memory loads complete in order); the compiler
  // does not track loads that write LDS directly
  __asm__ volatile("s_waitcnt vmcnt(24)" ::: "memory");  // kInFlight * kVmemPerBlk
  const int tl = cx.tl, hl = cx.hl;
  // scale/zero rows: lane l holds dword l of each array's span; share them
  // through LDS ([array][32 tokens] of 8-byte rows) so that each lane has the
  // four rows of its own tokens
  {
    uint32_t* w = reinterpret_cast<uint32_t*>(szw) + cx.lane;
#pragma unroll
    for (int a = 0; a < 4; ++a) w[64 * a] = x.sz[a];
  }
  __asm__ volatile("" ::: "memory");
  u2v sz[2][4];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
#pragma unroll
    for (int a = 0; a < 4; ++a) sz[st][a] = szw[32 * a + 16 * st + tl];
    // V scale and zero rows of tokens past the range are zeroed, so that the
    // zero weight of such a token cannot meet garbage from beyond the sequence
    if (t0 + 16 * st + tl >= cx.end) { sz[st][2] = u2v{0u, 0u}; sz[st][3] = u2v{0u, 0u}; }
  }
  // scores of tokens t0 + 16*st + tl for head hl
  float xs[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const v8i bk = widen_codes(x.kc[st]);
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(cx.qa_hi, bk, acc, 0, 0, 0, cx.sc_hi, 0, kCodeScale);
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(cx.qa_lo, bk, acc, 0, 0, 0, cx.sc_lo, 0, kCodeScale);
    float sc = 0.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      sc = __builtin_fmaf(half_at(sz[st][0], g), acc[g], sc);
      sc = __builtin_fmaf(half_at(sz[st][1], g), cx.qs[g], sc);
    }
    const bool live = t0 + 16 * st + tl < cx.end && !((lmask >> (16 * st + tl)) & 1u);
    xs[st] = live ? sc * cx.c : -__builtin_inff();
  }
  const float mx = row_max16(fmaxf(xs[0], xs[1]));
  const float m_new = fmaxf(S.m_run, mx);
  if (__builtin_amdgcn_ballot_w64(m_new > S.m_run) != 0) {
    const float fac = S.m_run == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(S.m_run - m_new);
    S.l_run *= fac;
#pragma unroll
    for (int g = 0; g < 4; ++g) S.Z[g] *= fac;
#pragma unroll
    for (int i = 0; i < 8; ++i) S.O[i] *= fac;
    S.m_run = m_new;
  }
  const float m_use = S.m_run == -__builtin_inff() ? 0.0f : S.m_run;
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    // tokens past the range have x = -inf (p = 0) and zeroed scale rows;
    // head rows beyond G are never read back
    const float p = __builtin_amdgcn_exp2f(xs[st] - m_use);
    S.l_run += p;
#pragma unroll
    for (int g = 0; g < 4; ++g) S.Z[g] = __builtin_fmaf(p, half_at(sz[st][3], g), S.Z[g]);
    // p * s in fp16 (p rounded to fp16 first: two roundings of 2^-11 each)
    const _Float16 ph = static_cast<_Float16>(p);
    const h2 pp = {ph, ph};
    // (the vector elements go through named scalars: __builtin_bit_cast of an
    // element expression like v[1] is compiled as a cast of element 0 by this
    // hipcc, so the second pair silently became a copy of the first)
    const uint32_t vs01 = sz[st][2][0], vs23 = sz[st][2][1];
    const h2 p01 = pp * __builtin_bit_cast(h2, vs01);
    const h2 p23 = pp * __builtin_bit_cast(h2, vs23);
    (st == 0 ? wr : wr2)[tl * 4 + hl] = uint2{__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23)};
  }
  __asm__ volatile("" ::: "memory");
  const s4 ra = __builtin_amdgcn_ds_read_tr16_b64_v4i16(rd0);
  const s4 rb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(rd1);
  __asm__ volatile("" ::: "memory");
  // A operand: row 4h+g, K slot e = token 4e + lane/16
  const v4i pai = __builtin_shufflevector(__builtin_bit_cast(v2i_t, ra), __builtin_bit_cast(v2i_t, rb), 0, 1, 2, 3);
  const v8h pA = __builtin_bit_cast(v8h, pai);
  // B operand of head_dim column 8*(lane%16) + dd, tokens 4e + lane/16:
  // byte kb of the lane's code dword holds columns 2kb (low nibble) and 2kb+1
  // (high nibble); each code becomes the fp16 subnormal 16*code*2^-24, i.e.
  // the nibble moved to bits 4..7 of a zero-extended byte
  // rows 4e + (lane/16), e = 0..7, dword lane%16 (K slot e of the B operand
  // is token 4e + lane/16; the A operand above uses the same order)
  typedef const __attribute__((address_space(3))) uint32_t lds_u32;
  lds_u32* vb = (lds_u32*)slot + 16 * hl + tl;
  uint32_t hiR[8], loR[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t v = vb[64 * e];
    hiR[e] = v & 0xF0F0F0F0u;
    loR[e] = (v << 4) & 0xF0F0F0F0u;
  }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const uint32_t sel = static_cast<uint32_t>(kb) | (0x0Cu << 8) | ((4u + kb) << 16) | (0x0Cu << 24);
    v4i bhi, blo;
#pragma unroll
    for (int rp = 0; rp < 4; ++rp) {
      bhi[rp] = static_cast<int>(__builtin_amdgcn_perm(hiR[2 * rp + 1], hiR[2 * rp], sel));
      blo[rp] = static_cast<int>(__builtin_amdgcn_perm(loR[2 * rp + 1], loR[2 * rp], sel));
    }
    S.O[2 * kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pA, __builtin_bit_cast(v8h, blo), S.O[2 * kb], 0, 0, 0);
    S.O[2 * kb + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pA, __builtin_bit_cast(v8h, bhi), S.O[2 * kb + 1], 0, 0, 0);
  }
}

template <int G, bool LINES>
__global__ void __launch_bounds__(256, 3) k_decode_split(DecodeArgs a) {
  __shared__ float s_o[kWaves][4][kD];
  __shared__ float s_ml[kWaves][4][2];
  // fp16 p*s_v of (token, head), 4 groups each: tokens 0..15, then 16..31
  __shared__ uint2 s_p[kWaves][kBlk / 2][4];
  __shared__ uint2 s_p2[kWaves][kBlk / 2][4];
  // INT4 blocks in flight, one array per slot (separate objects, so that
  // reads of one slot never wait for loads still landing in another)
  __shared__ __align__(16) char s_blk0[kWaves][kSlotBytes];
  __shared__ __align__(16) char s_blk1[kWaves][kSlotBytes];
  __shared__ __align__(16) char s_blk2[kWaves][kSlotBytes];
  __shared__ __align__(16) char s_blk3[kWaves][kSlotBytes];
  __shared__ u2v s_sz[kWaves][4 * kBlk];  // scale/zero rows of the block being computed
  const int s = blockIdx.x;
  const int hk = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int len = min(a.kv.seq_len[b], a.kv.L_cap);  // never read past the cache

  // Vertical lines (R33): lane e < 16 of every wave holds entry e's token when
  // it lies in the INT4 region [n_sink, len - n_recent) and exceeds every
  // earlier entry (an exclusive prefix maximum by DPP row shifts), else -1
  int lkey = -1;
  if constexpr (LINES) {
    const int e = lane & 15;
    const int raw = (lane < 16 && e < a.kv.n_lines)
                        ? a.kv.lines[(static_cast<int64_t>(b) * a.Hkv + hk) * a.kv.n_lines + e] : -1;
    constexpr int kMin = -2147483647 - 1;
    int pm = raw;
    pm = max(pm, __builtin_amdgcn_update_dpp(kMin, pm, 0x111, 0xF, 0xF, false));  // row_shr:1
    pm = max(pm, __builtin_amdgcn_update_dpp(kMin, pm, 0x112, 0xF, 0xF, false));  // row_shr:2
    pm = max(pm, __builtin_amdgcn_update_dpp(kMin, pm, 0x114, 0xF, 0xF, false));  // row_shr:4
    pm = max(pm, __builtin_amdgcn_update_dpp(kMin, pm, 0x118, 0xF, 0xF, false));  // row_shr:8
    const int before = __builtin_amdgcn_update_dpp(kMin, pm, 0x111, 0xF, 0xF, false);
    if (lane < 16 && raw >= a.kv.n_sink && raw < len - a.kv.n_recent && raw > before) lkey = raw;
  }
  // line tokens inside the 32-token block starting at t
  auto line_mask = [&](int t) -> uint32_t {
    if constexpr (!LINES) {
      return 0u;
    } else {
      uint64_t bal = __ballot(lkey >= t && lkey < t + kBlk);
      uint32_t m = 0;
      while (bal) {
        const int e = __builtin_ctzll(bal);
        m |= 1u << (__builtin_amdgcn_readlane(lkey, e) - t);
        bal &= bal - 1;
      }
      return m;
    }
  };

  if (s == a.S) {
    fp16_tokens<G, LINES>(a, hk, b, len, wave, lane, s_o, s_ml, lkey);
  } else {
    const int64_t bh = static_cast<int64_t>(b) * a.Hkv + hk;
    const int int_lo = min(a.kv.n_sink, len);
    const int int_hi = max(len - a.kv.n_recent, int_lo);
    const int beg = int_lo + s * a.tokens_per_split;
    const int end = min(beg + a.tokens_per_split, int_hi);

    // ---- q operands: row m = 4h + g of the block-diagonal A, lane group jg
    const int mrow = lane & 15, jg = lane >> 4;
    const int hr = mrow >> 2, gr = mrow & 3;
    v8i qa_hi = {0, 0, 0, 0, 0, 0, 0, 0}, qa_lo = {0, 0, 0, 0, 0, 0, 0, 0};
    int sc_hi = 127, sc_lo = 127;
    float qsum = 0.0f;
    if (hr < G) {
      const uint4* qp = reinterpret_cast<const uint4*>(a.q + (static_cast<int64_t>(b) * a.Hq + hk * G + hr) * kD + 32 * gr);
      float x[32];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint4 u = qp[w];
        const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[8 * w + 2 * k] = __uint_as_float(uu[k] << 16);
          x[8 * w + 2 * k + 1] = __uint_as_float(uu[k] & 0xFFFF0000u);
        }
      }
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) { amax = fmaxf(amax, fabsf(x[i])); qsum += x[i]; }
      // hi part: |x| * 2^-e_hi < 256 (E4M3 keeps 4 significant bits); the
      // residual, at most 8 * 2^e_hi, scaled by 2^5 stays below 256 as well
      const uint32_t ef = (__float_as_uint(amax) >> 23) & 0xFF;
      int e_hi = ef == 0 ? -120 : static_cast<int>(ef) - 127 - 7;
      e_hi = max(e_hi, -120);
      sc_hi = 127 + e_hi;
      sc_lo = 127 + e_hi - 5;
      if (jg == gr) {
        const float inv_hi = __builtin_ldexpf(1.0f, -e_hi);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // dword w: even elements 8w, 8w+2, 8w+4, 8w+6; dword 4+w: the odd ones
#pragma unroll
          for (int par = 0; par < 2; ++par) {
            const float y0 = x[8 * w + par] * inv_hi, y1 = x[8 * w + 2 + par] * inv_hi;
            const float y2 = x[8 * w + 4 + par] * inv_hi, y3 = x[8 * w + 6 + par] * inv_hi;
            int hb = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
            hb = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, hb, true);
            const float r0 = (y0 - __builtin_amdgcn_cvt_f32_fp8(hb, 0)) * 32.0f;
            const float r1 = (y1 - __builtin_amdgcn_cvt_f32_fp8(hb, 1)) * 32.0f;
            const float r2 = (y2 - __builtin_amdgcn_cvt_f32_fp8(hb, 2)) * 32.0f;
            const float r3 = (y3 - __builtin_amdgcn_cvt_f32_fp8(hb, 3)) * 32.0f;
            int lb = __builtin_amdgcn_cvt_pk_fp8_f32(r0, r1, 0, false);
            lb = __builtin_amdgcn_cvt_pk_fp8_f32(r2, r3, lb, true);
            qa_hi[4 * par + w] = hb;
            qa_lo[4 * par + w] = lb;
          }
        }
      }
    }
    // group sums of q for the (token, head) lanes: head lane/16, groups 0..3
    const int tl = lane & 15, hl = lane >> 4;
    float qs[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) qs[g] = __shfl(qsum, 4 * hl + g);

    // ---- stream the split's blocks
    St st_;
    st_.m_run = -__builtin_inff();
    st_.l_run = 0.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g) st_.Z[g] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) st_.O[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    Ctx<G> cx;
    cx.qa_hi = qa_hi; cx.qa_lo = qa_lo; cx.sc_hi = sc_hi; cx.sc_lo = sc_lo;
#pragma unroll
    for (int g = 0; g < 4; ++g) cx.qs[g] = qs[g];
    cx.c = a.c; cx.end = end; cx.tl = tl; cx.hl = hl;
    // transposed-read addresses of this lane: token 4(4r + (lane/4)%4) + lane/16, head lane%4
    const int rq = lane >> 4, rk = (lane >> 2) & 3, rh = lane & 3;
    cx.rd0 = (lds_s4*)(&s_p[wave][4 * rk + rq][rh]);
    cx.rd1 = (lds_s4*)(&s_p2[wave][4 * rk + rq][rh]);
    cx.wr = &s_p[wave][0][0];
    cx.wr2 = &s_p2[wave][0][0];
    cx.lane = lane;

    const int L = a.kv.L_cap;
    const uint32_t Lu = static_cast<uint32_t>(L);
    Rsrc rs;
    rs.kc = region(a.kv.k_codes, bh * L * (kD / 2), Lu * (kD / 2));
    rs.vc = region(a.kv.v_codes, bh * L * (kD / 2), Lu * (kD / 2));
    rs.sz[0] = region(a.kv.k_scale, bh * L * 8, Lu * 8);
    rs.sz[1] = region(a.kv.k_zero, bh * L * 8, Lu * 8);
    rs.sz[2] = region(a.kv.v_scale, bh * L * 8, Lu * 8);
    rs.sz[3] = region(a.kv.v_zero, bh * L * 8, Lu * 8);
    const int offk = tl * (kD / 2) + 16 * jg;
    constexpr int kStep = kBlk * kWaves;
    int t0 = beg + kBlk * wave;
    lds_char* sl0 = (lds_char*)&s_blk0[wave][0];
    lds_char* sl1 = (lds_char*)&s_blk1[wave][0];
    lds_char* sl2 = (lds_char*)&s_blk2[wave][0];
    lds_char* sl3 = (lds_char*)&s_blk3[wave][0];
    u2v* szw = &s_sz[wave][0];
    if (t0 < end) {
      // four blocks rotate through registers and LDS slots: a block is
      // computed while the next three blocks' loads are in flight, and its
      // registers and slot are refilled with the block four ahead right after.
      // The loop runs whole groups of four steps with one exit: a step past
      // the range computes nothing (all its tokens are masked), and its loads
      // are issued at token L_cap, past every descriptor's range, so they
      // return zeros without memory traffic (re-reading a block instead went
      // back to HBM once the L2 had moved on: 40 KB per split).  Every step
      // issues the same loads, so the wait count in process_blk holds.
      const int n_steps = (end - t0 + kStep - 1) / kStep;
      const int n_groups = (n_steps + 3) / 4;
      KBlk k0, k1, k2, k3;
#define MXQ_AT(d) (t0 + (d) * kStep < end ? t0 + (d) * kStep : L)
      issue_blk(k0, rs, t0, offk, lane, sl0);
      issue_blk(k1, rs, MXQ_AT(1), offk, lane, sl1);
      issue_blk(k2, rs, MXQ_AT(2), offk, lane, sl2);
      issue_blk(k3, rs, MXQ_AT(3), offk, lane, sl3);
      for (int grp = 0; grp < n_groups; ++grp) {
        process_blk<G>(st_, cx, k0, sl0, szw, cx.wr, cx.wr2, cx.rd0, cx.rd1, t0, line_mask(t0));
        issue_blk(k0, rs, MXQ_AT(4), offk, lane, sl0);
        t0 += kStep;
        process_blk<G>(st_, cx, k1, sl1, szw, cx.wr, cx.wr2, cx.rd0, cx.rd1, t0, line_mask(t0));
        issue_blk(k1, rs, MXQ_AT(4), offk, lane, sl1);
        t0 += kStep;
        process_blk<G>(st_, cx, k2, sl2, szw, cx.wr, cx.wr2, cx.rd0, cx.rd1, t0, line_mask(t0));
        issue_blk(k2, rs, MXQ_AT(4), offk, lane, sl2);
        t0 += kStep;
        process_blk<G>(st_, cx, k3, sl3, szw, cx.wr, cx.wr2, cx.rd0, cx.rd1, t0, line_mask(t0));
        issue_blk(k3, rs, MXQ_AT(4), offk, lane, sl3);
        t0 += kStep;
      }
#undef MXQ_AT
      // the loads past the end still write (zeros to) LDS: let them land
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    const float m_run = st_.m_run, l_run = st_.l_run;
    float Z[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) Z[g] = st_.Z[g];
    v4f O[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) O[i] = st_.O[i];

    // ---- this wave's partial: head hl, head_dim 8*tl .. 8*tl+7 (group tl/4)
    const float l_tot = row_sum16(l_run);
    float Zt[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) Zt[g] = row_sum16(Z[g]);
    const int gsel = tl >> 2;
    const float zsel = gsel == 0 ? Zt[0] : gsel == 1 ? Zt[1] : gsel == 2 ? Zt[2] : Zt[3];
    if (hl < G) {
      float ov[8];
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const v4f o = O[dd];
        const float v = gsel == 0 ? o[0] : gsel == 1 ? o[1] : gsel == 2 ? o[2] : o[3];
        ov[dd] = __builtin_fmaf(v, 1048576.0f, zsel);  // B held code * 2^-20
      }
      float4* dst = reinterpret_cast<float4*>(&s_o[wave][hl][8 * tl]);
      dst[0] = make_float4(ov[0], ov[1], ov[2], ov[3]);
      dst[1] = make_float4(ov[4], ov[5], ov[6], ov[7]);
      if (tl == 0) { s_ml[wave][hl][0] = m_run; s_ml[wave][hl][1] = l_tot; }
    }
  }
  __syncthreads();
  // thread (h, d) merges the 4 waves in order
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
    float* dst = a.ws + ((static_cast<int64_t>(b) * a.Hq + hk * G + h) * (a.S + 1) + s) * (kD + 2);
    dst[d] = ot;
    if (d == 0) { dst[kD] = M; dst[kD + 1] = lt; }
  }
}

// thread (sequence, query head, d): one pass over the splits in ascending
// order, rescaling the running sums whenever a later split's maximum is
// larger.  Partials are loaded 8 splits at a time so the loads overlap.
__global__ void __launch_bounds__(kD) k_decode_merge(const float* __restrict__ ws, float* __restrict__ out,
                                                     int Hq, int S1) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const float* base = ws + (static_cast<int64_t>(b) * Hq + h) * S1 * (kD + 2);
  float M = -__builtin_inff(), lt = 0.0f, ot = 0.0f;
  // 16 partials per round (one round for the default split counts): all loads
  // of a round are in flight together
  constexpr int R = 16;
  for (int s0 = 0; s0 < S1; s0 += R) {
    float ms[R], ls[R], os[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const float* part = base + min(s0 + j, S1 - 1) * (kD + 2);
      ms[j] = s0 + j < S1 ? part[kD] : -__builtin_inff();
      ls[j] = part[kD + 1];
      os[j] = part[d];
    }
#pragma unroll
    for (int j = 0; j < R; ++j) {
      if (ms[j] == -__builtin_inff()) continue;
      const float mn = fmaxf(M, ms[j]);
      const float fo = M == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(M - mn);
      const float fs = __builtin_amdgcn_exp2f(ms[j] - mn);
      lt = __builtin_fmaf(lt, fo, ls[j] * fs);
      ot = __builtin_fmaf(ot, fo, os[j] * fs);
      M = mn;
    }
  }
  out[(static_cast<int64_t>(b) * Hq + h) * kD + d] = ot / lt;
}

int pick_splits(int max_seq_len, int num_splits) {
  if (num_splits > 0) return num_splits;
  int s = (max_seq_len + 4095) / 4096;
  return s < 1 ? 1 : (s > 64 ? 64 : s);
}

}  // namespace
}  // namespace mxq

using namespace mxq;

extern "C" size_t attn_quantkv_decode_workspace(int32_t B, int32_t Hq, int32_t D, int32_t num_splits,
                                                int32_t max_seq_len) {
  if (B <= 0 || Hq <= 0 || D <= 0) return 0;
  const int S = pick_splits(max_seq_len, num_splits);
  return static_cast<size_t>(B) * Hq * (S + 1) * (D + 2) * sizeof(float);
}

namespace mxq {
namespace {

// Host checks shared by both decode entry points; nothing is launched on error.
mxq_status validate_decode(const uint16_t* q, const mxq_kv_cache* kv, int32_t B, int32_t Hq, int32_t Hkv,
                           int32_t D, int32_t max_seq_len, float softmax_scale, int32_t num_splits, float* out) {
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
  MXQ_REQUIRE(kv->n_lines >= 0 && kv->n_lines <= kMaxLines, MXQ_EINVAL,
              "attn_quantkv_decode: n_lines must be in [0, 16]");
  MXQ_REQUIRE(kv->n_lines == 0 || (kv->lines && kv->k_lines && kv->v_lines), MXQ_EINVAL,
              "attn_quantkv_decode: lines, k_lines and v_lines are required when n_lines > 0");
  MXQ_REQUIRE(max_seq_len >= 1 && max_seq_len <= kv->L_cap, MXQ_EINVAL,
              "attn_quantkv_decode: need 1 <= max_seq_len <= L_cap");
  // each (sequence, kv head) region of the code arrays is addressed with
  // 32-bit byte offsets (L_cap * 64 bytes)
  MXQ_REQUIRE(kv->L_cap <= (1 << 25), MXQ_EUNSUPPORTED, "attn_quantkv_decode: L_cap must be <= 2^25");
  MXQ_REQUIRE(num_splits >= 0 && num_splits <= 4096, MXQ_EINVAL, "attn_quantkv_decode: num_splits out of range");
  MXQ_REQUIRE(B <= 65535 && Hkv <= 65535, MXQ_EUNSUPPORTED, "attn_quantkv_decode: B, Hkv must be <= 65535");
  MXQ_REQUIRE(!(softmax_scale != softmax_scale), MXQ_EINVAL, "attn_quantkv_decode: softmax_scale is NaN");
  return MXQ_OK;
}

// Both decode launches on `stream`, with the split partials in `ws` (device
// memory of at least attn_quantkv_decode_workspace(...) bytes).
mxq_status launch_decode(const uint16_t* q, const mxq_kv_cache* kv, int32_t B, int32_t Hq, int32_t Hkv,
                         int32_t D, int32_t max_seq_len, float softmax_scale, int32_t num_splits, float* ws,
                         float* out, hipStream_t st) {
  const int G = Hq / Hkv;
  const int S = pick_splits(max_seq_len, num_splits);
  DecodeArgs a;
  a.q = q; a.kv = *kv; a.ws = ws; a.Hq = Hq; a.Hkv = Hkv; a.S = S;
  // INT4 tokens per split: at most max_seq_len in total, whole 32-token blocks per wave
  int tps = (max_seq_len + S - 1) / S;
  tps = (tps + kWaves * kBlk - 1) / (kWaves * kBlk) * (kWaves * kBlk);
  a.tokens_per_split = tps;
  const double sc = softmax_scale > 0.0f ? static_cast<double>(softmax_scale) : 1.0 / __builtin_sqrt(static_cast<double>(D));
  a.c = static_cast<float>(sc * 1.4426950408889634);
  dim3 grid(S + 1, Hkv, B);
  const bool lines = kv->n_lines > 0;
  switch (G * 2 + (lines ? 1 : 0)) {
    case 2: hipLaunchKernelGGL((k_decode_split<1, false>), grid, dim3(256), 0, st, a); break;
    case 3: hipLaunchKernelGGL((k_decode_split<1, true>), grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_decode_split<2, false>), grid, dim3(256), 0, st, a); break;
    case 5: hipLaunchKernelGGL((k_decode_split<2, true>), grid, dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL((k_decode_split<4, false>), grid, dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL((k_decode_split<4, true>), grid, dim3(256), 0, st, a); break;
  }
  mxq_status stt = check_launch("k_decode_split");
  if (stt != MXQ_OK) return stt;
  hipLaunchKernelGGL(k_decode_merge, dim3(Hq, B), dim3(kD), 0, st, a.ws, out, Hq, S + 1);
  return check_launch("k_decode_merge");
}

}  // namespace
}  // namespace mxq

extern "C" mxq_status attn_quantkv_decode(const uint16_t* q, const mxq_kv_cache* kv, int32_t B,
                                          int32_t Hq, int32_t Hkv, int32_t D, int32_t max_seq_len,
                                          float softmax_scale, int32_t num_splits, void* workspace,
                                          size_t ws_bytes, float* out, mxq_stream_t stream) {
  mxq_status st = validate_decode(q, kv, B, Hq, Hkv, D, max_seq_len, softmax_scale, num_splits, out);
  if (st != MXQ_OK) return st;
  MXQ_REQUIRE(workspace && ws_bytes >= attn_quantkv_decode_workspace(B, Hq, D, num_splits, max_seq_len),
              MXQ_EINVAL, "attn_quantkv_decode: workspace too small");
  return launch_decode(q, kv, B, Hq, Hkv, D, max_seq_len, softmax_scale, num_splits,
                       static_cast<float*>(workspace), out, as_stream(stream));
}

// ---- the allocation-free variant ---------------------------------------------
// The split partials live in this file-scope device array instead of a caller
// workspace.  Each GPU the library runs on holds its own copy for the life of
// the process.  In host code `scratch` names a host-side stand-in, not device
// memory: the device address of the current GPU's copy comes from
// hipGetSymbolAddress, taken once per device and kept in scratch_ptr[].
static __device__ __align__(256) uint8_t scratch[MXQ_DECODE_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (taken under a lock on the first
// call on that device).
mxq_status scratch_for_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return mxq::fail(MXQ_EHIP, std::string("attn_quantkv_decode_noalloc: hipGetDevice: ") +
                                                      hipGetErrorString(e));
  MXQ_REQUIRE(dev >= 0 && dev < kMaxDevices, MXQ_EUNSUPPORTED,
              "attn_quantkv_decode_noalloc: device index beyond 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return mxq::fail(MXQ_EHIP, std::string("attn_quantkv_decode_noalloc: hipGetSymbolAddress: ") +
                                     hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MXQ_OK;
}
}  // namespace

extern "C" mxq_status attn_quantkv_decode_noalloc(const uint16_t* q, const mxq_kv_cache* kv, int32_t B,
                                                  int32_t Hq, int32_t Hkv, int32_t D, int32_t max_seq_len,
                                                  float softmax_scale, int32_t num_splits, float* out,
                                                  mxq_stream_t stream) {
  mxq_status st = validate_decode(q, kv, B, Hq, Hkv, D, max_seq_len, softmax_scale, num_splits, out);
  if (st != MXQ_OK) return st;
  const size_t need = attn_quantkv_decode_workspace(B, Hq, D, num_splits, max_seq_len);
  MXQ_REQUIRE(need <= static_cast<size_t>(MXQ_DECODE_SCRATCH_BYTES), MXQ_EINVAL,
              "attn_quantkv_decode_noalloc: the split partials need " + std::to_string(need) +
                  " bytes, beyond the library's fixed scratch of " +
                  std::to_string(static_cast<size_t>(MXQ_DECODE_SCRATCH_BYTES)) +
                  " bytes (use fewer splits or sequences, or attn_quantkv_decode with a workspace)");
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != MXQ_OK) return st;
  return launch_decode(q, kv, B, Hq, Hkv, D, max_seq_len, softmax_scale, num_splits, static_cast<float*>(ws),
                       out, as_stream(stream));
}

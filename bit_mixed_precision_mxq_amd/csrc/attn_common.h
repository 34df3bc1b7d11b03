// Shared by the attention kernels (attn_mixed.hip: sequences of more than 256
// keys; attn_short.hip: at most 256): launch arguments, the constants of
// the P grid and the online-softmax references, the LDS layouts, lane and
// cross-lane helpers.
#pragma once

#include <type_traits>

#include "mxq_internal.h"

// Products and sums round on their own unless written as __builtin_fmaf: the
// reference exponent ceil(fl32(rowmax * c)) must be one rounded product.
#pragma clang fp contract(off)

namespace mxq {
mxq_status validate_attn_shape(const mxq_attn_shape* s);

namespace attn {

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
  const uint16_t* v_bf16;  // [B*Hkv][N][D]: the line keys' V when v_f16t is NULL
  const uint32_t* mask;
  const int32_t* lines;  // [B*Hq][n_lines] vertical-line keys
  void* out;
  float* lse;
  int Hq, Hkv, N, n_valid, n_qt, words, causal, mode, out_bf16;
  int sel_bq;  // query rows per selection tile (mask row = query row / sel_bq)
  int n_lines;
  int nbh;  // B * Hq
  float c;  // fl32(softmax_scale * log2(e))
  // short-sequence kernel: exact quotients n / d by a multiply-high with
  // ceil(2^32 / d) (0 for d = 1), valid for n * d <= 2^32, so that the
  // workgroup's indices stay scalar (a division would run on the vector ALU)
  uint32_t mg_nt, mg_hq, mg_g;  // for N / 64 query tiles, Hq, Hq / Hkv
  int sel_shift;                // log2(sel_bq)
};

// floor(n / d) from m = ceil(2^32 / d) (m = 0: d = 1); exact for n * d <= 2^32
__device__ __forceinline__ uint32_t mdiv(uint32_t n, uint32_t m) {
  return m ? static_cast<uint32_t>((static_cast<uint64_t>(n) * m) >> 32) : n;
}

// Work-item and workgroup ids straight from the hardware registers.  The
// attention files are compiled with IEEE mode off, so the device library's id
// helpers, built with it on, are not inlined: threadIdx/blockIdx become calls,
// and values derived from them land in vector registers.  The short-sequence
// kernel uses these (its prologue is a large share of its time); the long
// kernel keeps the library helpers, called once per workgroup, because its
// main loop was measured to schedule slower with the intrinsics.
__device__ __forceinline__ int lane_tid() { return static_cast<int>(__builtin_amdgcn_workitem_id_x()); }
__device__ __forceinline__ uint32_t wg_x() { return __builtin_amdgcn_workgroup_id_x(); }

constexpr float kGridMagic = kPGridMagic;  // 1.5 * 2^12: spacing 2^-11 in [2^12, 2^13)
constexpr float kExpOffset = 8.0f;     // P is stored as E4M3(2^(x + 8)) * 2^-8
constexpr int kPScale = 119;           // E8M0 code of 2^-8
constexpr float kMaxLag = 64.0f;       // largest gap kept between O's reference and the running one
constexpr float kMaxLag16 = 15.0f;     // the same for FP16 tiles, whose P must stay below 2^16
constexpr int kMaxChunks = 1024;       // 128-key chunks: 2048 key tiles of 64
constexpr int kMaxLines = 16;          // vertical-line keys per head: one 16-key MFMA block

// fp16 bits of a line key's V element: the fp16 V^T copy's value, or the
// bf16 value rounded to fp16 (to nearest, ties to even: the rounding of the
// fp16 copy) when the values come straight from bf16 V.
__device__ __forceinline__ uint32_t line_v_f16(uint32_t raw, bool from_bf16) {
  return from_bf16 ? __builtin_bit_cast(uint16_t, static_cast<_Float16>(__uint_as_float(raw << 16))) : raw;
}

// Key (within the 128-key chunk) that A-operand row r of S-block beta holds.
__device__ __forceinline__ int chunk_key(int beta, int r) {
  return 64 * (beta >> 2) + 16 * (r >> 2) + 4 * (beta & 3) + (r & 3);
}

__device__ __forceinline__ float wave_rowmax(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// max of three scores.  The attention files are compiled with NaNs not
// honoured and the IEEE mode bit off (scores are finite or -inf, never NaN), so fmaxf needs no
// canonicalising moves and maps to one v_max3_f32.
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Row maximum over the 4 lane groups (lanes col, col+16, col+32, col+48) with
// two cross-row swaps (v_permlane16_swap / v_permlane32_swap), no LDS traffic.
// Row maxima of two values at once (a: tile 0, b: tile 1): one swap pairs the
// groups of a with those of b, a second folds the halves, a third hands each
// lane the other value.  Three swaps and two maxima instead of four and four.
__device__ __forceinline__ void rowmax4x2(float a, float b, float& ra, float& rb) {
  const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  // group 0: a of groups 0/1, 1: b of 0/1, 2: a of 2/3, 3: b of 2/3
  const uint32_t m = __float_as_uint(fmaxf(__uint_as_float(p16[0]), __uint_as_float(p16[1])));
  const auto p32 = __builtin_amdgcn_permlane32_swap(m, m, false, false);
  // groups 0 and 2: max of a; groups 1 and 3: max of b
  const uint32_t r = __float_as_uint(fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1])));
  const auto q16 = __builtin_amdgcn_permlane16_swap(r, r, false, false);
  ra = __uint_as_float(q16[0]);
  rb = __uint_as_float(q16[1]);
}

__device__ __forceinline__ float rowmax4(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto p16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float m1 = fmaxf(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
  const uint32_t u1 = __float_as_uint(m1);
  const auto p32 = __builtin_amdgcn_permlane32_swap(u1, u1, false, false);
  return fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
}

// LDS layouts.  Low-bit chunks (128 keys) live in two rings: K (four
// buffers) and V (three buffers); the FP16 tile stage, the workgroup's bf16 Q
// rows and constants follow.  Codes and FP16 tiles are written by direct
// global-to-LDS loads, 1 KB (64 lanes x 16 B) per wave instruction, so every
// layout is a permutation of 16-byte units inside contiguous rows.
// Bank rule the swizzles are built for (gfx950, measured): a 16-byte-per-lane
// LDS read serves each 32-lane half of the wave in two cycles of 16 lanes, the
// lane quads of even index parity (lanes 0-3, 12-15, 20-23, 24-27 of the
// half) in one and the odd ones in the other; a cycle is conflict-free when
// its 16 lanes touch 16 distinct 16-byte slots modulo 256 bytes.
//  K buffer: FP4 K rows of D/2 bytes; D = 128: the 16-byte unit index XOR 2 *
//    key bit 5, D = 64: rows whose key bit 5 is set swap bit 2 of the row
//    index; then the K scales, byte [g][col][beta] = scale of block g of the
//    key that S block beta's row col holds (one 8-byte read per lane serves
//    all 8 QK MFMAs, op_sel picks the byte).
//  V buffer: FP8 V^T rows (one per head_dim element, 128 keys = 8 units), unit u
//    of row d stored at u ^ ((d >> 1) & 7) (an operand read takes units g and
//    g + 4); then the V scales, byte [g][col][db] = scale of key block g of
//    row 16*db+col.
//  FP16 stages, one per tile of a chunk (64 keys each): bf16 K rows of 2*D
//    bytes, unit index XOR-swizzled by 4 key bits; fp16 V^T rows of 128 bytes,
//    unit u of row d stored at u ^ (d bit 1) ^ 4 * (d bit 3) (an operand read
//    takes units 2g and 2g + 1).  (The bf16 Q the FP16 tiles multiply stays
//    in registers: each lane needs only its own row's slices.)
//  Vertical lines: bf16 K rows of the 16 line entries (swizzled like Q) and
//    their fp16 V as [d][entry], loaded once.
template <int D>
struct Lds {
  static constexpr int KROW = D / 2;
  static constexpr int NSB = D / 32;
  static constexpr int RK = 4, RV = 3;           // ring buffers
  static constexpr int KS_IN = 128 * KROW;       // K scales inside a K buffer
  static constexpr int K_BYTES = KS_IN + 512;
  static constexpr int VS_IN = D * 128;          // V scales inside a V buffer
  static constexpr int V_BYTES = VS_IN + 512;
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = K_OFF + RK * K_BYTES;
  static constexpr int HK_OFF = V_OFF + RV * V_BYTES;     // FP16 stage 0: bf16 K tile
  static constexpr int HV_OFF = HK_OFF + 64 * 2 * D;      //   and fp16 V^T tile
  static constexpr int STAGE = 64 * 2 * D + D * 128;      // bytes per FP16 stage (stage t: tile t of a chunk)
  static constexpr int LK_OFF = HK_OFF + 2 * STAGE;       // bf16 K rows of the line entries
  static constexpr int LV_OFF = LK_OFF + kMaxLines * 2 * D;  // fp16 V of the lines, [d][entry]
  static constexpr int BYTES = LV_OFF + D * kMaxLines * 2;
  // K codes of (key, 16-byte unit g) inside a K buffer
  __device__ static __forceinline__ int k_off(int key, int g) {
    if constexpr (D == 128) {
      return key * KROW + 16 * (g ^ (2 * ((key >> 5) & 1)));
    } else {
      return k_row(key) * KROW + 16 * g;
    }
  }
  // D = 64 row of a key (an involution: key bit 5 is left as it is)
  __device__ static __forceinline__ int k_row(int key) { return key ^ (((key >> 5) & 1) << 2); }
  // 128-byte row d, 16-byte unit u (FP8 V^T of 128 keys or fp16 V^T of 64)
  __device__ static __forceinline__ int vrow_off(int d, int u) { return d * 128 + 16 * (u ^ ((d >> 1) & 7)); }
  // fp16 V^T row d of an FP16 stage, unit u
  __device__ static __forceinline__ int hv_swz(int d) { return ((d >> 1) & 1) | (((d >> 3) & 1) << 2); }
  __device__ static __forceinline__ int hvrow_off(int d, int u) { return d * 128 + 16 * (u ^ hv_swz(d)); }
  __device__ static __forceinline__ int hk_swz(int key) {
    if constexpr (D == 128) return (key & 3) | ((key >> 2) & 12);
    else return ((key >> 1) & 1) | ((key >> 3) & 6);
  }
  __device__ static __forceinline__ int hk_off(int key, int cidx) {  // key in [0,64)
    return HK_OFF + key * 2 * D + 16 * (cidx ^ hk_swz(key));
  }
  __device__ static __forceinline__ int lk_off(int e, int u) {
    return LK_OFF + e * 2 * D + 16 * (u ^ (e & (D / 8 - 1)));
  }
};


// One FP4 x FP4 QK block: S^T[16 keys x 16 queries] over the whole head_dim.
// The key's scale byte is selected from the packed word by op_sel (beta & 3).
#define MXQ_QK_BLOCK(OPSEL) \
  __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qf4, v4f{0.f, 0.f, 0.f, 0.f}, 4, 4, OPSEL, sc, 0, qsc)
#define MXQ_PV_BLOCK(OPSEL) \
  __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(va, pb, o, 0, 0, OPSEL, vs, 0, psc)

// Launch of the short-sequence kernel (attn_short.hip), head_dim D = 64 or 128.
mxq_status launch_short(const AttnArgs& a, int D, hipStream_t st);

}  // namespace attn
}  // namespace mxq

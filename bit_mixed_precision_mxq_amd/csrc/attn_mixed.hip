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
  int sel_bq;  // query rows per selection tile (mask row = query row / sel_bq)
  float c;  // fl32(softmax_scale * log2(e))
};

constexpr float kGridMagic = 6144.0f;  // 1.5 * 2^12: spacing 2^-11 in [2^12, 2^13)
constexpr float kExpOffset = 8.0f;     // P is stored as E4M3(2^(x + 8)) * 2^-8
constexpr int kPScale = 119;           // E8M0 code of 2^-8
constexpr float kMaxLag = 64.0f;       // largest gap kept between O's reference and the running one
constexpr int kMaxChunks = 1024;       // 128-key chunks: 2048 key tiles of 64

// Key (within the 128-key chunk) that A-operand row r of S-block beta holds.
__device__ __forceinline__ int chunk_key(int beta, int r) {
  return 64 * (beta >> 2) + 16 * (r >> 2) + 4 * (beta & 3) + (r & 3);
}

__device__ __forceinline__ float wave_rowmax(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// max of three scores.  This file is compiled with NaNs not honoured and the
// IEEE mode bit off (scores are finite or -inf, never NaN), so fmaxf needs no
// canonicalising moves and maps to one v_max3_f32.
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Row maximum over the 4 lane groups (lanes col, col+16, col+32, col+48) with
// two cross-row swaps (v_permlane16_swap / v_permlane32_swap), no LDS traffic.
__device__ __forceinline__ float rowmax4(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto p16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float m1 = fmaxf(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
  const uint32_t u1 = __float_as_uint(m1);
  const auto p32 = __builtin_amdgcn_permlane32_swap(u1, u1, false, false);
  return fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
}

// LDS layouts.
//  Low-bit chunk (128 keys, a ring of three buffers):
//   K codes: FP4 rows of D/2 bytes (D/32 chunks of 16 bytes), the chunk index
//     XOR-swizzled with key bits so the 16 rows one MFMA operand read touches
//     fall in distinct banks (for D = 64 rows also swap 4 apart);
//   K scales: byte [g][col][beta] = scale of block g of the key that S block
//     beta's row col holds, so one 8-byte read per lane serves all 8 QK MFMAs
//     (op_sel picks the byte);
//   V codes: FP8 V^T rows (one per head_dim element, 128 keys) padded to 144 B;
//   V scales: byte [g][col][db] = scale of key block g of row 16*db+col.
//  FP16 tile (64 keys, one buffer): bf16 K rows of 2*D bytes with the 16-byte
//  chunk index XOR-swizzled by 4 key bits; fp16 V^T rows padded to 144 bytes.
//  bf16 Q of the workgroup's 128 rows (read by the FP16 tiles' QK), loaded once.
template <int D>
struct Lds {
  static constexpr int KROW = D / 2;
  static constexpr int NSB = D / 32;
  static constexpr int VSTRIDE = 144;
  static constexpr int K_OFF = 0;
  static constexpr int KS_OFF = K_OFF + 128 * KROW;
  static constexpr int V_OFF = KS_OFF + 512;
  static constexpr int VS_OFF = V_OFF + D * VSTRIDE;
  static constexpr int LO_BYTES = VS_OFF + 512;
  static constexpr int RING = 3;                          // low-bit chunk buffers
  static constexpr int HK_OFF = RING * LO_BYTES;          // bf16 K tile
  static constexpr int HV_OFF = HK_OFF + 64 * 2 * D;      // fp16 V^T tile
  static constexpr int ONES_OFF = HV_OFF + D * VSTRIDE;   // 32 B of E4M3 1.0, 16 B of fp16 1.0
  static constexpr int Q_OFF = ONES_OFF + 48;             // bf16 Q tile of the workgroup
  static constexpr int BYTES = Q_OFF + 128 * 2 * D;
  // bf16 Q row r, 16-byte unit u (8 head_dim elements), XOR-swizzled by the row
  __device__ static __forceinline__ int q_off(int r, int u) {
    return Q_OFF + r * 2 * D + 16 * (u ^ (r & (D / 8 - 1)));
  }
  __device__ static __forceinline__ int k_off(int key, int g) {
    if constexpr (D == 128) {
      return K_OFF + key * KROW + 16 * (g ^ ((key >> 4) & 3));
    } else {
      const int row = key ^ ((key >> 2) & 4);
      return K_OFF + row * KROW + 16 * (g ^ ((key >> 5) & 1));
    }
  }
  __device__ static __forceinline__ int hk_off(int key, int cidx) {  // key in [0,64)
    int f;
    if constexpr (D == 128) f = (key & 3) | ((key >> 2) & 12);
    else f = ((key >> 1) & 1) | ((key >> 3) & 6);
    return HK_OFF + key * 2 * D + 16 * (cidx ^ f);
  }
};


// One FP4 x FP4 QK block: S^T[16 keys x 16 queries] over the whole head_dim.
// The key's scale byte is selected from the packed word by op_sel (beta & 3).
#define MXQ_QK_BLOCK(OPSEL) \
  __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qf4, v4f{0.f, 0.f, 0.f, 0.f}, 4, 4, OPSEL, sc, 0, qsc)
#define MXQ_PV_BLOCK(OPSEL) \
  __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(va, pb, o, 0, 0, OPSEL, vs, 0, psc)

template <int D>
__global__ void __launch_bounds__(512, 1) k_attn_mixed(AttnArgs a) {
  using LY = Lds<D>;
  constexpr int BQ = 128;        // query rows per workgroup
  constexpr int NT = 512;        // 8 waves of 16 rows
  constexpr int KROW = D / 2;
  constexpr int NDB = D / 16;    // 16-row head_dim blocks of O^T
  constexpr int NSB = D / 32;    // MX blocks per row, and K=32 steps of the bf16 MFMA
  constexpr int KUNITS = 128 * KROW / 16;   // 16-byte K-code units per chunk
  constexpr int KU = (KUNITS + NT - 1) / NT;
  constexpr int VU = D * 8 / NT;            // 16-byte V-code units per thread
  static_assert(D * 8 % NT == 0, "V units must divide evenly");
  constexpr float NEG_INF = -__builtin_inff();

  __shared__ __attribute__((aligned(16))) uint8_t sm[LY::BYTES];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 15;   // query column within the wave's 16 rows
  const int g = lane >> 4;     // lane group 0..3
  // Work order: workgroups are dispatched in linear id order, round-robin
  // over the 8 XCDs.  Linear id L takes query tile n_qt-1 - L/Hq (longest
  // causal tiles of every head first, then shorter ones fill in) and, when Hq
  // is a multiple of 8, head (Hq/8)*(L%8) + (L%Hq)/8, so that each XCD (and
  // its L2) serves a contiguous block of query heads, i.e. whole kv groups.
  const int lin = static_cast<int>(blockIdx.x) + a.n_qt * static_cast<int>(blockIdx.y);
  const int it = a.n_qt - 1 - lin / a.Hq;
  const int hr = lin % a.Hq;
  const int h = (a.Hq % 8 == 0) ? (a.Hq / 8) * (hr % 8) + hr / 8 : hr;
  const int b = blockIdx.z;
  const int G = a.Hq / a.Hkv;
  const int64_t bhq = static_cast<int64_t>(b) * a.Hq + h;
  const int64_t bhk = static_cast<int64_t>(b) * a.Hkv + h / G;
  const int qs = it * BQ;
  const int q = qs + wave * 16 + col;  // this lane's query row

  if (qs >= a.n_valid) {  // a tile of padding rows: output 0, lse -inf
    for (int idx = tid; idx < BQ * D; idx += NT) {
      int64_t o = (bhq * a.N + qs) * D + idx;
      if (a.out_bf16) static_cast<uint16_t*>(a.out)[o] = 0;
      else static_cast<float*>(a.out)[o] = 0.0f;
    }
    if (a.lse)
      for (int r = tid; r < BQ; r += NT) a.lse[bhq * a.N + qs + r] = NEG_INF;
    return;
  }
  const int qe = min(qs + BQ, a.n_valid) - 1;
  int last_tile = (a.n_valid - 1) / 64;
  if (a.causal) last_tile = min(last_tile, qe / 64);
  const int n_chunks = (last_tile + 2) / 2;
  const int wq_lo = qs + wave * 16;                 // this wave's first row
  const bool wave_live = wq_lo < a.n_valid;

  // FP4 Q fragment (B operand of S^T = K Q^T), held for the whole pass
  v8i qf4 = {0, 0, 0, 0, 0, 0, 0, 0};
  int qsc = 127;
  if (a.mode != MXQ_ALL_FP16 && g < NSB) {
    const v4i w = *reinterpret_cast<const v4i*>(a.q_codes + (bhq * a.N + q) * KROW + 16 * g);
    qf4[0] = w[0]; qf4[1] = w[1]; qf4[2] = w[2]; qf4[3] = w[3];
    qsc = a.q_scales[(bhq * a.N + q) * NSB + g];
  }

  v4f O[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) O[i] = v4f{0.f, 0.f, 0.f, 0.f};
  v4f L = {0.f, 0.f, 0.f, 0.f};
  float m_run = NEG_INF;   // running integer reference (log2 units)
  float m_o = NEG_INF;     // reference O and L are currently expressed in
  const float c = a.c;

  // Promotion flags.  Selection tiles are 64 or 128 rows high, so the
  // workgroup's 128 rows lie in one or two mask rows (ra, rb) and each wave's
  // 16 rows in one of them.  Each wave uses the flags of its own row; staging
  // uses the union (FP16 data some wave needs) and the intersection (low-bit
  // data is needed unless every wave promotes the tile).  The two rows' bits
  // are unpacked once per workgroup into one byte per chunk in LDS.
  const int64_t mbase = bhq * (a.N / a.sel_bq);
  const uint32_t* mrow_a = a.mask ? a.mask + (mbase + qs / a.sel_bq) * a.words : nullptr;
  const uint32_t* mrow_b = a.mask ? a.mask + (mbase + (qs + BQ - 1) / a.sel_bq) * a.words : nullptr;
  const bool w_in_b = wq_lo / a.sel_bq != qs / a.sel_bq;
  auto row_flags = [&](const uint32_t* mr, int ch) -> int {  // bit t: tile t of chunk ch is FP16
    const int j0 = 2 * ch;
    const bool valid1 = j0 + 1 <= last_tile;
    if (a.mode == MXQ_ALL_FP16) return 1 | (valid1 ? 2 : 0);
    if (a.mode == MXQ_ALL_LOWBIT) return 0;
    const uint32_t wbits = mr[j0 >> 5];
    return static_cast<int>((wbits >> (j0 & 31)) & 1u) |
           (valid1 ? static_cast<int>(((wbits >> ((j0 + 1) & 31)) & 1u) << 1) : 0);
  };
  __shared__ uint8_t s_fl[kMaxChunks];  // per chunk: bits 0-1 row ra, bits 2-3 row rb
  for (int ch = tid; ch < n_chunks; ch += NT)
    s_fl[ch] = static_cast<uint8_t>(row_flags(mrow_a, ch) | (row_flags(mrow_b, ch) << 2));
  // packed: bits 0-1 this wave, 2-3 any wave, 4-5 every wave
  auto chunk_flags = [&](int ch) -> int {
    const int v = __builtin_amdgcn_readfirstlane(static_cast<int>(s_fl[ch]));
    const int fa = v & 3, fb = v >> 2;
    return (w_in_b ? fb : fa) | ((fa | fb) << 2) | ((fa & fb) << 4);
  };
  auto needs_low = [&](int ch, int fl) -> bool {
    const int all = (fl >> 4) & 3;
    return !(all & 1) || ((2 * ch + 1 <= last_tile) && !(all & 2));
  };
  auto rebase = [&](float m) {  // rescale O and L from m_o to m >= m_o (powers of two)
    if (__any(m != m_o)) {
      float f = 1.0f;
      if (m_o != NEG_INF && m != m_o) f = __builtin_ldexpf(1.0f, static_cast<int>(fmaxf(m_o - m, -256.0f)));
#pragma unroll
      for (int i = 0; i < NDB; ++i) O[i] *= f;
      L *= f;
    }
    m_o = m;
  };

  // ---- staging registers for one chunk of low-bit K and V
  v4i pk[KU], pv[VU];
  uint32_t pks = 0, pvs = 0;
  auto stage_load = [&](int ch) {
    const int kc = ch * 128;
    const v4i* kg = reinterpret_cast<const v4i*>(a.k_codes + (bhk * a.N + kc) * KROW);
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int u = tid + i * NT;
      if (u < KUNITS) pk[i] = kg[u];
    }
    if (tid < 128 * NSB) pks = a.k_scales[(bhk * a.N + kc) * NSB + tid];
#pragma unroll
    for (int i = 0; i < VU; ++i) {
      const int u = tid + i * NT;
      pv[i] = *reinterpret_cast<const v4i*>(a.v_codes + (bhk * D + (u >> 3)) * a.N + kc + 16 * (u & 7));
    }
    if (tid < D) pvs = *reinterpret_cast<const uint32_t*>(a.v_scales + (bhk * D + tid) * (a.N / 32) + kc / 32);
  };
  auto stage_store = [&](uint8_t* sb) {
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int u = tid + i * NT;
      if (u < KUNITS) *reinterpret_cast<v4i*>(sb + LY::k_off(u / NSB, u % NSB)) = pk[i];
    }
    if (tid < 128 * NSB) {  // K scale of (key, block kg) -> [kg][col][beta]
      const int key = tid / NSB, kg = tid % NSB;
      const int kcol = 4 * ((key >> 4) & 3) + (key & 3);
      const int kbeta = 4 * (key >> 6) + ((key >> 2) & 3);
      sb[LY::KS_OFF + (kg * 16 + kcol) * 8 + kbeta] = static_cast<uint8_t>(pks);
    }
#pragma unroll
    for (int i = 0; i < VU; ++i) {
      const int u = tid + i * NT;
      *reinterpret_cast<v4i*>(sb + LY::V_OFF + (u >> 3) * LY::VSTRIDE + 16 * (u & 7)) = pv[i];
    }
    if (tid < D) {  // V scales of row d for key blocks 0..3 -> [block][d%16][d/16]
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        sb[LY::VS_OFF + (kb * 16 + (tid & 15)) * 8 + (tid >> 4)] = static_cast<uint8_t>(pvs >> (8 * kb));
    }
  };
  // FP16 tile staging: global loads into registers, then LDS stores
  constexpr int HKU = 64 * 2 * D / 16;  // 16-byte units of the bf16 K tile
  constexpr int HKR = (HKU + NT - 1) / NT, HVR = (D * 8 + NT - 1) / NT;
  auto fp16_tile_load = [&](int kt0, v4i (&hk)[HKR], v4i (&hv)[HVR]) {
#pragma unroll
    for (int i = 0; i < HKR; ++i) {
      const int u = tid + i * NT;
      if (u < HKU) hk[i] = reinterpret_cast<const v4i*>(a.k_bf16 + (bhk * a.N + kt0 + u / (D / 8)) * D)[u % (D / 8)];
    }
#pragma unroll
    for (int i = 0; i < HVR; ++i) {
      const int u = tid + i * NT;
      if (u < D * 8) hv[i] = *reinterpret_cast<const v4i*>(a.v_f16t + (bhk * D + (u >> 3)) * a.N + kt0 + 8 * (u & 7));
    }
  };
  auto fp16_tile_store = [&](const v4i (&hk)[HKR], const v4i (&hv)[HVR]) {
#pragma unroll
    for (int i = 0; i < HKR; ++i) {
      const int u = tid + i * NT;
      if (u < HKU) *reinterpret_cast<v4i*>(sm + LY::hk_off(u / (D / 8), u % (D / 8))) = hk[i];
    }
#pragma unroll
    for (int i = 0; i < HVR; ++i) {
      const int u = tid + i * NT;
      if (u < D * 8) *reinterpret_cast<v4i*>(sm + LY::HV_OFF + (u >> 3) * LY::VSTRIDE + 16 * (u & 7)) = hv[i];
    }
  };

  if (tid < 12) reinterpret_cast<uint32_t*>(sm + LY::ONES_OFF)[tid] = tid < 8 ? 0x38383838u : 0x3C003C00u;
  if constexpr (NSB < 4) {
    // lane groups g >= D/32 carry no head_dim data: their K scale bytes must be
    // a finite E8M0 (0xFF would be NaN), so set them to 127 (= 1.0) once
    constexpr int PAD = (4 - NSB) * 16 * 8;
    for (int i = tid; i < LY::RING * PAD; i += NT)
      sm[(i / PAD) * LY::LO_BYTES + LY::KS_OFF + NSB * 16 * 8 + i % PAD] = 127;
  }

  // per-lane LDS byte offsets (constant over the pass)
  // K fragment of S block beta: a per-lane base plus a constant per block
  // (lane bits and block bits of chunk_key() do not interact in k_off()); no
  // array, so nothing is indexed at run time
  const int kbase0 = LY::k_off(chunk_key(0, col), g);
  const int kbase1 = LY::k_off(chunk_key(1, col), g);
  auto koff = [&](int beta) -> int {
    if constexpr (D == 128) {
      return kbase0 + LY::KROW * (64 * (beta >> 2) + 4 * (beta & 3));
    } else {  // the row swizzle flips key bit 2, i.e. block bit 0
      return (beta & 1 ? kbase1 : kbase0) + LY::KROW * (64 * (beta >> 2) + 4 * (beta & 2));
    }
  };
  const int ksoff = LY::KS_OFF + (g * 16 + col) * 8;
  auto qk_block = [&](const v8i& ka, int sc, int beta) -> v4f {
    switch (beta & 3) {
      case 0: return MXQ_QK_BLOCK(0);
      case 1: return MXQ_QK_BLOCK(1);
      case 2: return MXQ_QK_BLOCK(2);
      default: return MXQ_QK_BLOCK(3);
    }
  };
  auto pv_block = [&](const v8i& va, const v8i& pb, const v4f& o, int vs, int psc, int db) -> v4f {
    switch (db & 3) {
      case 0: return MXQ_PV_BLOCK(0);
      case 1: return MXQ_PV_BLOCK(1);
      case 2: return MXQ_PV_BLOCK(2);
      default: return MXQ_PV_BLOCK(3);
    }
  };
  const int voff = LY::V_OFF + col * LY::VSTRIDE + 16 * g;
  const int vsoff = LY::VS_OFF + (g * 16 + col) * 8;

  // ---- low-bit building blocks (chunk staged in LDS at sb)
  // S^T blocks of the chunk's 128 keys: one FP4 x FP4 MFMA per 16 keys
  auto qk_lowbit = [&](const uint8_t* sb, v4f (&S)[8]) {
    const uint32_t* ksw = reinterpret_cast<const uint32_t*>(sb + ksoff);
    const uint32_t ksc0 = ksw[0], ksc1 = ksw[1];
#pragma unroll
    for (int beta = 0; beta < 8; ++beta) {
      v8i ka = {0, 0, 0, 0, 0, 0, 0, 0};
      const v4i w = *reinterpret_cast<const v4i*>(sb + koff(beta));
      ka[0] = w[0]; ka[1] = w[1]; ka[2] = w[2]; ka[3] = w[3];
      const int sc = beta < 4 ? static_cast<int>(ksc0) : static_cast<int>(ksc1);
      S[beta] = qk_block(ka, sc, beta);
    }
  };
  // running reference after an unmasked low-bit chunk: integer per-tile
  // references m0 <= m1 and, when O's reference lags too far, a rebase
  auto chunk_max = [&](const v4f (&S)[8], float& m0, float& m1) {
    float mx0 = max3f(S[0][0], S[0][1], S[0][2]);
    float mx1 = max3f(S[4][0], S[4][1], S[4][2]);
    mx0 = max3f(mx0, S[0][3], S[1][0]);
    mx1 = max3f(mx1, S[4][3], S[5][0]);
#pragma unroll
    for (int e = 5; e < 16; e += 2) {  // remaining 11 values of each tile, two per v_max3
      const float a0 = S[e >> 2][e & 3], b0 = e + 1 < 16 ? S[(e + 1) >> 2][(e + 1) & 3] : a0;
      const float a1 = S[4 + (e >> 2)][e & 3], b1 = e + 1 < 16 ? S[4 + ((e + 1) >> 2)][(e + 1) & 3] : a1;
      mx0 = max3f(mx0, a0, b0);
      mx1 = max3f(mx1, a1, b1);
    }
    mx0 = rowmax4(mx0);
    mx1 = rowmax4(mx1);
    m0 = fmaxf(m_run, ceilf(mx0 * c));
    m1 = fmaxf(m0, ceilf(mx1 * c));
    m_run = m1;
  };
  auto chunk_lag = [&](float m0, float m1) {
    // O and L stay expressed against a lagging reference m_o <= m0: each
    // tile's contribution is scaled by 2^(m_t - m_o) through the E8M0 scale
    // of its P blocks, so O is only rescaled when the gap grows large
    if (m_o == NEG_INF) m_o = m0;
    if (__any(m1 - m_o > kMaxLag)) rebase(m1);
  };
  auto chunk_refs = [&](const v4f (&S)[8], float& m0, float& m1) {
    chunk_max(S, m0, m1);
    chunk_lag(m0, m1);
  };
  // P = E4M3(2^xq) of one S block (4 scores per lane -> 4 bytes)
  auto p_block = [&](const v4f& s4, float off) -> int {
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s4[i], c, off) - kGridMagic);
    const int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
  };
  // O^T += V^T P^T (FP8 x FP8) and L += sum(P) for a staged chunk
  auto pv_lowbit = [&](const uint8_t* sb, const v8i& pb, int psc) {
    const uint32_t* vsw = reinterpret_cast<const uint32_t*>(sb + vsoff);
    const uint32_t vsc0 = vsw[0], vsc1 = NDB > 4 ? vsw[1] : 0u;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const uint8_t* vrow = sb + voff + 16 * db * LY::VSTRIDE;
      const v4i w0 = *reinterpret_cast<const v4i*>(vrow);
      const v4i w1 = *reinterpret_cast<const v4i*>(vrow + 64);
      const v8i va = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
      const int vs = db < 4 ? static_cast<int>(vsc0) : static_cast<int>(vsc1);
      O[db] = pv_block(va, pb, O[db], vs, psc, db);
    }
    const v8i ones8 = *reinterpret_cast<const v8i*>(sm + LY::ONES_OFF);
    L = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones8, pb, L, 0, 0, 0, 127, 0, psc);
  };

  // ---- main loop over 128-key chunks.
  // Ring protocol: chunk ch+1's low-bit data (loaded into registers during
  // iteration ch-1) is written to its ring buffer at the top of iteration ch,
  // the loads for chunk ch+2 are issued, then one barrier.  After it, chunks ch
  // and ch+1 are both visible, and ring buffer (ch+2)%3 may be overwritten in
  // the next iteration (its previous chunk, ch-1, was finished by every wave
  // before this barrier).
  // Software pipeline for runs of unmasked all-low-bit chunks: while the
  // exponentials of chunk ch are computed, the FP4 QK MFMAs of chunk ch+1 are
  // issued into the score registers just consumed, and the row maxima of chunk
  // ch+1 are taken while the PV MFMAs of chunk ch run.
  v4f S[8];
  float hm0 = 0.0f, hm1 = 0.0f;   // tile references of the chunk whose scores S holds
  bool s_ready = false;           // S already holds the scores of chunk ch
  auto is_hot = [&](int ch, int fl) -> bool {
    const int kc = ch * 128;
    const bool valid1 = 2 * ch + 1 <= last_tile;
    const bool need_mask = (kc + 127 >= a.n_valid) || (a.causal && kc + 127 > wq_lo) || (qe < qs + BQ - 1);
    return !((fl >> 2) & 3) && valid1 && !need_mask;
  };
  // P blocks of the chunk held in S (references hm0, hm1)
  auto p_scale = [&]() -> int {
    // 2^-8 * 2^(m_t - m_o); below 2^-127 (after a forced rebase) the tile adds nothing visible
    return static_cast<int>(fminf(fmaxf(static_cast<float>(kPScale) + ((g < 2 ? hm0 : hm1) - m_o), 0.0f), 254.0f));
  };
  // last chunk of a run: exponentials and PV only
  auto hot_chunk = [&](const uint8_t* sb) {
    const float off0 = kGridMagic + kExpOffset - hm0;  // hm0 is finite: key 0.. are valid
    const float off1 = kGridMagic + kExpOffset - hm1;
    v8i pb;
#pragma unroll
    for (int beta = 0; beta < 8; ++beta) pb[beta] = p_block(S[beta], beta < 4 ? off0 : off1);
    pv_lowbit(sb, pb, p_scale());
  };
  // chunk ch (scores in S) followed by another hot chunk at sbn.  Issue order,
  // fixed with scheduling barriers: the next chunk's K fragments; per S block
  // its exponentials and then the FP4 QK MFMA of the next chunk into the same
  // registers (the vector ALU and the matrix core work side by side); per
  // head_dim block the V fragments two blocks ahead, one PV MFMA and a slice of
  // the next chunk's row maxima.
  auto hot_chunk_next = [&](const uint8_t* sb, const uint8_t* sbn) {
    const float off0 = kGridMagic + kExpOffset - hm0;
    const float off1 = kGridMagic + kExpOffset - hm1;
    const uint32_t* ksw = reinterpret_cast<const uint32_t*>(sbn + ksoff);
    const uint32_t nks0 = ksw[0], nks1 = ksw[1];
    constexpr int KAHEAD = 3;  // K fragments in flight ahead of their MFMA
    v4i kn[8];
#pragma unroll
    for (int beta = 0; beta < KAHEAD; ++beta) kn[beta] = *reinterpret_cast<const v4i*>(sbn + koff(beta));
    __builtin_amdgcn_sched_barrier(0);
    v8i pb;
#pragma unroll
    for (int beta = 0; beta < 8; ++beta) {
      if (beta + KAHEAD < 8) kn[beta + KAHEAD] = *reinterpret_cast<const v4i*>(sbn + koff(beta + KAHEAD));
      pb[beta] = p_block(S[beta], beta < 4 ? off0 : off1);
      const v8i ka = {kn[beta][0], kn[beta][1], kn[beta][2], kn[beta][3], 0, 0, 0, 0};
      S[beta] = qk_block(ka, beta < 4 ? static_cast<int>(nks0) : static_cast<int>(nks1), beta);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int psc = p_scale();
    const uint32_t* vsw = reinterpret_cast<const uint32_t*>(sb + vsoff);
    const uint32_t vsc0 = vsw[0], vsc1 = NDB > 4 ? vsw[1] : 0u;
    auto vload = [&](int db) -> v8i {
      const uint8_t* vrow = sb + voff + 16 * db * LY::VSTRIDE;
      const v4i w0 = *reinterpret_cast<const v4i*>(vrow);
      const v4i w1 = *reinterpret_cast<const v4i*>(vrow + 64);
      return v8i{w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
    };
    v8i va[NDB];
    va[0] = vload(0);
    va[1] = vload(1);
    constexpr int SPB = 8 / NDB;  // S blocks reduced per PV step
    float mx0 = NEG_INF, mx1 = NEG_INF;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      if (db + 2 < NDB) va[db + 2] = vload(db + 2);
      O[db] = pv_block(va[db], pb, O[db], db < 4 ? static_cast<int>(vsc0) : static_cast<int>(vsc1), psc, db);
#pragma unroll
      for (int j = 0; j < SPB; ++j) {
        const int beta = db * SPB + j;
        float& mx = beta < 4 ? mx0 : mx1;
        mx = max3f(mx, S[beta][0], S[beta][1]);
        mx = max3f(mx, S[beta][2], S[beta][3]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    const v8i ones8 = *reinterpret_cast<const v8i*>(sm + LY::ONES_OFF);
    L = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones8, pb, L, 0, 0, 0, 127, 0, psc);
    mx0 = rowmax4(mx0);
    mx1 = rowmax4(mx1);
    hm0 = fmaxf(m_run, ceilf(mx0 * c));
    hm1 = fmaxf(hm0, ceilf(mx1 * c));
    m_run = hm1;
    chunk_lag(hm0, hm1);
  };

  if (a.mode != MXQ_ALL_LOWBIT) {  // bf16 Q rows of the workgroup -> LDS (rows past N are never read)
    constexpr int QU = 128 * D / 8;  // 16-byte units
#pragma unroll
    for (int i = 0; i < (QU + NT - 1) / NT; ++i) {
      const int u = tid + i * NT;
      if (u < QU) {
        const int r = u / (D / 8), cu = u % (D / 8);
        *reinterpret_cast<v4i*>(sm + LY::q_off(r, cu)) =
            *reinterpret_cast<const v4i*>(a.q_bf16 + (bhq * a.N + qs + r) * D + 8 * cu);
      }
    }
  }
  // the Q fragment is used in every chunk: wait for it here, once
  asm volatile("" ::"v"(qsc), "v"(qf4[0]), "v"(qf4[1]), "v"(qf4[2]), "v"(qf4[3]));
  __syncthreads();  // s_fl and the constant LDS words are written
  int f_cur = chunk_flags(0);
  int f_nxt = n_chunks > 1 ? chunk_flags(1) : 0;
  if (needs_low(0, f_cur)) {  // chunk 0 is published before the first barrier
    stage_load(0);
    stage_store(sm);
  }
  bool have_next = false;
  if (n_chunks > 1 && needs_low(1, f_nxt)) {
    stage_load(1);
    have_next = true;
  }
  int slot = 0;  // ring buffer of chunk ch

  for (int ch = 0; ch < n_chunks; ++ch) {
    const int kc = ch * 128;
    const bool valid1 = 2 * ch + 1 <= last_tile;
    const int slot1 = slot == LY::RING - 1 ? 0 : slot + 1;
    const uint8_t* sb = sm + slot * LY::LO_BYTES;
    uint8_t* sbn = sm + slot1 * LY::LO_BYTES;
    if (have_next) stage_store(sbn);
    have_next = false;
    int f_nn = 0;
    if (ch + 2 < n_chunks) {
      f_nn = chunk_flags(ch + 2);
      if (needs_low(ch + 2, f_nn)) {
        stage_load(ch + 2);
        have_next = true;
      }
    }
    // A general chunk with FP16 tiles: the first such tile's K and V and this
    // wave's bf16 Q fragment are fetched before the barrier, so their latency
    // overlaps the wait.
    const bool hot = is_hot(ch, f_cur);
    const int t_first = (f_cur & 4) ? 0 : 1;  // first tile some wave promotes
    v4i hk[HKR], hv[HVR];
    v8bf qb[NSB];
    __syncthreads();

    if (hot) {
      // ================= hot path: both tiles low-bit for every wave, no masks
      if (!s_ready) {
        qk_lowbit(sb, S);
        chunk_refs(S, hm0, hm1);
      }
      const bool hot_next = ch + 1 < n_chunks && is_hot(ch + 1, f_nxt);
      if (hot_next) hot_chunk_next(sb, sbn);
      else hot_chunk(sb);
      s_ready = hot_next;
    } else {
      s_ready = false;
      const bool need_mask = (kc + 127 >= a.n_valid) || (a.causal && kc + 127 > wq_lo) || (qe < qs + BQ - 1);
      // ================= general path: masks, FP16 tiles, a lone last tile
      const bool low_w = !(f_cur & 1) || (valid1 && !(f_cur & 2));  // this wave runs FP8 PV
      v8i pb = {0, 0, 0, 0, 0, 0, 0, 0};
      float m_tile0 = NEG_INF;
#pragma unroll 1
      for (int t = 0; t < 2; ++t) {
        if (t == 1 && !valid1) break;
        const bool prom = (f_cur >> t) & 1;            // this wave's tile t is FP16
        const bool stage_hi = (f_cur >> (2 + t)) & 1;  // some wave's tile t is FP16
        if (stage_hi) {
          // the stage's previous users finished before the chunk barrier,
          // unless it holds this chunk's tile 0
          if (t != t_first) __syncthreads();
          fp16_tile_load(kc + 64 * t, hk, hv);
          fp16_tile_store(hk, hv);
          __syncthreads();
        }
        v4f S[4];
        if (prom) {
#pragma unroll
          for (int st = 0; st < NSB; ++st) qb[st] = *reinterpret_cast<const v8bf*>(sm + LY::q_off(wave * 16 + col, 4 * st + g));
#pragma unroll
          for (int st = 0; st < NSB; ++st) {
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
              const int key = 16 * (col >> 2) + 4 * bb + (col & 3);
              const v8bf ka = *reinterpret_cast<const v8bf*>(sm + LY::hk_off(key, 4 * st + g));
              S[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[st], st == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : S[bb], 0, 0, 0);
            }
          }
        } else {
          const uint32_t kscw = reinterpret_cast<const uint32_t*>(sb + ksoff)[t];
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            v8i ka = {0, 0, 0, 0, 0, 0, 0, 0};
            const v4i w = *reinterpret_cast<const v4i*>(sb + (t ? koff(4 + bb) : koff(bb)));
            ka[0] = w[0]; ka[1] = w[1]; ka[2] = w[2]; ka[3] = w[3];
            const int sc = static_cast<int>(kscw >> (8 * bb)) & 0xFF;
            S[bb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qf4, v4f{0.f, 0.f, 0.f, 0.f}, 4, 4, 0,
                                                                       sc, 0, qsc);
          }
        }
        if (need_mask) {
#pragma unroll
          for (int bb = 0; bb < 4; ++bb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = kc + 64 * t + 16 * g + 4 * bb + i;
              const bool ok = key < a.n_valid && q < a.n_valid && (!a.causal || key <= q);
              if (!ok) S[bb][i] = NEG_INF;
            }
        }
        float mx = NEG_INF;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) mx = fmaxf(fmaxf(mx, fmaxf(S[bb][0], S[bb][1])), fmaxf(S[bb][2], S[bb][3]));
        mx = rowmax4(mx);
        const float m_t = fmaxf(m_run, ceilf(mx * c));
        m_run = m_t;
        if (t == 0) m_tile0 = m_t;
        const float m_safe = m_t == NEG_INF ? 0.0f : m_t;
        if (prom) {
          rebase(m_t);
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            v8h ph;
#pragma unroll
            for (int e = 0; e < 8; ++e)
              ph[e] = static_cast<_Float16>(__builtin_amdgcn_exp2f(__builtin_fmaf(S[2 * st + (e >> 2)][e & 3], c, -m_safe)));
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
              const v8h va = *reinterpret_cast<const v8h*>(sm + LY::HV_OFF + (16 * db + col) * LY::VSTRIDE + 32 * g + 16 * st);
              O[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, ph, O[db], 0, 0, 0);
            }
            const v8h ones16 = *reinterpret_cast<const v8h*>(sm + LY::ONES_OFF + 32);
            L = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones16, ph, L, 0, 0, 0);
          }
        } else {
          const float off = kGridMagic + kExpOffset - m_safe;
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            float y[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[bb][i], c, off) - kGridMagic);
            int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
            pb[4 * t + bb] = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
          }
        }
      }
      if (low_w) {
        rebase(m_run);
        int psc = kPScale;
        if (g < 2) {
          const float gap = m_run - m_tile0;
          psc = (m_tile0 == NEG_INF || gap >= static_cast<float>(kPScale)) ? 0 : kPScale - static_cast<int>(gap);
        }
        const uint32_t* vsw = reinterpret_cast<const uint32_t*>(sb + vsoff);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const uint8_t* vrow = sb + voff + 16 * db * LY::VSTRIDE;
          const v4i w0 = *reinterpret_cast<const v4i*>(vrow);
          const v4i w1 = *reinterpret_cast<const v4i*>(vrow + 64);
          const v8i va = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
          const int vs = static_cast<int>(vsw[db >> 2] >> (8 * (db & 3))) & 0xFF;
          O[db] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(va, pb, O[db], 0, 0, 0, vs, 0, psc);
        }
        const v8i ones8 = *reinterpret_cast<const v8i*>(sm + LY::ONES_OFF);
        L = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones8, pb, L, 0, 0, 0, 127, 0, psc);
      }
    }
    f_cur = f_nxt;
    f_nxt = f_nn;
    slot = slot1;
  }

  // ---------------------------------------------------------------- epilogue
  // out = O / l is independent of the reference; lse uses O's reference m_o
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
      uint2 pk2 = make_uint2(bf(o0) | (bf(o1) << 16), bf(o2) | (bf(o3) << 16));
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + obase + d0) = pk2;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(a.out) + obase + d0) = make_float4(o0, o1, o2, o3);
    }
  }
  if (a.lse && g == 0) {
    a.lse[bhq * a.N + q] = row_ok ? (m_o + __log2f(l)) * 0.69314718055994531f : NEG_INF;
  }
  (void)wave_live;
}

template <int D>
mxq_status launch(const AttnArgs& a, int n_qt, int Hq, int B, hipStream_t st) {
  hipLaunchKernelGGL((k_attn_mixed<D>), dim3(n_qt, Hq, B), dim3(512), 0, st, a);
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
  a.sel_bq = s->Bq;
  a.c = static_cast<float>(sc * 1.4426950408889634);
  hipStream_t strm = as_stream(stream);
  // 128-row workgroups of 8 waves whatever the selection tile height (the
  // mask row is looked up per row block); two workgroups share a CU.
  const int n_qt = s->N / 128;
  a.n_qt = n_qt;
  if (s->D == 128) return launch<128>(a, n_qt, s->Hq, s->B, strm);
  return launch<64>(a, n_qt, s->Hq, s->B, strm);
}

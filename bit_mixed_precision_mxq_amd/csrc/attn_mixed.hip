// attn_mixed_fwd: stage 2 of ThriftAttention (abstract) -- selected query-key
// tiles in FP16, the rest in block-scaled low bit, merged through one online
// softmax into a single output.  HyQuant (abstract): sink and local-window
// tiles are among the high-precision ones (the selection mask carries them).
//
// Work decomposition (gfx950, wave64):
//   workgroup = (batch, query head, query tile of 128 rows), 8 waves, one per
//               CU (two waves per SIMD);
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
//   Softmax: row max within a lane (v_max3) and across the 4 lane groups
//   (permlane swaps), integer-snapped running reference per tile,
//   P = E4M3(2^xq) with xq on the 2^-11 grid (one FMA, one subtraction,
//   v_exp_f32, v_cvt_pk_fp8_f32), FP16 tiles fp16(2^x).
//   O^T[d x 16 queries] += V^T . P^T: v_mfma_scale_f32_16x16x128_f8f6f4 (FP8 x
//   FP8) per 16 head_dim rows; each 64-key tile's reference enters through
//   the E8M0 scale of its P blocks (2^-8 times 2^(tile reference - O's
//   reference)), so O is rescaled only when that gap grows large; one more
//   MFMA with an all-ones A operand accumulates l = sum(P).  FP16 tiles add
//   their contribution with v_mfma_f32_16x16x32_f16.
// Vertical-line tokens (HyQuant): up to 16 single keys per head, listed by the
// caller, run as one FP16 tile ahead of the chunks: S^T[16 entries x 16
// queries] with the bf16 MFMA, P = fp16(2^x), PV with the 16x16x16 fp16 MFMA;
// those keys are masked out of their own tiles, so the chunks holding them
// take the general path.  A kernel variant without lines carries none of it.
// Runs of unmasked all-low-bit chunks are software-pipelined inside each wave:
// the QK MFMAs of chunk c+1 are issued between the exponentials of chunk c,
// and the row maxima of chunk c+1 between its PV MFMAs.  Masked chunks (the
// causal diagonal, padding) and chunks holding FP16 tiles take a general path.
// Exact skips: a 16-key block whose largest score gives P = 0 for every row
// of the wave (the same grid FMA the exponentials use decides) gets P = 0
// without exponentials; a chunk with no such block skips its PV; an FP16
// tile's 32-key half whose fp16 P rounds to 0 everywhere skips its work.
// Staging: the workgroup's K and V chunks arrive in LDS by direct
// global-to-LDS copies, K two chunks and V one chunk before they are needed
// (rings of four and three buffers, one barrier per chunk); a promoted tile's
// bf16 K and fp16 V^T are copied into a stage one chunk ahead when the stage
// is free; each lane's bf16 Q slices for the FP16 tiles stay in registers.
#include "attn_common.h"

namespace mxq {
namespace attn {
namespace {

// LINES: vertical-line tokens are present (n_lines > 0); without them the
// kernel carries none of their code.
// GH: query heads per workgroup.  GH = 1: the workgroup's 8 waves take 128
// rows of one head.  GH = G = Hq / Hkv (2 or 4): one workgroup serves the G
// query heads of a kv group (HyQuant's signals shared by the heads of a
// group): 8 / G waves per head, 128 / G rows of each, and the mask row and
// line list of the group's first head apply to all of them (attn_select_blocks
// and attn_select_lines with group_shared write identical rows for the G
// heads, reading R35 and R31).  Each row's arithmetic is the same either way.
template <int D, bool LINES, int GH>
__global__ void __launch_bounds__(512, 1) k_attn_mixed(AttnArgs a) {
  using LY = Lds<D>;
  constexpr int BQ = 128 / GH;   // query rows per head and workgroup
  constexpr int WPH = 8 / GH;    // waves per head
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
  // over the 8 XCDs.  Linear id L takes query tile n_qt-1 - L/H (longest
  // causal tiles of every head first, then shorter ones fill in; H = Hq, or
  // Hkv when a workgroup serves a kv group) and, when H is a multiple of 8,
  // head (H/8)*(L%8) + (L%H)/8, so that each XCD (and its L2) serves a
  // contiguous block of heads, i.e. whole kv groups.
  const int nh = GH == 1 ? a.Hq : a.Hkv;
  const int lin = static_cast<int>(blockIdx.x) + a.n_qt * static_cast<int>(blockIdx.y);
  const int it = a.n_qt - 1 - lin / nh;
  const int hr = lin % nh;
  const int hs = (nh % 8 == 0) ? (nh / 8) * (hr % 8) + hr / 8 : hr;  // head, or kv head when GH > 1
  const int b = blockIdx.z;
  const int G = a.Hq / a.Hkv;
  const int h = GH == 1 ? hs : hs * GH + wave / WPH;  // this wave's query head
  const int64_t bhq = static_cast<int64_t>(b) * a.Hq + h;
  const int64_t bhq0 = GH == 1 ? bhq : static_cast<int64_t>(b) * a.Hq + hs * GH;  // mask and line rows
  const int64_t bhk = static_cast<int64_t>(b) * a.Hkv + h / G;
  const int qs = it * BQ;
  const int wrow = (GH == 1 ? wave : wave % WPH) * 16;  // this wave's first row within the tile
  const int q = qs + wrow + col;  // this lane's query row

  if (qs >= a.n_valid) {  // a tile of padding rows: output 0, lse -inf
    if constexpr (GH == 1) {
      for (int idx = tid; idx < BQ * D; idx += NT) {
        int64_t o = (bhq * a.N + qs) * D + idx;
        if (a.out_bf16) static_cast<uint16_t*>(a.out)[o] = 0;
        else static_cast<float*>(a.out)[o] = 0.0f;
      }
      if (a.lse)
        for (int r = tid; r < BQ; r += NT) a.lse[bhq * a.N + qs + r] = NEG_INF;
    } else {  // each wave its own head's 16 rows
      for (int idx = lane; idx < 16 * D; idx += 64) {
        int64_t o = (bhq * a.N + qs + wrow) * D + idx;
        if (a.out_bf16) static_cast<uint16_t*>(a.out)[o] = 0;
        else static_cast<float*>(a.out)[o] = 0.0f;
      }
      if (a.lse && lane < 16) a.lse[bhq * a.N + qs + wrow + lane] = NEG_INF;
    }
    return;
  }
  const int qe = min(qs + BQ, a.n_valid) - 1;
  int last_tile = (a.n_valid - 1) / 64;
  if (a.causal) last_tile = min(last_tile, qe / 64);
  last_tile = __builtin_amdgcn_readfirstlane(last_tile);
  const int n_chunks = (last_tile + 2) / 2;
  const int wq_lo = __builtin_amdgcn_readfirstlane(qs + wrow);  // this wave's first row
  const bool wave_live = wq_lo < a.n_valid;

  // Buffer resources over slices of the operands: reads past a slice return
  // zeros instead of faulting.
  // (base, size) pass through readfirstlane so that the resource is built in
  // scalar registers even where its offset arithmetic ran on the vector ALU
  auto rsrc = [](const void* base, int64_t off_bytes, int64_t bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base) + (base ? off_bytes : 0);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32));
    const int n = __builtin_amdgcn_readfirstlane(static_cast<int>(base ? bytes : 0));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo), 0, n,
                                             0x00020000);
  };

  // FP4 Q fragment (B operand of S^T = K Q^T), held for the whole pass.  Lane
  // groups g >= D/32 carry no head_dim block: their offsets fall past the
  // slice, so they read zero codes and a zero scale byte (2^-127, finite).
  // Unconditional buffer loads land straight in the fragment's registers, so
  // nothing waits for them before the prologue's other loads are out.
  // (In MXQ_ALL_FP16 mode the codes may be absent: a null base gives an empty
  // slice, so the loads return zeros there too.)
  const auto r_qc = rsrc(a.q_codes, bhq * a.N * KROW, static_cast<int64_t>(a.N) * KROW);
  const auto r_qs = rsrc(a.q_scales, bhq * a.N * NSB, static_cast<int64_t>(a.N) * NSB);
  const v4i qw = __builtin_bit_cast(
      v4i, __builtin_amdgcn_raw_buffer_load_b128(r_qc, g < NSB ? q * KROW + 16 * g : a.N * KROW, 0, 0));
  const v8i qf4 = {qw[0], qw[1], qw[2], qw[3], 0, 0, 0, 0};
  const int qsc = __builtin_amdgcn_raw_buffer_load_b8(r_qs, g < NSB ? q * NSB + g : a.N * NSB, 0, 0);

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
  const int64_t mbase = bhq0 * (a.N / a.sel_bq);
  const uint32_t* mrow_a = a.mask ? a.mask + (mbase + qs / a.sel_bq) * a.words : nullptr;
  const uint32_t* mrow_b = a.mask ? a.mask + (mbase + (qs + BQ - 1) / a.sel_bq) * a.words : nullptr;
  const bool w_in_b = __builtin_amdgcn_readfirstlane(static_cast<int>(wq_lo / a.sel_bq != qs / a.sel_bq)) != 0;
  // bit t: tile t of chunk ch is FP16; wbits is the mask word holding tile 2ch
  auto row_flags = [&](uint32_t wbits, int ch) -> int {
    const int j0 = 2 * ch;
    const bool valid1 = j0 + 1 <= last_tile;
    if (a.mode == MXQ_ALL_FP16) return 1 | (valid1 ? 2 : 0);
    if (a.mode == MXQ_ALL_LOWBIT) return 0;
    return static_cast<int>((wbits >> (j0 & 31)) & 1u) |
           (valid1 ? static_cast<int>(((wbits >> ((j0 + 1) & 31)) & 1u) << 1) : 0);
  };
  auto mask_word = [&](const uint32_t* mr, int ch) -> uint32_t {
    return a.mode == MXQ_MIXED ? mr[(2 * ch) >> 5] : 0u;
  };
  // The prologue's loads go out before anything waits: this thread's first
  // mask words (chunk tid) and line entry here, the first chunks' K/V copies
  // and scales and the Q rows below; the flags, lines and scales are then
  // unpacked while the copies land.
  const uint32_t mw_a = tid < n_chunks ? mask_word(mrow_a, tid) : 0u;
  const uint32_t mw_b = tid < n_chunks ? mask_word(mrow_b, tid) : 0u;
  // the line list through the scalar unit (its own wait counter, so the
  // dependent gathers below need not wait for the vector loads in flight):
  // 16 loads with indices clamped to the row, then entry e to lane e
  int line_raw = -1;
  if constexpr (LINES) {
    const uint64_t pa = reinterpret_cast<uint64_t>(a.lines + bhq0 * a.n_lines);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(pa));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(pa >> 32));
    typedef const __attribute__((address_space(4))) int32_t cint;
    cint* lrow = reinterpret_cast<cint*>((static_cast<uint64_t>(hi) << 32) | lo);
    int raw_s[kMaxLines];
#pragma unroll
    for (int e = 0; e < kMaxLines; ++e) raw_s[e] = lrow[min(e, a.n_lines - 1)];
#pragma unroll
    for (int e = 0; e < kMaxLines; ++e) line_raw = (lane == e && e < a.n_lines) ? raw_s[e] : line_raw;
  }
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

  // ---- staging.  Buffer resources (built above) over this (batch, kv
  // head)'s slices: reads past a slice return zeros instead of faulting.
  const bool lowbit = a.mode != MXQ_ALL_FP16;  // low-bit operands exist
  const auto r_kc = rsrc(a.k_codes, bhk * a.N * KROW, static_cast<int64_t>(a.N) * KROW);
  const auto r_ks = rsrc(a.k_scales, bhk * a.N * NSB, static_cast<int64_t>(a.N) * NSB);
  const auto r_vc = rsrc(a.v_codes, bhk * D * a.N, static_cast<int64_t>(D) * a.N);
  const auto r_vs = rsrc(a.v_scales, bhk * D * (a.N / 32), static_cast<int64_t>(D) * (a.N / 32));
  const auto r_hk = rsrc(a.k_bf16, bhk * a.N * D * 2, static_cast<int64_t>(a.N) * D * 2);
  const auto r_hv = rsrc(a.v_f16t, bhk * D * a.N * 2, static_cast<int64_t>(D) * a.N * 2);
  const bool lv_bf16 = a.v_f16t == nullptr;  // line V from bf16 V rows (no FP16 tile is promoted)
  const auto r_lv = lv_bf16 ? rsrc(a.v_bf16, bhk * a.N * D * 2, static_cast<int64_t>(a.N) * D * 2) : r_hv;
  uint8_t* const kring = sm + LY::K_OFF;
  uint8_t* const vring = sm + LY::V_OFF;
  // One wave's share of a direct global -> LDS copy: 64 lanes x 16 B land
  // contiguously at dst (a wave-uniform LDS address).
  auto dma16 = [](const __amdgpu_buffer_rsrc_t& r, uint8_t* dst, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, 0, 0, 0);
  };
  // Per iteration every wave issues the same vector-memory instructions in
  // the same order: the scale loads (registers), one K-code copy and D/64
  // V-code copies.  kRegOps is the fewest of them any wave issues.
  constexpr int kRegOps = D == 128 ? 4 : 2;
  // keeps the compiler from moving memory operations across it: the wait
  // counts rely on the order in which the copies are issued
  auto issue_fence = []() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // K codes of chunk ch -> K buffer kb: wave w fills rows 16w..16w+15
  auto k_dma = [&](int ch, uint8_t* kb) {
    const int kc = ch * 128;
    if constexpr (D == 128) {
      const int key = 16 * wave + (lane >> 2);
      const int gu = (lane & 3) ^ (2 * ((key >> 5) & 1));
      dma16(r_kc, kb + 1024 * wave, (kc + key) * KROW + 16 * gu);
    } else {
      if (lane < 32) {
        const int key = LY::k_row(16 * wave + (lane >> 1));
        dma16(r_kc, kb + 512 * wave, (kc + key) * KROW + 16 * (lane & 1));
      }
    }
  };
  // V^T codes of chunk ch -> V buffer vb: 8 rows per 1 KB
  auto v_dma = [&](int ch, uint8_t* vb) {
    const int kc = ch * 128;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
      const int blk = i * 8 + wave;
      const int d = blk * 8 + (lane >> 3);
      const int u = (lane & 7) ^ ((d >> 1) & 7);
      dma16(r_vc, vb + 1024 * blk, d * a.N + kc + 16 * u);
    }
  };
  uint32_t pks = 0, pvs = 0;  // scales in flight (one iteration)
  auto ks_fetch = [&](int ch) -> uint32_t {
    return tid < 128 * NSB ? __builtin_amdgcn_raw_buffer_load_b8(r_ks, ch * 128 * NSB + tid, 0, 0) : 0u;
  };
  auto ks_load = [&](int ch) {
    if (tid < 128 * NSB) pks = __builtin_amdgcn_raw_buffer_load_b8(r_ks, ch * 128 * NSB + tid, 0, 0);
  };
  auto vs_load = [&](int ch) {
    if (tid < D) pvs = __builtin_amdgcn_raw_buffer_load_b32(r_vs, tid * (a.N / 32) + ch * 4, 0, 0);
  };
  auto ks_store = [&](uint8_t* kb) {  // K scale of (key, block kg) -> [kg][col][beta]
    if (tid < 128 * NSB) {
      const int key = tid / NSB, kg = tid % NSB;
      const int kcol = 4 * ((key >> 4) & 3) + (key & 3);
      const int kbeta = 4 * (key >> 6) + ((key >> 2) & 3);
      kb[LY::KS_IN + (kg * 16 + kcol) * 8 + kbeta] = static_cast<uint8_t>(pks);
    }
  };
  auto vs_store = [&](uint8_t* vb) {  // V scales of row d for key blocks 0..3 -> [block][d%16][d/16]
    if (tid < D) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        vb[LY::VS_IN + (kb * 16 + (tid & 15)) * 8 + (tid >> 4)] = static_cast<uint8_t>(pvs >> (8 * kb));
    }
  };
  // FP16 tile (64 keys from kt0) -> stage t: bf16 K rows and fp16 V^T rows
  auto fp16_dma = [&](int kt0, int t) {
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {  // bf16 K: 2*D bytes per key
      const int blk = i * 8 + wave;
      const int o = blk * 1024 + 16 * lane;
      const int key = o / (2 * D), cu = (o % (2 * D)) / 16;
      dma16(r_hk, sm + LY::HK_OFF + t * LY::STAGE + 1024 * blk, (kt0 + key) * 2 * D + 16 * (cu ^ LY::hk_swz(key)));
    }
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {  // fp16 V^T: 128 bytes per row
      const int blk = i * 8 + wave;
      const int d = blk * 8 + (lane >> 3);
      const int u = (lane & 7) ^ LY::hv_swz(d);
      dma16(r_hv, sm + LY::HV_OFF + t * LY::STAGE + 1024 * blk, d * a.N * 2 + kt0 * 2 + 16 * u);
    }
  };

  auto kbuf = [&](int ch) { return kring + (ch & (LY::RK - 1)) * LY::K_BYTES; };
  auto vbuf = [&](int vslot) { return vring + vslot * LY::V_BYTES; };
  if constexpr (NSB < 4) {
    // lane groups g >= D/32 carry no head_dim data: their K scale bytes must be
    // a finite E8M0 (0xFF would be NaN), so set them to 127 (= 1.0) once
    constexpr int PAD = (4 - NSB) * 16 * 8;
    for (int i = tid; i < LY::RK * PAD; i += NT)
      sm[LY::K_OFF + (i / PAD) * LY::K_BYTES + LY::KS_IN + NSB * 16 * 8 + i % PAD] = 127;
  }
  // chunks 0, 1 (K) and 0 (V) in full, as iterations -3 and -2 would have
  // staged them: copies and scale loads now, scale stores before the barrier
  uint32_t pks0 = 0, pks1 = 0;
  if (lowbit) {
    pks0 = ks_fetch(0);
    pks1 = ks_fetch(1);
    k_dma(0, kbuf(0));
    k_dma(1, kbuf(1));
  }
  issue_fence();

  // Vertical-line keys (HyQuant): entry e of the head's list takes part when
  // 0 <= key < n_valid and it exceeds every earlier entry.  Lane e < 16 of
  // every wave holds entry e's key in lkey (else -1) and, for a used entry,
  // lslot = the rank of its 128-key chunk among the chunks holding line keys.
  // (Cross-lane steps use DPP row shifts and readlane, vector-ALU
  // operations: an LDS permute here would have to wait for the copies in
  // flight, since they also write LDS.)
  int lkey = -1, lslot = 0, n_line = 0;
  // exclusive prefix maximum within each row of 16 lanes (INT_MIN before the first)
  auto prefix_max_excl = [](int v) -> int {
    constexpr int kMin = -2147483647 - 1;
    v = max(v, __builtin_amdgcn_update_dpp(kMin, v, 0x111, 0xF, 0xF, false));  // row_shr:1
    v = max(v, __builtin_amdgcn_update_dpp(kMin, v, 0x112, 0xF, 0xF, false));  // row_shr:2
    v = max(v, __builtin_amdgcn_update_dpp(kMin, v, 0x114, 0xF, 0xF, false));  // row_shr:4
    v = max(v, __builtin_amdgcn_update_dpp(kMin, v, 0x118, 0xF, 0xF, false));  // row_shr:8
    return __builtin_amdgcn_update_dpp(kMin, v, 0x111, 0xF, 0xF, false);
  };
  if constexpr (LINES) {
    const int e = lane & 15;
    const int raw = line_raw;
    if (lane < 16 && raw >= 0 && raw < a.n_valid && raw > prefix_max_excl(raw)) lkey = raw;
    // chunk ranks: an entry opens a new chunk when its chunk exceeds every
    // earlier used entry's (used keys ascend)
    const int cb = prefix_max_excl(lkey >= 0 ? (lkey >> 7) : -1);
    const uint64_t opens = __ballot(lane < 16 && lkey >= 0 && (lkey >> 7) > cb);
    lslot = __popcll(opens & ((2ull << e) - 1)) - 1;
    n_line = __popcll(__ballot(lkey >= 0));
  }
  // lkey of lane e (0..15) for a per-lane e: readlanes and selects
  auto lane_key = [&](int e) -> int {
    int k = -1;
#pragma unroll
    for (int x = 0; x < kMaxLines; ++x) k = e == x ? __builtin_amdgcn_readlane(lkey, x) : k;
    return k;
  };
  // the entries' bf16 K rows and fp16 V (zeros for unused entries), one
  // unit of each per thread, issued here with the other prologue loads:
  // buffer loads with out-of-range offsets for unused entries (they read zero)
  constexpr int LU = kMaxLines * D / 8;       // 16-byte units of K
  constexpr int LV = D * (kMaxLines / 4);     // 4-entry groups of V
  static_assert(LU <= NT && LV <= NT, "one line unit per thread");
  const int ke = tid / (D / 8), kcu = tid % (D / 8);
  const int vd = tid / (kMaxLines / 4), ve0 = 4 * (tid % (kMaxLines / 4));
  v4i kw = {0, 0, 0, 0};
  uint32_t hv[4] = {0u, 0u, 0u, 0u};
  if constexpr (LINES) {  // unconditional inside the variant: no merge of values forces a wait
    constexpr int kOut = 0x7FFFFFF0;  // past every slice
    const int kkey = lane_key(ke & 15);
    kw = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                                     r_hk, (tid < LU && kkey >= 0) ? kkey * 2 * D + 16 * kcu : kOut, 0, 0));
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int key = lane_key(ve0 + x);
      const int off = lv_bf16 ? (key * D + vd) * 2 : (vd * a.N + key) * 2;
      hv[x] = __builtin_amdgcn_raw_buffer_load_b16(r_lv, (tid < LV && key >= 0) ? off : kOut, 0, 0);
    }
  }
  issue_fence();

  // all-ones MFMA operands for the row sums (E4M3 1.0 and fp16 1.0), kept in
  // registers: an LDS read here would be made to wait for copies in flight
  constexpr int kOne8 = 0x38383838, kOne16 = 0x3C003C00;
  v8i ones8 = {kOne8, kOne8, kOne8, kOne8, kOne8, kOne8, kOne8, kOne8};
  __asm__ volatile("" : "+v"(ones8));  // kept in registers, not rebuilt before every use

  // per-lane LDS byte offsets (constant over the pass)
  // K fragment of S block beta: a per-lane base plus a constant per block
  // (lane bits and block bits of chunk_key() do not interact in k_off()); no
  // array, so nothing is indexed at run time
  const int kbase0 = LY::k_off(chunk_key(0, col), g);
  const int kbase1 = LY::k_off(chunk_key(1, col), g);
  auto koff = [&](int beta) -> int {
    if constexpr (D == 128) {
      return kbase0 + LY::KROW * (64 * (beta >> 2) + 4 * (beta & 3));
    } else {  // the row swizzle flips key bit 2 (block bit 0) by a lane bit
      return (beta & 1 ? kbase1 : kbase0) + LY::KROW * (64 * (beta >> 2) + 4 * (beta & 2));
    }
  };
  const int ksoff = LY::KS_IN + (g * 16 + col) * 8;  // inside a K buffer
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
  // V fragment of head_dim block db: row 16*db+col, units g and g+4 (keys
  // 16g.. and 64+16g..); the row swizzle depends on col only, and unit g+4
  // sits 64 bytes from unit g's slot (bit 6 flipped)
  const int voff = LY::vrow_off(col, g);  // + 2048*db inside a V buffer
  const int vsoff = LY::VS_IN + (g * 16 + col) * 8;
  auto vfrag = [&](const uint8_t* vb, int db) -> v8i {
    const v4i w0 = *reinterpret_cast<const v4i*>(vb + 2048 * db + voff);
    const v4i w1 = *reinterpret_cast<const v4i*>(vb + 2048 * db + (voff ^ 64));
    return v8i{w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
  };

  // ---- low-bit building blocks (chunk staged in K buffer kb, V buffer vb)
  // S^T blocks of the chunk's 128 keys: one FP4 x FP4 MFMA per 16 keys
  auto qk_lowbit = [&](const uint8_t* kb, v4f (&S)[8]) {
    const uint32_t* ksw = reinterpret_cast<const uint32_t*>(kb + ksoff);
    const uint32_t ksc0 = ksw[0], ksc1 = ksw[1];
#pragma unroll
    for (int beta = 0; beta < 8; ++beta) {
      v8i ka = {0, 0, 0, 0, 0, 0, 0, 0};
      const v4i w = *reinterpret_cast<const v4i*>(kb + koff(beta));
      ka[0] = w[0]; ka[1] = w[1]; ka[2] = w[2]; ka[3] = w[3];
      const int sc = beta < 4 ? static_cast<int>(ksc0) : static_cast<int>(ksc1);
      S[beta] = qk_block(ka, sc, beta);
    }
  };
  auto chunk_lag = [&](float m0, float m1) {
    // O and L stay expressed against a lagging reference m_o <= m0: each
    // tile's contribution is scaled by 2^(m_t - m_o) through the E8M0 scale
    // of its P blocks, so O is only rescaled when the gap grows large
    if (m_o == NEG_INF) m_o = m0;
    if (__any(m1 - m_o > kMaxLag)) rebase(m1);
  };
  // P = E4M3(2^xq) of one S block (4 scores per lane -> 4 bytes)
  auto p_block = [&](const v4f& s4, float off) -> int { return p4_e4m3(s4, c, off); };

  // ---- main loop over 128-key chunks.
  // Ring protocol: at the top of iteration ch the scale bytes of K chunk ch+2
  // and V chunk ch (loaded into registers in iteration ch-1) are written to
  // their buffers, each wave waits for its own copies issued up to iteration
  // ch-2, then one barrier publishes them; after it iteration ch issues K chunk
  // ch+3 and V chunk ch+1.  A K buffer is rewritten three iterations after the
  // QK MFMAs of its chunk, a V buffer two iterations after its PV MFMAs, both
  // past a barrier that every reader has passed.
  // Software pipeline, one step per chunk: S holds chunk ch's FP4 scores (its
  // QK MFMAs were issued in iteration ch-1).  Iteration ch turns them into P
  // blocks while the QK MFMAs of chunk ch+1 go into the registers just read
  // and the PV MFMAs of chunk ch-1 (the pending P) run beside them, so the
  // vector ALU and the matrix core always have independent work.  Chunks that
  // need masks, FP16 tiles or line keys first rewrite their S blocks (-inf where
  // a key adds nothing to the low-bit PV) and then take the same step.
  v4f S[8];
  float mxa = NEG_INF, mxb = NEG_INF;  // per-lane partial row maxima of S's two tiles
  float hm0 = 0.0f, hm1 = 0.0f;        // per-tile P references of chunk ch
  v8i pb_p = {0, 0, 0, 0, 0, 0, 0, 0};  // pending P (chunk ch-1); 0 adds nothing
  float hp0 = NEG_INF, hp1 = NEG_INF;  // its per-tile references
  // chunks [0, hot_end) have both tiles valid and need no mask for this wave:
  // no padded key, no key past the wave's first row, no padded query row
  int hot_end = (last_tile + 1) >> 1;
  hot_end = min(hot_end, a.n_valid >> 7);
  if (a.causal) hot_end = min(hot_end, (wq_lo + 1) >> 7);
  if (qe < qs + BQ - 1) hot_end = 0;
  hot_end = __builtin_amdgcn_readfirstlane(hot_end);
  auto is_hot = [&](int ch, int fl) -> bool {
    return ch < hot_end && !((fl >> 2) & 3) && !(LINES && (fl & 64));
  };
  // E8M0 scale of the pending P: 2^-8 * 2^(m_t - m_o), taken when it is
  // applied (after any rebase since it was formed); below 2^-127 the tile adds
  // nothing visible, and a tile with no valid key for this row adds nothing
  auto pend_scale = [&]() -> int {
    const float mt = g < 2 ? hp0 : hp1;
    if (mt == NEG_INF || m_o == NEG_INF) return 0;
    return static_cast<int>(fminf(fmaxf(static_cast<float>(kPScale) + (mt - m_o), 0.0f), 254.0f));
  };
  // partial maxima of S block beta (tile beta / 4)
  auto s_max = [&](int beta) {
    float& mx = beta < 4 ? mxa : mxb;
    mx = max3f(mx, S[beta][0], S[beta][1]);
    mx = max3f(mx, S[beta][2], S[beta][3]);
  };
  // One pipeline step (see above).  Issue order, fixed with scheduling
  // barriers, per S block: the K fragment two blocks ahead, the block's
  // exponentials, its QK MFMA for the next chunk, every 8/NDB blocks one PV
  // MFMA of the pending chunk (V fragments one head_dim block ahead), and the
  // partial maxima of the block whose QK MFMA was issued three blocks before.
  // The exponentials of a block run only where some of its P can be nonzero:
  // in a live tile (see tile_live), and there only for the 16-key blocks whose
  // largest score passes the same exact test (a block of zero P costs one
  // maximum, one FMA and a compare); every other block's P is 0.
  // Variants of the step: PV, the pending chunk had a live tile, so its PV
  // MFMAs and their V reads run; the choice is one scalar branch per chunk.
  // kpre: the first two K fragments, read by the caller after the barrier.
  bool live0 = true, live1 = true;  // tiles of chunk ch with a nonzero low-bit P (this wave)
  auto pipe = [&](auto PVc, const uint8_t* kbn, const uint8_t* vbp, int pscp, v8i& pb, auto&& copies,
                  const v4i (&kpre)[2]) {
    constexpr bool PV = decltype(PVc)::value;
    float off0 = kGridMagic + kExpOffset - (hm0 == NEG_INF ? 0.0f : hm0);
    float off1 = kGridMagic + kExpOffset - (hm1 == NEG_INF ? 0.0f : hm1);
    // opaque from here on: the exponentials cannot be moved out of this step
    // (the compiler would otherwise compute them where the references are set)
    __asm__ volatile("" : "+v"(off0), "+v"(off1));
    const uint32_t* ksw = reinterpret_cast<const uint32_t*>(kbn + ksoff);
    const uint32_t nks0 = ksw[0], nks1 = ksw[1];
    uint32_t vsc0 = 0u, vsc1 = 0u;
    if constexpr (PV) {
      const uint32_t* vsw = reinterpret_cast<const uint32_t*>(vbp + vsoff);
      vsc0 = vsw[0];
      vsc1 = NDB > 4 ? vsw[1] : 0u;
    }
    constexpr int KAHEAD = 2;  // K fragments in flight ahead of their MFMA
    constexpr int SPB = 8 / NDB;  // S blocks per PV MFMA
    v4i kn[8];
    v8i va[NDB];
#pragma unroll
    for (int beta = 0; beta < KAHEAD; ++beta) kn[beta] = kpre[beta];
    if constexpr (PV) va[0] = vfrag(vbp, 0);
    mxa = NEG_INF;
    mxb = NEG_INF;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int beta = 0; beta < 8; ++beta) {
      if (beta + KAHEAD < 8) kn[beta + KAHEAD] = *reinterpret_cast<const v4i*>(kbn + koff(beta + KAHEAD));
      if (beta == 1) copies();  // this iteration's copies, among the step's work
      {
        const float offb = beta < 4 ? off0 : off1;
        bool lvb = beta < 4 ? live0 : live1;
        if (lvb) {  // P = 0 for the whole block when its largest score gives y <= 6134 (see tile_live)
          const float m4 = fmaxf(max3f(S[beta][0], S[beta][1], S[beta][2]), S[beta][3]);
          lvb = __any(__builtin_fmaf(m4, c, offb) > kGridMagic - 10.0f);
        }
        if (lvb) pb[beta] = p_block(S[beta], offb);
        else pb[beta] = 0;
        __asm__ volatile("" ::"v"(pb[beta]));  // formed here, not where it is next read
      }
      const v8i ka = {kn[beta][0], kn[beta][1], kn[beta][2], kn[beta][3], 0, 0, 0, 0};
      S[beta] = qk_block(ka, beta < 4 ? static_cast<int>(nks0) : static_cast<int>(nks1), beta);
      if constexpr (PV) {
        if (beta % SPB == SPB - 1) {
          const int db = beta / SPB;
          if (db + 1 < NDB) va[db + 1] = vfrag(vbp, db + 1);
          O[db] = pv_block(va[db], pb_p, O[db], db < 4 ? static_cast<int>(vsc0) : static_cast<int>(vsc1), pscp, db);
        }
      }
      if (beta >= 3) s_max(beta - 3);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (PV) L = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones8, pb_p, L, 0, 0, 0, 127, 0, pscp);
    s_max(5);
    s_max(6);
    s_max(7);
  };
  // the pending chunk's PV on its own (after the last chunk)
  auto pv_flush = [&](const uint8_t* vbp, int pscp) {
    const uint32_t* vsw = reinterpret_cast<const uint32_t*>(vbp + vsoff);
    const uint32_t vsc0 = vsw[0], vsc1 = NDB > 4 ? vsw[1] : 0u;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      O[db] = pv_block(vfrag(vbp, db), pb_p, O[db], db < 4 ? static_cast<int>(vsc0) : static_cast<int>(vsc1), pscp, db);
    L = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones8, pb_p, L, 0, 0, 0, 127, 0, pscp);
  };

  // bf16 Q of this lane's row, head_dim elements 32 st + 8 g .. +7: the B
  // operand of the bf16 QK MFMAs of FP16 tiles and of the line tile
  v8bf qbr[NSB];
#pragma unroll
  for (int st = 0; st < NSB; ++st) qbr[st] = v8bf{};
  if (a.mode != MXQ_ALL_LOWBIT || LINES) {
#pragma unroll
    for (int st = 0; st < NSB; ++st)
      qbr[st] = *reinterpret_cast<const v8bf*>(a.q_bf16 + (bhq * a.N + q) * D + 8 * (4 * st + g));
  }
  // per chunk, the decoded flags (see chunk_flags) of the waves on mask row ra
  // in the low half and of those on row rb in the high half
  using FlagT = typename std::conditional<LINES, uint32_t, uint16_t>::type;
  constexpr int kFlShift = LINES ? 16 : 8;
  __shared__ FlagT s_fl[kMaxChunks];
  // per slot and lane group g: the group's line keys in the chunk, bit
  // 16t + (key & 15) for key = chunk start + 64t + 16g + (key & 15)
  __shared__ uint32_t s_lm[kMaxLines * 4];
  for (int ch = tid; ch < n_chunks; ch += NT) {
    int add = 0;
    if (LINES && n_line > 0) {
#pragma unroll
      for (int e = 0; e < kMaxLines; ++e) {
        const int key = __builtin_amdgcn_readlane(lkey, e);
        if (key >= 0 && (key >> 7) == ch) add = 16 | (__builtin_amdgcn_readlane(lslot, e) << 8);
      }
    }
    const uint32_t wa = ch == tid ? mw_a : mask_word(mrow_a, ch);
    const uint32_t wb = ch == tid ? mw_b : mask_word(mrow_b, ch);
    // bits 0-1 this wave's promoted tiles, 2-3 any wave's, 4-5 every wave's,
    // 6 a line key in the chunk, 8-11 the chunk's line slot
    const int fa = row_flags(wa, ch), fb = row_flags(wb, ch);
    const int common = ((fa | fb) << 2) | ((fa & fb) << 4) | ((add & 16) << 2) | (add & 0xF00);
    s_fl[ch] = static_cast<FlagT>((fa | common) | ((fb | common) << kFlShift));
  }
  // the line tile's keys: entries 4g..4g+3 of this lane's rows
  int lkey4[4] = {-1, -1, -1, -1};
  if constexpr (LINES) {
#pragma unroll
    for (int i = 0; i < 4; ++i) lkey4[i] = lane_key(4 * g + i);
  }
  if (LINES && n_line > 0) {
    if (wave == 0) {
      uint32_t m = 0;
#pragma unroll
      for (int e = 0; e < kMaxLines; ++e) {
        const int key = __builtin_amdgcn_readlane(lkey, e);
        const int sl = __builtin_amdgcn_readlane(lslot, e);
        if (key >= 0 && sl == (lane >> 2) && ((key >> 4) & 3) == (lane & 3))
          m |= 1u << ((((key & 127) >> 6) << 4) | (key & 15));
      }
      s_lm[lane] = m;
    }
    // the gathered line rows (loaded in the prologue) -> LDS
    if (tid < LU) *reinterpret_cast<v4i*>(sm + LY::lk_off(ke, kcu)) = kw;
    if (tid < LV)
      *reinterpret_cast<uint2*>(sm + LY::LV_OFF + (vd * kMaxLines + ve0) * 2) =
          make_uint2(line_v_f16(hv[0], lv_bf16) | (line_v_f16(hv[1], lv_bf16) << 16),
                     line_v_f16(hv[2], lv_bf16) | (line_v_f16(hv[3], lv_bf16) << 16));
  }
  // this wave's half of a chunk's flags
  const int fl_shift = w_in_b ? kFlShift : 0;
  auto fl_decode = [&](int raw) -> int {
    return (__builtin_amdgcn_readfirstlane(raw) >> fl_shift) & ((1 << kFlShift) - 1);
  };
  auto chunk_flags = [&](int ch) -> int { return fl_decode(static_cast<int>(s_fl[ch])); };

  if (lowbit) {
    pks = pks0;
    ks_store(kbuf(0));
    pks = pks1;
    ks_store(kbuf(1));
    // the first pipeline step runs the PV MFMAs of a pending chunk that does
    // not exist yet (P = 0) on V buffer RV-1, which no copy fills before
    // iteration 1: zero codes and scales there, since bytes left in LDS by an
    // earlier kernel may be E4M3 or E8M0 NaNs, and 0 * NaN would poison O
    for (int i = tid; i < LY::V_BYTES / 16; i += NT)
      reinterpret_cast<v4i*>(vbuf(LY::RV - 1))[i] = v4i{0, 0, 0, 0};
  } else {
    // no low-bit operands: the rings are never filled, yet every chunk's
    // pipeline step runs its QK and PV MFMAs (with P = 0); zero codes and
    // scales keep them finite so that they add exactly 0
    for (int i = tid; i < (LY::RK * LY::K_BYTES + LY::RV * LY::V_BYTES) / 16; i += NT)
      reinterpret_cast<v4i*>(kring)[i] = v4i{0, 0, 0, 0};
  }
  // the Q fragment is used in every chunk: wait for it here, once
  asm volatile("" ::"v"(qsc), "v"(qf4[0]), "v"(qf4[1]), "v"(qf4[2]), "v"(qf4[3]));
#pragma unroll
  for (int st = 0; st < NSB; ++st) asm volatile("" ::"v"(qbr[st]));
  __syncthreads();  // s_fl and the constant LDS words are written
  int f_cur = chunk_flags(0);
  int f_nxt = n_chunks > 1 ? chunk_flags(1) : 0;
  // chunk ch+2's flags word, read from LDS one iteration before it is decoded
  // (so that no iteration waits for that read); entries past the chunks are
  // never decoded
  int fl_raw = static_cast<int>(s_fl[min(2, kMaxChunks - 1)]);

  // Staging schedule (K ring of 4, V ring of 3, one barrier per chunk).
  // Iteration ch issues (in this order): after its barrier, the FP16 tile of
  // chunk ch or ch+1 when one is due (below); from inside its step, the K and
  // V scale loads into registers, the K codes of chunk ch+3 and the V codes of
  // chunk ch+1.  At the top of iteration ch+1 the scales are written to LDS
  // and each wave waits until at most kRegOps of its loads are in flight,
  // i.e. everything issued before iteration ch's scale loads has landed: the
  // K codes of chunk ch+2, the V codes of chunk ch and any FP16 tile issued
  // in iteration ch.  The barrier then publishes them to all waves.  A K
  // buffer is rewritten three iterations after its chunk was last read, a V
  // buffer two, both after a barrier that every reader has passed.
  // Workgroup barrier without the memory fence __syncthreads() carries (that
  // fence waits for every load in flight, copies for later chunks included):
  // this wave's LDS writes are complete, then s_barrier.  Copies are waited
  // for explicitly before it.
  auto lds_barrier = []() {
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // FP16 tiles of chunk 0, then iteration -1's regular loads
  int hi_rdy = 0;  // bit t: stage t holds chunk ch's tile t
  issue_fence();
#pragma unroll
  for (int t = 0; t < 2; ++t)
    if ((f_cur >> (2 + t)) & 1) {
      fp16_dma(64 * t, t);
      hi_rdy |= 1 << t;
    }
  issue_fence();
  if (lowbit) {
    ks_load(2);
    vs_load(0);
    k_dma(2, kbuf(2));
    v_dma(0, vbuf(0));
  }
  if (LINES && n_line > 0) {
    // ---- the vertical-line tile, first in the reference order: S^T[16
    // entries x 16 queries] = K_lines . Q^T (bf16, exact in fp16), lane (col,
    // g) holding entries 4g..4g+3 of query col, which is also the P^T operand
    // layout of the 16x16x16 fp16 MFMA that adds V_lines^T P^T to O^T
    v4f SL = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < NSB; ++st) {
      const v8bf ka = *reinterpret_cast<const v8bf*>(sm + LY::lk_off(col, 4 * st + g));
      SL = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qbr[st], SL, 0, 0, 0);
    }
    float mx = NEG_INF;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = lkey4[i];
      const bool ok = key >= 0 && q < a.n_valid && (!a.causal || key <= q);
      if (!ok) SL[i] = NEG_INF;
      mx = fmaxf(mx, SL[i]);
    }
    mx = rowmax4(mx);
    m_run = ceilf(mx * c);  // -inf when the row sees no line
    m_o = m_run;
    const float m_ref = m_run == NEG_INF ? 0.0f : m_run;
    v4h ph;
#pragma unroll
    for (int i = 0; i < 4; ++i) ph[i] = static_cast<_Float16>(__builtin_amdgcn_exp2f(__builtin_fmaf(SL[i], c, -m_ref)));
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const v4h va = *reinterpret_cast<const v4h*>(sm + LY::LV_OFF + ((16 * db + col) * kMaxLines + 4 * g) * 2);
      O[db] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, ph, O[db], 0, 0, 0);
    }
    const v4h ones4 = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f),
                       static_cast<_Float16>(1.0f)};
    L = __builtin_amdgcn_mfma_f32_16x16x16f16(ones4, ph, L, 0, 0, 0);
  }
  // integer tile references of an unmasked all-low-bit chunk from the partial
  // maxima of its scores; O's reference follows when it lags too far
  // A tile is live for this wave when some row's low-bit P there can be
  // nonzero: P = E4M3(2^x) is 0 exactly when x = fl32(S*c + off) - 6144 <= -10
  // (2^-10 is the tie between 0 and the smallest subnormal), and the fused
  // multiply-add is monotonic in S, so the row maximum decides for the row.
  auto tile_live = [&](float rmax, float href) -> bool {
    const float off = kGridMagic + kExpOffset - (href == NEG_INF ? 0.0f : href);
    return __any(__builtin_fmaf(rmax, c, off) > kGridMagic - 10.0f);
  };
  bool pend_live = false;           // the pending chunk has a live tile
  // integer tile references of an unmasked all-low-bit chunk from the partial
  // maxima of its scores; O's reference follows when it lags too far
  auto hot_refs = [&]() {
    float ra, rb;
    rowmax4x2(mxa, mxb, ra, rb);
    hm0 = fmaxf(m_run, ceilf(ra * c));
    hm1 = fmaxf(hm0, ceilf(rb * c));
    m_run = hm1;
    chunk_lag(hm0, hm1);
    live0 = tile_live(ra, hm0);
    live1 = tile_live(rb, hm1);
  };
  int vslot = 0;    // V buffer of chunk ch
  int vslot_p = LY::RV - 1;  // V buffer of the pending chunk (none yet: P = 0 over the zeroed buffer)
  if (lowbit) {     // chunk 0's FP4 scores (K chunks 0 and 1 are in place)
    qk_lowbit(kbuf(0), S);
#pragma unroll
    for (int beta = 0; beta < 8; ++beta) s_max(beta);
  } else {          // every tile is FP16 and rewrites its blocks
#pragma unroll
    for (int beta = 0; beta < 8; ++beta) S[beta] = v4f{NEG_INF, NEG_INF, NEG_INF, NEG_INF};
  }

  for (int ch = 0; ch < n_chunks; ++ch) {
    const int kc = ch * 128;
    const bool valid1 = 2 * ch + 1 <= last_tile;
    const int vslot1 = vslot == LY::RV - 1 ? 0 : vslot + 1;
    const int f_nn = ch + 2 < n_chunks ? fl_decode(fl_raw) : 0;
    fl_raw = static_cast<int>(s_fl[min(ch + 3, kMaxChunks - 1)]);
    if (lowbit) {
      ks_store(kbuf(ch + 2));
      vs_store(vbuf(vslot));
      __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(kRegOps) : "memory");
    } else {
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    lds_barrier();
    // FP16 tile issue, stage t for tile t: chunk ch's promoted tiles not staged
    // yet, and chunk ch+1's where chunk ch leaves the stage alone (a stage's
    // previous users finished before this barrier)
    // (the flags promote no tile when there are no FP16 operands; f_nxt is 0
    // past the last chunk)
    const int pc = (f_cur >> 2) & 3;
    const int hi_now = pc & ~hi_rdy;                  // issued just now: waited for before use
    const int hi_rdy_next = ((f_nxt >> 2) & 3) & ~pc;  // prefetched for chunk ch+1
    if (hi_now | hi_rdy_next) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if ((hi_now >> t) & 1) fp16_dma(kc + 64 * t, t);
        else if ((hi_rdy_next >> t) & 1) fp16_dma(kc + 128 + 64 * t, t);
      }
    }
    issue_fence();
    // the step's first K fragments (chunk ch+1, published by this barrier),
    // read now so that their latency overlaps what follows
    v4i kpre[2];
#pragma unroll
    for (int beta = 0; beta < 2; ++beta) kpre[beta] = *reinterpret_cast<const v4i*>(kbuf(ch + 1) + koff(beta));
    // an unmasked all-low-bit chunk: its integer tile references from the
    // partial maxima of its scores (issued in the previous step), computed
    // after the barrier (the previous chunk's PV is done, so a rebase of O
    // stays between two PV updates)
    if (is_hot(ch, f_cur)) hot_refs();
    // this iteration's copies (scale loads, K codes of chunk ch+3, V codes of
    // chunk ch+1), issued in this order from inside the step, so that their
    // issue overlaps its arithmetic instead of following the barrier
    auto copies = [&]() {
      if (lowbit) {
        ks_load(ch + 3);
        vs_load(ch + 1);
        k_dma(ch + 3, kbuf(ch + 3));
        v_dma(ch + 1, vbuf(vslot1));
      }
    };

    if (!is_hot(ch, f_cur)) {
      // (a chunk with both tiles low-bit for every wave and no masks had its
      // tile references set at the end of the previous iteration)
      // ================= masks, FP16 tiles, line keys, a lone last tile: the
      // S blocks are rewritten tile by tile (masked keys and FP16 tiles -inf)
      const bool need_mask = (kc + 127 >= a.n_valid) || (a.causal && kc + 127 > wq_lo) || (qe < qs + BQ - 1);
      const bool has_line = LINES && (f_cur & 64);  // line keys run in the line tile, not here
      const bool low_w = !(f_cur & 1) || (valid1 && !(f_cur & 2));  // this wave runs FP8 PV
      float m_tile0 = NEG_INF;
      float low0 = NEG_INF, low1 = NEG_INF;  // row maxima of the low-bit scores left in each tile
      if (hi_now) {  // FP16 tiles issued after this chunk's barrier: let them land, then publish
        // (a chunk with a promoted tile is masked-path for every wave; the
        // tiles are the last copies issued so far in this iteration)
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
      }
      // (both tiles in one unrolled body: the second tile's MFMAs and loads
      // overlap the first tile's softmax)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (t == 1 && !valid1) break;
        const bool prom = (f_cur >> t) & 1;  // this wave's tile t is FP16 (in stage t)
        uint8_t* const stg = sm + t * LY::STAGE;
        v4f St[4];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) St[bb] = t ? S[4 + bb] : S[bb];
        if (prom) {
#pragma unroll
          for (int st = 0; st < NSB; ++st) {
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
              const int key = 16 * (col >> 2) + 4 * bb + (col & 3);
              const v8bf ka = *reinterpret_cast<const v8bf*>(stg + LY::hk_off(key, 4 * st + g));
              St[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qbr[st], st == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : St[bb], 0, 0, 0);
            }
          }
        }
        if (need_mask) {
#pragma unroll
          for (int bb = 0; bb < 4; ++bb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = kc + 64 * t + 16 * g + 4 * bb + i;
              const bool ok = key < a.n_valid && q < a.n_valid && (!a.causal || key <= q);
              if (!ok) St[bb][i] = NEG_INF;
            }
        }
        if (has_line) {  // bit 4bb + i: key kc + 64t + 16g + 4bb + i is a line key
          const uint32_t lm = s_lm[4 * ((f_cur >> 8) & 15) + g] >> (16 * t);
#pragma unroll
          for (int bb = 0; bb < 4; ++bb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if ((lm >> (4 * bb + i)) & 1u) St[bb][i] = NEG_INF;
        }
        float mx = NEG_INF;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) mx = fmaxf(fmaxf(mx, fmaxf(St[bb][0], St[bb][1])), fmaxf(St[bb][2], St[bb][3]));
        mx = rowmax4(mx);
        const float m_t = fmaxf(m_run, ceilf(mx * c));
        m_run = m_t;
        if (t == 0) m_tile0 = m_t;
        if (!prom) {
          if (t == 0) low0 = mx;
          else low1 = mx;
        }
        if (prom) {
          // P relative to O's reference m_o <= m_t: the same fp16 values scaled
          // by 2^(m_t - m_o) (exact while normal), so O needs no rescale unless
          // the largest one, 2^(m_t - m_o), would leave fp16's range
          if (m_o == NEG_INF) m_o = m_t;
          else if (__any(m_t - m_o > kMaxLag16)) rebase(m_t);
          const float m_ref = m_o == NEG_INF ? 0.0f : m_o;
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            // 32 keys whose fp16 P is 0 for every row add nothing: skip their
            // exponentials and MFMAs.  fp16 rounds 2^x to 0 for x < -25, and
            // x <= -25.5 keeps v_exp_f32's error far from that tie
            const float m8 = fmaxf(fmaxf(max3f(St[2 * st][0], St[2 * st][1], St[2 * st][2]),
                                         max3f(St[2 * st][3], St[2 * st + 1][0], St[2 * st + 1][1])),
                                   fmaxf(St[2 * st + 1][2], St[2 * st + 1][3]));
            if (!__any(__builtin_fmaf(m8, c, -m_ref) > -25.5f)) continue;
            v8h ph;
#pragma unroll
            for (int e = 0; e < 8; ++e)
              ph[e] = static_cast<_Float16>(__builtin_amdgcn_exp2f(__builtin_fmaf(St[2 * st + (e >> 2)][e & 3], c, -m_ref)));
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
              const v8h va = *reinterpret_cast<const v8h*>(stg + LY::HV_OFF + LY::hvrow_off(16 * db + col, 2 * g + st));
              O[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, ph, O[db], 0, 0, 0);
            }
            const v8h ones16 = __builtin_bit_cast(v8h, v4i{kOne16, kOne16, kOne16, kOne16});
            L = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones16, ph, L, 0, 0, 0);
          }
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) St[bb] = v4f{NEG_INF, NEG_INF, NEG_INF, NEG_INF};  // no low-bit P
        }
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          if (t) S[4 + bb] = St[bb];
          else S[bb] = St[bb];
        }
      }
      if (!valid1) {  // a lone last tile: the second one adds nothing
#pragma unroll
        for (int bb = 4; bb < 8; ++bb) S[bb] = v4f{NEG_INF, NEG_INF, NEG_INF, NEG_INF};
      }
      // tile references of the low-bit P: each tile's running maximum
      hm0 = m_tile0;
      hm1 = m_run;
      live0 = tile_live(low0, hm0);
      live1 = tile_live(low1, hm1);
      if (low_w) {
        // as for unmasked chunks (the same reference choices, so a row's
        // result does not depend on which path its chunk took): each tile's
        // P enters through the E8M0 scale 2^-8 * 2^(m_t - m_o); O starts at
        // the first tile's reference and is rescaled when the lag grows large
        chunk_lag(m_tile0 == NEG_INF ? m_run : m_tile0, m_run);
      }
    }
    // ================= the pipeline step: P of chunk ch, QK of chunk ch+1, PV of chunk ch-1
    v8i pb;
    {
      const std::true_type T{};
      const std::false_type F{};
      const uint8_t* kbn = kbuf(ch + 1);
      const uint8_t* vbp = vbuf(vslot_p);
      // (one step with PV MFMAs, so that O has a single update site: two
      // would make the compiler copy O between register sets every chunk)
      if (pend_live) pipe(T, kbn, vbp, pend_scale(), pb, copies, kpre);
      else pipe(F, kbn, vbp, 0, pb, copies, kpre);
    }
    pb_p = pb;
    pend_live = live0 || live1;
    hp0 = hm0;
    hp1 = hm1;
    vslot_p = vslot;
    f_cur = f_nxt;
    f_nxt = f_nn;
    vslot = vslot1;
    hi_rdy = hi_rdy_next;
  }
  // no copy may still be landing when the workgroup's LDS is handed on; the
  // last chunk's V codes (copied in the previous iteration by every wave) are
  // published by this barrier for the last PV
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lds_barrier();
  if (pend_live) pv_flush(vbuf(vslot_p), pend_scale());

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
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + obase + d0) =
          make_uint2(bf16x2_rne(o0, o1), bf16x2_rne(o2, o3));
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
  if (a.n_lines > 0) hipLaunchKernelGGL((k_attn_mixed<D, true, 1>), dim3(n_qt, Hq, B), dim3(512), 0, st, a);
  else hipLaunchKernelGGL((k_attn_mixed<D, false, 1>), dim3(n_qt, Hq, B), dim3(512), 0, st, a);
  return check_launch("k_attn_mixed");
}

// one workgroup per (query tile of 128 / G rows, kv head, batch) serving the
// G query heads of the group
template <int D, int GH>
mxq_status launch_group(const AttnArgs& a, int Hkv, int B, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.n_qt), static_cast<unsigned>(Hkv), static_cast<unsigned>(B));
  if (a.n_lines > 0) hipLaunchKernelGGL((k_attn_mixed<D, true, GH>), grid, dim3(512), 0, st, a);
  else hipLaunchKernelGGL((k_attn_mixed<D, false, GH>), grid, dim3(512), 0, st, a);
  return check_launch("k_attn_mixed");
}

}  // namespace
}  // namespace attn
}  // namespace mxq


using namespace mxq;
using namespace mxq::attn;

extern "C" mxq_status attn_mixed_fwd(const uint8_t* q_codes, const uint8_t* q_scales,
                                     const uint8_t* k_codes, const uint8_t* k_scales,
                                     const uint8_t* v_codes, const uint8_t* v_scales,
                                     const uint16_t* q_bf16, const uint16_t* k_bf16,
                                     const uint16_t* v_f16t, const uint16_t* v_bf16, const uint32_t* mask,
                                     const int32_t* lines, int32_t n_lines,
                                     const mxq_attn_shape* s, float softmax_scale, mxq_mode mode,
                                     void* out, mxq_out_dtype out_dtype, float* lse,
                                     mxq_stream_t stream) {
  mxq_status st = validate_attn_shape(s);
  if (st != MXQ_OK) return st;
  const bool group_heads = (static_cast<int>(mode) & MXQ_GROUP_HEADS) != 0;
  mode = static_cast<mxq_mode>(static_cast<int>(mode) & ~MXQ_GROUP_HEADS);
  MXQ_REQUIRE(mode == MXQ_MIXED || mode == MXQ_ALL_LOWBIT || mode == MXQ_ALL_FP16, MXQ_EINVAL,
              "attn_mixed_fwd: bad mode");
  MXQ_REQUIRE(!group_heads || ((s->Hq / s->Hkv == 2 || s->Hq / s->Hkv == 4) && s->N > 256), MXQ_EUNSUPPORTED,
              "attn_mixed_fwd: MXQ_GROUP_HEADS needs Hq / Hkv in {2, 4} and N > 256");
  MXQ_REQUIRE(out_dtype == MXQ_OUT_F32 || out_dtype == MXQ_OUT_BF16, MXQ_EINVAL,
              "attn_mixed_fwd: bad out_dtype");
  MXQ_REQUIRE(out != nullptr, MXQ_EINVAL, "attn_mixed_fwd: out is NULL");
  const bool lowbit = mode != MXQ_ALL_FP16;
  MXQ_REQUIRE(!lowbit || (q_codes && q_scales && k_codes && k_scales && v_codes && v_scales),
              MXQ_EINVAL, "attn_mixed_fwd: low-bit operands are required in this mode");
  MXQ_REQUIRE(mode != MXQ_ALL_FP16 || (q_bf16 && k_bf16 && v_f16t), MXQ_EINVAL,
              "attn_mixed_fwd: bf16 Q/K and fp16 V^T are required in this mode");
  MXQ_REQUIRE(mode != MXQ_MIXED || (q_bf16 && k_bf16 && (v_f16t || v_bf16)), MXQ_EINVAL,
              "attn_mixed_fwd: bf16 Q/K and fp16 V^T (or, when no tile is promoted, bf16 V) are required in this mode");
  MXQ_REQUIRE(mode != MXQ_MIXED || mask != nullptr, MXQ_EINVAL, "attn_mixed_fwd: mask required in MIXED mode");
  MXQ_REQUIRE(n_lines >= 0 && n_lines <= kMaxLines, MXQ_EINVAL, "attn_mixed_fwd: n_lines must be in [0, 16]");
  MXQ_REQUIRE(n_lines == 0 || (lines && q_bf16 && k_bf16 && (v_f16t || v_bf16)), MXQ_EINVAL,
              "attn_mixed_fwd: vertical lines need lines, bf16 Q/K and fp16 V^T or bf16 V");
  MXQ_REQUIRE(!(softmax_scale != softmax_scale), MXQ_EINVAL, "attn_mixed_fwd: softmax_scale is NaN");
  double sc = softmax_scale > 0.0f ? static_cast<double>(softmax_scale) : 1.0 / __builtin_sqrt(static_cast<double>(s->D));
  AttnArgs a;
  a.q_codes = q_codes; a.q_scales = q_scales; a.k_codes = k_codes; a.k_scales = k_scales;
  a.v_codes = v_codes; a.v_scales = v_scales; a.q_bf16 = q_bf16; a.k_bf16 = k_bf16;
  a.v_f16t = v_f16t; a.v_bf16 = v_bf16; a.mask = mask; a.out = out; a.lse = lse;
  a.lines = lines; a.n_lines = n_lines;
  a.Hq = s->Hq; a.Hkv = s->Hkv; a.N = s->N; a.n_valid = s->n_valid; a.n_qt = s->N / s->Bq;
  a.words = (s->N / s->Bk + 31) / 32; a.causal = s->causal; a.mode = mode;
  a.out_bf16 = out_dtype == MXQ_OUT_BF16;
  a.sel_bq = s->Bq;
  a.nbh = 0;
  a.c = static_cast<float>(sc * 1.4426950408889634);
  hipStream_t strm = as_stream(stream);
  // 128-row workgroups of 8 waves whatever the selection tile height (the
  // mask row is looked up per row block); one workgroup per CU.
  const int n_qt = s->N / 128;
  a.n_qt = n_qt;
  // at most two 128-key chunks: small workgroups that stage the whole head
  if (s->N <= 256) {
    // one-dimensional grid: at most 2^21 heads x 4 query tiles x 256 threads
    MXQ_REQUIRE(static_cast<int64_t>(s->B) * s->Hq <= (1 << 21), MXQ_EUNSUPPORTED,
                "attn_mixed_fwd: at most 2^21 (batch, head) pairs when N <= 256");
    MXQ_REQUIRE((static_cast<int64_t>(s->B) * s->Hq + 8) * s->Hq <= (int64_t{1} << 32), MXQ_EUNSUPPORTED,
                "attn_mixed_fwd: (B * Hq + 8) * Hq must not exceed 2^32 when N <= 256");
    a.nbh = s->B * s->Hq;
    auto magic = [](int d) -> uint32_t {
      return d == 1 ? 0u : static_cast<uint32_t>(((int64_t{1} << 32) + d - 1) / d);
    };
    a.mg_nt = magic(s->N / 64);
    a.mg_hq = magic(s->Hq);
    a.mg_g = magic(s->Hq / s->Hkv);
    a.sel_shift = s->Bq == 128 ? 7 : 6;
    return launch_short(a, s->D, strm);
  }
  if (group_heads) {
    const int G = s->Hq / s->Hkv;
    a.n_qt = s->N / (128 / G);
    if (s->D == 128) return G == 2 ? launch_group<128, 2>(a, s->Hkv, s->B, strm) : launch_group<128, 4>(a, s->Hkv, s->B, strm);
    return G == 2 ? launch_group<64, 2>(a, s->Hkv, s->B, strm) : launch_group<64, 4>(a, s->Hkv, s->B, strm);
  }
  if (s->D == 128) return launch<128>(a, n_qt, s->Hq, s->B, strm);
  return launch<64>(a, n_qt, s->Hq, s->B, strm);
}
